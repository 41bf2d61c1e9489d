// Internal launch interface between the C ABI host code and the HIP kernels of libkvq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// consecutive pages of one (sequence, kv head, K|V) that one append wave processes
constexpr int kAppendPagesPerWave = 4;

struct AppendParams {
  uint8_t* pool;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* cu_new;
  const int32_t* start_pos;
  const int32_t* block_table;
  int32_t hkv;
  int32_t num_seqs;
  int32_t max_pages;
  int32_t max_new;
  const float* quat;   // had_block 4: unit quaternions [32][4] or [32][8] (quat_full)
  int32_t quat_full;
};

struct DecodePlan {
  int32_t pages_per_split;  // pages one workgroup handles (fixed splits)
  int32_t nsplit;           // workgroups per (sequence, kv head); the grid is units * nsplit
  int32_t waves;            // waves per workgroup
  int32_t depth;            // pages in flight per wave (register prefetch pipeline)
  // Balanced cut (narrow batches): the units are cut on the device, from seq_lens, into
  // near-equal pieces of at most C = max(ceil(total pages / slots), min_piece) pages; workgroup
  // k takes piece k.  units * nsplit >= slots + units covers every cut.
  int32_t balanced;
  int32_t slots;
  int32_t min_piece;
};

struct DecodeParams {
  uint8_t* pool;     // written only by the fused step (the appended token's bytes)
  const void* q;
  const int32_t* seq_lens;
  const int32_t* block_table;
  void* out;
  float* part_o;     // [units][nsplit][G][128] split partials (unnormalised o')
  float* part_ml;    // [units][nsplit][G][2]   running max (log2 domain) and sum
  uint32_t* counters;  // [units] runs finished; zero between calls (each call wraps it back)
  int32_t hkv;
  int32_t group;     // q heads per kv head (1..8)
  int32_t hq;
  int32_t num_seqs;
  int32_t max_pages;
  int32_t had_block;  // 1, 64, 128: Hadamard block width; 4: quaternion block rotation
  const float* quat;
  int32_t quat_full;
  int32_t q_dtype;
  int32_t out_dtype;
  int32_t out_rotated;
  float q_scale;
  float sm_scale_log2;  // sm_scale * log2(e)
  int32_t e8_shift;     // 23: see ue8m0_scale
  // fused step (append != 0): token seq_lens[b]-1 of every sequence is appended from
  // knew/vnew [num_seqs][hkv][128] (kv_dtype F16 or BF16) before it is attended
  const uint8_t* knew;
  const uint8_t* vnew;
  int32_t kv_dtype;
  int32_t append;
  DecodePlan plan;
};

struct PrefillParams {
  const uint8_t* pool;
  const void* q;             // [num_tokens][hq][128]
  const int32_t* cu_q;       // [num_seqs + 1]: chunk tokens of sequence b
  const int32_t* seq_lens;   // [num_seqs]: positions in the cache, the chunk included
  const int32_t* block_table;
  void* out;                 // [num_tokens][hq][128]
  int32_t hkv;
  int32_t group;
  int32_t hq;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_pages;
  int32_t had_block;  // 1, 64, 128: Hadamard block width; 4: quaternion block rotation
  const float* quat;
  int32_t quat_full;
  int32_t q_dtype;
  int32_t out_dtype;
  int32_t out_rotated;
  int32_t tiles;             // query tiles per (sequence, kv head)
  float q_scale;
  float sm_scale_log2;
  int32_t e8_shift;          // 23: see ue8m0_scale
};

struct DequantParams {
  const uint8_t* pool;
  const int32_t* page_ids;
  float* out_k;
  float* out_v;
  int32_t n;
  int32_t hkv;
  int32_t had_block;  // 1, 64, 128: Hadamard block width; 4: quaternion block rotation
  const float* quat;
  int32_t quat_full;
  int32_t unrotate;
  int32_t fmt;
};

// KVQ_DEBUG_CHECKS: validation of a call's device-side tables (kvq_check.hip)
enum CheckKind { kCheckAppend = 0, kCheckDecode = 1, kCheckPrefill = 2, kCheckDequant = 3 };
enum CheckCode { kCheckOk = 0, kBadSeqLen = 1, kBadPageId = 2, kBadCumulative = 3, kBadStartPos = 4, kBadChunk = 5 };
struct CheckParams {
  int32_t kind;
  const int32_t* cu;           // append: cu_new; prefill: cu_q
  const int32_t* start_pos;    // append
  const int32_t* seq_lens;     // decode, prefill
  const int32_t* block_table;  // append, decode, prefill
  const int32_t* page_ids;     // dequant
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_pages;
  int32_t max_len;             // decode / prefill: max_seq_len; append: max_new_tokens
  int32_t max_q_len;           // prefill
  int32_t n;                   // dequant: page ids
  int64_t num_pages;
};
// Runs the check on `stream` and waits for it: *code is a CheckCode, *index the sequence or page
// index of the first violation found.
hipError_t run_check(const CheckParams& c, hipStream_t stream, int* code, int* index);

hipError_t launch_append(const AppendParams& p, bool bf16, int had_block, int fmt, hipStream_t stream);
DecodePlan plan_decode(int num_seqs, int hkv, int max_seq_len);
// the decode workspace's counter region has room for this many (sequence, kv head) units for
// every call with at most that many, so such calls share one workspace layout
constexpr size_t kCounterUnits = 16384;
size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int hkv, int group);
void carve_workspace(void* ws, const DecodePlan& plan, int num_seqs, int hkv, int group, float** part_ml,
                     float** part_o, uint32_t** counters);
// variant: 0 INT4, 1 MXFP4, 2 MXFP4 with q.K and p.V on the scaled FP8 x FP4 matrix cores
hipError_t launch_decode(const DecodeParams& p, int variant, hipStream_t stream);
hipError_t launch_dequant(const DequantParams& p, hipStream_t stream);
int prefill_tokens_per_tile(int group);
hipError_t launch_prefill(const PrefillParams& p, int fmt, hipStream_t stream);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_fold4(const void* src, void* dst, size_t dst_bytes, hipStream_t stream);
hipError_t launch_append_pattern(const void* k, const void* v, const int32_t* block_table, void* pool, int hkv,
                                 int num_seqs, int new_tokens, int max_pages, int order, hipStream_t stream);
hipError_t launch_decode_pattern(const void* pool, const int32_t* block_table, int hkv, int num_seqs,
                                 int pages_per_seq, int max_pages, int waves, int depth, int pages_per_split,
                                 uint32_t* sink, hipStream_t stream);

}  // namespace kvq
