/*
 * kvq.h -- C ABI of libkvq: a rotated 4-bit paged KV cache for AMD MI355X (gfx950).
 *
 * The method (SAW-INT4 summary, aissential.tech, "Summary" and "Method"; UltraQuant
 * article, oracore.dev, section on how the method works):
 *   write path  every new K/V token vector is rotated by a block-diagonal Walsh-Hadamard
 *               matrix R_b = blockdiag(H_b / sqrt(b)), quantized token-wise to 4 bits and
 *               written into a paged cache through a block table (kvq_append);
 *   read path   decode attention reads the 4-bit pages back, dequantizes in registers and
 *               computes softmax(q'.K'^T) V' with q' = R_b q, rotating the result back
 *               (kvq_decode_attn).  An orthogonal R_b preserves q.k (IsoQuant abstract).
 * Two 4-bit formats: token-wise asymmetric INT4 with an fp16 scale and zero per vector,
 * and MXFP4 (e2m1 codes, one UE8M0 power-of-two scale per 32 channels, UltraQuant).
 * Alternative rotation stage: IsoQuant's quaternion block-4 rotation (had_block 4, below).
 * Also: chunked-prefill attention over the cache (kvq_prefill_attn), the write and read of a
 * decode step in one launch (kvq_decode_step), page dequantization (kvq_dequant_page).
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to device memory (hipMalloc / a torch
 *     CUDA tensor) owned by the caller; `cache` and scalars are host values.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only enqueued: the
 *     library never synchronizes and never allocates device memory, and apart from two
 *     documented exceptions (kvq_decode_step_noalloc's fixed scratch and the KVQ_DEBUG_CHECKS
 *     verdict slot, one of each per device) it keeps no mutable global state, so calls are
 *     thread-safe; calls on one stream run in order.
 *   - Host-side argument checks run before any HIP call and return a negative kvq_status;
 *     kvq_last_error() then names the argument.  Device-side data (token counts, sequence
 *     lengths, page ids) is trusted: out-of-range values are undefined behaviour -- except when
 *     the environment variable KVQ_DEBUG_CHECKS is set (not "0"; read on every call): each
 *     entry point then first validates its device tables on its stream (cu_new / cu_q
 *     non-decreasing within [0, num_tokens]; 1 <= seq_lens <= max_seq_len; chunks no longer
 *     than their sequence or max_q_len; start_pos >= 0 with the appended positions inside
 *     max_pages*16; every block-table entry or page id the call reads inside [0, num_pages)),
 *     waits for the verdict, and returns KVQ_ERR_INVALID_ARG naming the violation and its index
 *     instead of launching.  That wait synchronizes the stream: a debugging aid, not for graph
 *     capture.  The verdict lives in one slot per device, so checked calls on one device must
 *     not overlap in time (on other streams or threads).
 *   - A failed kernel launch returns KVQ_ERR_HIP with the HIP error text in kvq_last_error().
 *   - No C++ exception crosses this boundary.
 *
 * Cache geometry: head_dim 128, page 16 tokens.  One page-head block (one page, one
 * kv head) is 2176 bytes; the pool is uint8[num_pages][num_kv_heads][2176]:
 *   [0,1024)     K code rows: slot s at 64*s; row byte 4a+q (a=0..15, q=0..3) holds channel
 *                a+32q in its low nibble and channel a+32q+16 in its high nibble (channels
 *                of the rotated vector; row word a carries channel a+16i in nibble i).
 *   [1024,2048)  V code rows, same row bytes, interleaved by slot quads: byte j of slot s at
 *                1024 + 256*(s/4) + 4*j + (s%4).
 *   [2048,2112)  K parameters, slot s at 2048+4s;  [2112,2176) V parameters, same.
 *                INT4: fp16 scale then fp16 zero (little-endian); value = scale*code + zero.
 *                MXFP4: UE8M0 bytes of channel groups [0,32),[32,64),[64,96),[96,128);
 *                value = e2m1(code) * 2^(E-127); code bit 3 is the sign.
 * Only the bytes of appended slots are ever written.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 2
#define KVQ_HEAD_DIM 128
#define KVQ_PAGE_SIZE 16
#define KVQ_PAGE_HEAD_BYTES 2176

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent geometry       */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not implemented: head_dim, page size, dtype... */
  KVQ_ERR_WORKSPACE = -3,   /* decode workspace missing or smaller than required         */
  KVQ_ERR_HIP = -4          /* a HIP call (kernel launch) failed                          */
} kvq_status;

typedef enum { KVQ_FMT_INT4_TOKEN = 0, KVQ_FMT_MXFP4_G32 = 1 } kvq_format;

typedef enum { KVQ_F16 = 0, KVQ_BF16 = 1, KVQ_F32 = 2, KVQ_FP8_E4M3 = 3 } kvq_dtype;

/* kvq_decode_attn flags */
#define KVQ_OUT_ROTATED 1u /* leave the output in the rotated basis (skip the final R_b) */
#define KVQ_MX_SCALED_MFMA 2u /* MXFP4 caches: q.K and p.V on the scaled FP8 x FP4 matrix cores */
/* kvq_dequant_page flags */
#define KVQ_UNROTATE 1u    /* return R_b * y^ (the original basis) instead of y^          */

/* Description of one cache (one layer).  Host struct; `pool` is a device pointer. */
typedef struct {
  int32_t format;       /* kvq_format                                                     */
  int32_t num_kv_heads; /* >= 1                                                           */
  int32_t head_dim;     /* must be 128                                                    */
  int32_t page_size;    /* must be 16                                                     */
  int32_t had_block;    /* rotation before quantizing: Walsh-Hadamard block width b = 1   */
                        /* (no rotation, "plain INT4"), 64 or 128; or KVQ_ROT_QUAT4 (4):  */
                        /* the quaternion block-4 rotation below.  MXFP4 takes 128, 4, or */
                        /* 1 (for tests).                                                 */
  int32_t quat_full;    /* had_block 4: 0 = IsoQuant-Fast, 1 = IsoQuant-Full; else 0       */
  int64_t num_pages;    /* pages in the pool                                              */
  void* pool;           /* device uint8[num_pages][num_kv_heads][2176], 16-byte aligned   */
  const float* quat;    /* had_block 4: device fp32 unit quaternions (w, x, y, z), 16-byte */
                        /* aligned: [32][4] q_L (Fast) or [32][8] q_L, q_R (Full); else   */
                        /* NULL.  Channels 4k..4k+3 of a vector, as the quaternion v, are */
                        /* rotated to q_L v conj(q_R) (IsoQuant abstract: the isoclinic   */
                        /* decomposition of SO(4); Fast keeps the left factor, q_R = 1);  */
                        /* the way back is the transpose.  The caller draws them.         */
} kvq_cache;

#define KVQ_ROT_QUAT4 4

/* Version of this ABI (KVQ_ABI_VERSION). */
int kvq_abi_version(void);

/* Bytes of one page across all kv heads: num_kv_heads * 2176; 0 if `cache` is invalid. */
size_t kvq_page_bytes(const kvq_cache* cache);

/*
 * kvq_append -- fused rotate + 4-bit quantize + paged write of new K and V tokens.
 * (SAW-INT4 summary, "Summary": a fused rotation-quantization kernel writing directly into
 * paged KV-cache layouts.)
 *
 *   k, v         device, [num_tokens][num_kv_heads][128], dtype kv_dtype (KVQ_F16 or
 *                KVQ_BF16), contiguous, 16-byte aligned.
 *   cu_new       device int32[num_seqs+1], non-decreasing, cu_new[0] = 0 and
 *                cu_new[num_seqs] <= num_tokens: tokens cu_new[b]..cu_new[b+1]-1 belong to
 *                sequence b.
 *   start_pos    device int32[num_seqs]: position of sequence b's first new token.  Token i
 *                goes to position p = start_pos[b] + i - cu_new[b], i.e. page
 *                block_table[b*max_pages + p/16], slot p%16.
 *   block_table  device int32[num_seqs][max_pages]; entries used must be < num_pages.
 *   max_new_tokens  host hint: >= every cu_new[b+1]-cu_new[b] (sizes the grid); tokens
 *                beyond it are not written.
 * Writes each vector's 64 code bytes and 4 parameter bytes; nothing else in the pool.
 * Positions appended by one call must be distinct.
 */
int kvq_append(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
               int32_t num_tokens, int32_t num_seqs, const int32_t* cu_new,
               const int32_t* start_pos, const int32_t* block_table, int32_t max_pages,
               int32_t max_new_tokens, void* stream);

/*
 * Bytes of workspace kvq_decode_attn and kvq_decode_step need for these sizes (same
 * arguments as there).  No passage of the pages defines it: it is the storage of the split
 * form of the online softmax (per split, the running maximum, the running sum and the
 * unnormalised output of every query head), which a long sequence's decode uses to spread its
 * pages over several workgroups, and which the pages' decode attention implies only as an
 * implementation of the same softmax(q'.K'^T) V' result.  The workspace holds the partial results of (sequence, kv head) pairs
 * split over several workgroups and one counter per pair, which the last of a pair's
 * workgroups to finish uses to know that it merges the partials.  It must be zero-filled once
 * before its first use (e.g. hipMemset when it is allocated).  Every call leaves its counters
 * at zero again, and the counters have the same place for every call of at most 16384 (sequence,
 * kv head) pairs, so a workspace serves any number of later such calls, of any sizes that fit
 * it, without being cleared.  Clear it again before a call with more pairs than that if it
 * served smaller calls, and after a call that did not run to completion (a launch error).
 * Returns 0 when no workspace is needed (then `workspace` may be NULL), or (size_t)-1 on
 * invalid arguments.
 */
size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t num_q_heads,
                                  int32_t num_seqs, int32_t max_seq_len);

/*
 * kvq_decode_attn -- paged decode attention over the 4-bit cache, dequantizing in registers.
 * (SAW-INT4 summary, "Summary": attention served straight from the paged 4-bit cache;
 * UltraQuant: queries attend against FP4 KV tensors with group scales.)
 *
 *   q            device [num_seqs][num_q_heads][128], dtype q_dtype (F16, BF16, F32,
 *                FP8_E4M3), contiguous.  The kernel uses q_scale * q.
 *   num_q_heads  a multiple of num_kv_heads, with group G = num_q_heads/num_kv_heads <= 8;
 *                query head h reads kv head h / G.
 *   seq_lens     device int32[num_seqs]: tokens attended, positions [0, seq_lens[b]);
 *                1 <= seq_lens[b] <= max_seq_len.
 *   max_seq_len  host hint used to size the grid; must be <= max_pages*16.
 *   sm_scale     softmax scale (1/sqrt(128) is the usual value).
 *   out          device [num_seqs][num_q_heads][128], dtype out_dtype (F32, F16, BF16):
 *                o = R^T sum_t softmax_t(sm_scale * q'.k^'_t) v^'_t (q' = R q; R^T = R_b for
 *                the Hadamard rotation), or the rotated-basis
 *                result with KVQ_OUT_ROTATED.
 *   flags        KVQ_OUT_ROTATED (above) and, for MXFP4 caches only, KVQ_MX_SCALED_MFMA: both
 *                contractions then run on the scaled FP8 x FP4 matrix cores straight on the
 *                stored e2m1 codes (UltraQuant article, section on how the method works: FP8
 *                queries, FP4 KV, UE8M0 group scales, native scaled MFMA on CDNA4).  q.K:
 *                v_mfma_scale_f32_16x16x128_f8f6f4 on the K codes and their UE8M0 bytes, q'
 *                carried as three MXFP8 limbs.  p.V: v_mfma_scale_f32_32x32x64_f8f6f4 on the V
 *                codes, 64 tokens and one 32-channel group per product, with the attention
 *                weights FP8-quantized: p times the token's V group scale as three e4m3 limbs,
 *                one UE8M0 scale per 32 tokens.  The default (fp16 tiles) is the faster one and
 *                the more exact: a scaled MFMA sums its products to about 2^-14.5 of the largest
 *                one (measured), so the scores carry an error that grows with
 *                sm_scale * max|q'_i k'_i|; the row error stays within 2e-3 up to about 50 for
 *                that product.  The default path dequantizes K and V of an MXFP4 cache into fp16
 *                tiles, so their values must stay below 65504 in magnitude; the scaled path has
 *                no such limit.  KVQ_ERR_UNSUPPORTED on an INT4 cache; any other bit is
 *                KVQ_ERR_INVALID_ARG.
 *   workspace    device, >= kvq_decode_workspace_bytes(...) bytes, 256-byte aligned; calls
 *                that overlap in time (other streams) need workspaces of their own.
 * Decode does not append: a decode step is kvq_append then kvq_decode_attn on one stream, or
 * kvq_decode_step.
 */
int kvq_decode_attn(const kvq_cache* cache, const void* q, int32_t q_dtype, float q_scale,
                    int32_t num_q_heads, int32_t num_seqs, const int32_t* seq_lens,
                    int32_t max_seq_len, const int32_t* block_table, int32_t max_pages,
                    float sm_scale, void* out, int32_t out_dtype, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_decode_step -- one decode step in one launch: append then attend.
 * (SAW-INT4 summary, "Summary": the fused rotation-quantization write into the paged layout;
 * both halves of the method in a single pass over the cache.)
 *
 * Same result as kvq_append(cache, k, v, kv_dtype, num_seqs, num_seqs, cu_new = 0..num_seqs,
 * start_pos = seq_lens - 1, block_table, max_pages, 1) followed by kvq_decode_attn(...) with
 * the remaining arguments, up to the rounding of the rotation (a butterfly here, a matrix
 * product there; both fp32, so an appended code may differ where its pre-rounding value lies
 * within a few 1e-6 of a rounding boundary).
 *   k, v         device [num_seqs][num_kv_heads][128], dtype kv_dtype (KVQ_F16 or KVQ_BF16):
 *                the new token of every sequence, written at position seq_lens[b] - 1
 *                (page block_table[b*max_pages + (seq_lens[b]-1)/16], slot (seq_lens[b]-1)%16).
 *   seq_lens     device int32[num_seqs], >= 1: tokens attended, including the new one.
 * All other arguments and the workspace are those of kvq_decode_attn.  The new token's
 * bytes are the only pool bytes written.
 */
int kvq_decode_step(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
                    const void* q, int32_t q_dtype, float q_scale, int32_t num_q_heads,
                    int32_t num_seqs, const int32_t* seq_lens, int32_t max_seq_len,
                    const int32_t* block_table, int32_t max_pages, float sm_scale, void* out,
                    int32_t out_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * kvq_decode_step_noalloc -- kvq_decode_step without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It allocates nothing.  The split-run partials and merge counters live in a
 * fixed scratch array inside the library, 16 MiB per device, held by every device the library
 * runs on until the process ends.
 *
 * Arguments and result are those of kvq_decode_step without `workspace` / `workspace_bytes`;
 * the same kernels run.  `stream` must belong to the current device.
 * Limits: at most 16384 (sequence, kv head) pairs, and a call whose kvq_decode_workspace_bytes
 * exceeds 16 MiB (16777216 bytes) returns KVQ_ERR_WORKSPACE before any HIP call.
 * The first call on a device looks the scratch up and clears its merge counters with a kernel on
 * `stream` (a clear recorded into a graph under capture is repeated by later calls until one runs
 * eagerly); every call that runs to completion leaves them at zero again.
 * All calls on one device share that device's scratch: calls that overlap in time on one device
 * (other streams, other threads, concurrent graph replays) race and give wrong results.
 */
int kvq_decode_step_noalloc(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
                            const void* q, int32_t q_dtype, float q_scale, int32_t num_q_heads,
                            int32_t num_seqs, const int32_t* seq_lens, int32_t max_seq_len,
                            const int32_t* block_table, int32_t max_pages, float sm_scale, void* out,
                            int32_t out_dtype, uint32_t flags, void* stream);

/*
 * kvq_prefill_attn -- chunked-prefill attention over the 4-bit cache: the new tokens of a turn
 * attend over the resident prefix and, causally, over each other.
 * (UltraQuant article, section on what it showed: prefixes kept resident in the 4-bit cache
 * spare the re-prefill of later turns; SAW-INT4 summary, "Summary": attention served from the
 * paged 4-bit cache.)
 *
 *   q            device [num_tokens][num_q_heads][128], dtype q_dtype (F16, BF16, F32,
 *                FP8_E4M3); the kernel uses q_scale * q.
 *   num_q_heads  as for kvq_decode_attn (G = num_q_heads/num_kv_heads <= 8).
 *   cu_q         device int32[num_seqs+1], non-decreasing, cu_q[0] = 0, cu_q[num_seqs] <=
 *                num_tokens: tokens cu_q[b] .. cu_q[b+1]-1 are the chunk of sequence b.
 *   seq_lens     device int32[num_seqs]: positions in the cache, the chunk included (the
 *                chunk's K/V must already be appended): chunk token j of sequence b sits at
 *                position seq_lens[b] - (cu_q[b+1]-cu_q[b]) + j and attends positions 0 .. that.
 *   max_seq_len  host hint >= every seq_lens[b], <= max_pages*16 and <= 131072.
 *   max_q_len    host hint >= every cu_q[b+1]-cu_q[b] (sizes the grid).
 *   out          device [num_tokens][num_q_heads][128], dtype out_dtype (F32, F16, BF16); rows
 *                of tokens outside every chunk are not written.
 *   flags        0 or KVQ_OUT_ROTATED, as for kvq_decode_attn.
 * Needs no workspace and writes nothing but `out`.
 */
int kvq_prefill_attn(const kvq_cache* cache, const void* q, int32_t q_dtype, float q_scale,
                     int32_t num_q_heads, int32_t num_tokens, int32_t num_seqs,
                     const int32_t* cu_q, const int32_t* seq_lens, int32_t max_seq_len,
                     int32_t max_q_len, const int32_t* block_table, int32_t max_pages,
                     float sm_scale, void* out, int32_t out_dtype, uint32_t flags, void* stream);

/*
 * kvq_dequant_page -- dequantize whole pages (all 16 slots, all kv heads) to fp32.
 * (SAW-INT4 summary, "Method": token-wise INT4 quantization -- read here as asymmetric, a
 * value being the vector's stored fp16 scale times the code plus its stored fp16 zero;
 * UltraQuant article, section on how the method works: FP4 KV elements with UE8M0 group
 * scales, a value being the e2m1 element times its group's power of two.  The rotation undone
 * with KVQ_UNROTATE is the block-diagonal Hadamard rotation of the SAW-INT4 "Method", or
 * IsoQuant's quaternion block rotation.)
 *   page_ids     device int32[n], each < num_pages.
 *   out_k, out_v device float[n][num_kv_heads][16][128]; channel order is natural.
 *   flags        0: values in the rotated basis (y^ = scale*code + zero, one fp32 rounding,
 *                or e2m1*2^(E-127) exactly); KVQ_UNROTATE: R^T y^, the original basis (R_b^T =
 *                R_b; for the quaternion rotation the transposed block matrices).
 * Slots never written hold whatever bytes the pool had.
 */
int kvq_dequant_page(const kvq_cache* cache, const int32_t* page_ids, int32_t n,
                     float* out_k, float* out_v, uint32_t flags, void* stream);

/* Static description of a kvq_status. */
const char* kvq_strerror(int status);

/* Detail of the last error on the calling thread (empty string if none). */
const char* kvq_last_error(void);

/*
 * kvq_hbm_copy -- plain device-to-device copy kernel (16-byte vector loads and stores).
 * Not part of the method: it measures achievable HBM bandwidth and calibrates memory
 * traffic counters.  bytes must be a multiple of 16; src and dst 16-byte aligned.
 */
int kvq_hbm_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * kvq_hbm_read -- read-only streaming kernel: every 16-byte vector of src is loaded once and
 * XORed into its workgroup's 32-bit word.  Not part of the method: it measures the achievable
 * HBM read bandwidth, the ceiling of decode attention (which only reads the cache).
 * src: device, 16-byte aligned, bytes a multiple of 16.  sink: device uint32[4096], 4-byte
 * aligned; the call writes words [0, w) with w <= 2048 and leaves the rest as they are, so that
 * after a call on a zeroed sink the XOR of all 4096 words equals the XOR of all 32-bit words of
 * src.  bytes == 0 writes nothing and returns KVQ_OK.
 */
int kvq_hbm_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * kvq_hbm_fold4 -- a 4:1 read:write streaming kernel over 16-byte vectors in groups of 256
 * output vectors: dst vector 256 m + t = XOR of src vectors 1024 m + t + 256 k, k = 0..3.  Not
 * part of the method: it measures the HBM bandwidth of a contiguous stream with the append's
 * read:write mix (about 3.8:1 for bf16 in, 4-bit out), its ceiling.
 * src: device, 4 * dst_bytes bytes; dst: device, dst_bytes bytes (a multiple of 4096); both
 * 16-byte aligned, not overlapping.  dst_bytes == 0 writes nothing and returns KVQ_OK.
 */
int kvq_hbm_fold4(const void* src, void* dst, size_t dst_bytes, void* stream);

/*
 * kvq_hbm_append_pattern -- the memory traffic of kvq_append without its arithmetic.  Not part
 * of the method: it measures what the append's access pattern allows (the caller's K and V rows
 * read per kv head, 16 tokens per page, the page-head blocks written through the block table),
 * with the same waves, lane map and cache policies as the append.
 * k, v: device [num_seqs * new_tokens][num_kv_heads][128] 2-byte elements, sequence b's tokens
 * at rows b * new_tokens ..; block_table: device int32 [num_seqs][max_pages] (page ids trusted,
 * as for kvq_append); pool: device [pages][num_kv_heads][2176].  k, v and pool 16-byte aligned;
 * new_tokens a multiple of 16, at most 16 * max_pages; 1 <= num_kv_heads <= 1024.
 * Written, for sequence b, kv head h, page p = block_table[b][j] (j < new_tokens / 16), token
 * slot n (0..15) and g = 0..3, with X = the XOR of the 16-byte words at bytes 16 g + 64 i
 * (i = 0..3) of the row of token 16 j + n:  K: X at byte 64 n + 16 g of the page-head block
 * and its first 32-bit word at 2048 + 4 n (g = 0 only); V: X at 1024 + 256 (n / 4) + 64 g +
 * 16 (n % 4) and the first word at 2112 + 4 n.  Nothing else is written.
 * order 0: the append's own order (one wave per (sequence, kv head, K|V) and run of 4 pages, four
 * such waves per workgroup); order 1: one workgroup per (sequence, page) holding a wave per
 * (K|V, kv head), which reads the page's token rows of all kv heads together and writes all of
 * its head blocks (at most 8 kv heads, else KVQ_ERR_UNSUPPORTED).  Both write the same bytes.
 * order 2: as order 1, with the pages written in the order of their ids: block_table is then a
 * list of exactly num_seqs * P items (P = new_tokens / 16, so max_pages must equal P, else
 * KVQ_ERR_INVALID_ARG), and workgroup i (launched as order 1 launches the i-th (sequence, page)
 * in row-major order) takes item e = block_table[i] (0 <= e < num_seqs * P, trusted): it reads
 * the rows of sequence e / P's page e % P and writes them to page i, as order 1 would with that
 * page's table entry equal to i.  The pool must hold num_seqs * P pages.
 */
int kvq_hbm_append_pattern(const void* k, const void* v, int32_t num_kv_heads, int32_t num_seqs,
                           int32_t new_tokens, const int32_t* block_table, int32_t max_pages, void* pool,
                           uint32_t order, void* stream);

/*
 * kvq_hbm_decode_pattern -- the memory traffic of the decode's page stream without its arithmetic.
 * Not part of the method: it measures what the decode's access pattern allows (page-head blocks
 * gathered through the block table, each kv head's 17 KiB apart), with the workgroups, waves,
 * lane map, prefetch depth and cache policy of kvq_decode_attn's fixed-split plan.
 * pool: device [pages][num_kv_heads][2176] (only read; any format), 16-byte aligned;
 * block_table: device int32 [num_seqs][max_pages] (page ids trusted, as for kvq_decode_attn);
 * every sequence holds pages_per_seq full pages (1 <= pages_per_seq <= max_pages);
 * waves 4 or 8, depth 2, 3 or 4, 1 <= pages_per_split <= 64 * waves; 1 <= num_kv_heads <= 1024.
 * The grid has num_seqs * num_kv_heads * ceil(pages_per_seq / pages_per_split) workgroups in
 * split-major order (workgroup j: split j / (num_seqs * num_kv_heads), sequence and kv head from
 * j mod that, the kv head fastest); wave w of a workgroup streams pages p0 + w, p0 + w + waves, ..
 * of its split (p0 = split * pages_per_split).  Lane l (n = l % 16, g = l / 16) loads, from each
 * of those page-head blocks, the 16 bytes at 64 n + 16 g, the 16 bytes at 1024 + 16 l and the
 * 32-bit words at 2048 + 4 n and 2112 + 4 n.  sink: device uint32, one word per wave (index
 * waves * j + w): the sum mod 2^32 of every 32-bit word its lanes loaded.  Nothing else is
 * written.
 */
int kvq_hbm_decode_pattern(const void* pool, int32_t num_kv_heads, int32_t num_seqs, int32_t pages_per_seq,
                           const int32_t* block_table, int32_t max_pages, int32_t waves, int32_t depth,
                           int32_t pages_per_split, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
