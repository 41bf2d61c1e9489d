// C ABI of libkvq (declared in include/kvq.h): argument validation, launch planning, errors.
// Validation runs before any HIP call, so invalid calls fail the same way with or without a GPU.
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kvq_internal.h"

// Scratch of kvq_decode_step_noalloc: the split-run partials and merge counters that the other
// decode entry points keep in the caller's workspace.  One copy per device, held until the
// process ends.  Host code never passes this name to a kernel: it is a host-side stand-in, and
// the device address comes from hipGetSymbolAddress (scratch_for_device below).
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVQ_OK;
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Common cache checks.  Returns KVQ_OK or an error status (with the message set).
int check_cache(const kvq_cache* c) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (!c->pool) return fail(KVQ_ERR_INVALID_ARG, "cache->pool is NULL");
  if (c->num_kv_heads < 1) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", c->num_kv_heads);
  // the kernels address a page's 16 token rows through one 32-bit buffer range
  if (c->num_kv_heads > 1024) return fail(KVQ_ERR_UNSUPPORTED, "num_kv_heads %d above 1024", c->num_kv_heads);
  if (c->num_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "num_pages must be >= 1");

  if (c->head_dim != KVQ_HEAD_DIM) return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", c->head_dim);
  if (c->page_size != KVQ_PAGE_SIZE) return fail(KVQ_ERR_UNSUPPORTED, "page_size %d unsupported (only 16)", c->page_size);
  if (c->format != KVQ_FMT_INT4_TOKEN && c->format != KVQ_FMT_MXFP4_G32)
    return fail(KVQ_ERR_UNSUPPORTED, "format %d unknown", c->format);
  if (c->had_block != 1 && c->had_block != KVQ_ROT_QUAT4 && c->had_block != 64 && c->had_block != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "had_block %d unsupported (1, 4, 64 or 128)", c->had_block);
  if (c->format == KVQ_FMT_MXFP4_G32 && c->had_block == 64)
    return fail(KVQ_ERR_UNSUPPORTED, "MXFP4 takes had_block 128 or 4 (or 1, for tests)");
  if (c->had_block == KVQ_ROT_QUAT4) {
    if (!c->quat) return fail(KVQ_ERR_INVALID_ARG, "had_block 4 needs cache->quat");
    if (((uintptr_t)c->quat) & 15) return fail(KVQ_ERR_INVALID_ARG, "cache->quat must be 16-byte aligned");
    if (c->quat_full != 0 && c->quat_full != 1) return fail(KVQ_ERR_INVALID_ARG, "cache->quat_full must be 0 or 1");
  } else {
    if (c->quat_full != 0) return fail(KVQ_ERR_INVALID_ARG, "cache->quat_full must be 0 unless had_block is 4");
    if (c->quat) return fail(KVQ_ERR_INVALID_ARG, "cache->quat must be NULL unless had_block is 4");
  }
  if (((uintptr_t)c->pool) & 15) return fail(KVQ_ERR_INVALID_ARG, "pool must be 16-byte aligned");
  return KVQ_OK;
}

// KVQ_DEBUG_CHECKS (environment, read on every call; unset, empty or "0": off): validate the
// call's device-side tables on its stream, wait for the verdict, and refuse the call before its
// kernels run.  The check synchronizes the stream, so it is for debugging, not graph capture.
bool debug_checks() {
  const char* e = getenv("KVQ_DEBUG_CHECKS");
  return e && e[0] && strcmp(e, "0") != 0;
}

// KVQ_LOG (environment, read on every call): one line per launching call on stderr with the
// call's shape and the launch plan the library chose for it.
bool log_on() {
  const char* e = getenv("KVQ_LOG");
  return e && e[0] && strcmp(e, "0") != 0;
}

void log_line(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  fputs("kvq: ", stderr);
  vfprintf(stderr, fmt, ap);
  fputc('\n', stderr);
  va_end(ap);
}

int device_check(const kvq::CheckParams& c, void* stream, const char* what) {
  int code = 0, index = 0;
  const hipError_t e = kvq::run_check(c, (hipStream_t)stream, &code, &index);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: KVQ_DEBUG_CHECKS: %s", what, hipGetErrorString(e));
  const char* msg = nullptr;
  switch (code) {
    case kvq::kCheckOk: return KVQ_OK;
    case kvq::kBadSeqLen: msg = "seq_lens out of [1, max_seq_len]"; break;
    case kvq::kBadPageId: msg = "a block-table entry / page id outside [0, num_pages)"; break;
    case kvq::kBadCumulative: msg = "cumulative counts not non-decreasing within [0, num_tokens]"; break;
    case kvq::kBadStartPos: msg = "start_pos negative or the appended positions beyond max_pages*16"; break;
    case kvq::kBadChunk: msg = "chunk longer than its sequence or than max_q_len"; break;
    default: msg = "unknown violation"; break;
  }
  return fail(KVQ_ERR_INVALID_ARG, "%s: KVQ_DEBUG_CHECKS: %s (index %d)", what, msg, index);
}

// Zero n 32-bit words (the scratch's merge counters).  A kernel rather than hipMemsetAsync, so
// that a call made under stream capture records an ordinary kernel node.
__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int n) {
  const int i = (int)(__builtin_amdgcn_workgroup_id_x() * 256 + __builtin_amdgcn_workitem_id_x());
  if (i < n) p[i] = 0u;
}

// Per device: the device address of `scratch`, and whether its counter region has been cleared
// by a launch that ran eagerly (not into a graph being captured).
constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
  void* ptr;
  bool cleared;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxScratchDevices];

// The scratch of the device that `stream` runs on (it must be the current device).  The first
// call on a device looks up the array's address (hipGetSymbolAddress, with that device current)
// and clears the merge counters on `stream`; every call that runs to completion leaves them at
// zero again.  A clear recorded into a graph under capture is repeated until one runs eagerly.
int scratch_for_device(hipStream_t stream, void** out) {
  int dev = 0, sdev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
  if (sdev != dev) return fail(KVQ_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d", sdev, dev);
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(KVQ_ERR_UNSUPPORTED, "device %d: scratch kept for devices 0..%d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[dev];
  if (!slot.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    slot.ptr = p;
  }
  if (!slot.cleared) {
    hipLaunchKernelGGL(zero_words, dim3((unsigned)((kvq::kCounterUnits + 255) / 256)), dim3(256), 0, stream,
                       (uint32_t*)slot.ptr, (int)kvq::kCounterUnits);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "scratch counter clear launch");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) slot.cleared = true;
  }
  *out = slot.ptr;
  return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

size_t kvq_page_bytes(const kvq_cache* cache) {
  if (!cache || cache->num_kv_heads < 1) return 0;
  return (size_t)cache->num_kv_heads * KVQ_PAGE_HEAD_BYTES;
}

const char* kvq_strerror(int status) {
  switch (status) {
    case KVQ_OK: return "success";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* kvq_last_error(void) { return g_last_error; }

int kvq_append(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
               int32_t num_tokens, int32_t num_seqs, const int32_t* cu_new,
               const int32_t* start_pos, const int32_t* block_table, int32_t max_pages,
               int32_t max_new_tokens, void* stream) {
  g_last_error[0] = 0;
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k and v must not be NULL");
  if (!cu_new || !start_pos || !block_table) return fail(KVQ_ERR_INVALID_ARG, "cu_new, start_pos and block_table must not be NULL");
  if (kv_dtype != KVQ_F16 && kv_dtype != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "kv_dtype %d unsupported (F16 or BF16)", kv_dtype);
  if (num_tokens < 0 || num_seqs < 0) return fail(KVQ_ERR_INVALID_ARG, "num_tokens and num_seqs must be >= 0");
  if (max_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (max_pages > (1 << 24)) return fail(KVQ_ERR_UNSUPPORTED, "max_pages %d above 2^24", max_pages);
  if (max_new_tokens < 0) return fail(KVQ_ERR_INVALID_ARG, "max_new_tokens must be >= 0");
  if ((((uintptr_t)k) | ((uintptr_t)v)) & 15) return fail(KVQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (num_seqs > 65535) return fail(KVQ_ERR_UNSUPPORTED, "num_seqs %d above 65535", num_seqs);
  if (num_tokens == 0 || num_seqs == 0 || max_new_tokens == 0) return KVQ_OK;
  kvq::AppendParams p;
  p.pool = (uint8_t*)cache->pool;
  p.k = (const uint8_t*)k;
  p.v = (const uint8_t*)v;
  p.cu_new = cu_new;
  p.start_pos = start_pos;
  p.block_table = block_table;
  p.hkv = cache->num_kv_heads;
  p.num_seqs = num_seqs;
  p.max_pages = max_pages;
  p.max_new = max_new_tokens;
  p.quat = cache->quat;
  p.quat_full = cache->quat_full;
  if (debug_checks()) {
    kvq::CheckParams c;
    memset(&c, 0, sizeof(c));
    c.kind = kvq::kCheckAppend;
    c.cu = cu_new;
    c.start_pos = start_pos;
    c.block_table = block_table;
    c.num_seqs = num_seqs;
    c.num_tokens = num_tokens;
    c.max_pages = max_pages;
    c.max_len = max_new_tokens;
    c.num_pages = cache->num_pages;
    if (int st = device_check(c, stream, "kvq_append")) return st;
  }
  if (log_on())
    log_line("kvq_append: %d tokens, %d seqs, %d kv heads, max_new_tokens %d, had_block %d, format %d, "
             "grid %d x %d x %d workgroups of 4 waves (%d pages per wave)",
             num_tokens, num_seqs, cache->num_kv_heads, max_new_tokens, cache->had_block, cache->format,
             ((max_new_tokens + 15) / 16 + 1 + kvq::kAppendPagesPerWave - 1) / kvq::kAppendPagesPerWave, num_seqs,
             (2 * cache->num_kv_heads + 3) / 4, kvq::kAppendPagesPerWave);
  return hip_status(kvq::launch_append(p, kv_dtype == KVQ_BF16, cache->had_block, cache->format, (hipStream_t)stream),
                    "kvq_append launch");
}

static int decode_geometry(const kvq_cache* cache, int32_t num_q_heads, int32_t num_seqs, int32_t max_seq_len) {
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads, cache->num_kv_heads);
  if (num_q_heads / cache->num_kv_heads > 8)
    return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d above 8", num_q_heads / cache->num_kv_heads);
  if (num_seqs < 0) return fail(KVQ_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (max_seq_len < 1) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t num_q_heads, int32_t num_seqs,
                                  int32_t max_seq_len) {
  if (decode_geometry(cache, num_q_heads, num_seqs, max_seq_len) != KVQ_OK) return (size_t)-1;
  const kvq::DecodePlan plan = kvq::plan_decode(num_seqs, cache->num_kv_heads, max_seq_len);
  return kvq::decode_workspace_bytes(plan, num_seqs, cache->num_kv_heads, num_q_heads / cache->num_kv_heads);
}

// Shared body of kvq_decode_attn and kvq_decode_step (knew == NULL: no append).
static int decode_common(const kvq_cache* cache, const void* knew, const void* vnew, int32_t kv_dtype,
                         const void* q, int32_t q_dtype, float q_scale, int32_t num_q_heads, int32_t num_seqs,
                         const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                         int32_t max_pages, float sm_scale, void* out, int32_t out_dtype, uint32_t flags,
                         void* workspace, size_t workspace_bytes, void* stream, const char* what,
                         bool use_scratch = false) {
  int st = decode_geometry(cache, num_q_heads, num_seqs, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!q || !seq_lens || !block_table || !out) return fail(KVQ_ERR_INVALID_ARG, "q, seq_lens, block_table and out must not be NULL");
  if (q_dtype < KVQ_F16 || q_dtype > KVQ_FP8_E4M3) return fail(KVQ_ERR_UNSUPPORTED, "q_dtype %d unknown", q_dtype);
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d unsupported (F32, F16 or BF16)", out_dtype);
  if (max_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (max_pages > (1 << 24)) return fail(KVQ_ERR_UNSUPPORTED, "max_pages %d above 2^24", max_pages);
  // the query (and new K/V) tensors are addressed through one 32-bit buffer range each
  if ((int64_t)num_seqs * num_q_heads * KVQ_HEAD_DIM * 4 >= (1ll << 30))
    return fail(KVQ_ERR_UNSUPPORTED, "num_seqs * num_q_heads %lld too large", (long long)num_seqs * num_q_heads);
  if ((int64_t)max_seq_len > (int64_t)max_pages * KVQ_PAGE_SIZE)
    return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds max_pages*16 = %lld", max_seq_len, (long long)max_pages * KVQ_PAGE_SIZE);
  if (flags & ~(KVQ_OUT_ROTATED | KVQ_MX_SCALED_MFMA)) return fail(KVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & KVQ_MX_SCALED_MFMA) && cache->format != KVQ_FMT_MXFP4_G32)
    return fail(KVQ_ERR_UNSUPPORTED, "KVQ_MX_SCALED_MFMA needs an MXFP4 cache");
  if (!std::isfinite(q_scale) || !std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARG, "q_scale and sm_scale must be finite");
  const bool append = knew != nullptr || vnew != nullptr;
  if (append) {
    if (!knew || !vnew) return fail(KVQ_ERR_INVALID_ARG, "k and v must both be given");
    if (kv_dtype != KVQ_F16 && kv_dtype != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "kv_dtype %d unsupported (F16 or BF16)", kv_dtype);
  }
  if (num_seqs == 0) return KVQ_OK;
  const int hkv = cache->num_kv_heads;
  const int group = num_q_heads / hkv;
  const kvq::DecodePlan plan = kvq::plan_decode(num_seqs, hkv, max_seq_len);
  const size_t need = kvq::decode_workspace_bytes(plan, num_seqs, hkv, group);
  if ((int64_t)num_seqs * hkv * plan.nsplit > 0x7FFFFFFF) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  kvq::DecodeParams p;
  memset(&p, 0, sizeof(p));
  if (use_scratch && need > 0) {
    // the library's fixed scratch stands in for the workspace
    if ((size_t)num_seqs * hkv > kvq::kCounterUnits)
      return fail(KVQ_ERR_WORKSPACE, "%lld (sequence, kv head) pairs: the fixed scratch serves at most %zu",
                  (long long)num_seqs * hkv, kvq::kCounterUnits);
    if (need > kScratchBytes)
      return fail(KVQ_ERR_WORKSPACE, "this call needs %zu bytes of scratch, above the fixed maximum of %zu", need,
                  kScratchBytes);
    workspace_bytes = kScratchBytes;
    if (int s2 = scratch_for_device((hipStream_t)stream, &workspace)) return s2;
  }
  if (need > 0) {
    if (!workspace) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (workspace_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes given, %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace) & 255) return fail(KVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    kvq::carve_workspace(workspace, plan, num_seqs, hkv, group, &p.part_ml, &p.part_o, &p.counters);
  }
  p.pool = (uint8_t*)cache->pool;
  p.q = q;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.out = out;
  p.hkv = hkv;
  p.group = group;
  p.hq = num_q_heads;
  p.num_seqs = num_seqs;
  p.max_pages = max_pages;
  p.had_block = cache->had_block;
  p.quat = cache->quat;
  p.quat_full = cache->quat_full;
  p.q_dtype = q_dtype;
  p.out_dtype = out_dtype;
  p.out_rotated = (flags & KVQ_OUT_ROTATED) ? 1 : 0;
  p.q_scale = q_scale;
  p.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  p.e8_shift = 23;
  p.knew = (const uint8_t*)knew;
  p.vnew = (const uint8_t*)vnew;
  p.kv_dtype = append ? kv_dtype : KVQ_BF16;
  p.append = append ? 1 : 0;
  p.plan = plan;
  if (debug_checks()) {
    kvq::CheckParams c;
    memset(&c, 0, sizeof(c));
    c.kind = kvq::kCheckDecode;
    c.seq_lens = seq_lens;
    c.block_table = block_table;
    c.num_seqs = num_seqs;
    c.max_pages = max_pages;
    c.max_len = max_seq_len;
    c.num_pages = cache->num_pages;
    if (int st = device_check(c, stream, what)) return st;
  }
  // kernel variant 2: MXFP4 with q.K and p.V on the scaled matrix cores
  const int variant = (flags & KVQ_MX_SCALED_MFMA) ? 2 : cache->format;
  if (log_on())
    log_line("%s: %d seqs, %d q / %d kv heads, max_seq_len %d, variant %d (0 INT4, 1 MXFP4, 2 MXFP4 scaled), "
             "%d waves, depth %d, %s, up to %d runs of at most %d pages per (sequence, kv head), %lld workgroups",
             what, num_seqs, num_q_heads, cache->num_kv_heads, max_seq_len, variant, plan.waves, plan.depth,
             plan.balanced ? "balanced cut" : "fixed splits", plan.nsplit, plan.pages_per_split,
             (long long)num_seqs * cache->num_kv_heads * plan.nsplit);
  return hip_status(kvq::launch_decode(p, variant, (hipStream_t)stream), what);
}

int kvq_decode_attn(const kvq_cache* cache, const void* q, int32_t q_dtype, float q_scale,
                    int32_t num_q_heads, int32_t num_seqs, const int32_t* seq_lens,
                    int32_t max_seq_len, const int32_t* block_table, int32_t max_pages,
                    float sm_scale, void* out, int32_t out_dtype, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  return decode_common(cache, nullptr, nullptr, 0, q, q_dtype, q_scale, num_q_heads, num_seqs, seq_lens,
                       max_seq_len, block_table, max_pages, sm_scale, out, out_dtype, flags, workspace,
                       workspace_bytes, stream, "kvq_decode_attn launch");
}

int kvq_decode_step(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype, const void* q,
                    int32_t q_dtype, float q_scale, int32_t num_q_heads, int32_t num_seqs,
                    const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                    int32_t max_pages, float sm_scale, void* out, int32_t out_dtype, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k and v must not be NULL");
  return decode_common(cache, k, v, kv_dtype, q, q_dtype, q_scale, num_q_heads, num_seqs, seq_lens,
                       max_seq_len, block_table, max_pages, sm_scale, out, out_dtype, flags, workspace,
                       workspace_bytes, stream, "kvq_decode_step launch");
}

int kvq_decode_step_noalloc(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype, const void* q,
                            int32_t q_dtype, float q_scale, int32_t num_q_heads, int32_t num_seqs,
                            const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                            int32_t max_pages, float sm_scale, void* out, int32_t out_dtype, uint32_t flags,
                            void* stream) {
  g_last_error[0] = 0;
  if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k and v must not be NULL");
  return decode_common(cache, k, v, kv_dtype, q, q_dtype, q_scale, num_q_heads, num_seqs, seq_lens,
                       max_seq_len, block_table, max_pages, sm_scale, out, out_dtype, flags, nullptr, 0, stream,
                       "kvq_decode_step_noalloc launch", true);
}

int kvq_prefill_attn(const kvq_cache* cache, const void* q, int32_t q_dtype, float q_scale, int32_t num_q_heads,
                     int32_t num_tokens, int32_t num_seqs, const int32_t* cu_q, const int32_t* seq_lens,
                     int32_t max_seq_len, int32_t max_q_len, const int32_t* block_table, int32_t max_pages,
                     float sm_scale, void* out, int32_t out_dtype, uint32_t flags, void* stream) {
  g_last_error[0] = 0;
  int st = decode_geometry(cache, num_q_heads, num_seqs, max_seq_len);
  if (st != KVQ_OK) return st;
  const int group = num_q_heads / cache->num_kv_heads;
  if (!q || !cu_q || !seq_lens || !block_table || !out)
    return fail(KVQ_ERR_INVALID_ARG, "q, cu_q, seq_lens, block_table and out must not be NULL");
  if (q_dtype < KVQ_F16 || q_dtype > KVQ_FP8_E4M3) return fail(KVQ_ERR_UNSUPPORTED, "q_dtype %d unknown", q_dtype);
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_F16 && out_dtype != KVQ_BF16)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d unsupported (F32, F16 or BF16)", out_dtype);
  if (num_tokens < 0 || max_q_len < 0) return fail(KVQ_ERR_INVALID_ARG, "num_tokens and max_q_len must be >= 0");
  if (max_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  if (max_pages > (1 << 24)) return fail(KVQ_ERR_UNSUPPORTED, "max_pages %d above 2^24", max_pages);
  if ((int64_t)max_seq_len > (int64_t)max_pages * KVQ_PAGE_SIZE)
    return fail(KVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds max_pages*16 = %lld", max_seq_len, (long long)max_pages * KVQ_PAGE_SIZE);
  if (max_seq_len > 131072) return fail(KVQ_ERR_UNSUPPORTED, "prefill attends at most 131072 positions (max_seq_len %d)", max_seq_len);
  if (max_q_len > max_seq_len) return fail(KVQ_ERR_INVALID_ARG, "max_q_len %d exceeds max_seq_len %d", max_q_len, max_seq_len);
  if ((int64_t)num_tokens * num_q_heads * KVQ_HEAD_DIM * 4 >= (1ll << 30))
    return fail(KVQ_ERR_UNSUPPORTED, "num_tokens * num_q_heads %lld too large", (long long)num_tokens * num_q_heads);
  if (flags & ~KVQ_OUT_ROTATED) return fail(KVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!std::isfinite(q_scale) || !std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARG, "q_scale and sm_scale must be finite");
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return KVQ_OK;
  const int tpt = kvq::prefill_tokens_per_tile(group);
  const int64_t tiles = (max_q_len + tpt - 1) / tpt;
  if ((int64_t)num_seqs * cache->num_kv_heads * tiles > 0x7FFFFFFF) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  kvq::PrefillParams p;
  memset(&p, 0, sizeof(p));
  p.pool = (const uint8_t*)cache->pool;
  p.q = q;
  p.cu_q = cu_q;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.out = out;
  p.hkv = cache->num_kv_heads;
  p.group = group;
  p.hq = num_q_heads;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.max_pages = max_pages;
  p.had_block = cache->had_block;
  p.quat = cache->quat;
  p.quat_full = cache->quat_full;
  p.q_dtype = q_dtype;
  p.out_dtype = out_dtype;
  p.out_rotated = (flags & KVQ_OUT_ROTATED) ? 1 : 0;
  p.tiles = (int32_t)tiles;
  p.q_scale = q_scale;
  p.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  p.e8_shift = 23;
  if (debug_checks()) {
    kvq::CheckParams c;
    memset(&c, 0, sizeof(c));
    c.kind = kvq::kCheckPrefill;
    c.cu = cu_q;
    c.seq_lens = seq_lens;
    c.block_table = block_table;
    c.num_seqs = num_seqs;
    c.num_tokens = num_tokens;
    c.max_pages = max_pages;
    c.max_len = max_seq_len;
    c.max_q_len = max_q_len;
    c.num_pages = cache->num_pages;
    if (int st = device_check(c, stream, "kvq_prefill_attn")) return st;
  }
  if (log_on())
    log_line("kvq_prefill_attn: %d tokens, %d seqs, %d q / %d kv heads, max_q_len %d, format %d, %d tiles of %d "
             "tokens, %lld workgroups of 8 waves",
             num_tokens, num_seqs, num_q_heads, cache->num_kv_heads, max_q_len, cache->format, (int)tiles,
             kvq::prefill_tokens_per_tile(group), (long long)num_seqs * cache->num_kv_heads * tiles);
  return hip_status(kvq::launch_prefill(p, cache->format, (hipStream_t)stream), "kvq_prefill_attn launch");
}

int kvq_dequant_page(const kvq_cache* cache, const int32_t* page_ids, int32_t n, float* out_k,
                     float* out_v, uint32_t flags, void* stream) {
  g_last_error[0] = 0;
  int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (n < 0) return fail(KVQ_ERR_INVALID_ARG, "n must be >= 0");
  if (flags & ~KVQ_UNROTATE) return fail(KVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (n == 0) return KVQ_OK;
  if (!page_ids || !out_k || !out_v) return fail(KVQ_ERR_INVALID_ARG, "page_ids, out_k and out_v must not be NULL");
  if ((int64_t)n * cache->num_kv_heads > 0x7FFFFFFF) return fail(KVQ_ERR_UNSUPPORTED, "too many pages");
  kvq::DequantParams p;
  p.pool = (const uint8_t*)cache->pool;
  p.page_ids = page_ids;
  p.out_k = out_k;
  p.out_v = out_v;
  p.n = n;
  p.hkv = cache->num_kv_heads;
  p.had_block = cache->had_block;
  p.quat = cache->quat;
  p.quat_full = cache->quat_full;
  p.unrotate = (flags & KVQ_UNROTATE) ? 1 : 0;
  p.fmt = cache->format;
  if (debug_checks()) {
    kvq::CheckParams c;
    memset(&c, 0, sizeof(c));
    c.kind = kvq::kCheckDequant;
    c.page_ids = page_ids;
    c.n = n;
    c.num_pages = cache->num_pages;
    if (int st = device_check(c, stream, "kvq_dequant_page")) return st;
  }
  if (log_on())
    log_line("kvq_dequant_page: %d pages, %d kv heads, format %d, had_block %d, %s, %lld workgroups", n,
             cache->num_kv_heads, cache->format, cache->had_block,
             !p.unrotate ? "rotated basis"
                         : (p.fmt == 0 && (p.had_block == 64 || p.had_block == 128) ? "rotated back on the matrix cores"
                                                                                    : "rotated back by butterfly"),
             (long long)n * cache->num_kv_heads);
  return hip_status(kvq::launch_dequant(p, (hipStream_t)stream), "kvq_dequant_page launch");
}

int kvq_hbm_copy(const void* src, void* dst, size_t bytes, void* stream) {
  g_last_error[0] = 0;
  if (!src || !dst) return fail(KVQ_ERR_INVALID_ARG, "src and dst must not be NULL");
  if (bytes % 16) return fail(KVQ_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) return fail(KVQ_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if (bytes == 0) return KVQ_OK;
  return hip_status(kvq::launch_copy(src, dst, bytes, (hipStream_t)stream), "kvq_hbm_copy launch");
}

int kvq_hbm_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  g_last_error[0] = 0;
  if (!src || !sink) return fail(KVQ_ERR_INVALID_ARG, "src and sink must not be NULL");
  if (bytes % 16) return fail(KVQ_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (((uintptr_t)src & 15) || ((uintptr_t)sink & 3)) return fail(KVQ_ERR_INVALID_ARG, "src must be 16-byte and sink 4-byte aligned");
  if (bytes == 0) return KVQ_OK;
  return hip_status(kvq::launch_read(src, bytes, sink, (hipStream_t)stream), "kvq_hbm_read launch");
}

int kvq_hbm_fold4(const void* src, void* dst, size_t dst_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!src || !dst) return fail(KVQ_ERR_INVALID_ARG, "src and dst must not be NULL");
  if (dst_bytes % 4096) return fail(KVQ_ERR_INVALID_ARG, "dst_bytes must be a multiple of 4096");
  if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) return fail(KVQ_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if (dst_bytes == 0) return KVQ_OK;
  return hip_status(kvq::launch_fold4(src, dst, dst_bytes, (hipStream_t)stream), "kvq_hbm_fold4 launch");
}

int kvq_hbm_append_pattern(const void* k, const void* v, int32_t num_kv_heads, int32_t num_seqs,
                           int32_t new_tokens, const int32_t* block_table, int32_t max_pages, void* pool,
                           uint32_t order, void* stream) {
  g_last_error[0] = 0;
  if (!k || !v || !block_table || !pool) return fail(KVQ_ERR_INVALID_ARG, "k, v, block_table and pool must not be NULL");
  if ((((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)pool)) & 15)
    return fail(KVQ_ERR_INVALID_ARG, "k, v and pool must be 16-byte aligned");
  if ((uintptr_t)block_table & 3) return fail(KVQ_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  if (num_kv_heads < 1 || num_kv_heads > 1024) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be in [1, 1024]");
  if (num_seqs < 0 || num_seqs > 65535) return fail(KVQ_ERR_INVALID_ARG, "num_seqs must be in [0, 65535]");
  if (new_tokens < 0 || new_tokens % 16) return fail(KVQ_ERR_INVALID_ARG, "new_tokens must be a non-negative multiple of 16");
  if (max_pages < 0 || (int64_t)new_tokens > 16 * (int64_t)max_pages)
    return fail(KVQ_ERR_INVALID_ARG, "new_tokens must be at most 16 * max_pages");
  if (order > 2) return fail(KVQ_ERR_INVALID_ARG, "order must be 0, 1 or 2");
  if (order != 0 && num_kv_heads > 8) return fail(KVQ_ERR_UNSUPPORTED, "orders 1 and 2 take at most 8 kv heads");
  if (order == 2 && (int64_t)max_pages * 16 != new_tokens)
    return fail(KVQ_ERR_INVALID_ARG, "order 2 takes a list of exactly num_seqs * new_tokens / 16 items");
  if (num_seqs == 0 || new_tokens == 0) return KVQ_OK;
  return hip_status(kvq::launch_append_pattern(k, v, block_table, pool, num_kv_heads, num_seqs, new_tokens, max_pages,
                                               (int)order, (hipStream_t)stream),
                    "kvq_hbm_append_pattern launch");
}

int kvq_hbm_decode_pattern(const void* pool, int32_t num_kv_heads, int32_t num_seqs, int32_t pages_per_seq,
                           const int32_t* block_table, int32_t max_pages, int32_t waves, int32_t depth,
                           int32_t pages_per_split, uint32_t* sink, void* stream) {
  g_last_error[0] = 0;
  if (!pool || !block_table || !sink) return fail(KVQ_ERR_INVALID_ARG, "pool, block_table and sink must not be NULL");
  if ((uintptr_t)pool & 15) return fail(KVQ_ERR_INVALID_ARG, "pool must be 16-byte aligned");
  if ((((uintptr_t)block_table) | ((uintptr_t)sink)) & 3)
    return fail(KVQ_ERR_INVALID_ARG, "block_table and sink must be 4-byte aligned");
  if (num_kv_heads < 1 || num_kv_heads > 1024) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be in [1, 1024]");
  if (num_seqs < 0) return fail(KVQ_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (pages_per_seq < 1 || pages_per_seq > max_pages)
    return fail(KVQ_ERR_INVALID_ARG, "pages_per_seq must be in [1, max_pages]");
  if (waves != 4 && waves != 8) return fail(KVQ_ERR_INVALID_ARG, "waves must be 4 or 8");
  if (depth < 2 || depth > 4) return fail(KVQ_ERR_INVALID_ARG, "depth must be 2, 3 or 4");
  if (pages_per_split < 1 || pages_per_split > 64 * waves)
    return fail(KVQ_ERR_INVALID_ARG, "pages_per_split must be in [1, 64 * waves]");
  const int64_t grid = (int64_t)num_seqs * num_kv_heads * ((pages_per_seq + pages_per_split - 1) / pages_per_split);
  if (grid > 0x7FFFFFFF) return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  if (num_seqs == 0) return KVQ_OK;
  return hip_status(kvq::launch_decode_pattern(pool, block_table, num_kv_heads, num_seqs, pages_per_seq, max_pages,
                                               waves, depth, pages_per_split, sink, (hipStream_t)stream),
                    "kvq_hbm_decode_pattern launch");
}

}  // extern "C"
