// KVQ_DEBUG_CHECKS: validation of a call's device-side tables (sequence lengths, cumulative token
// counts, start positions, block-table entries, page ids) before the call's own kernels run.
// Without it those values are trusted and out-of-range ones are undefined behaviour.  One thread
// per sequence (or page id); the first violation found is recorded with its index.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

__device__ int g_check[2];  // [0] first violation code (0: none), [1] its sequence / page index

__device__ __forceinline__ void report(int code, int index) {
  if (atomicCAS(&g_check[0], 0, code) == 0) g_check[1] = index;
}

// pages [p0, p1] of sequence b must hold page ids in [0, num_pages)
__device__ __forceinline__ bool pages_ok(const CheckParams& c, int b, int p0, int p1) {
  const int32_t* row = c.block_table + (int64_t)b * c.max_pages;
  for (int j = max(p0, 0); j <= p1 && j < c.max_pages; ++j) {
    const int32_t id = row[j];
    if (id < 0 || (int64_t)id >= c.num_pages) return false;
  }
  return true;
}

}  // namespace

__global__ __launch_bounds__(256) void check_kernel(CheckParams c) {
  const int stride = (int)(gridDim.x * 256);
  const int count = c.kind == kCheckDequant ? c.n : c.num_seqs;
  for (int i = block_id_x() * 256 + thread_id(); i < count; i += stride) {
    if (c.kind == kCheckDequant) {
      const int32_t id = c.page_ids[i];
      if (id < 0 || (int64_t)id >= c.num_pages) report(kBadPageId, i);
      continue;
    }
    if (c.kind == kCheckDecode) {
      const int L = c.seq_lens[i];
      if (L < 1 || L > c.max_len) {
        report(kBadSeqLen, i);
        continue;
      }
      if (!pages_ok(c, i, 0, (L - 1) / kPage)) report(kBadPageId, i);
      continue;
    }
    // append / prefill: cumulative counts
    const int32_t c0 = c.cu[i], c1 = c.cu[i + 1];
    if (c0 < 0 || c1 < c0 || c1 > c.num_tokens) {
      report(kBadCumulative, i);
      continue;
    }
    const int n = c1 - c0;
    if (c.kind == kCheckAppend) {
      const int s0 = c.start_pos[i];
      const int n_w = min(n, c.max_len);  // tokens past max_new_tokens are not written
      if (s0 < 0 || (int64_t)s0 + n_w > (int64_t)c.max_pages * kPage) {
        report(kBadStartPos, i);
        continue;
      }
      if (n_w > 0 && !pages_ok(c, i, s0 / kPage, (s0 + n_w - 1) / kPage)) report(kBadPageId, i);
    } else {
      if (n == 0) continue;
      const int L = c.seq_lens[i];
      if (L < 1 || L > c.max_len) {
        report(kBadSeqLen, i);
        continue;
      }
      if (n > L || n > c.max_q_len) {
        report(kBadChunk, i);
        continue;
      }
      if (!pages_ok(c, i, 0, (L - 1) / kPage)) report(kBadPageId, i);
    }
  }
}

hipError_t run_check(const CheckParams& c, hipStream_t stream, int* code, int* index) {
  const int zero[2] = {0, 0};
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_check), zero, sizeof(zero), 0, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  const int count = c.kind == kCheckDequant ? c.n : c.num_seqs;
  const int blocks = count <= 0 ? 1 : (count + 255) / 256 > 1024 ? 1024 : (count + 255) / 256;
  hipLaunchKernelGGL(check_kernel, dim3(blocks), dim3(256), 0, stream, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int out[2] = {0, 0};
  e = hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(g_check), sizeof(out), 0, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  *code = out[0];
  *index = out[1];
  return hipSuccess;
}

}  // namespace kvq
