// kvq_dequant_page: whole pages of the 4-bit cache back to fp32, plus the copy and read-only
// kernels used to measure HBM bandwidth (kvq_hbm_copy, kvq_hbm_read).
//   INT4   y^ = fma(scale, code, zero): a single rounding of the exact value (token-wise INT4 with an
//          fp16 scale and zero, SAW-INT4 summary, "Summary"/"Method").
//   MXFP4  y^ = e2m1(code) * 2^(E-127), exact (FP4 with UE8M0 group scales, UltraQuant article).
// With KVQ_UNROTATE the rotation is undone, x^ = R^T y^: for R_b (symmetric) by the fp32
// Walsh-Hadamard butterfly of the attention kernels, for the quaternion block rotation by the
// transposed 4 x 4 block matrices (IsoQuant abstract), both in registers.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t idx = c & 7u;
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6: (2 + (idx&1)) * 2^((idx>>1) - 2) for idx >= 2
  float mag = idx < 2u ? 0.5f * (float)idx : ldexpf(1.0f + 0.5f * (float)(idx & 1u), (int)(idx >> 1) - 1);
  return (c & 8u) ? -mag : mag;
}

}  // namespace

// One workgroup per (page, kv head), 256 threads.  Load: thread = (slot s = tid/16, column
// a = tid%16) takes row bytes 4a..4a+3 of slot s, i.e. channels a + 32q + 16e (q = 0..3, e = 0..1),
// and writes the dequantized values to LDS.  With KVQ_UNROTATE, wave w then takes 8 of the
// page-head's 32 token vectors (waves 0, 1: K slots 0-7, 8-15; waves 2, 3: V slots) as the
// attention kernels hold a 128-vector (channel `lane` in x0, `lane + 64` in x1), undoes the
// rotation in registers (lane exchanges, all 8 vectors at once) and puts them back.  Store: the
// workgroup writes K and V as interleaved 1 KiB runs.  (Measured: loading each wave's vectors
// straight into that layout, one byte load per channel pair, took 36.4 us against 25.5 for the
// bench's 1024 pages x 8 kv heads, with or without the rotation.)
template <bool UNROTATE>
__global__ __launch_bounds__(256) void dequant_kernel(DequantParams p) {
  __shared__ float buf[2][kPage][kHeadDim];
  const int tid = thread_id();
  const int s = tid >> 4, col = tid & 15;
  const int i = block_id_x() / p.hkv, h = block_id_x() % p.hkv;
  const uint8_t* base = p.pool + ((int64_t)p.page_ids[i] * p.hkv + h) * kPageHeadBytes;
  for (int which = 0; which < 2; ++which) {
    uint32_t word;  // row bytes 4col..4col+3 of slot s
    if (which == 0) {
      word = *(const uint32_t*)(base + 64 * s + 4 * col);
    } else {
      const uint8_t* vb = base + kVCodesOff + 256 * (s >> 2) + 16 * col + (s & 3);
      word = (uint32_t)vb[0] | ((uint32_t)vb[4] << 8) | ((uint32_t)vb[8] << 16) | ((uint32_t)vb[12] << 24);
    }
    const uint32_t pw = *(const uint32_t*)(base + (which ? kVParamsOff : kKParamsOff) + 4 * s);
    for (int q = 0; q < 4; ++q) {
      for (int e = 0; e < 2; ++e) {
        const uint32_t c = (word >> (8 * q + 4 * e)) & 15u;
        const int ch = col + 32 * q + 16 * e;
        float y;
        if (p.fmt == 0) {
          y = fmaf(f16_bits_to_f32(pw & 0xFFFFu), (float)c, f16_bits_to_f32(pw >> 16));
        } else {
          const int ex = (int)((pw >> (8 * (ch >> 5))) & 255u);
          y = ldexpf(e2m1_value(c), ex - 127);
        }
        buf[which][s][ch] = y;
      }
    }
  }
  __syncthreads();
  if constexpr (UNROTATE) {
    const int lane = tid & 63, wave = tid >> 6;
    const int which = wave >> 1, s0 = 8 * (wave & 1);
    float x0[8], x1[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x0[r] = buf[which][s0 + r][lane];
      x1[r] = buf[which][s0 + r][lane + 64];
    }
    attn::rotate_rows<8>(x0, x1, p.had_block, p.quat, p.quat_full, lane, true);
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // each wave rewrites only the rows it read
      buf[which][s0 + r][lane] = x0[r];
      buf[which][s0 + r][lane + 64] = x1[r];
    }
    __syncthreads();
  }
  const int64_t out_base = ((int64_t)i * p.hkv + h) * kPage * kHeadDim;
  for (int k = tid; k < kPage * kHeadDim; k += 256) {
    __builtin_nontemporal_store((&buf[0][0][0])[k], p.out_k + out_base + k);
    __builtin_nontemporal_store((&buf[1][0][0])[k], p.out_v + out_base + k);
  }
}

// Bandwidth probes.  Each workgroup streams one contiguous chunk of the buffer, 4 KiB per
// wave-group step (256 lanes x 16 B), several steps' loads in flight before they are used:
// whole DRAM rows are read while open, which a grid-stride walk (neighbouring kilobytes from
// different workgroups at different times) does not get.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                  int64_t n16, int64_t per_block) {
  const int64_t b0 = (int64_t)block_id_x() * per_block;
  const int64_t b1 = b0 + per_block < n16 ? b0 + per_block : n16;
  int64_t i = b0 + thread_id();
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    u32x4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = src[i + j * 256];
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(a[j], &dst[i + j * 256]);
  }
  for (; i < b1; i += 256) __builtin_nontemporal_store(src[i], &dst[i]);
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t per_block,
                                                  uint32_t* __restrict__ sink) {
  // non-temporal loads (streamed once); the workgroup's XOR of everything it read goes to
  // sink[workgroup], so every load feeds a stored result
  __shared__ uint32_t red[4];
  const int64_t b0 = (int64_t)block_id_x() * per_block;
  const int64_t b1 = b0 + per_block < n16 ? b0 + per_block : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = b0 + thread_id();
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    u32x4 a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __builtin_nontemporal_load(&src[i + j * 256]);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= a[j];
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(&src[i]);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  if ((thread_id() & 63) == 0) red[thread_id() >> 6] = x;
  __syncthreads();
  if (thread_id() == 0) sink[block_id_x()] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_dequant(const DequantParams& p, hipStream_t stream) {
  if (p.unrotate)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)((int64_t)p.n * p.hkv)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)((int64_t)p.n * p.hkv)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  // 4096 workgroups (16 per CU) of 4 x 4 KiB steps, fewer for small copies
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 256 * 4 - 1) / (256 * 4);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const int64_t per_block = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst, n16,
                     per_block);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  // 2048 workgroups (8 per CU) of 8 x 4 KiB steps, fewer for small reads
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 256 * 8 - 1) / (256 * 8);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  const int64_t per_block = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src, n16, per_block,
                     sink);
  return hipGetLastError();
}

}  // namespace kvq
