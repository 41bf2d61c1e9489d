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

// INT4 pages rotated back with the Hadamard block b in {64, 128}: x = R (s c + z 1) =
// (s / sqrt(b)) H c + z sqrt(b) e_0 per block (H_b 1 = b e_0 for the Sylvester matrix; the first
// channel is taken with centred codes, below).  H c is a
// product of integers, so it runs on the f16 matrix cores exactly: the codes enter as the fp16
// subnormals c 2^-24 (a nibble mask), H as +-1, and the fp32 sums of at most 128 products of
// 4-bit codes are exact.  v_mfma_f32_16x16x32_f16 with A = rows of H (16 output channels) and
// B = 32 codes x 16 tokens: lane (n, q) of the B operand of step kb holds the 8 nibbles of code
// row word 4q + kb of token n, i.e. input channels (4q + kb) + 16e, e = 0..7; the output leaves
// lane (n, q) with output channels 16 tile + 4q .. +3 of token n (one 16-byte store).  With
// input channel c = a + 16e (a < 16) and output channel j = n + 16 tile, H[j][c] =
// (-1)^popc(n & a) (-1)^popc(tile & e) (b = 64: zero unless e / 4 == tile / 4, and tile & e
// taken mod 4), so a lane's A operand for (tile, step) is one pattern over e per tile, negated
// by the lane's sign (-1)^popc(n & (4q + kb)).  Waves 0, 1 take K (output tiles 0-3, 4-7),
// waves 2, 3 take V.
template <int HB>
__global__ __launch_bounds__(256) void dequant_rot_i4_kernel(DequantParams p) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  const int which = wave >> 1, upper = wave & 1;  // K | V; output tiles 4 upper .. 4 upper + 3
  const int n = lane & 15, q = lane >> 4;
  const int i = block_id_x() / p.hkv, h = block_id_x() % p.hkv;
  const uint8_t* base = p.pool + ((int64_t)p.page_ids[i] * p.hkv + h) * kPageHeadBytes;

  // ---- the code row words 4q .. 4q+3 of token n, and the token's parameters ----
  uint32_t w[4];
  if (which == 0) {
    const u32x4 x = *(const u32x4*)(base + 64 * n + 16 * q);
    w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
  } else {
    // V: byte s of row word 4q + r of token n sits at 1024 + 256 (n/4) + 64 q + 16 r + 4 s + n%4
    const uint8_t* vb = base + kVCodesOff + 256 * (n >> 2) + 64 * q;
    const uint32_t m = n & 3;
    const uint32_t sel = 0x0C0C0000u | ((4u + m) << 8) | m;  // byte m of each of two words
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x4 x = *(const u32x4*)(vb + 16 * r);
      w[r] = perm(perm(x[3], x[2], sel), perm(x[1], x[0], sel), 0x05040100u);
    }
  }
  const uint32_t pw = *(const uint32_t*)(base + (which ? kVParamsOff : kKParamsOff) + 4 * n);

  // ---- B operands: nibble e of word 4q + kb -> element e, as c 2^-24 ----
  f16x8 bop[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t lo = w[kb] & 0x0F0F0F0Fu, hi = (w[kb] >> 4) & 0x0F0F0F0Fu;
    bop[kb] = __builtin_bit_cast(f16x8, u32x4{perm(hi, lo, 0x0C040C00u), perm(hi, lo, 0x0C050C01u),
                                               perm(hi, lo, 0x0C060C02u), perm(hi, lo, 0x0C070C03u)});
  }

  // ---- the products ----
  f32x4 acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    // pattern over e of output tile 4 upper + tt (+1 0x3C00, -1 0xBC00, 0)
    uint32_t pat[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int e = 2 * d + hlf;
        uint32_t v16;
        if (HB == 128) {
          const int par = (__builtin_popcount(tt & e) + (upper & (e >> 2))) & 1;
          v16 = par ? 0xBC00u : 0x3C00u;
        } else {
          const bool same = (e >> 2) == upper;
          v16 = same ? (((__builtin_popcount(tt & e & 3)) & 1) ? 0xBC00u : 0x3C00u) : 0u;
        }
        word |= v16 << (16 * hlf);
      }
      pat[d] = word;
    }
    acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t flip = (__builtin_popcount(n & (4 * q + kb)) & 1) ? 0x80008000u : 0u;
      const f16x8 aop = __builtin_bit_cast(f16x8, u32x4{pat[0] ^ flip, pat[1] ^ flip, pat[2] ^ flip, pat[3] ^ flip});
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[kb], acc[tt], 0, 0, 0);
    }
  }

  // ---- x = (s 2^24 / sqrt(b)) acc + z sqrt(b) at the first channel of each block; store ----
  constexpr float kIsb = HB == 128 ? 0.08838834764831845f : 0.125f;
  constexpr float kSb = HB == 128 ? 11.313708498984761f : 8.0f;
  // At a block's first channel the two terms are each about (s / sqrt(b)) sum(c), up to ~100 times
  // the result, and would cancel in fp32.  With the codes centred, H (c - 8) = H c - 8 b e_0, that
  // channel is (acc - 8 b 2^-24) s' + (z + 8 s) sqrt(b): the subtraction and z + 8 s are exact in
  // fp32 (the first an integer times 2^-24 below 2^12, the second from two fp16 values).
  const float s16 = f16_bits_to_f32(pw & 0xFFFFu);
  const float sc = s16 * (16777216.0f * kIsb);
  const float zb = (f16_bits_to_f32(pw >> 16) + 8.0f * s16) * kSb;
  constexpr float k8b = 8.0f * HB / 16777216.0f;
  // the tiles go through LDS, so that the workgroup writes K and V as whole 512-byte token rows
  // (16-byte stores straight from the tile layout cover 64-byte pieces 512 bytes apart: slower)
  __shared__ __attribute__((aligned(16))) float buf[2][kPage][kHeadDim];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tile = 4 * upper + tt;
    // output channel 16 tile + 4q + r; the block's first channel: r = 0, q = 0 and tile 0 (b = 128)
    // or tile 0, 4 (b = 64)
    const bool first = q == 0 && (HB == 128 ? tile == 0 : (tile & 3) == 0);
    *(f32x4*)&buf[which][n][16 * tile + 4 * q] =
        f32x4{first ? fmaf(acc[tt][0] - k8b, sc, zb) : acc[tt][0] * sc, acc[tt][1] * sc, acc[tt][2] * sc, acc[tt][3] * sc};
  }
  __syncthreads();
  const int64_t out_base = (int64_t)block_id_x() * kPage * kHeadDim;
  const int tid = thread_id();
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

__global__ __launch_bounds__(256) void fold4_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n_groups, int64_t per_block) {
  // a 4:1 read:write stream in groups of 256 output vectors: output vector 256 m + t is the XOR
  // of input vectors 1024 m + t + 256 k (k = 0..3), so every load and store instruction of a
  // wave covers 1 KiB of consecutive bytes; each workgroup walks one contiguous chunk of groups,
  // two groups (32 KiB read, 8 KiB written) per step.  Nontemporal loads (streamed once),
  // default-policy stores.
  const int64_t g0 = (int64_t)block_id_x() * per_block;
  const int64_t g1 = g0 + per_block < n_groups ? g0 + per_block : n_groups;
  const int t = thread_id();
  int64_t g = g0;
  for (; g + 1 < g1; g += 2) {
    u32x4 a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = __builtin_nontemporal_load(&src[1024 * (g + (k >> 2)) + t + 256 * (k & 3)]);
    dst[256 * g + t] = a[0] ^ a[1] ^ a[2] ^ a[3];
    dst[256 * (g + 1) + t] = a[4] ^ a[5] ^ a[6] ^ a[7];
  }
  if (g < g1) {
    u32x4 a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = __builtin_nontemporal_load(&src[1024 * g + t + 256 * k]);
    dst[256 * g + t] = a[0] ^ a[1] ^ a[2] ^ a[3];
  }
}

// The append's memory traffic without its arithmetic: same grid, waves, pages per wave, lane
// map, buffer descriptors and cache policies as append_kernel, for sequences of new_tokens
// tokens from position 0.  Lane (n, g) reads the 16-byte words at bytes 16 g + 64 j (j = 0..3)
// of token 16 p + n's row and stores their XOR where the append stores its code row piece, plus
// the first word where the append stores the token's parameters (lanes g = 0).
__global__ __launch_bounds__(256) void append_pattern_kernel(const uint8_t* __restrict__ k,
                                                             const uint8_t* __restrict__ v,
                                                             const int32_t* __restrict__ block_table,
                                                             uint8_t* __restrict__ pool, int hkv, int new_tokens,
                                                             int max_pages) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  const int hk = block_id_z() * 4 + wave;
  if (hk >= 2 * hkv) return;
  const int is_v = hk >= hkv;
  const int h = is_v ? hk - hkv : hk;
  const int b = block_id_y();
  const int pg_begin = block_id_x() * kAppendPagesPerWave;
  const int pg_end = min(pg_begin + kAppendPagesPerWave, new_tokens / kPage);
  if (pg_begin >= pg_end) return;
  const int npg = pg_end - pg_begin;
  const int page_ids = lane < npg ? block_table[(int64_t)b * max_pages + pg_begin + lane] : 0;
  const int n = lane & 15, g = lane >> 4;
  const int row_stride = hkv * kHeadDim * 2;
  const uint8_t* src = (is_v ? v : k) + ((int64_t)b * new_tokens * hkv + h) * (kHeadDim * 2);
  for (int i = 0; i < npg; ++i) {
    const int pos0 = (pg_begin + i) * kPage;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (int64_t)pos0 * row_stride, kPage * row_stride);
    u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, n * row_stride + 16 * g + 64 * j, 0, 0));
    const int page_id = __builtin_amdgcn_readlane(page_ids, i);
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(pool + ((int64_t)page_id * hkv + h) * (int64_t)kPageHeadBytes, kPageHeadBytes);
    const int off = is_v ? kVCodesOff + 256 * (n >> 2) + 64 * g + 16 * (n & 3) : 64 * n + 16 * g;
    __builtin_amdgcn_raw_buffer_store_b128(x, pr, off, 0, 2);  // 2: nontemporal, as the append
    const int poff = g == 0 ? (is_v ? kVParamsOff : kKParamsOff) + 4 * n : attn::kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(x[0], pr, poff, 0, 2);
  }
}

// The same traffic in another order: one workgroup per (page, sequence) with one wave per (K|V,
// kv head), so the workgroup reads the page's tokens of all kv heads (one contiguous run of
// 16 token rows for K and one for V) and writes all of the page's head blocks.  With a list
// (the destination order), workgroup i = b P + pg (P pages per sequence) takes list item
// e = list[i] instead: it reads sequence e / P's page e % P and writes page i, so the pages are
// written in launch order whatever order the rows are read in.
__global__ __launch_bounds__(1024) void append_pattern_page_kernel(const uint8_t* __restrict__ k,
                                                                  const uint8_t* __restrict__ v,
                                                                  const int32_t* __restrict__ block_table,
                                                                  uint8_t* __restrict__ pool, int hkv,
                                                                  int new_tokens, int max_pages, bool list) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  if (wave >= 2 * hkv) return;
  const int is_v = wave >= hkv;
  const int h = is_v ? wave - hkv : wave;
  int b = block_id_y(), pg = block_id_x();
  const int npg = new_tokens / kPage;
  const int dest = b * npg + pg;  // list form: the page written
  if (list) {
    const int e = __builtin_amdgcn_readfirstlane(block_table[dest]);
    b = e / npg;
    pg = e - b * npg;
  }
  const int n = lane & 15, g = lane >> 4;
  const int row_stride = hkv * kHeadDim * 2;
  const uint8_t* src = (is_v ? v : k) + (((int64_t)b * new_tokens + pg * kPage) * hkv + h) * (kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, kPage * row_stride);
  u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, n * row_stride + 16 * g + 64 * j, 0, 0));
  const int page_id = list ? dest : block_table[(int64_t)b * max_pages + pg];
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(pool + ((int64_t)page_id * hkv + h) * (int64_t)kPageHeadBytes, kPageHeadBytes);
  const int off = is_v ? kVCodesOff + 256 * (n >> 2) + 64 * g + 16 * (n & 3) : 64 * n + 16 * g;
  __builtin_amdgcn_raw_buffer_store_b128(x, pr, off, 0, 2);
  const int poff = g == 0 ? (is_v ? kVParamsOff : kKParamsOff) + 4 * n : attn::kOutOfRange;
  __builtin_amdgcn_raw_buffer_store_b32(x[0], pr, poff, 0, 2);
}

// The decode's page stream without its arithmetic: the grid (a workgroup per (sequence, kv head,
// split) in split-major order), W waves with the pages dealt round-robin (wave w takes pages
// p_begin + w + W i), each lane's page loads (K row bytes 64 n + 16 g, V words 1024 + 16 l, the K
// and V parameter words of token n; n = l % 16, g = l / 16), the buffer descriptors, nontemporal
// policy and prefetch depth D of decode_kernel, for sequences of pages_per_seq full pages.  Each
// lane adds up the 32-bit words it loaded (mod 2^32); wave w of workgroup j stores the sum over
// its lanes at sink[W j + w].
template <int W, int D>
__global__ __launch_bounds__(W * 64) void decode_pattern_kernel(const uint8_t* __restrict__ pool,
                                                                const int32_t* __restrict__ block_table, int hkv,
                                                                int num_seqs, int pages_per_seq, int max_pages,
                                                                int pages_per_split, uint32_t* __restrict__ sink) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  const int units = num_seqs * hkv;
  const int split = block_id_x() / units, unit = block_id_x() % units;
  const int kvh = unit % hkv, b = unit / hkv;
  const int p_begin = split * pages_per_split;
  const int p_end = min(p_begin + pages_per_split, pages_per_seq);
  const int pw0 = p_begin + wave;
  const int npw = max(0, (p_end - pw0 + W - 1) / W);  // <= 64: pages_per_split <= 64 W
  const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(block_table + (int64_t)b * max_pages, max_pages * 4);
  const int pid_vec =
      (int)__builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, lane < npw ? 4 * (pw0 + W * lane) : attn::kOutOfRange, 0, 0);
  const uint8_t* pool_h = pool + (int64_t)kvh * kPageHeadBytes;
  const int64_t page_stride = (int64_t)hkv * kPageHeadBytes;
  const int n = lane & 15, g = lane >> 4;
  const int koff = 64 * n + 16 * g, voff = kVCodesOff + 16 * lane, poff = 4 * n;
  struct Words {
    u32x4 k, v;
    uint32_t kp, vp;
  };
  // page i of the wave (past its last: out-of-range offsets, the loads return zeros)
  auto load = [&](int i) {
    const uint64_t addr = (uint64_t)(pool_h + (int64_t)__builtin_amdgcn_readlane(pid_vec, min(i, 63)) * page_stride);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const __amdgpu_buffer_rsrc_t r = make_rsrc((const uint8_t*)(((uint64_t)hi << 32) | lo), kPageHeadBytes);
    const bool live = i < npw;
    Words d;
    d.k = __builtin_amdgcn_raw_buffer_load_b128(r, live ? koff : attn::kOutOfRange, 0, 2);
    d.v = __builtin_amdgcn_raw_buffer_load_b128(r, live ? voff : attn::kOutOfRange, 0, 2);
    d.kp = __builtin_amdgcn_raw_buffer_load_b32(r, live ? poff : attn::kOutOfRange, kKParamsOff, 2);
    d.vp = __builtin_amdgcn_raw_buffer_load_b32(r, live ? poff : attn::kOutOfRange, kVParamsOff, 2);
    return d;
  };
  constexpr int NB = D + 1;
  Words st[NB];
#pragma unroll
  for (int d = 0; d < D; ++d) st[d] = load(d);
  uint32_t acc = 0u;
  for (int i0 = 0; i0 < npw; i0 += NB) {
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      st[(d + D) % NB] = load(i0 + d + D);
      const Words& w = st[d];
      acc += w.k[0] + w.k[1] + w.k[2] + w.k[3] + w.v[0] + w.v[1] + w.v[2] + w.v[3] + w.kp + w.vp;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += (uint32_t)__shfl_xor((int)acc, m, 64);
  if (lane == 0) sink[(int64_t)W * block_id_x() + wave] = acc;
}

hipError_t launch_dequant(const DequantParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)p.n * p.hkv);
  if (p.unrotate && p.fmt == 0 && p.had_block == 128)
    hipLaunchKernelGGL(dequant_rot_i4_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  else if (p.unrotate && p.fmt == 0 && p.had_block == 64)
    hipLaunchKernelGGL(dequant_rot_i4_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  else if (p.unrotate)
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

hipError_t launch_fold4(const void* src, void* dst, size_t dst_bytes, hipStream_t stream) {
  // groups of 256 output vectors (4 KiB); 2048 workgroups (8 per CU), each a contiguous chunk
  const int64_t groups = (int64_t)(dst_bytes / 4096);
  int64_t blocks = groups < 2048 ? groups : 2048;
  if (blocks < 1) blocks = 1;
  const int64_t per_block = (groups + blocks - 1) / blocks;
  hipLaunchKernelGGL(fold4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst,
                     groups, per_block);
  return hipGetLastError();
}

hipError_t launch_append_pattern(const void* k, const void* v, const int32_t* block_table, void* pool, int hkv,
                                 int num_seqs, int new_tokens, int max_pages, int order, hipStream_t stream) {
  const int pages = new_tokens / kPage;
  if (order != 0) {
    hipLaunchKernelGGL(append_pattern_page_kernel, dim3((unsigned)pages, (unsigned)num_seqs), dim3(1024), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, block_table, (uint8_t*)pool, hkv, new_tokens, max_pages, order == 2);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((pages + kAppendPagesPerWave - 1) / kAppendPagesPerWave), (unsigned)num_seqs,
                  (unsigned)((2 * hkv + 3) / 4));
  hipLaunchKernelGGL(append_pattern_kernel, grid, dim3(256), 0, stream, (const uint8_t*)k, (const uint8_t*)v,
                     block_table, (uint8_t*)pool, hkv, new_tokens, max_pages);
  return hipGetLastError();
}

hipError_t launch_decode_pattern(const void* pool, const int32_t* block_table, int hkv, int num_seqs,
                                 int pages_per_seq, int max_pages, int waves, int depth, int pages_per_split,
                                 uint32_t* sink, hipStream_t stream) {
  const int nsplit = (pages_per_seq + pages_per_split - 1) / pages_per_split;
  const dim3 grid((unsigned)((int64_t)num_seqs * hkv * nsplit));
#define KVQ_PATTERN_CASE(WV, DV)                                                                        \
  if (waves == WV && depth == DV) {                                                                     \
    hipLaunchKernelGGL((decode_pattern_kernel<WV, DV>), grid, dim3(WV * 64), 0, stream, (const uint8_t*)pool, \
                       block_table, hkv, num_seqs, pages_per_seq, max_pages, pages_per_split, sink);     \
  } else
  KVQ_PATTERN_CASE(4, 2) KVQ_PATTERN_CASE(4, 3) KVQ_PATTERN_CASE(4, 4)
  KVQ_PATTERN_CASE(8, 2) KVQ_PATTERN_CASE(8, 3) KVQ_PATTERN_CASE(8, 4) { return hipErrorInvalidValue; }
#undef KVQ_PATTERN_CASE
  return hipGetLastError();
}

}  // namespace kvq
