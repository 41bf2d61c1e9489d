// Device-side helpers shared by the libkvq HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kPageHeadBytes = 2176;
constexpr int kVCodesOff = 1024;
constexpr int kKParamsOff = 2048;
constexpr int kVParamsOff = 2112;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// dtype codes (same values as kvq_dtype in kvq.h; duplicated so kernels need no C header)
enum : int { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2, DT_E4M3 = 3 };

// Work-item and workgroup ids straight from the hardware registers.  (The threadIdx/blockIdx
// accessors go through device-library functions that this build's floating-point flags keep
// from inlining, which would turn every use into a subroutine call.)
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_id_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int block_id_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int block_id_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }
__device__ __forceinline__ int lane_id() { return thread_id() & 63; }

// ---- DPP row (16-lane) reductions; every lane of the row ends with the same bits ----
// All patterns used below read lanes inside the same row, so bound_ctrl never applies; setting it
// lets the compiler fuse the move into the consuming VALU op (v_max_f32_dpp ...).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<kQuadSwap1>(x));
  x = fmaxf(x, dpp_f<kQuadSwap2>(x));
  x = fmaxf(x, dpp_f<kRowHalfMirror>(x));
  x = fmaxf(x, dpp_f<kRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x = x + dpp_f<kQuadSwap1>(x);
  x = x + dpp_f<kQuadSwap2>(x);
  x = x + dpp_f<kRowHalfMirror>(x);
  x = x + dpp_f<kRowMirror>(x);
  return x;
}

// ---- lane exchanges ----
// x from lane (lane ^ M) of the wave, for M = 1 .. 32, without the LDS unit's permute where the
// VALU can do it: quad permutes (1, 2), row shifts by 4 with complementary bank masks (lanes
// with bit 2 clear read lane + 4, the others lane - 4), a row rotation by 8, a swizzle (16, LDS
// unit but no address operand), and the gfx950 32-lane swap (32).  Every lane read lies in the
// same 16-lane row (M <= 8), so no bound control is involved.
template <int CTRL, int BANK>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, 0xF, BANK, false);
}
template <int M>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(dpp_i<0xB1, 0xF>(0, x));        // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return __int_as_float(dpp_i<0x4E, 0xF>(0, x));   // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return __int_as_float(dpp_i<0x114, 0xA>(dpp_i<0x104, 0x5>(0, x), x));  // row_shl/shr:4
  else if constexpr (M == 8) return __int_as_float(dpp_i<0x128, 0xF>(0, x));  // row_ror:8
  else if constexpr (M == 16) {
    // swap: the odd 16-lane rows of the first copy take the even rows of the second, and back
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return __int_as_float((lane & 16) ? (int)r[0] : (int)r[1]);
  } else {
    static_assert(M == 32, "lane exchange distance");
    // swap: lanes 32..63 of the first copy take lanes 0..31 of the second, and back
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return __int_as_float(lane < 32 ? (int)r[1] : (int)r[0]);
  }
}

// Inclusive prefix sum over the wave's 64 lanes: shifts by 1, 2, 4, 8 inside each 16-lane row
// (lanes whose source lies before the row add 0), then the last lane of row 0 / rows 0-1 is
// broadcast into rows 1, 3 / rows 2, 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += dpp_rows<0x111, 0xF>(x);  // row_shr:1
  x += dpp_rows<0x112, 0xF>(x);  // row_shr:2
  x += dpp_rows<0x114, 0xF>(x);  // row_shr:4
  x += dpp_rows<0x118, 0xF>(x);  // row_shr:8
  x += dpp_rows<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_rows<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

// Full-wave reductions (prologue/epilogue only): the row reduction, then rows 16 and 32 apart.
__device__ __forceinline__ float wave_max(float x) {
  x = row_max16(x);
  x = fmaxf(x, xor_lane<16>(x, lane_id()));
  x = fmaxf(x, xor_lane<32>(x, lane_id()));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
  x = row_sum16(x);
  x += xor_lane<16>(x, lane_id());
  x += xor_lane<32>(x, lane_id());
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dpp_i<kQuadSwap1, 0xF>(0, x);
  x += dpp_i<kQuadSwap2, 0xF>(0, x);
  x += dpp_i<kRowHalfMirror, 0xF>(0, x);
  x += dpp_i<kRowMirror, 0xF>(0, x);
  x += __float_as_int(xor_lane<16>(__int_as_float(x), lane_id()));
  x += __float_as_int(xor_lane<32>(__int_as_float(x), lane_id()));
  return x;
}

// ---- quaternion block rotation (IsoQuant abstract: a 4-channel block v -> qL v conj(qR)) ----
// Rotation codes carried in the kernels' had_block argument besides the Hadamard widths.
constexpr int kQuatBlock = 4;

// M = L(a) R(conj(b)), where L(a) v = a v and R(c) v = v c are the Hamilton products of
// quaternions (w, x, y, z); b = 1 (IsoQuant-Fast) leaves M = L(a).
__device__ __forceinline__ void quat_matrix(const float (&a)[4], const float (&b)[4], float (&m)[4][4]) {
  const float l[4][4] = {{a[0], -a[1], -a[2], -a[3]},
                         {a[1], a[0], -a[3], a[2]},
                         {a[2], a[3], a[0], -a[1]},
                         {a[3], -a[2], a[1], a[0]}};
  const float c0 = b[0], c1 = -b[1], c2 = -b[2], c3 = -b[3];
  const float r[4][4] = {{c0, -c1, -c2, -c3}, {c1, c0, c3, -c2}, {c2, -c3, c0, c1}, {c3, c2, -c1, c0}};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m[i][j] = fmaf(l[i][3], r[3][j], fmaf(l[i][2], r[2][j], fmaf(l[i][1], r[1][j], l[i][0] * r[0][j])));
}

// The coefficients with which channel r of 4-channel block `block` is formed from the block's
// four inputs: row r of M (forward, y = M x) or column r (inverse, x = M^T y).  `quat` holds
// q_L per block ([32][4], IsoQuant-Fast) or q_L then q_R ([32][8], IsoQuant-Full).
__device__ __forceinline__ void quat_coeffs(const float* quat, int full, int block, int r, bool inverse,
                                            float (&c)[4]) {
  const float* q = quat + block * (full ? 8 : 4);
  const float a[4] = {q[0], q[1], q[2], q[3]};
  float b[4] = {1.0f, 0.0f, 0.0f, 0.0f};
  if (full) {
    b[0] = q[4];
    b[1] = q[5];
    b[2] = q[6];
    b[3] = q[7];
  }
  float m[4][4];
  quat_matrix(a, b, m);
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = m[0][j];
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i == r) c[j] = m[i][j];
  if (inverse) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = m[j][0];
#pragma unroll
      for (int i = 1; i < 4; ++i) c[j] = i == r ? m[j][i] : c[j];
    }
  }
}

// One 4-channel block held by the four lanes of a DPP quad (lane 4m + r holds channel r):
// channel r of the result = sum_j c[j] * (channel j of the input).
__device__ __forceinline__ float quat_apply_quad(float x, const float (&c)[4]) {
  const float g0 = dpp_f<0x00>(x), g1 = dpp_f<0x55>(x), g2 = dpp_f<0xAA>(x), g3 = dpp_f<0xFF>(x);
  return fmaf(c[3], g3, fmaf(c[2], g2, fmaf(c[1], g1, c[0] * g0)));
}

// ---- scalar conversions ----
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;  // NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
}
// OCP FP8 E4M3 (FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits; 0x7F/0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);  // NaN (bit pattern: the build assumes no NaN math)
  else if (e == 0u) v = (float)m * 0x1p-9f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return s ? -v : v;
}

// Low bits of `bits` (an element already shifted down from its 32-bit word) as dtype `dt`.
__device__ __forceinline__ float raw_to_f32(uint32_t bits, int dt) {
  switch (dt) {
    case DT_F16: return f16_bits_to_f32(bits & 0xFFFFu);
    case DT_BF16: return bf16_bits_to_f32(bits & 0xFFFFu);
    case DT_F32: return __uint_as_float(bits);
    default: return e4m3_to_f32(bits & 0xFFu);
  }
}

// Nontemporal: the outputs are not read again by the kernel that writes them (measured: the
// llama decode step 25.60-25.63 -> 25.46-25.52 us in graph replays).
__device__ __forceinline__ void store_elem(void* p, int64_t i, int dt, float x) {
  switch (dt) {
    case DT_F16: __builtin_nontemporal_store((uint16_t)f32_to_f16_bits(x), (uint16_t*)p + i); break;
    case DT_BF16: __builtin_nontemporal_store((uint16_t)f32_to_bf16_bits(x), (uint16_t*)p + i); break;
    default: __builtin_nontemporal_store(x, (float*)p + i); break;
  }
}

// Byte permute: bytes of {hi, lo} selected by `sel` (0..3 = lo bytes, 4..7 = hi bytes, 0x0C = 0).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ int popc(uint32_t x) { return __builtin_popcount(x); }

// Round |r| (< 8) to the e2m1 grid {0,.5,1,1.5,2,3,4,6}: nearest, ties to the even index,
// saturating at 6.  Adding then subtracting 2^22/2^23/2^24 rounds to steps 0.5/1/2 (RNE).
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  float m = fabsf(r);
  float c = m < 2.0f ? 4194304.0f : (m < 4.0f ? 8388608.0f : 16777216.0f);
  float v = __builtin_fminf((m + c) - c, 6.0f);
  uint32_t idx = v < 1.0f ? (uint32_t)(v * 2.0f) : ((__float_as_uint(v) >> 22) - 252u);
  return idx | (r < 0.0f ? 8u : 0u);
}

// Raw buffer resource over `bytes` bytes at `p` (gfx9 dword3 0x00020000); loads past the end
// return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

}  // namespace kvq
