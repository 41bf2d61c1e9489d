// Device pieces shared by the attention kernels of libkvq (decode and chunked prefill): the
// page-head load, the per-page INT4 / MXFP4 score + online softmax + p.V step on the matrix
// cores, and the wave-level Walsh-Hadamard butterfly.  See kvq_decode.hip for the method.
#pragma once

#include "kvq_device.h"

namespace kvq {
namespace attn {


constexpr int kMaxG = 8;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float inv_sqrt_block(int hb) {
  return hb == 128 ? 0.08838834764831845f : (hb == 64 ? 0.125f : 1.0f);
}

// One butterfly stage of the Walsh-Hadamard transform over lanes `lane` and `lane ^ M`.
template <int M>
__device__ __forceinline__ void fwht_stage(float& x0, float& x1, int lane) {
  const float y0 = xor_lane<M>(x0, lane), y1 = xor_lane<M>(x1, lane);
  const bool upper = (lane & M) != 0;
  x0 = upper ? y0 - x0 : x0 + y0;
  x1 = upper ? y1 - x1 : x1 + y1;
}

// Walsh-Hadamard transform of one 128-vector held by a wave, element `lane` in x0 and element
// `lane + 64` in x1 (unnormalised, blocks of hb channels, natural Sylvester order; hb is 64 or
// 128, and 1 leaves x as it is).  Cross-lane stages use lane exchanges, so no workgroup barrier
// is needed; the stage across the two halves (hb 128) stays in registers.
__device__ __forceinline__ void fwht_wave(float& x0, float& x1, int hb, int lane) {
  if (hb < 64) return;
  fwht_stage<1>(x0, x1, lane);
  fwht_stage<2>(x0, x1, lane);
  fwht_stage<4>(x0, x1, lane);
  fwht_stage<8>(x0, x1, lane);
  fwht_stage<16>(x0, x1, lane);
  fwht_stage<32>(x0, x1, lane);
  if (hb == 128) {
    const float t = x0;
    x0 = t + x1;
    x1 = t - x1;
  }
}

// The same transform of R vectors at once (row r in x0[r], x1[r]).
template <int R>
__device__ __forceinline__ void fwht_rows(float (&x0)[R], float (&x1)[R], int hb, int lane) {
  if (hb < 64) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    fwht_stage<1>(x0[r], x1[r], lane);
    fwht_stage<2>(x0[r], x1[r], lane);
    fwht_stage<4>(x0[r], x1[r], lane);
    fwht_stage<8>(x0[r], x1[r], lane);
    fwht_stage<16>(x0[r], x1[r], lane);
    fwht_stage<32>(x0[r], x1[r], lane);
  }
  if (hb == 128) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = x0[r];
      x0[r] = t + x1[r];
      x1[r] = t - x1[r];
    }
  }
}

// The quaternion block rotation of one 128-vector held by a wave (element lane in x0, lane + 64
// in x1): the four lanes of a quad hold one 4-channel block.  inverse: the transpose.
__device__ __forceinline__ void quat_wave(float& x0, float& x1, const float* quat, int full, int lane,
                                          bool inverse) {
  float c0[4], c1[4];
  quat_coeffs(quat, full, lane >> 2, lane & 3, inverse, c0);
  quat_coeffs(quat, full, 16 + (lane >> 2), lane & 3, inverse, c1);
  x0 = quat_apply_quad(x0, c0);
  x1 = quat_apply_quad(x1, c1);
}

// y = R x for the cache's rotation (normalised Hadamard of width hb, or the quaternion block
// rotation when hb is kQuatBlock), wave layout as above.
__device__ __forceinline__ void rotate_wave(float& x0, float& x1, int hb, const float* quat, int full, int lane) {
  if (hb == kQuatBlock) {
    quat_wave(x0, x1, quat, full, lane, false);
    return;
  }
  fwht_wave(x0, x1, hb, lane);
  const float isb = inv_sqrt_block(hb);
  x0 *= isb;
  x1 *= isb;
}

// x = R^T y (R_b is symmetric)
__device__ __forceinline__ void unrotate_wave(float& x0, float& x1, int hb, const float* quat, int full,
                                              int lane) {
  if (hb == kQuatBlock) {
    quat_wave(x0, x1, quat, full, lane, true);
    return;
  }
  fwht_wave(x0, x1, hb, lane);
  const float isb = inv_sqrt_block(hb);
  x0 *= isb;
  x1 *= isb;
}

// Rows r = 0..R-1 at once (x0[r], x1[r]); the coefficients are shared by the rows.
template <int R>
__device__ __forceinline__ void rotate_rows(float (&x0)[R], float (&x1)[R], int hb, const float* quat, int full,
                                            int lane, bool inverse) {
  if (hb == kQuatBlock) {
    float c0[4], c1[4];
    quat_coeffs(quat, full, lane >> 2, lane & 3, inverse, c0);
    quat_coeffs(quat, full, 16 + (lane >> 2), lane & 3, inverse, c1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      x0[r] = quat_apply_quad(x0[r], c0);
      x1[r] = quat_apply_quad(x1[r], c1);
    }
    return;
  }
  fwht_rows<R>(x0, x1, hb, lane);
  const float isb = inv_sqrt_block(hb);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    x0[r] *= isb;
    x1[r] *= isb;
  }
}

template <int FMT>
struct PageData {
  u32x4 k;      // K row bytes 16*jg..16*jg+15 of token n
  u32x4 v;      // V words: row bytes 4n..4n+3 of tokens 4jg..4jg+3
  uint32_t kp;  // K params of token n
  uint32_t vp;  // INT4: V params of token n
};
template <>
struct PageData<1> {
  u32x4 k;
  u32x4 v;
  uint32_t kp;  // UE8M0 bytes of token n (K)
  u32x4 vp4;    // UE8M0 bytes of tokens 4jg..4jg+3 (V)
};

// Offset past the end of every buffer range used here: a load with it returns zeros without a
// memory access.  Loads that are not needed still issue with it, so every path through a kernel
// issues the same sequence of loads and the compiler's memory-counter waits stay exact (a load
// skipped on some path makes it wait for everything issued after the value it needs).
constexpr int kOutOfRange = 0x40000000;

// `base` is wave-uniform: the buffer descriptor lives in scalar registers and the per-lane offsets
// are loop invariant, so a page costs no vector address arithmetic.  `live` false turns the four
// loads into out-of-range ones.
template <int FMT>
__device__ __forceinline__ PageData<FMT> load_page(const uint8_t* base, bool live, int koff, int voff, int poff,
                                                   int qoff) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, kPageHeadBytes);
  if (!live) koff = voff = poff = qoff = kOutOfRange;
  PageData<FMT> d;
  // cache policy 2 = nontemporal: the pages are streamed once per step
  d.k = __builtin_amdgcn_raw_buffer_load_b128(r, koff, 0, 2);
  d.v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2);
  d.kp = __builtin_amdgcn_raw_buffer_load_b32(r, poff, kKParamsOff, 2);
  if constexpr (FMT == 0) d.vp = __builtin_amdgcn_raw_buffer_load_b32(r, poff, kVParamsOff, 2);
  else d.vp4 = __builtin_amdgcn_raw_buffer_load_b128(r, qoff, kVParamsOff, 2);
  return d;
}

// 2^(E-127) for the UE8M0 byte E at bit `shift` of w (E = 0 gives 0: an all-zero or sub-2^-125 group):
// E moved into the fp32 exponent field.  e8sh is that field's position, 23, passed in as a kernel
// argument: with the amount unknown at compile time the byte extraction stays a byte-select
// operand of the one shift instruction, instead of being rewritten into a shift and a mask (two
// instructions for three of the four bytes).
__device__ __forceinline__ float ue8m0_scale(uint32_t w, int shift, int e8sh) {
  return __uint_as_float(((w >> shift) & 0xFFu) << e8sh);
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
// Two e2m1 codes of byte `sel` of w -> two fp16 values times `scale` (low nibble first).
__device__ __forceinline__ f16x2 cvt_fp4(uint32_t w, float scale, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3);
  }
}

// Per-wave streaming state.
struct WaveState {
  float m0, m1, l0, l1, pz0, pz1;
  f32x4 acc[8];
};

// The row-independent operands of an INT4 page: the K codes as int8 B tiles (low and high
// nibbles), the V codes as centred fp16 subnormal B tiles, and the token's parameters.
struct PageI4 {
  i32x4 kb0, kb1;
  f16x4 blo[4], bhi[4];
  float sk, zk, sv, zv;
};

// vlimit (wave-uniform): slots of the page that exist in the sequence.  Past it the V parameters
// are taken as 0, so whatever bytes the pool held there stay finite in the p.V terms (their p is
// 0: an inf or NaN scale would still poison the sums).
__device__ __forceinline__ PageI4 unpack_i4(const PageData<0>& pg, int vlimit, int n) {
  const uint32_t M4 = 0x0F0F0F0Fu, M16 = 0x000F000Fu;
  PageI4 u;
  // parameters of slots past the attended count are zeroed: those slots hold whatever the pool
  // held (fp16 inf / NaN possible), and a masked score must stay -inf after the lo limb's share
  // s_k * lo joins it
  const bool live = n < vlimit;
  const uint32_t vp = live ? pg.vp : 0u, kp = live ? pg.kp : 0u;
  u.kb0 = i32x4{(int)(pg.k[0] & M4), (int)(pg.k[1] & M4), (int)(pg.k[2] & M4), (int)(pg.k[3] & M4)};
  u.kb1 = i32x4{(int)((pg.k[0] >> 4) & M4), (int)((pg.k[1] >> 4) & M4), (int)((pg.k[2] >> 4) & M4),
                (int)((pg.k[3] >> 4) & M4)};
  u.sk = f16_bits_to_f32(kp & 0xFFFFu);
  u.zk = f16_bits_to_f32(kp >> 16);
  u.sv = f16_bits_to_f32(vp & 0xFFFFu);
  u.zv = f16_bits_to_f32(vp >> 16);
  // V codes as fp16 subnormals: word q of the lane holds row byte 4n+q of 4 tokens.  Low nibbles
  // (channel n+32q) are masked to c*2^-24, high nibbles (channel n+32q+16) are masked in place to
  // 16c*2^-24 (their accumulators carry that factor 16 until the end).  One exact packed fp16
  // subtraction centres the codes, c -> c - 8: all products p~*c would otherwise share one sign,
  // and the MFMA accumulation error would not average out (the centre 8*sv moves into the zero
  // point, zv + 8*sv).
  typedef __attribute__((ext_vector_type(2))) _Float16 h2;
  const h2 c8lo = __builtin_bit_cast(h2, 0x00080008u), c8hi = __builtin_bit_cast(h2, 0x00800080u);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t Y = pg.v[q], Y8 = Y >> 8;
    const h2 l0 = __builtin_bit_cast(h2, Y & M16) - c8lo, l1 = __builtin_bit_cast(h2, Y8 & M16) - c8lo;
    const h2 u0 = __builtin_bit_cast(h2, Y & (M16 << 4)) - c8hi;
    const h2 u1 = __builtin_bit_cast(h2, Y8 & (M16 << 4)) - c8hi;
    u.blo[q] = f16x4{l0[0], l0[1], l1[0], l1[1]};  // tokens 0,2 | 1,3
    u.bhi[q] = f16x4{u0[0], u0[1], u1[0], u1[1]};
  }
  return u;
}

// The INT4 score path holds q' of a head as a 24-bit fixed-point number Q = rne(q' / delta),
// delta = max|q'| / kQFix, split into three int8 limbs Q = 65536 hi + 256 mid + lo (hi in
// [-122, 122], mid and lo in [-128, 127]); the limbs are A-tile rows of the integer MFMA, whose
// output row r lands in lane group r / 4.  Two layouts:
//   one head per lane group (at most 4 heads): rows 4g, 4g+1, 4g+2 hold hi, mid, lo of head g
//     (row 4g+3 zero), so lane group g holds all of head g's partial sums; its p~ parts take
//     rows 4g, 4g+1 of the p.V tile, so its accumulators are lane group g's rows too;
//   two heads per lane group (5 to 8 heads, and the chunked prefill's row sets): rows 2g, 2g+1
//     hold hi, mid of head g and row 2g of a second tile its lo (row 2g+1 zero), two more MFMAs
//     per page; p~ parts in rows 2g, 2g+1.
// Q carries ~23 bits of q' (an error of at most max|q'| / 1.6e7 per channel), far below the
// fp32 arithmetic after it.
constexpr float kQFix = 8000000.0f;

// Byte of channel ch in a head's limb block [a2][jg][16] (the A-tile byte order): channel
// (4 jg + w) + 32 q2 + 16 a2 sits at byte 4w + q2 of operand a2, lane group jg.
__device__ __forceinline__ int qlimb_byte(int ch) {
  const int c16 = ch & 15, c_hi = ch >> 4;
  return (c_hi & 1) * 64 + (c16 >> 2) * 16 + 4 * (c16 & 3) + (c_hi >> 1);
}

// Quantize one head's q' (element lane in v0, lane + 64 in v1) to the three limbs, written at
// block[0][byte], block[plane][byte], block[2 plane][byte] (plane: bytes between limb planes).
// Returns 256 delta, the weight of the mid limb; *qsum gets delta * sum(Q), the sum of the q'
// actually used.
__device__ __forceinline__ float q_limbs(float v0, float v1, uint8_t* block, int plane, int lane, float* qsum) {
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float delta = amax > 0.0f ? amax / kQFix : 1.0f;
  const int q0 = (int)rintf(v0 / delta), q1 = (int)rintf(v1 / delta);
  *qsum = delta * (float)wave_sum_i(q0 + q1);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    // balanced base-256 digits from the bottom, each in [-128, 127] (the top one within +-122)
    const int Q = e ? q1 : q0;
    const int lo = ((Q + 128) & 255) - 128, Q1 = (Q - lo) >> 8;
    const int mid = ((Q1 + 128) & 255) - 128, hi = (Q1 - mid) >> 8;
    uint8_t* dst = block + qlimb_byte(lane + 64 * e);
    dst[0] = (uint8_t)(hi & 255);
    dst[plane] = (uint8_t)(mid & 255);
    dst[2 * plane] = (uint8_t)(lo & 255);
  }
  return 256.0f * delta;
}

// One set of 8 rows (two heads per lane group: A-tile rows 2g+limb) against an unpacked INT4
// page.  valid0 / valid1: tokens of the page that rows x0 / x1 attend (decode: the same count).
__device__ __forceinline__ void rows_i4(const PageI4& u, int valid0, int valid1, WaveState& s,
                                        const i32x4 (&qa)[4], float alpha0, float beta0, float alpha1,
                                        float beta1, bool has0, bool has1, int n, int jg, bool a_row_used,
                                        _Float16 (*ptile)[kPage]) {
  const bool tv0 = n < valid0, tv1 = n < valid1;

  // Q.c_t on the integer matrix cores, exactly: hi and mid limbs in sc, lo in sl.  alpha = 256
  // delta sm_scale log2(e) weighs the mid limb (|256 hi.c + mid.c| < 2^26 is exact in int32).
  // The hi and mid limbs give the score to 2^-15 of its largest term, and that sets the running
  // maximum (any reference value gives the same softmax); the lo limb's share joins while the
  // maximum is reduced, off its dependency chain.
  i32x4 sc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], u.kb0, i32x4{0, 0, 0, 0}, 0, 0, 0);
  sc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], u.kb1, sc, 0, 0, 0);
  i32x4 sl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[2], u.kb0, i32x4{0, 0, 0, 0}, 0, 0, 0);
  sl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[3], u.kb1, sl, 0, 0, 0);
  const int lo0 = sl[0], lo1 = sl[2];

  float x0 = fmaf((float)(sc[0] * 256 + sc[1]) * alpha0, u.sk, u.zk * beta0);
  float x1 = fmaf((float)(sc[2] * 256 + sc[3]) * alpha1, u.sk, u.zk * beta1);
  x0 = tv0 ? x0 : -INFINITY;
  x1 = tv1 ? x1 : -INFINITY;

  const float pm0 = row_max16(x0), pm1 = row_max16(x1);
  x0 = fmaf((float)lo0 * (alpha0 * (1.0f / 256.0f)), u.sk, x0);
  x1 = fmaf((float)lo1 * (alpha1 * (1.0f / 256.0f)), u.sk, x1);
  const float sv = u.sv, zv = u.zv;
  // The reference max m only moves when a score exceeds it by more than 2^8 (or when p~ = p * sv
  // could leave the fp16 range): any m gives the same softmax, and p <= 2^8 keeps the fp16 and
  // fp32 partial sums in range.  exp2 of very negative arguments may flush to zero: harmless here.
  if (__any(pm0 > s.m0 + 8.0f || pm1 > s.m1 + 8.0f || ((pm0 > s.m0 || pm1 > s.m1) && sv > 128.0f))) {
    const float mn0 = fmaxf(s.m0, pm0), mn1 = fmaxf(s.m1, pm1);
    const float f0 = __builtin_amdgcn_exp2f(s.m0 - mn0), f1 = __builtin_amdgcn_exp2f(s.m1 - mn1);
#pragma unroll
    for (int i = 0; i < 8; ++i) s.acc[i] *= f32x4{f0, f0, f1, f1};
    s.l0 *= f0;
    s.l1 *= f1;
    s.pz0 *= f0;
    s.pz1 *= f1;
    s.m0 = mn0;
    s.m1 = mn1;
  }
  const float p0 = __builtin_amdgcn_exp2f(x0 - s.m0), p1 = __builtin_amdgcn_exp2f(x1 - s.m1);
  s.l0 += p0;
  s.l1 += p1;
  // A masked score is -inf, so its p is exactly 0, and sv, zv are finite (zeroed past the
  // sequence's end): masked tokens add nothing below without a select.
  const float zc = fmaf(8.0f, sv, zv);  // zero point of the centred codes (exact: fp16 inputs)
  s.pz0 = fmaf(p0, zc, s.pz0);
  s.pz1 = fmaf(p1, zc, s.pz1);

  // p~ = p * sv as fp16 high + low parts, stored at A-tile rows 2g+limb in the k order of the
  // V words (tokens 0, 2, 1, 3 of each quad: bits 0 and 1 of the token swapped)
  const float pt0 = p0 * sv, pt1 = p1 * sv;
  const _Float16 h0 = (_Float16)pt0, h1 = (_Float16)pt1;
  const _Float16 r0 = (_Float16)(pt0 - (float)h0), r1 = (_Float16)(pt1 - (float)h1);
  const int pos = (n & ~3) | ((n & 1) << 1) | ((n >> 1) & 1);
  if (has0) {
    ptile[4 * jg + 0][pos] = h0;
    ptile[4 * jg + 1][pos] = r0;
  }
  if (has1) {
    ptile[4 * jg + 2][pos] = h1;
    ptile[4 * jg + 3][pos] = r1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f16x4 pa = a_row_used ? *(const f16x4*)&ptile[n][4 * jg] : f16x4{0, 0, 0, 0};
  __builtin_amdgcn_wave_barrier();

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s.acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, u.blo[q], s.acc[2 * q], 0, 0, 0);
    s.acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, u.bhi[q], s.acc[2 * q + 1], 0, 0, 0);
  }
}

// One head per lane group (at most 4 heads, layout above): head jg's scores, online softmax
// (statistics in s.m0, s.l0, s.pz0) and p.V (accumulator rows 0, 1 of lane group jg).
__device__ __forceinline__ void rows_i4_one(const PageI4& u, int valid, WaveState& s, const i32x4 (&qa)[2],
                                            float alpha, float beta, bool has, int n, int jg, bool a_row_used,
                                            _Float16 (*ptile)[kPage]) {
  const bool tv = n < valid;
  // hi, mid, lo limb sums in sc[0], sc[1], sc[2]; the lo share joins after the maximum (as above)
  i32x4 sc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], u.kb0, i32x4{0, 0, 0, 0}, 0, 0, 0);
  sc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], u.kb1, sc, 0, 0, 0);
  float x = fmaf((float)(sc[0] * 256 + sc[1]) * alpha, u.sk, u.zk * beta);
  x = tv ? x : -INFINITY;
  const float pm = row_max16(x);
  x = fmaf((float)sc[2] * (alpha * (1.0f / 256.0f)), u.sk, x);
  const float sv = u.sv, zv = u.zv;
  // the reference maximum moves as in rows_i4
  if (__any(pm > s.m0 + 8.0f || (pm > s.m0 && sv > 128.0f))) {
    const float mn = fmaxf(s.m0, pm);
    const float f = __builtin_amdgcn_exp2f(s.m0 - mn);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s.acc[i][0] *= f;
      s.acc[i][1] *= f;
    }
    s.l0 *= f;
    s.pz0 *= f;
    s.m0 = mn;
  }
  const float p = __builtin_amdgcn_exp2f(x - s.m0);
  s.l0 += p;
  const float zc = fmaf(8.0f, sv, zv);
  s.pz0 = fmaf(p, zc, s.pz0);
  // p~ = p * sv as fp16 high + low parts at p-tile rows 4 jg, 4 jg + 1 (token order as in rows_i4)
  const float pt = p * sv;
  const _Float16 h = (_Float16)pt;
  const _Float16 r = (_Float16)(pt - (float)h);
  const int pos = (n & ~3) | ((n & 1) << 1) | ((n >> 1) & 1);
  if (has) {
    ptile[4 * jg + 0][pos] = h;
    ptile[4 * jg + 1][pos] = r;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f16x4 pa = a_row_used ? *(const f16x4*)&ptile[n][4 * jg] : f16x4{0, 0, 0, 0};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s.acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, u.blo[q], s.acc[2 * q], 0, 0, 0);
    s.acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, u.bhi[q], s.acc[2 * q + 1], 0, 0, 0);
  }
}

// HPL heads per lane group: 1 (rows_i4_one: head jg, statistics and operands of slot 0) or 2
// (rows_i4: heads 2jg, 2jg+1).
template <int HPL>
__device__ __forceinline__ void process_page(const PageData<0>& pg, int valid0, int valid1, WaveState& s,
                                             const i32x4 (&qa)[4],
                                             float alpha0, float beta0, float alpha1, float beta1,
                                             bool has0, bool has1, int n, int jg, bool a_row_used,
                                             _Float16 (*ptile)[kPage]) {
  if constexpr (HPL == 1) {
    const i32x4 q2[2] = {qa[0], qa[1]};
    rows_i4_one(unpack_i4(pg, valid0, n), valid0, s, q2, alpha0, beta0, has0, n, jg, a_row_used, ptile);
  } else {
    rows_i4(unpack_i4(pg, max(valid0, valid1), n), valid0, valid1, s, qa, alpha0, beta0, alpha1, beta1, has0, has1,
            n, jg, a_row_used, ptile);
  }
}

// The A operands of the INT4 q.K tiles for lane row n (layouts above); limbs(l, g, a2) is the
// 16-byte operand a2 of limb l of head g for this lane's row group.
template <int HPL, typename Limbs>
__device__ __forceinline__ void q_tiles_i4(const Limbs& limbs, int G, int n, i32x4 (&qa)[4]) {
  const i32x4 zero = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int a2 = 0; a2 < 2; ++a2) {
    if constexpr (HPL == 1) {
      const int g = n >> 2, limb = n & 3;
      qa[a2] = (g < G && limb < 3) ? limbs(limb, g, a2) : zero;
      qa[2 + a2] = zero;
    } else {
      const int g = n >> 1, limb = n & 1;
      qa[a2] = g < G ? limbs(limb, g, a2) : zero;
      qa[2 + a2] = (g < G && limb == 0) ? limbs(2, g, a2) : zero;
    }
  }
}

// MXFP4 page: K and V are dequantized to fp16 tiles with their UE8M0 group scales by the gfx950
// fp4 conversion (two codes of one byte -> two fp16), then both contractions run on f16 MFMA.
//   q.K: v_mfma_f32_16x16x32_f16, A = q' as fp16 high/low parts (rows 2g, 2g+1), B = K tile;
//        dword kk of the lane's K chunk feeds MFMA kk: byte q -> channels (4jg+kk)+32q (+16),
//        all in channel group q (one scale).
//   p.V: v_mfma_f32_16x16x16_f16, A = p split high/low, B = V tile: byte r of V word q is token
//        4jg+r, channels n+32q and n+32q+16 (group q), repacked so one register holds two tokens.
struct KTileMx {
  f16x8 kb[4];
};

__device__ __forceinline__ KTileMx unpack_k_mx(const PageData<1>& pg, int e8sh) {
  KTileMx t;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t w = pg.k[kk];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x2 h2 = cvt_fp4(w, ue8m0_scale(pg.kp, 8 * q, e8sh), q);
      t.kb[kk][2 * q] = h2[0];
      t.kb[kk][2 * q + 1] = h2[1];
    }
  }
  return t;
}

__device__ __forceinline__ f32x4 scores_mx(const KTileMx& t, const f16x8 (&qh)[4]) {
  f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh[kk], t.kb[kk], sc, 0, 0, 0);
  return sc;
}

// The V tile of an MXFP4 page as fp16 B operands.  vlimit (wave-uniform): tokens of the page
// that exist in the sequence; the slots past it hold whatever the pool held, and their V scale
// is taken as 0: dequantized with a stray scale byte they could overflow fp16, and 0 * inf in
// the p.V contraction would poison every row even though their p is 0.
struct VTileMx {
  f16x4 blo[4], bhi[4];
};

__device__ __forceinline__ VTileMx unpack_v_mx(const PageData<1>& pg, int vlimit, int jg, int e8sh) {
  VTileMx t;
  uint32_t vw[4];  // the scale words of tokens 4jg .. 4jg+3, zero past the sequence's end
#pragma unroll
  for (int r = 0; r < 4; ++r) vw[r] = 4 * jg + r < vlimit ? pg.vp4[r] : 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t Y = pg.v[q];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f16x2 h2 = cvt_fp4(Y, ue8m0_scale(vw[r], 8 * q, e8sh), r);
      t.blo[q][r] = h2[0];
      t.bhi[q][r] = h2[1];
    }
  }
  return t;
}

typedef __attribute__((ext_vector_type(8))) int i32x8;

// The q.K scores of an MXFP4 page on the scaled matrix cores (UltraQuant article, section on how
// the method works: FP8 queries against FP4 KV with UE8M0 group scales on CDNA4's native scaled
// MFMA): v_mfma_scale_f32_16x16x128_f8f6f4 with A = q' as MXFP8 (e4m3 elements, one UE8M0 scale
// per 32 channels) and B = the stored e2m1 K codes with their stored UE8M0 bytes, no conversion.
//
// The MFMA takes one scale per (B column, 32-long K block), so a lane's 32 B nibbles must all be
// codes of one channel group.  A code row word a carries channel a + 16i in nibble i: byte q of
// every word belongs to group q.  group_codes() turns the 16 row bytes a lane loads (words
// 4jg..4jg+3 of token n) into the 32 codes of group jg of token n: a 4x4 byte transpose inside
// the lane (byte q of the four words -> dword q) and a 4x4 dword transpose across the four
// 16-lane rows (two permlane swap stages).  Dword k then holds byte jg of words 4k..4k+3, so B
// nibble i = 8k + 2w + h is channel 4k + w + 32jg + 16h; mxfp8_k_index() gives the A tiles the
// same order.
__device__ __forceinline__ u32x4 group_codes(const u32x4& w) {
  const uint32_t p01l = perm(w[1], w[0], 0x05010400u), p01h = perm(w[1], w[0], 0x07030602u);
  const uint32_t p23l = perm(w[3], w[2], 0x05010400u), p23h = perm(w[3], w[2], 0x07030602u);
  uint32_t s0 = perm(p23l, p01l, 0x05040100u), s1 = perm(p23l, p01l, 0x07060302u);
  uint32_t s2 = perm(p23h, p01h, 0x05040100u), s3 = perm(p23h, p01h, 0x07060302u);
  // dword q of lane row r is element (r, q) of a 4x4 matrix; transpose it: swap the off-diagonal
  // 2x2 blocks (rows 2,3 of dwords 0,1 <-> rows 0,1 of dwords 2,3), then the off-diagonal
  // elements inside each block (odd rows of dwords 0 / 2 <-> even rows of dwords 1 / 3)
  const auto x = __builtin_amdgcn_permlane32_swap(s0, s2, false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(s1, s3, false, false);
  const auto u = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
  const auto v = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
  return u32x4{u[0], u[1], v[0], v[1]};
}

// K index of channel ch in the scaled q.K contraction (the inverse of the order above)
__device__ __forceinline__ int mxfp8_k_index(int ch) {
  return (ch & ~31) + 8 * ((ch >> 2) & 3) + 2 * (ch & 3) + ((ch >> 4) & 1);
}

// q' of one head (channel `lane` in v0, `lane + 64` in v1) as three MXFP8 limbs: limb t is q'
// minus the limbs before it, in e4m3 with one UE8M0 scale per 32 channels (OCP MX rule:
// 2^(floor(log2 amax) - 8), elements rounded to nearest even and clamped at 448), subtracted as the
// matrix cores will decode it.  Limb t goes to A tile t/2, row 2g + t%2, bytes in K order;
// q8s[tile][row][group] gets its scales.  One scaled MFMA pass sums its products to ~2^-14 of the
// largest one, so three limbs (~12 bits) keep the scores as exact as that pass allows.
__device__ __forceinline__ void mxfp8_limbs(float v0, float v1, int g, int lane, uint8_t (*q8)[16][kHeadDim],
                                            uint8_t (*q8s)[16][4]) {
  // lanes 0-31 / 32-63 of v0 hold channel groups 0 / 1, of v1 groups 2 / 3
  const int k0 = mxfp8_k_index(lane), k1 = mxfp8_k_index(lane + 64);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float m0 = row_max16(fabsf(v0)), m1 = row_max16(fabsf(v1));
    m0 = fmaxf(m0, xor_lane<16>(m0, lane_id()));
    m1 = fmaxf(m1, xor_lane<16>(m1, lane_id()));
    const int e0 = min(max((int)((__float_as_uint(m0) >> 23) & 255u) - 8, 0), 254);
    const int e1 = min(max((int)((__float_as_uint(m1) >> 23) & 255u) - 8, 0), 254);
    const float y0 = fminf(fmaxf(ldexpf(v0, 127 - e0), -448.0f), 448.0f);
    const float y1 = fminf(fmaxf(ldexpf(v1, 127 - e1), -448.0f), 448.0f);
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    v0 -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 0), e0 - 127);
    v1 -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 1), e1 - 127);
    const int tile = t >> 1, row = 2 * g + (t & 1);
    q8[tile][row][k0] = (uint8_t)(pk & 255);
    q8[tile][row][k1] = (uint8_t)((pk >> 8) & 255);
    if ((lane & 31) == 0) {
      q8s[tile][row][lane >> 5] = (uint8_t)e0;
      q8s[tile][row][2 + (lane >> 5)] = (uint8_t)e1;
    }
  }
}

// A tiles of lane (jg, n): fp8 A operands hold K 16jg..16jg+15 in bytes 0-15 and K 64+16jg..
// in bytes 16-31, row n; the lane's scale is that of row n, K block (channel group) jg.  Tile 1
// uses its even rows only.
__device__ __forceinline__ void mxfp8_a_tiles(const uint8_t (*q8)[16][kHeadDim], const uint8_t (*q8s)[16][4],
                                              bool a_row_used, int limb, int n, int jg, i32x8 (&qa8)[2],
                                              int (&qsa)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool used = a_row_used && (t == 0 || limb == 0);
    const u32x4 lo = used ? *(const u32x4*)&q8[t][n][16 * jg] : u32x4{0, 0, 0, 0};
    const u32x4 hi = used ? *(const u32x4*)&q8[t][n][64 + 16 * jg] : u32x4{0, 0, 0, 0};
    qa8[t] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    qsa[t] = used ? (int)q8s[t][n][jg] : 127;
  }
}

__device__ __forceinline__ f32x4 scores_mx_scaled(const PageData<1>& pg, const i32x8 (&qa8)[2],
                                                  const int (&qsa)[2], int jg) {
  const int sb = (int)(pg.kp >> (8 * jg));  // the MFMA reads bits 7:0: group jg of token n
  const u32x4 c = group_codes(pg.k);
  const i32x8 kb = i32x8{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
  // format codes: 0 = fp8 e4m3 (A), 4 = fp4 e2m1 (B)
  f32x4 sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa8[0], kb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0,
                                                               qsa[0], 0, sb);
  sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa8[1], kb, sc, 0, 4, 0, qsa[1], 0, sb);
  return sc;
}

// Online softmax and p.V of an MXFP4 page, from its q.K scores (C layout: column n = token n,
// rows 4jg..4jg+3 = A rows 2g+part of heads 2jg, 2jg+1) and its V tile.
__device__ __forceinline__ void softmax_pv_mx(const VTileMx& vt, f32x4 sc, int valid0, int valid1, WaveState& s,
                                              float c2, bool has0, bool has1, int n, int jg, bool a_row_used,
                                              _Float16 (*ptile)[kPage]) {
  const bool tv0 = n < valid0, tv1 = n < valid1;
  float x0 = (sc[0] + sc[1]) * c2, x1 = (sc[2] + sc[3]) * c2;
  x0 = tv0 ? x0 : -INFINITY;
  x1 = tv1 ? x1 : -INFINITY;

  const float pm0 = row_max16(x0), pm1 = row_max16(x1);
  // p <= 2^8 stays far inside fp16 (no value scale is folded into p here)
  if (__any(pm0 > s.m0 + 8.0f || pm1 > s.m1 + 8.0f)) {
    const float mn0 = fmaxf(s.m0, pm0), mn1 = fmaxf(s.m1, pm1);
    const float f0 = __builtin_amdgcn_exp2f(s.m0 - mn0), f1 = __builtin_amdgcn_exp2f(s.m1 - mn1);
#pragma unroll
    for (int i = 0; i < 8; ++i) s.acc[i] *= f32x4{f0, f0, f1, f1};
    s.l0 *= f0;
    s.l1 *= f1;
    s.m0 = mn0;
    s.m1 = mn1;
  }
  const float p0 = __builtin_amdgcn_exp2f(x0 - s.m0), p1 = __builtin_amdgcn_exp2f(x1 - s.m1);
  s.l0 += p0;
  s.l1 += p1;

  // p as fp16 high + low parts at A-tile rows 2g+limb, natural token order (a masked score is
  // -inf: its p is exactly 0)
  const float pt0 = p0, pt1 = p1;
  const _Float16 h0 = (_Float16)pt0, h1 = (_Float16)pt1;
  const _Float16 r0 = (_Float16)(pt0 - (float)h0), r1 = (_Float16)(pt1 - (float)h1);
  if (has0) {
    ptile[4 * jg + 0][n] = h0;
    ptile[4 * jg + 1][n] = r0;
  }
  if (has1) {
    ptile[4 * jg + 2][n] = h1;
    ptile[4 * jg + 3][n] = r1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f16x4 pa = a_row_used ? *(const f16x4*)&ptile[n][4 * jg] : f16x4{0, 0, 0, 0};
  __builtin_amdgcn_wave_barrier();

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s.acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vt.blo[q], s.acc[2 * q], 0, 0, 0);
    s.acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vt.bhi[q], s.acc[2 * q + 1], 0, 0, 0);
  }
}

__device__ __forceinline__ void process_page_mx(const PageData<1>& pg, int valid0, int valid1, int vlimit,
                                                WaveState& s, const f16x8 (&qh)[4], float c2, bool has0, bool has1,
                                                int n, int jg, bool a_row_used, _Float16 (*ptile)[kPage], int e8sh) {
  softmax_pv_mx(unpack_v_mx(pg, vlimit, jg, e8sh), scores_mx(unpack_k_mx(pg, e8sh), qh), valid0, valid1, s, c2, has0,
                has1, n, jg, a_row_used, ptile);
}

// Two MXFP4 pages at once (pages a and b of the wave, ptile2 two p tiles): both pages' scores,
// one update of the running maxima for the pair, then both pages' p.V products.  The two pages'
// chains are independent, and the row reductions, the vote and the LDS round trip of p are
// paid once per pair.
__device__ __forceinline__ void process_pages_mx2(const PageData<1>& pa, const PageData<1>& pb, int valid_a,
                                                  int valid_b, WaveState& s, const f16x8 (&qh)[4], float c2, bool has0,
                                                  bool has1, int n, int jg, bool a_row_used,
                                                  _Float16 (*ptile2)[2 * kMaxG][kPage], int e8sh) {
  const VTileMx va = unpack_v_mx(pa, valid_a, jg, e8sh), vb = unpack_v_mx(pb, valid_b, jg, e8sh);
  const f32x4 sa = scores_mx(unpack_k_mx(pa, e8sh), qh), sb = scores_mx(unpack_k_mx(pb, e8sh), qh);
  const bool ta = n < valid_a, tb = n < valid_b;
  const float xa0 = ta ? (sa[0] + sa[1]) * c2 : -INFINITY, xa1 = ta ? (sa[2] + sa[3]) * c2 : -INFINITY;
  const float xb0 = tb ? (sb[0] + sb[1]) * c2 : -INFINITY, xb1 = tb ? (sb[2] + sb[3]) * c2 : -INFINITY;
  const float pm0 = row_max16(fmaxf(xa0, xb0)), pm1 = row_max16(fmaxf(xa1, xb1));
  // p <= 2^8 stays far inside fp16 (no value scale is folded into p here)
  if (__any(pm0 > s.m0 + 8.0f || pm1 > s.m1 + 8.0f)) {
    const float mn0 = fmaxf(s.m0, pm0), mn1 = fmaxf(s.m1, pm1);
    const float f0 = __builtin_amdgcn_exp2f(s.m0 - mn0), f1 = __builtin_amdgcn_exp2f(s.m1 - mn1);
#pragma unroll
    for (int i = 0; i < 8; ++i) s.acc[i] *= f32x4{f0, f0, f1, f1};
    s.l0 *= f0;
    s.l1 *= f1;
    s.m0 = mn0;
    s.m1 = mn1;
  }
  const float pa0 = __builtin_amdgcn_exp2f(xa0 - s.m0), pa1 = __builtin_amdgcn_exp2f(xa1 - s.m1);
  const float pb0 = __builtin_amdgcn_exp2f(xb0 - s.m0), pb1 = __builtin_amdgcn_exp2f(xb1 - s.m1);
  s.l0 += pa0 + pb0;
  s.l1 += pa1 + pb1;
  // p as fp16 high + low parts at A-tile rows 2g+limb of each page's tile (a masked score is
  // -inf: its p is exactly 0)
  const float pv[2][2] = {{pa0, pa1}, {pb0, pb1}};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const _Float16 h0 = (_Float16)pv[t][0], h1 = (_Float16)pv[t][1];
    const _Float16 r0 = (_Float16)(pv[t][0] - (float)h0), r1 = (_Float16)(pv[t][1] - (float)h1);
    if (has0) {
      ptile2[t][4 * jg + 0][n] = h0;
      ptile2[t][4 * jg + 1][n] = r0;
    }
    if (has1) {
      ptile2[t][4 * jg + 2][n] = h1;
      ptile2[t][4 * jg + 3][n] = r1;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f16x4 a0 = a_row_used ? *(const f16x4*)&ptile2[0][n][4 * jg] : f16x4{0, 0, 0, 0};
  const f16x4 a1 = a_row_used ? *(const f16x4*)&ptile2[1][n][4 * jg] : f16x4{0, 0, 0, 0};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s.acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, va.blo[q], s.acc[2 * q], 0, 0, 0);
    s.acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, va.bhi[q], s.acc[2 * q + 1], 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s.acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, vb.blo[q], s.acc[2 * q], 0, 0, 0);
    s.acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, vb.bhi[q], s.acc[2 * q + 1], 0, 0, 0);
  }
}

// p.V of an MXFP4 cache on the scaled matrix cores as well (UltraQuant article, section on how
// the method works: FP8-quantized attention weights against the FP4 V tensors with their UE8M0
// group scales): v_mfma_scale_f32_32x32x64_f8f6f4, 64 tokens (4 pages) per MFMA, one MFMA per V
// channel group of 32 (the output columns).  Operand layouts (checked on the device): A (e4m3)
// lane l is row l%32, bytes 0-15 hold K 16(l/32)+j and bytes 16-31 hold K 32+16(l/32)+j; B (e2m1)
// lane l is column l%32, nibble i (low nibble first) holds K 32(l/32)+i; each lane supplies the
// scale of its row / column for the 32-long K block l/32; D register i of lane l is row
// 8(i/4)+4(l/32)+i%4, column l%32.
//
// The V codes go in raw (B scale 1); V's UE8M0 scale belongs to (token, channel group), which the
// MFMA's per-(column, K block) B scale cannot express, so it moves into the A side:
// p~[h][t] = p[h][t] * 2^(E_v[t][group] - 127), one A operand per channel group.  p~ enters as
// three e4m3 limbs (rows 8(h/2)+4(h%2)+t of the A tile, t = limb; row t = 3 stays zero), each with
// one UE8M0 scale per 32 tokens: limb 0 scales the block's largest magnitude into [128, 256),
// limb t > 0 is what the limbs before it left, at 2^-4 of the previous scale (a bound on that
// remainder).  Three limbs keep ~11 bits of p~ relative to its block maximum.  Per page, the wave stages the V codes transposed (channel-major nibbles)
// and the V exponents in LDS; every fourth page it updates the running maximum once for the four
// pages, builds the limbs (lane 8h + 2g + kb: head h, channel group g, 32-token block kb) and
// runs the four MFMAs.
struct ScaledStage {
  uint8_t vt[4][32][32];   // V codes of group g, column c (channel 32g+c), 64 tokens as nibbles
  int32_t ve[4][64];       // V exponent - 127 of group g, token
  union {
    float p[kMaxG][64];              // p of the group's tokens, per head
    uint8_t a8[4][3 * kMaxG][64];    // e4m3 limbs of p~: group, row 3h+t, token
  };
  uint8_t as[4][3 * kMaxG][2];       // their UE8M0 scales per 32-token block
};

// Scores of one page on the scaled matrix cores, masked, into x0 / x1 (heads 2jg, 2jg+1 of
// token n), and the page's V codes and exponents staged for slot d of the 4-page group.
__device__ __forceinline__ void scaled_stage_page(const PageData<1>& pg, int valid, const i32x8 (&qa8)[2],
                                                  const int (&qsa)[2], float c2, int n, int jg, int d,
                                                  ScaledStage& st, float& x0, float& x1) {
  const f32x4 sc = scores_mx_scaled(pg, qa8, qsa, jg);
  const bool tv = n < valid;
  x0 = tv ? (sc[0] + sc[1]) * c2 : -INFINITY;
  x1 = tv ? (sc[2] + sc[3]) * c2 : -INFINITY;
  // V word q: row bytes 4n+q of tokens 4jg .. 4jg+3 (byte r: token 4jg+r); its low nibbles are
  // channel n+32q (column n of group q), its high nibbles channel n+32q+16 (column n+16).  The
  // four nibbles of a column go to token positions 16d+4jg .. +3: one 16-bit store.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t Y = pg.v[q];
    const uint32_t lo = Y & 0x0F0F0F0Fu, hi = (Y >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo2 = lo | (lo >> 4), hi2 = hi | (hi >> 4);  // bytes 0 and 2 hold the pairs
    *(uint16_t*)&st.vt[q][n][8 * d + 2 * jg] = (uint16_t)perm(0u, lo2, 0x0C0C0200u);
    *(uint16_t*)&st.vt[q][n + 16][8 * d + 2 * jg] = (uint16_t)perm(0u, hi2, 0x0C0C0200u);
  }
  // exponents of token 4jg + n (lanes n < 4), zero past the sequence's end: their p is 0 anyway,
  // and a stray byte then cannot matter
  if (n < 4) {
    const int t = 4 * jg + n;
    const uint32_t wn = n == 0 ? pg.vp4[0] : (n == 1 ? pg.vp4[1] : (n == 2 ? pg.vp4[2] : pg.vp4[3]));
    const uint32_t w = t < valid ? wn : 0x7F7F7F7Fu;
#pragma unroll
    for (int g = 0; g < 4; ++g) st.ve[g][16 * d + t] = (int)((w >> (8 * g)) & 255u) - 127;
  }
}

// p.V accumulators of the scaled path: one 32x32 tile per channel group.
struct ScaledAcc {
  f32x16 c[4];
};

// The 4-page group's softmax and p.V on the scaled matrix cores (layout above).  xs0 / xs1: the
// masked scores of the group's pages (heads 2jg, 2jg+1 of token n; -inf for pages past the
// wave's last).
__device__ __forceinline__ void scaled_flush(const float (&xs0)[4], const float (&xs1)[4], WaveState& s,
                                             ScaledAcc& acc, ScaledStage& st, int G, bool has0, bool has1, int n,
                                             int jg, int lane) {
  // ---- running maximum, once for the four pages (p <= 2^8 keeps every partial sum in range) ----
  const float pm0 = row_max16(fmaxf(fmaxf(xs0[0], xs0[1]), fmaxf(xs0[2], xs0[3])));
  const float pm1 = row_max16(fmaxf(fmaxf(xs1[0], xs1[1]), fmaxf(xs1[2], xs1[3])));
  if (__any(pm0 > s.m0 + 8.0f || pm1 > s.m1 + 8.0f)) {
    const float mn0 = fmaxf(s.m0, pm0), mn1 = fmaxf(s.m1, pm1);
    const float f0 = __builtin_amdgcn_exp2f(s.m0 - mn0), f1 = __builtin_amdgcn_exp2f(s.m1 - mn1);
    s.l0 *= f0;
    s.l1 *= f1;
    s.m0 = mn0;
    s.m1 = mn1;
    // accumulator rows of lane half b hold heads 2a + b (registers 4a .. 4a+3): head 2a is lane
    // group a's first head, 2a+1 its second
    const int b = lane >> 5;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float fa0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), 16 * a));
      const float fa1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f1), 16 * a));
      const float f = b ? fa1 : fa0;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 3; ++t) acc.c[g][4 * a + t] *= f;
    }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float p0 = __builtin_amdgcn_exp2f(xs0[d] - s.m0), p1 = __builtin_amdgcn_exp2f(xs1[d] - s.m1);
    s.l0 += p0;
    s.l1 += p1;
    if (has0) st.p[2 * jg][16 * d + n] = p0;
    if (has1) st.p[2 * jg + 1][16 * d + n] = p1;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- e4m3 limbs of p~ = p * 2^(E_v - 127): lane 8h + 2g + kb, 32 tokens ----
  const int h = lane >> 3, g = (lane >> 1) & 3, kb = lane & 1;
  float v[32];
  if (h < G) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x4 pv = *(const f32x4*)&st.p[h][32 * kb + 4 * w];
      const i32x4 ev = *(const i32x4*)&st.ve[g][32 * kb + 4 * w];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * w + r] = ldexpf(pv[r], ev[r]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  // every lane has read its p before any limb overwrites them (a8 shares their bytes)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // limb 0's UE8M0 scale: 2^(floor(log2 m) - 7) for the block's largest magnitude m, which then
  // scales into [128, 256), inside e4m3's range (448), so no element saturates.  A limb's rounding
  // error is at most half an e4m3 step in the binade of that maximum, i.e. 8 in the scaled units,
  // so the next limb's scale is 2^-4 of this one: its elements scale into (-128, 128)
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, v[i]);  // p~ >= 0
  int sc = max((int)((__float_as_uint(m) >> 23) & 255u) - 7, 0);
#pragma unroll
  for (int t = 0; t < 3; ++t, sc = max(sc - 4, 0)) {
    const float inv = ldexpf(1.0f, 127 - sc), scl = ldexpf(1.0f, sc - 127);
    uint32_t wd[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w] * inv, v[4 * w + 1] * inv, 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2] * inv, v[4 * w + 3] * inv, pk, true);
      wd[w] = (uint32_t)pk;
      if (t < 2) {
        const f32x2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false), d23 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
        v[4 * w + 0] = fmaf(-d01[0], scl, v[4 * w + 0]);
        v[4 * w + 1] = fmaf(-d01[1], scl, v[4 * w + 1]);
        v[4 * w + 2] = fmaf(-d23[0], scl, v[4 * w + 2]);
        v[4 * w + 3] = fmaf(-d23[1], scl, v[4 * w + 3]);
      }
    }
    if (h < G) {
      *(u32x4*)&st.a8[g][3 * h + t][32 * kb] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      *(u32x4*)&st.a8[g][3 * h + t][32 * kb + 16] = u32x4{wd[4], wd[5], wd[6], wd[7]};
      st.as[g][3 * h + t][kb] = (uint8_t)sc;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- the four MFMAs: A row r = 8(h/2) + 4(h%2) + t of lane r + 32 b ----
  const int r = lane & 31, b = lane >> 5;
  const int ha = 2 * (r >> 3) + ((r >> 2) & 1), ta = r & 3;
  const bool used = ta < 3 && ha < G;
  const int row = 3 * ha + ta;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    const u32x4 a0 = used ? *(const u32x4*)&st.a8[gg][row][16 * b] : u32x4{0, 0, 0, 0};
    const u32x4 a1 = used ? *(const u32x4*)&st.a8[gg][row][32 + 16 * b] : u32x4{0, 0, 0, 0};
    const int sa = used ? (int)st.as[gg][row][b] : 127;
    const u32x4 bv = *(const u32x4*)&st.vt[gg][r][16 * b];
    const i32x8 A = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 B = i32x8{(int)bv[0], (int)bv[1], (int)bv[2], (int)bv[3], 0, 0, 0, 0};
    // format codes: 0 = fp8 e4m3 (A), 4 = fp4 e2m1 (B); B scale 127 = 1
    acc.c[gg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc.c[gg], 0, 4, 0, sa, 0, 127);
  }
  // the operands are in registers before the next group's staging overwrites them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rotate one row's normalised o' (element lane in o0, lane + 64 in o1) back and store it at
// row `row` of a [rows][128] output of dtype `out_dtype`.
__device__ __forceinline__ void store_row(void* out, int64_t row, int out_dtype, int rotated, int had_block,
                                          const float* quat, int quat_full, float o0, float o1, int lane) {
  if (!rotated) unrotate_wave(o0, o1, had_block, quat, quat_full, lane);
  const int64_t base = row * kHeadDim;
  store_elem(out, base + lane, out_dtype, o0);
  store_elem(out, base + lane + 64, out_dtype, o1);
}

}  // namespace attn
}  // namespace kvq
