// kvq_decode_attn: paged decode attention that reads the rotated 4-bit cache and dequantizes in
// registers (SAW-INT4 summary, "Summary": attention served from paged 4-bit KV; UltraQuant
// article, section on how the method works: queries attend over 4-bit KV with group scales).
//
// A workgroup (4 waves) owns one (sequence, kv head, split): a run of pages of one sequence.
// Per page (16 tokens x 128 channels, one 2176-byte page-head block) each wave does:
//   scores   S[g][t] = sk_t * (q'_g . c_t) + zk_t * sum(q'_g)      (INT4: y^ = s*c + z)
//            q'_g . c_t runs on v_mfma_i32_16x16x64_i8 straight on the 4-bit codes: q' is held as
//            a 16-bit fixed-point number split into two int8 limbs (rows 2g, 2g+1 of the A tile),
//            so the contraction is exact integer arithmetic;
//   softmax  online, in the log2 domain; DPP row reductions over the 16 tokens;
//   p.V      O'[g][ch] += sum_t (p_t sv_t) c_t[ch] + sum_t p_t zv_t
//            sum_t (p_t sv_t) c_t runs on v_mfma_f32_16x16x16_f16: the codes enter as the exact
//            fp16 subnormals c * 2^-24 (a mask of the nibbles, no conversion), p_t*sv_t enters
//            split into an fp16 high part and an fp16 low part (rows 2g and 2g+1), which keeps
//            ~22 bits of it.
// The page layout puts V codes of four consecutive tokens in one 32-bit word per row byte, which
// is the B-operand shape of the p.V MFMA, so one 16-byte load per lane feeds it directly.
// The waves' partials merge in LDS; with several splits per (sequence, kv head) the last
// workgroup to finish merges the splits (arrival counter in the workspace).  The output is
// rotated back with an in-LDS fp32 Walsh-Hadamard butterfly.
#include "kvq_device.h"
#include "kvq_internal.h"

#include <stdlib.h>

namespace kvq {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxG = 8;
constexpr float kNegBig = -1.0e30f;

struct DecodeSmem {
  float qf[kMaxG][kHeadDim];
  float qdelta[kMaxG];
  float qsum[kMaxG];
  float ptile[kWaves][kMaxG][kPage];
  float wo[kWaves][kMaxG][kHeadDim];
  float wm[kWaves][kMaxG];
  float wl[kWaves][kMaxG];
  int is_last;
};

__device__ __forceinline__ float inv_sqrt_block(int hb) {
  return hb == 128 ? 0.08838834764831845f : (hb == 64 ? 0.125f : 1.0f);
}

// In-place unnormalised Walsh-Hadamard transform of G rows of 128 floats in LDS over blocks of hb
// channels (natural Sylvester order).  Callers synchronise before; returns synchronised.
__device__ void fwht_rows(float* x, int rows, int hb, int tid, int nthreads) {
  for (int len = 1; len < hb; len <<= 1) {
    for (int i = tid; i < rows * 64; i += nthreads) {
      const int g = i >> 6, k = i & 63;
      const int jj = (k / len) * 2 * len + (k % len);
      float* r = x + g * kHeadDim;
      const float u = r[jj], v = r[jj + len];
      r[jj] = u + v;
      r[jj + len] = u - v;
    }
    __syncthreads();
  }
}

}  // namespace

template <int FMT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams a) {
  __shared__ DecodeSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nsplit = a.plan.nsplit;
  const int P = a.plan.pages_per_split;
  const int split = blockIdx.x % nsplit;
  const int unit = blockIdx.x / nsplit;
  const int kvh = unit % a.hkv;
  const int b = unit / a.hkv;
  const int G = a.group;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const int p_begin = split * P;
  if (p_begin >= n_pages) return;  // uniform over the workgroup
  const int p_end = min(p_begin + P, n_pages);
  const int nsplit_b = (n_pages + P - 1) / P;
  const float isb = inv_sqrt_block(a.had_block);

  // ---- 1. q' = R_b (q_scale q) for the G query heads of this kv head ----
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int g = i >> 7, d = i & 127;
    sm.qf[g][d] = a.q_scale * load_elem(a.q, ((int64_t)b * a.hq + kvh * G + g) * kHeadDim + d, a.q_dtype);
  }
  __syncthreads();
  fwht_rows(&sm.qf[0][0], G, a.had_block, tid, 256);

  // ---- 2. q' as 16-bit fixed point per head: q' ~= delta_g * Q, |Q| <= 32000 ----
  for (int g = wave; g < G; g += kWaves) {
    const float v0 = sm.qf[g][lane] * isb, v1 = sm.qf[g][lane + 64] * isb;
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float delta = amax > 0.0f ? amax / 32000.0f : 1.0f;
    const int q0 = (int)rintf(v0 / delta), q1 = (int)rintf(v1 / delta);
    const int qs = wave_sum_i(q0 + q1);
    sm.qf[g][lane] = (float)q0;
    sm.qf[g][lane + 64] = (float)q1;
    if (lane == 0) {
      sm.qdelta[g] = delta;
      sm.qsum[g] = delta * (float)qs;  // sum of the q' actually used
    }
  }
  __syncthreads();

  const int n = lane & 15;     // token (QK, softmax) / output column (p.V)
  const int jg = lane >> 4;    // row group: heads 2jg, 2jg+1
  const int ga = n >> 1;       // A-tile row 2g+limb -> head of this lane's A row
  const int limb = n & 1;      // 0: high limb / high fp16 part, 1: low
  // A tile of the q.K MFMA: byte p = 4w+q2 of operand a2 is channel (4jg+w) + 32q2 + 16a2, which is
  // where the K row word that lane group jg loads keeps that channel after the nibble split.
  i32x4 qa[2];
#pragma unroll
  for (int a2 = 0; a2 < 2; ++a2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
      if (ga < G) {
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int Q = (int)sm.qf[ga][4 * jg + w + 32 * q2 + 16 * a2];
          const int hi = (Q + 128) >> 8;
          const int lo = Q - 256 * hi;
          word |= (uint32_t)((limb == 0 ? hi : lo) & 255) << (8 * q2);
        }
      }
      qa[a2][w] = (int)word;
    }
  }
  const int g0 = 2 * jg, g1 = 2 * jg + 1;
  const bool has0 = g0 < G, has1 = g1 < G;
  const float c2 = a.sm_scale_log2;
  const float alpha0 = has0 ? sm.qdelta[g0] * c2 : 0.0f, beta0 = has0 ? sm.qsum[g0] * c2 : 0.0f;
  const float alpha1 = has1 ? sm.qdelta[g1] * c2 : 0.0f, beta1 = has1 ? sm.qsum[g1] * c2 : 0.0f;

  // ---- 3. stream this wave's pages ----
  const int chunk = (p_end - p_begin + kWaves - 1) / kWaves;
  const int wp0 = p_begin + wave * chunk;
  const int wp1 = min(wp0 + chunk, p_end);
  float mrun0 = kNegBig, mrun1 = kNegBig;
  float l0 = 0.f, l1 = 0.f, pz0 = 0.f, pz1 = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int64_t head_off = (int64_t)kvh * kPageHeadBytes;
  const int64_t page_stride = (int64_t)a.hkv * kPageHeadBytes;
  const uint32_t M4 = 0x0F0F0F0Fu, M16 = 0x000F000Fu;

  for (int p = wp0; p < wp1; ++p) {
    const uint8_t* base = a.pool + (int64_t)bt[p] * page_stride + head_off;
    const u32x4 kv4 = *(const u32x4*)(base + 64 * n + 16 * jg);
    const u32x4 vv4 = *(const u32x4*)(base + kVCodesOff + 16 * lane);
    const uint32_t kp = *(const uint32_t*)(base + kKParamsOff + 4 * n);
    const uint32_t vp = *(const uint32_t*)(base + kVParamsOff + 4 * n);
    const bool tv = n < L - p * kPage;

    // q'.c_t on the integer matrix cores
    const i32x4 kb0 = i32x4{(int)(kv4[0] & M4), (int)(kv4[1] & M4), (int)(kv4[2] & M4), (int)(kv4[3] & M4)};
    const i32x4 kb1 = i32x4{(int)((kv4[0] >> 4) & M4), (int)((kv4[1] >> 4) & M4), (int)((kv4[2] >> 4) & M4),
                            (int)((kv4[3] >> 4) & M4)};
    i32x4 s = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[0], kb0, i32x4{0, 0, 0, 0}, 0, 0, 0);
    s = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[1], kb1, s, 0, 0, 0);

    const float sk = f16_bits_to_f32(kp & 0xFFFFu), zk = f16_bits_to_f32(kp >> 16);
    float x0 = fmaf((float)(s[0] * 256 + s[1]) * alpha0, sk, zk * beta0);
    float x1 = fmaf((float)(s[2] * 256 + s[3]) * alpha1, sk, zk * beta1);
    x0 = tv ? x0 : -INFINITY;
    x1 = tv ? x1 : -INFINITY;

    const float mn0 = fmaxf(mrun0, row_max16(x0));
    const float mn1 = fmaxf(mrun1, row_max16(x1));
    const float f0 = exp2f(mrun0 - mn0), f1 = exp2f(mrun1 - mn1);
    if (__any(f0 < 1.0f || f1 < 1.0f)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][0] *= f0;
        acc[i][1] *= f0;
        acc[i][2] *= f1;
        acc[i][3] *= f1;
      }
    }
    mrun0 = mn0;
    mrun1 = mn1;
    const float p0 = exp2f(x0 - mn0), p1 = exp2f(x1 - mn1);
    const float sv = f16_bits_to_f32(vp & 0xFFFFu), zv = f16_bits_to_f32(vp >> 16);
    l0 = fmaf(l0, f0, p0);
    l1 = fmaf(l1, f1, p1);
    pz0 = tv ? fmaf(p0, zv, pz0 * f0) : pz0 * f0;
    pz1 = tv ? fmaf(p1, zv, pz1 * f1) : pz1 * f1;

    // p~ = p * sv, moved from the (token-lane) softmax layout to the A layout of the p.V MFMA
    if (has0) sm.ptile[wave][g0][n] = tv ? p0 * sv : 0.0f;
    if (has1) sm.ptile[wave][g1][n] = tv ? p1 * sv : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f16x4 pa = f16x4{0, 0, 0, 0};
    if (ga < G) {
      const f32x4 pv = *(const f32x4*)&sm.ptile[wave][ga][4 * jg];
      const float v4[4] = {pv[0], pv[2], pv[1], pv[3]};  // k order of the V words: t0, t2, t1, t3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const _Float16 hi = (_Float16)v4[i];
        pa[i] = limb == 0 ? hi : (_Float16)(v4[i] - (float)hi);
      }
    }
    __builtin_amdgcn_wave_barrier();

    // V codes as fp16 subnormals c*2^-24: word q of the lane holds row byte 4n+q of 4 tokens
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t Y = vv4[q];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w0 = (Y >> (4 * e)) & M16;       // tokens 0, 2
        const uint32_t w1 = (Y >> (8 + 4 * e)) & M16;   // tokens 1, 3
        const f16x4 bv = __builtin_bit_cast(f16x4, u32x2{w0, w1});
        acc[2 * q + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, bv, acc[2 * q + e], 0, 0, 0);
      }
    }
  }

  // ---- 4. wave partial -> LDS ----
  l0 = row_sum16(l0);
  l1 = row_sum16(l1);
  pz0 = row_sum16(pz0);
  pz1 = row_sum16(pz1);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = n + 32 * q + 16 * e;
      const f32x4 v = acc[2 * q + e];
      if (has0) sm.wo[wave][g0][ch] = 16777216.0f * (v[0] + v[1]) + pz0;
      if (has1) sm.wo[wave][g1][ch] = 16777216.0f * (v[2] + v[3]) + pz1;
    }
  }
  if (n == 0) {
    if (has0) { sm.wm[wave][g0] = mrun0; sm.wl[wave][g0] = l0; }
    if (has1) { sm.wm[wave][g1] = mrun1; sm.wl[wave][g1] = l1; }
  }
  __syncthreads();

  // ---- 5. merge the waves; then either finish or hand over a split partial ----
  float* fo = &sm.qf[0][0];  // reuse: final o' [G][128]
  const int64_t slot = (int64_t)unit * nsplit + split;
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int g = i >> 7, ch = i & 127;
    float M = sm.wm[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][g]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(sm.wm[w][g] - M);
      O = fmaf(f, sm.wo[w][g][ch], O);
      Ls = fmaf(f, sm.wl[w][g], Ls);
    }
    if (nsplit_b == 1) {
      fo[i] = O / Ls;
    } else {
      a.part_o[(slot * G + g) * kHeadDim + ch] = O;
      if (ch == 0) {
        a.part_ml[(slot * G + g) * 2 + 0] = M;
        a.part_ml[(slot * G + g) * 2 + 1] = Ls;
      }
    }
  }
  if (nsplit_b > 1) {
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&a.counters[unit], 1);
      sm.is_last = prev == nsplit_b - 1;
    }
    __syncthreads();
    if (!sm.is_last) return;
    __threadfence();
    const int64_t s0 = (int64_t)unit * nsplit;
    for (int i = tid; i < G * kHeadDim; i += 256) {
      const int g = i >> 7, ch = i & 127;
      float M = kNegBig;
      for (int s = 0; s < nsplit_b; ++s) M = fmaxf(M, a.part_ml[((s0 + s) * G + g) * 2]);
      float O = 0.f, Ls = 0.f;
      for (int s = 0; s < nsplit_b; ++s) {
        const float f = exp2f(a.part_ml[((s0 + s) * G + g) * 2] - M);
        O = fmaf(f, a.part_o[((s0 + s) * G + g) * kHeadDim + ch], O);
        Ls = fmaf(f, a.part_ml[((s0 + s) * G + g) * 2 + 1], Ls);
      }
      fo[i] = O / Ls;
    }
    if (tid == 0) a.counters[unit] = 0;
  }
  __syncthreads();

  // ---- 6. rotate back (o = R_b o') and store ----
  float oscale = 1.0f;
  if (!a.out_rotated) {
    fwht_rows(fo, G, a.had_block, tid, 256);
    oscale = isb;
  }
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int g = i >> 7, ch = i & 127;
    store_elem(a.out, ((int64_t)b * a.hq + kvh * G + g) * kHeadDim + ch, a.out_dtype, fo[i] * oscale);
  }
}

DecodePlan plan_decode(int num_seqs, int hkv, int max_seq_len) {
  DecodePlan plan;
  plan.waves = kWaves;
  const int max_pg = (max_seq_len + kPage - 1) / kPage;
  const int64_t units = (int64_t)num_seqs * hkv;
  int target = 1024;
  if (const char* env = getenv("KVQ_DECODE_TARGET_WGS")) target = atoi(env);
  int P = 256;
  if (const char* env = getenv("KVQ_DECODE_PAGES_PER_SPLIT")) {
    P = atoi(env);
  } else {
    while (P > 16 && units * ((max_pg + P / 2 - 1) / (P / 2)) <= target) P /= 2;
  }
  if (P < 4) P = 4;
  plan.pages_per_split = P;
  plan.nsplit = max_pg > 0 ? (max_pg + P - 1) / P : 1;
  return plan;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int hkv, int group) {
  if (plan.nsplit <= 1) return 0;
  const size_t units = (size_t)num_seqs * hkv;
  const size_t slots = units * plan.nsplit;
  return align256(units * 4) + align256(slots * group * 2 * 4) + slots * group * kHeadDim * 4;
}

void carve_workspace(void* ws, const DecodePlan& plan, int num_seqs, int hkv, int group,
                     int32_t** counters, float** part_ml, float** part_o) {
  const size_t units = (size_t)num_seqs * hkv;
  const size_t slots = units * plan.nsplit;
  uint8_t* p = (uint8_t*)ws;
  *counters = (int32_t*)p;
  p += align256(units * 4);
  *part_ml = (float*)p;
  p += align256(slots * group * 2 * 4);
  *part_o = (float*)p;
}

hipError_t launch_decode(const DecodeParams& p, int fmt, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_seqs * p.hkv * p.plan.nsplit;
  if (fmt == 0) {
    hipLaunchKernelGGL(decode_kernel<0>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;  // MXFP4 decode is provided by its own kernel file
  }
  return hipGetLastError();
}

}  // namespace kvq
