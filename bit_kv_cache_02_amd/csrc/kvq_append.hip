// kvq_append: fused block-diagonal Walsh-Hadamard rotation + token-wise 4-bit quantization +
// paged write (SAW-INT4 summary, "Summary"/"Method": a fused rotation-quantization kernel that
// writes straight into paged KV-cache layouts; UltraQuant article, section on how the method
// works: Walsh-Hadamard rotation before FP4 quantization with UE8M0 group scales).
//
// One wave owns one (sequence, page, kv head, K|V) page-head: the up-to-16 new tokens of that
// page.  The rotation y*sqrt(b) = X * H_b is a dense +-1 matrix product: it runs on the matrix
// cores as v_mfma_f32_16x16x32_{bf16,f16} (16 tokens x 128 channels times 128 x 128 signs).  The
// inputs are exact bf16/fp16 values and the signs are exact, so every product is exact and only
// the fp32 accumulation rounds.  The MFMA output leaves lane l with tokens 4*(l/16)+r (r = 0..3)
// and channels 16*nb + l%16 (nb = 0..7); the page layout is chosen so that this is exactly what
// a lane stores: a 4-byte K row word per token, and a 16-byte V word for a quad of tokens.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

template <bool BF16>
struct Sign {
  static constexpr uint16_t kPlus = BF16 ? 0x3F80 : 0x3C00;
  static constexpr uint16_t kMinus = BF16 ? 0xBF80 : 0xBC00;
};

// Pack the low bytes of eight "magic-rounded" code words (0x4B400000 + c, c in 0..15) into one
// code row word: byte q = c[2q] | c[2q+1] << 4.
__device__ __forceinline__ uint32_t pack8(const uint32_t* c) {
  uint32_t even = perm(c[2], c[0], 0x0C0C0400u) | perm(c[6], c[4], 0x04000C0Cu);
  uint32_t odd = perm(c[3], c[1], 0x0C0C0400u) | perm(c[7], c[5], 0x04000C0Cu);
  return even | (odd << 4);
}

// Round |r| (< 8) to the e2m1 grid {0,.5,1,1.5,2,3,4,6}: nearest, ties to the even index,
// saturating at 6.  Adding then subtracting 2^22/2^23/2^24 rounds to steps 0.5/1/2 (RNE).
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  float m = fabsf(r);
  float c = m < 2.0f ? 4194304.0f : (m < 4.0f ? 8388608.0f : 16777216.0f);
  float v = __builtin_fminf((m + c) - c, 6.0f);
  uint32_t idx = v < 1.0f ? (uint32_t)(v * 2.0f) : ((__float_as_uint(v) >> 22) - 252u);
  return idx | (r < 0.0f ? 8u : 0u);
}

}  // namespace

template <bool BF16, int HB, int FMT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hk = blockIdx.z * 4 + wave;  // (K|V, kv head) combination
  if (hk >= 2 * a.hkv) return;
  const int is_v = hk >= a.hkv;
  const int h = is_v ? hk - a.hkv : hk;
  const int b = blockIdx.y;
  const int j = blockIdx.x;

  const int t0 = a.cu_new[b];
  const int n_new = min(a.cu_new[b + 1] - t0, a.max_new);
  if (n_new <= 0) return;
  const int s0 = a.start_pos[b];
  const int page_idx = s0 / kPage + j;
  const int pos0 = page_idx * kPage;
  if (pos0 >= s0 + n_new) return;
  const int slot_lo = max(s0 - pos0, 0);
  const int slot_hi = min(s0 + n_new - pos0, kPage);
  const int page_id = a.block_table[(int64_t)b * a.max_pages + page_idx];

  const int n = lane & 15;   // MFMA column / row of the tile this lane feeds
  const int kg = lane >> 4;  // lane group

  // ---- load 16 tokens x 128 channels as the MFMA A operand (zeros for slots not appended) ----
  const uint8_t* src = is_v ? a.v : a.k;
  const int slot_a = n;  // A row = token slot
  const bool valid_a = slot_a >= slot_lo && slot_a < slot_hi;
  u32x4 xa[4];
  {
    const int64_t tok = (int64_t)t0 + pos0 + slot_a - s0;
    const uint8_t* row = src + (tok * a.hkv + h) * (int64_t)(kHeadDim * 2) + kg * 16;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (valid_a) xa[kb] = *(const u32x4*)(row + kb * 64);
      else xa[kb] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- B tiles: signs of H (or the identity for HB = 1) for this lane's (k, n) entries ----
  // Entry (k, n) of tile (kb, nb) is H[32kb + k][16nb + n]; the sign factors into a base pattern
  // that depends on nb&1 and a global sign that depends on (kb, nb).
  uint32_t tp[2][4], tm[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word_p = 0, word_m = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k = 8 * kg + 2 * w + half;
        uint16_t vp, vm;
        if (HB == 1) {
          vp = (k == 16 * p + n) ? Sign<BF16>::kPlus : 0;
          vm = vp;
        } else {
          const int par = (popc((uint32_t)((k & 15) & n)) + ((k >> 4) & p)) & 1;
          vp = par ? Sign<BF16>::kMinus : Sign<BF16>::kPlus;
          vm = par ? Sign<BF16>::kPlus : Sign<BF16>::kMinus;
        }
        word_p |= (uint32_t)vp << (16 * half);
        word_m |= (uint32_t)vm << (16 * half);
      }
      tp[p][w] = word_p;
      tm[p][w] = word_m;
    }
  }

  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      bool use;
      int neg;
      if (HB == 128) {
        use = true;
        neg = popc((uint32_t)(kb & (nb >> 1))) & 1;
      } else if (HB == 64) {
        use = (kb >> 1) == (nb >> 2);
        neg = (kb & 1) & ((nb >> 1) & 1);
      } else {
        use = kb == (nb >> 1);
        neg = 0;
      }
      if (!use) continue;
      const uint32_t* t = neg ? tm[nb & 1] : tp[nb & 1];
      u32x4 bt = u32x4{t[0], t[1], t[2], t[3]};
      if (BF16) {
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[kb]),
                                                          __builtin_bit_cast(bf16x8, bt), acc[nb], 0, 0, 0);
      } else {
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, xa[kb]),
                                                         __builtin_bit_cast(f16x8, bt), acc[nb], 0, 0, 0);
      }
    }
  }

  // acc[nb][r] = sqrt(b) * y[token slot 4*kg + r][channel 16*nb + n]
  constexpr float inv_sqrt_b = HB == 128 ? 0.08838834764831845f : (HB == 64 ? 0.125f : 1.0f);

  uint32_t rowword[4];   // K-row word of each of this lane's 4 token slots
  uint32_t paramword[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (FMT == 0) {
      // token-wise asymmetric INT4: fp16 scale = (max - min)/15, fp16 zero = min
      float mn = acc[0][r], mx = acc[0][r];
#pragma unroll
      for (int nb = 1; nb < 8; ++nb) {
        mn = fminf(mn, acc[nb][r]);
        mx = fmaxf(mx, acc[nb][r]);
      }
      mn = row_min16(mn);
      mx = row_max16(mx);
      const float lo = mn * inv_sqrt_b;
      const float hi = mx * inv_sqrt_b;
      const uint32_t s_bits = f32_to_f16_bits((hi - lo) / 15.0f);
      const uint32_t z_bits = f32_to_f16_bits(lo);
      const float sf = f16_bits_to_f32(s_bits);
      const float zf = f16_bits_to_f32(z_bits);
      const float inv_s = sf > 0.0f ? 1.0f / sf : 0.0f;
      uint32_t cw[8];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const float t = fmaf(acc[nb][r], inv_sqrt_b, -zf);
        const float d = __builtin_amdgcn_fmed3f(t * inv_s, 0.0f, 15.0f);
        cw[nb] = __float_as_uint(d + 12582912.0f);  // 1.5 * 2^23: round to nearest even
      }
      rowword[r] = pack8(cw);
      paramword[r] = s_bits | (z_bits << 16);
    } else {
      // MXFP4: e2m1 codes, UE8M0 exponent per 32 channels (nb pairs {2g, 2g+1})
      uint32_t cw[8];
      uint32_t ebytes = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float y0 = acc[2 * g][r] * inv_sqrt_b;
        const float y1 = acc[2 * g + 1][r] * inv_sqrt_b;
        const float amax = row_max16(fmaxf(fabsf(y0), fabsf(y1)));
        const int e = min(max((int)((__float_as_uint(amax) >> 23) & 255u) - 2, 0), 254);
        ebytes |= (uint32_t)e << (8 * g);
        cw[2 * g] = e2m1_code(ldexpf(y0, 127 - e));
        cw[2 * g + 1] = e2m1_code(ldexpf(y1, 127 - e));
      }
      uint32_t word = 0;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) word |= cw[nb] << (4 * nb);
      rowword[r] = word;
      paramword[r] = ebytes;
    }
  }

  // ---- paged stores ----
  uint8_t* base = a.pool + ((int64_t)page_id * a.hkv + h) * (int64_t)kPageHeadBytes;
  const int slot0 = 4 * kg;
  if (!is_v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = slot0 + r;
      if (s >= slot_lo && s < slot_hi) *(uint32_t*)(base + 64 * s + 4 * n) = rowword[r];
    }
  } else {
    // transpose the 4x4 bytes: V word q holds row byte (4n + q) of slots slot0..slot0+3
    const uint32_t a01 = perm(rowword[1], rowword[0], 0x05010400u);
    const uint32_t b01 = perm(rowword[1], rowword[0], 0x07030602u);
    const uint32_t a23 = perm(rowword[3], rowword[2], 0x05010400u);
    const uint32_t b23 = perm(rowword[3], rowword[2], 0x07030602u);
    u32x4 vw;
    vw[0] = perm(a23, a01, 0x05040100u);
    vw[1] = perm(a23, a01, 0x07060302u);
    vw[2] = perm(b23, b01, 0x05040100u);
    vw[3] = perm(b23, b01, 0x07060302u);
    uint8_t* dst = base + kVCodesOff + 256 * kg + 16 * n;
    if (slot0 >= slot_lo && slot0 + 4 <= slot_hi) {
      *(u32x4*)dst = vw;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = slot0 + r;
        if (s >= slot_lo && s < slot_hi) {
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[4 * q + r] = (uint8_t)(vw[q] >> (8 * r));
        }
      }
    }
  }
  if (n == 0) {
    uint8_t* pdst = base + (is_v ? kVParamsOff : kKParamsOff) + 4 * slot0;
    if (slot0 >= slot_lo && slot0 + 4 <= slot_hi) {
      *(u32x4*)pdst = u32x4{paramword[0], paramword[1], paramword[2], paramword[3]};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = slot0 + r;
        if (s >= slot_lo && s < slot_hi) *(uint32_t*)(pdst + 4 * r) = paramword[r];
      }
    }
  }
}

template <bool BF16, int HB, int FMT>
static hipError_t launch_t(const AppendParams& p, int grid_x, hipStream_t stream) {
  dim3 grid(grid_x, p.num_seqs, (2 * p.hkv + 3) / 4);
  hipLaunchKernelGGL((append_kernel<BF16, HB, FMT>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, bool bf16, int had_block, int fmt, hipStream_t stream) {
  // pages one sequence's new tokens can touch: ceil(max_new/16), plus one when misaligned
  const int grid_x = (p.max_new + kPage - 1) / kPage + 1;
#define KVQ_APPEND_CASE(BF, HBV, F) \
  if (bf16 == BF && had_block == HBV && fmt == F) return launch_t<BF, HBV, F>(p, grid_x, stream);
  KVQ_APPEND_CASE(true, 128, 0)
  KVQ_APPEND_CASE(true, 64, 0)
  KVQ_APPEND_CASE(true, 1, 0)
  KVQ_APPEND_CASE(false, 128, 0)
  KVQ_APPEND_CASE(false, 64, 0)
  KVQ_APPEND_CASE(false, 1, 0)
  KVQ_APPEND_CASE(true, 128, 1)
  KVQ_APPEND_CASE(true, 1, 1)
  KVQ_APPEND_CASE(false, 128, 1)
  KVQ_APPEND_CASE(false, 1, 1)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
