// kvq_append: fused block-diagonal Walsh-Hadamard rotation + token-wise 4-bit quantization +
// paged write (SAW-INT4 summary, "Summary"/"Method": a fused rotation-quantization kernel that
// writes straight into paged KV-cache layouts; UltraQuant article, section on how the method
// works: Walsh-Hadamard rotation before FP4 quantization with UE8M0 group scales).
//
// One wave owns one (sequence, kv head, K|V) and walks kAppendPagesPerWave consecutive pages of
// it, loading the next page's tokens while it quantizes the current one.  Per page the rotation
// y*sqrt(b) = H_b^T X^T is a dense +-1 matrix product on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}: 128 x 128 signs times 128 channels x 16 tokens).  The inputs
// are exact bf16/fp16 values and the signs are exact, so every product is exact and only the
// fp32 accumulation rounds.  With the signs as the A operand the output tile nb leaves lane l
// with channels 16*nb + 4*(l/16) + r (r = 0..3) of token slot l%16: each lane holds 32 channels
// of one token, so the token-wise min/max is a 32-value in-lane reduction plus two cross-lane
// steps, and the per-token scale arithmetic runs once per lane.  The same lane holds exactly
// K row words 4*(l/16) .. 4*(l/16)+3 of its token (word a carries channels a + 16i in nibble i),
// which it stores as one 16-byte write; V rows are exchanged inside lane quads (DPP) so that
// each lane writes one 16-byte piece of the token-interleaved V block.
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

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// 4x4 word transpose across the lanes of a quad: afterwards lane m holds in w[r] what lane r held
// in w[m].  Two exchange stages (partner m^1, then m^2), each swapping the off-diagonal halves.
__device__ __forceinline__ void quad_transpose(uint32_t (&w)[4], int m) {
  const bool b0 = m & 1, b1 = m & 2;
#pragma unroll
  for (int r = 0; r < 4; r += 2) {
    const uint32_t recv = dpp_u<kQuadSwap1>(b0 ? w[r] : w[r + 1]);
    if (b0) w[r] = recv;
    else w[r + 1] = recv;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t recv = dpp_u<kQuadSwap2>(b1 ? w[r] : w[r + 2]);
    if (b1) w[r] = recv;
    else w[r + 2] = recv;
  }
}

}  // namespace

template <bool BF16, int HB, int FMT>
__global__ __launch_bounds__(256) void append_kernel(AppendParams a) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  const int hk = block_id_z() * 4 + wave;  // (K|V, kv head) combination
  if (hk >= 2 * a.hkv) return;
  const int is_v = hk >= a.hkv;
  const int h = is_v ? hk - a.hkv : hk;
  const int b = block_id_y();

  const int t0 = a.cu_new[b];
  const int n_new = min(a.cu_new[b + 1] - t0, a.max_new);
  if (n_new <= 0) return;
  const int s0 = a.start_pos[b];
  const int end_pos = s0 + n_new;
  const int pg_begin = s0 / kPage + block_id_x() * kAppendPagesPerWave;
  const int pg_end = min(pg_begin + kAppendPagesPerWave, (end_pos - 1) / kPage + 1);
  if (pg_begin >= pg_end) return;

  // page ids of this wave's pages, one per lane (read back with readlane): one load up front
  // instead of a dependent load per page
  const int npg = pg_end - pg_begin;
  const int page_ids = lane < npg ? a.block_table[(int64_t)b * a.max_pages + pg_begin + lane] : 0;

  const int n = lane & 15;  // token slot of this lane (B column, output column)
  const int g = lane >> 4;  // lane group: input channels 8g.. of each 32-block, output rows 4g..

  // ---- A tiles: signs of H (or the identity for HB = 1) for this lane's (row n, k) entries ----
  // Entry (n, k) of tile (kb, nb) is H[32kb + k][16nb + n]; the sign factors into a base pattern
  // that depends on nb&1 and a global sign that depends on (kb, nb).
  uint32_t tp[2][4], tm[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word_p = 0, word_m = 0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k = 8 * g + 2 * w + half;
        uint16_t vp, vm;
        if (HB == 1 || HB == kQuatBlock) {
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

  // quaternion block rotation: each wave stages the 32 block matrices in its own LDS slice (lane
  // k < 32 builds block k), so no workgroup barrier is needed after the early exits above
  __shared__ __attribute__((aligned(16))) float qm[HB == kQuatBlock ? 4 : 1][HB == kQuatBlock ? kHeadDim / 4 : 1][4][4];
  if constexpr (HB == kQuatBlock) {
    if (lane < kHeadDim / 4) {
      float c[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        quat_coeffs(a.quat, a.quat_full, lane, r, false, c);
        *(f32x4*)&qm[wave][lane][r][0] = f32x4{c[0], c[1], c[2], c[3]};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  const uint8_t* src = is_v ? a.v : a.k;
  const int row_stride = a.hkv * (kHeadDim * 2);  // bytes from one token's row to the next
  // Every page step issues the same buffer loads and stores whatever its slots: lanes with
  // nothing to move use an offset past the end of the buffer range (loads return zero, stores
  // are dropped).  Fixed counts keep the compiler's memory-counter waits exact, so the loads of
  // the next page stay in flight while the current page is processed and stored.
  constexpr int kOutOfRange = 0x40000000;

  struct PageIn {
    u32x4 x[4];  // 16 tokens x 128 channels as the B operand (zeros for slots not appended)
    u32x4 vold;  // current bytes of this lane's V piece when its quad is only partly appended
  };
  auto page_rsrc = [&](int i) {
    const int page_id = __builtin_amdgcn_readlane(page_ids, i);
    return make_rsrc(a.pool + ((int64_t)page_id * a.hkv + h) * (int64_t)kPageHeadBytes, kPageHeadBytes);
  };
  auto load_page = [&](int i, PageIn& in) {
    const bool live = i < npg;
    const int pos0 = (pg_begin + i) * kPage;
    const int slot_lo = max(s0 - pos0, 0), slot_hi = min(end_pos - pos0, kPage);
    const uint8_t* base = src + ((int64_t)(t0 + pos0 - s0) * a.hkv + h) * (int64_t)(kHeadDim * 2);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, kPage * row_stride);
    const int off = (live && n >= slot_lo && n < slot_hi) ? n * row_stride + 16 * g : kOutOfRange;
    // default cache policy for the inputs, nontemporal for the page stores below: of the
    // combinations measured on the prefill append this one is the fastest (~4% over nontemporal
    // loads with default stores)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      in.x[kb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 64 * kb, 0, 0));
    const int q0 = n & ~3;
    const bool partial = is_v && live && q0 + 3 >= slot_lo && q0 < slot_hi && (q0 < slot_lo || q0 + 4 > slot_hi);
    const int voff = partial ? kVCodesOff + 256 * (n >> 2) + 64 * g + 16 * (n & 3) : kOutOfRange;
    in.vold = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(page_rsrc(live ? i : 0), voff, 0, 0));
  };

  auto process = [&](int i, const PageIn& in) {
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
        const u32x4 at = u32x4{t[0], t[1], t[2], t[3]};
        if (BF16) {
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, at),
                                                            __builtin_bit_cast(bf16x8, in.x[kb]), acc[nb], 0, 0, 0);
        } else {
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, at),
                                                           __builtin_bit_cast(f16x8, in.x[kb]), acc[nb], 0, 0, 0);
        }
      }
    }
    if constexpr (HB == kQuatBlock) {
      // acc[nb] holds channels 16nb + 4g .. +3 of slot n: block 4nb + g, rotated in fp32
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const f32x4 x = acc[nb];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 m = *(const f32x4*)&qm[wave][4 * nb + g][r][0];
          acc[nb][r] = fmaf(m[3], x[3], fmaf(m[2], x[2], fmaf(m[1], x[1], m[0] * x[0])));
        }
      }
    }
    // acc[nb][r] = sqrt(b) * y[slot n][channel 16*nb + 4*g + r]  (b = 1: no Hadamard)
    constexpr float isb = HB == 128 ? 0.08838834764831845f : (HB == 64 ? 0.125f : 1.0f);

    uint32_t row[4];   // K row words 4g + r of slot n
    uint32_t param;    // (scale, zero) or four UE8M0 bytes of slot n
    if (FMT == 0) {
      // token-wise asymmetric INT4: fp16 scale = (max - min)/15, fp16 zero = min
      float mn = acc[0][0], mx = acc[0][0];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mn = fminf(mn, acc[nb][r]);
          mx = fmaxf(mx, acc[nb][r]);
        }
      mn = fminf(mn, __shfl_xor(mn, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mn = fminf(mn, __shfl_xor(mn, 32));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float lo = mn * isb;
      const float hi = mx * isb;
      const uint32_t s_bits = f32_to_f16_bits((hi - lo) * (1.0f / 15.0f));
      const uint32_t z_bits = f32_to_f16_bits(lo);
      const float sf = f16_bits_to_f32(s_bits);
      const float zf = f16_bits_to_f32(z_bits);
      // e = clamp((y - z) / (15 s), 0, 1); the code is rne(15 e), rounded by the magic addend
      // 1.5 * 2^23 inside one fma.  15 s is exact in fp32 (an fp16 times a 4-bit integer).
      const float r15 = sf > 0.0f ? __builtin_amdgcn_rcpf(15.0f * sf) : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t cw[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const float t = fmaf(acc[nb][r], isb, -zf);
          const float e = __builtin_amdgcn_fmed3f(t * r15, 0.0f, 1.0f);
          cw[nb] = __float_as_uint(fmaf(e, 15.0f, 12582912.0f));
        }
        row[r] = pack8(cw);
      }
      param = s_bits | (z_bits << 16);
    } else {
      // MXFP4: e2m1 codes, UE8M0 exponent per 32 channels (tiles nb = 2G, 2G+1)
      param = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) row[r] = 0;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fmaxf(fabsf(acc[2 * G][r]), fabsf(acc[2 * G + 1][r])));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float amax = m * isb;
        const int e = min(max((int)((__float_as_uint(amax) >> 23) & 255u) - 2, 0), 254);
        param |= (uint32_t)e << (8 * G);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          row[r] |= e2m1_code(ldexpf(acc[2 * G][r] * isb, 127 - e)) << (8 * G);
          row[r] |= e2m1_code(ldexpf(acc[2 * G + 1][r] * isb, 127 - e)) << (8 * G + 4);
        }
      }
    }

    // ---- paged stores ----
    const int pos0 = (pg_begin + i) * kPage;
    const int slot_lo = max(s0 - pos0, 0), slot_hi = min(end_pos - pos0, kPage);
    const __amdgpu_buffer_rsrc_t pr = page_rsrc(i);
    const bool valid = n >= slot_lo && n < slot_hi;
    u32x4 out;
    int off;
    if (!is_v) {
      out = u32x4{row[0], row[1], row[2], row[3]};
      off = valid ? 64 * n + 16 * g : kOutOfRange;
    } else {
      // lane m of the quad takes row word 4g + m of the quad's four slots, then transposes the
      // bytes: V word q holds row byte (16g + 4m + q) of slots 4(n/4) .. 4(n/4)+3
      const int m = n & 3, q0 = n & ~3;
      quad_transpose(row, m);
      const uint32_t a01 = perm(row[1], row[0], 0x05010400u);
      const uint32_t b01 = perm(row[1], row[0], 0x07030602u);
      const uint32_t a23 = perm(row[3], row[2], 0x05010400u);
      const uint32_t b23 = perm(row[3], row[2], 0x07030602u);
      out[0] = perm(a23, a01, 0x05040100u);
      out[1] = perm(a23, a01, 0x07060302u);
      out[2] = perm(b23, b01, 0x05040100u);
      out[3] = perm(b23, b01, 0x07060302u);
      // byte r of every word belongs to slot q0 + r: keep the current bytes of slots outside
      // the appended range (they were read with this page's inputs)
      uint32_t keep = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) keep |= (q0 + r >= slot_lo && q0 + r < slot_hi) ? 0u : 0xFFu << (8 * r);
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = (out[q] & ~keep) | (in.vold[q] & keep);
      off = keep != 0xFFFFFFFFu ? kVCodesOff + 256 * (n >> 2) + 64 * g + 16 * m : kOutOfRange;
    }
    __builtin_amdgcn_raw_buffer_store_b128(out, pr, off, 0, 2);  // 2: nontemporal
    const int poff = (g == 0 && valid) ? (is_v ? kVParamsOff : kKParamsOff) + 4 * n : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(param, pr, poff, 0, 2);
  };

  // Pages i = 0..npg-1: page i+1 loads while page i is processed.  The loop is unrolled and each
  // step is reached only through the previous one, so every wait sees the same sequence of earlier
  // loads and stores.
  PageIn buf[2];
  load_page(0, buf[0]);
  __builtin_amdgcn_sched_barrier(0);  // page 0's V read-back issues before page 1's loads
#pragma unroll
  for (int i = 0; i < kAppendPagesPerWave; ++i) {
    if (i + 1 < kAppendPagesPerWave) load_page(i + 1, buf[(i + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);  // the next page's loads issue before this page waits
    process(i, buf[i & 1]);
    if (i + 1 >= npg) break;
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
  const int pages = (p.max_new + kPage - 1) / kPage + 1;
  const int grid_x = (pages + kAppendPagesPerWave - 1) / kAppendPagesPerWave;
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
  KVQ_APPEND_CASE(true, kQuatBlock, 0)
  KVQ_APPEND_CASE(false, kQuatBlock, 0)
  KVQ_APPEND_CASE(true, kQuatBlock, 1)
  KVQ_APPEND_CASE(false, kQuatBlock, 1)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
