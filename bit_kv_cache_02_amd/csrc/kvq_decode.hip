// kvq_decode_attn: paged decode attention that reads the rotated 4-bit cache and dequantizes in
// registers (SAW-INT4 summary, "Summary": attention served from paged 4-bit KV; UltraQuant
// article, section on how the method works: queries attend over 4-bit KV with group scales).
//
// A workgroup (W waves) owns one (sequence, kv head, split): a run of pages of one sequence.
// Per page (16 tokens x 128 channels, one 2176-byte page-head block) each wave does:
//   scores   S[g][t] = sk_t * (q'_g . c_t) + zk_t * sum(q'_g)      (INT4: y^ = s*c + z)
//            q'_g . c_t runs on v_mfma_i32_16x16x64_i8 straight on the 4-bit codes: q' is held as
//            a 24-bit fixed-point number split into three int8 limbs (A-tile rows; layouts in
//            kvq_attn.h), so the contraction is exact integer arithmetic;
//   softmax  online, in the log2 domain; DPP row reductions over the 16 tokens;
//   p.V      O'[g][ch] += sum_t (p_t sv_t) (c_t[ch] - 8) + sum_t p_t (zv_t + 8 sv_t)
//            the first sum runs on v_mfma_f32_16x16x16_f16: the codes enter as the exact fp16
//            subnormals c * 2^-24 (a mask of the nibbles, no conversion), centred by one exact
//            packed fp16 subtraction so that the fp32 accumulation sees terms of both signs;
//            p_t*sv_t enters split into an fp16 high part and an fp16 low part (rows 2g and
//            2g+1), which keeps ~22 bits of it.
// MXFP4 pages convert to fp16 tiles with the group scale applied (v_cvt_scalef32_pk_f16_fp4) and
// run both contractions on the f16 matrix cores, two pages at a time (one softmax update per
// pair); with KVQ_MX_SCALED_MFMA both run on the scaled
// FP8 x FP4 matrix cores straight on the stored codes instead (layouts in kvq_attn.h).
// kvq_decode_step runs the same kernel with the append folded in: in the workgroup that streams a
// sequence's last page, the wave that streams that page also rotates and quantizes that step's
// new K/V token (a wave butterfly) after the workgroup barrier, while its first pages are in
// flight, writes it into the page, and substitutes its bytes into the page registers it streams.
// The page layout puts V codes of four consecutive tokens in one 32-bit word per row byte, which
// is the B-operand shape of the p.V MFMA, so one 16-byte load per lane feeds it directly.
// Each wave streams its pages through a register prefetch pipeline (the query loads and the
// first page loads are issued before anything waits).  The waves' partials merge in LDS; when a
// (sequence, kv head) is split over several workgroups, each writes its partial and the last to
// finish merges them all (a counter per unit in the workspace).  The query rotation and the final
// rotation back run in fp32 in registers, one head per wave, with lane shuffles for the
// cross-lane butterfly stages.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

#include <stdlib.h>

#include <type_traits>

namespace kvq {

namespace {

using namespace attn;

template <int W, int FMT>
struct DecodeSmem {
  // INT4: q' limbs (hi, mid, lo) in the byte order of the q.K A tile: [limb][g][a2][jg][16 bytes]
  uint8_t qlimb[3][kMaxG][2][4][16];
  // MXFP4: q' as fp16 high/low parts in the A-tile order of the f16 q.K MFMA: [part][g][kk][jg][8]
  _Float16 qh[2][kMaxG][4][4][8];
  // MXFP4 on the scaled matrix cores: q' limbs as the e4m3 A tiles [tile][row][K] and their
  // UE8M0 scales [tile][row][channel group] (row 2g+t: limb t+1; tile 1 row 2g: limb 3)
  uint8_t q8[2][16][kHeadDim];
  uint8_t q8s[2][16][4];
  float qdelta[kMaxG];  // INT4: weight of the mid limb, 256 delta
  float qsum[kMaxG];
  // p~ split into fp16 high/low parts, A-tile rows 2g+limb (MXFP4: one tile for each page of a pair)
  _Float16 ptile[W][FMT == 1 ? 2 : 1][2 * kMaxG][kPage];
  // each wave's partial output (after its pages); on the scaled MXFP4 path the same bytes hold
  // the wave's staging while it streams
  union WaveBuf {
    float wo[kMaxG][kHeadDim];
    std::conditional_t<FMT == 2, ScaledStage, float> st;
  };
  WaveBuf wb[W];
  float wm[W][kMaxG];
  float wl[W][kMaxG];
  // fused step: codes of the appended K (0) and V (1) vectors, their packed 64-byte rows and
  // their parameter words
  uint8_t acode[2][kHeadDim];
  uint32_t arow[2][16];
  uint32_t aparam[2];
  // balanced cut: wave totals of the block scans, and the piece this workgroup takes
  int red[16];
  int cut[4];
  int last;  // this workgroup finished its unit's last run: it merges the unit
  int prog[W];  // page groups each wave has streamed (8-wave pacing)
};

// Split partials cross workgroups, possibly on other XCDs (each with its own L2), within one
// launch.  They are written and read as relaxed agent-scope atomics: the stores write through
// to the device-coherent level and the loads read from it, so no L2 write-back or invalidate
// of the whole cache is needed.  A writer waits for its stores to complete before it counts
// its run done; the merging workgroup loads only after its count came back as the last.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix sum of v over the workgroup's threads (in thread order); *total gets the sum.
// Every thread of the workgroup (nw waves) must call it; red holds one int per wave.
__device__ __forceinline__ int block_scan_excl(int v, int nw, int* red, int* total) {
  const int lane = lane_id(), wave = thread_id() >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d);
    if (lane >= d) x += t;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
  for (int w = 0; w < nw; ++w) {
    const int r = red[w];
    before += w < wave ? r : 0;
    sum += r;
  }
  __syncthreads();  // red is free again for the next scan
  *total = sum;
  return before + x - v;
}

// The balanced cut, computed alike by every workgroup from seq_lens: sequence b has np_b pages;
// with T = hkv * sum(np_b) and C = max(ceil(T / slots), min_piece), each of its kv heads is cut
// into n_b = ceil(np_b / C) pieces, piece j holding pages [j np_b / n_b, (j+1) np_b / n_b).
// Pieces are numbered in (sequence, kv head, piece) order; sequence b's first is
// hkv * sum_{b' < b} n_b'.  At most slots + units pieces: rounding up adds less than one per unit.
struct Cut {
  int b;      // the sequence whose pieces hold piece number `key`, or -1
  int first;  // its first piece
  int n;      // its pieces per kv head
  int np;     // its pages
};

// Up to 64 sequences every wave computes the cut alone (lane = sequence; DPP scans, no LDS, no
// barrier); more (at most the workgroup's threads) take one thread per sequence, block scans
// through red and the answer broadcast through cut (4 ints).  The planner keeps sum(np_b) below
// 2^30.
__device__ __forceinline__ Cut balanced_cut(const DecodeParams& a, int key, int nw, int* red, int* cut) {
  Cut c;
  if (a.num_seqs <= 64) {
    const int lane = lane_id();
    const int L = lane < a.num_seqs ? a.seq_lens[lane] : 0;
    const int np = (max(L, 0) + kPage - 1) / kPage;
    const int total = __builtin_amdgcn_readlane(wave_scan_incl(np), 63);
    const int64_t T = (int64_t)total * a.hkv;
    const int C = max((int)((T + a.plan.slots - 1) / a.plan.slots), a.plan.min_piece);
    const int n = (np + C - 1) / C;
    const int first = (wave_scan_incl(n) - n) * a.hkv;
    const uint64_t m = __ballot(lane < a.num_seqs && n > 0 && key >= first && key < first + a.hkv * n);
    if (m == 0) {
      c.b = -1;
      return c;
    }
    const int src = __builtin_ctzll(m);
    c.b = src;
    c.first = __builtin_amdgcn_readlane(first, src);
    c.n = __builtin_amdgcn_readlane(n, src);
    c.np = __builtin_amdgcn_readlane(np, src);
    return c;
  }
  const int t = thread_id();
  const int L = t < a.num_seqs ? a.seq_lens[t] : 0;
  const int np = (max(L, 0) + kPage - 1) / kPage;
  if (t == 0) cut[0] = -1;
  int total;
  block_scan_excl(np, nw, red, &total);
  const int64_t T = (int64_t)total * a.hkv;
  const int C = max((int)((T + a.plan.slots - 1) / a.plan.slots), a.plan.min_piece);
  const int n = (np + C - 1) / C;
  int ntotal;
  const int first = block_scan_excl(n, nw, red, &ntotal) * a.hkv;
  if (t < a.num_seqs && n > 0 && key >= first && key < first + a.hkv * n) {
    cut[0] = t;
    cut[1] = first;
    cut[2] = n;
    cut[3] = np;
  }
  __syncthreads();
  c.b = __builtin_amdgcn_readfirstlane(cut[0]);
  c.first = __builtin_amdgcn_readfirstlane(cut[1]);
  c.n = __builtin_amdgcn_readfirstlane(cut[2]);
  c.np = __builtin_amdgcn_readfirstlane(cut[3]);
  return c;
}

// Fused step: put the appended token's bytes (staged in LDS) into the registers of the page that
// holds it, whatever the page load returned for that slot.
template <int FMT>
__device__ __forceinline__ void patch_appended(PageData<FMT>& pg, const uint32_t (&arow)[2][16],
                                               const uint32_t (&aparam)[2], int slot, int n, int jg) {
  if (n == slot) {
    pg.k = u32x4{arow[0][4 * jg], arow[0][4 * jg + 1], arow[0][4 * jg + 2], arow[0][4 * jg + 3]};
    pg.kp = aparam[0];
    if constexpr (FMT == 0) pg.vp = aparam[1];
  }
  if (jg == (slot >> 2)) {
    // V word q holds row byte 4n+q of tokens 4jg .. 4jg+3, one byte each
    const int sh = 8 * (slot & 3);
    const uint8_t* vrow = (const uint8_t*)arow[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) pg.v[q] = (pg.v[q] & ~(0xFFu << sh)) | ((uint32_t)vrow[4 * n + q] << sh);
    if constexpr (FMT == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pg.vp4[r] = (slot & 3) == r ? aparam[1] : pg.vp4[r];  // no dynamic index
    }
  }
}

// Rotate one head's normalised o' (element lane in o0, lane + 64 in o1) back and store it.
__device__ __forceinline__ void store_head(const DecodeParams& a, float o0, float o1, int b, int h, int lane) {
  store_row(a.out, (int64_t)b * a.hq + h, a.out_dtype, a.out_rotated, a.had_block, a.quat, a.quat_full, o0, o1,
            lane);
}

// Merge the partials of one (sequence, kv head)'s runs, in slots s0 .. s0 + n - 1, for heads
// wave, wave + nw, ...; rotate back and store.  The partials are taken 16 at a time: lane j < 16
// loads partial j's running maximum and weight while every lane loads its two channels of all
// 16 partial outputs, all in one round of loads; the passes merge online (rescaled by the
// change of maximum), so a unit of at most 16 runs costs one round trip.
__device__ __forceinline__ void merge_runs(const DecodeParams& a, int64_t s0, int n, int b, int kvh, int wave,
                                           int nw) {
  constexpr int kBatch = 16;
  const int lane = lane_id();
  const int G = a.group;
  for (int g = wave; g < G; g += nw) {
    float M = kNegBig, Ls = 0.f, O0 = 0.f, O1 = 0.f;
    for (int c = 0; c < n; c += kBatch) {
      const int cnt = min(kBatch, n - c);
      // partial j of this pass at slot s0 + c + j; indexes past the unit's last run re-read it
      // and get weight 0
      const int jl = min(lane, cnt - 1);
      const float* ml = a.part_ml + ((s0 + c + jl) * G + g) * 2;
      const float mj = ld_coherent(ml), lj = ld_coherent(ml + 1);
      const float* po = a.part_o + ((s0 + c) * G + g) * kHeadDim;
      float x[kBatch][2];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int ju = min(u, cnt - 1);
        x[u][0] = ld_coherent(po + (int64_t)ju * G * kHeadDim + lane);
        x[u][1] = ld_coherent(po + (int64_t)ju * G * kHeadDim + lane + 64);
      }
      const float mv = lane < cnt ? mj : kNegBig;
      const float Mn = fmaxf(M, wave_max(mv));
      // exponents <= 0: the hardware exp2 (1 ulp) is enough, the library one costs ~15 instructions
      const float r = __builtin_amdgcn_exp2f(M - Mn);
      const float f = lane < cnt ? __builtin_amdgcn_exp2f(mj - Mn) : 0.0f;
      Ls = fmaf(Ls, r, wave_sum_f(f * lj));
      O0 *= r;
      O1 *= r;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u));
        O0 = fmaf(fu, x[u][0], O0);
        O1 = fmaf(fu, x[u][1], O1);
      }
      M = Mn;
    }
    const float il = __builtin_amdgcn_rcpf(Ls);  // Ls >= 1: 1 ulp
    store_head(a, O0 * il, O1 * il, b, kvh * G + g, lane);
  }
}

}  // namespace


// FMT: 0 INT4; 1 MXFP4 (f16 tiles); 2 MXFP4 with q.K and p.V on the scaled FP8 x FP4 matrix cores.
// HPL: heads per lane group of the INT4 page step (1: at most 4 heads, 2: more; MXFP4: 2).
template <int FMT, int W, int D, int HPL>
__global__ __launch_bounds__(W * 64) void decode_kernel(DecodeParams a) {
  constexpr int PF = FMT == 0 ? 0 : 1;  // page format
  __shared__ DecodeSmem<W, FMT> sm;
  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // This workgroup's run: pages [p_begin, p_begin + span) of (sequence b, kv head kvh), one of
  // the unit's runs; its partial goes to workspace slot `slot`.
  int b, kvh, p_begin, span, pieces_cut = 0;
  int64_t slot, unit_s0;  // this run's slot and the unit's first
  if (a.plan.balanced) {
    const Cut c = balanced_cut(a, block_id_x(), W, sm.red, sm.cut);
    if (c.b < 0) return;  // past the last piece (uniform)
    b = c.b;
    const int r = block_id_x() - c.first;
    const int nb = c.n, np = c.np;
    kvh = r / nb;
    const int j = r - kvh * nb;
    p_begin = (int)((int64_t)j * np / nb);
    // at most 64 W pages by the plan; the clamp keeps lengths beyond the host hint in bounds
    span = min((int)((int64_t)(j + 1) * np / nb) - p_begin, 64 * W);
    pieces_cut = nb;
    slot = block_id_x();
    unit_s0 = slot - j;
  } else {
    // split-major order: every unit's first split is dispatched before any second split, so the
    // workgroups that have pages spread over the CUs and the empty ones (splits past a short
    // sequence's end) come last and exit at once
    const int units = a.num_seqs * a.hkv;
    const int split = block_id_x() / units;
    const int unit = block_id_x() % units;
    kvh = unit % a.hkv;
    b = unit / a.hkv;
    p_begin = split * a.plan.pages_per_split;
    span = a.plan.pages_per_split;
    slot = (int64_t)unit * a.plan.nsplit + split;
    unit_s0 = (int64_t)unit * a.plan.nsplit;
  }
  const int G = a.group;
  const int n = lane & 15;   // token (QK, softmax) / output column (p.V)
  const int jg = lane >> 4;  // row group: head jg (HPL 1) or heads 2jg, 2jg+1

  // ---- 0. loads that depend on nothing: the query words, then this wave's block-table entries
  //         (the page loads wait for those, and with them for the query words issued just
  //         before).  Pages are dealt to the waves round-robin (wave w takes pages
  //         p_begin + w + W*i), so the entries a wave needs do not depend on the sequence length.
  // Wave w holds heads w, w+W, ...; a wave without a head in a slot loads head G-1 and ignores it.
  // Each element is fetched as the aligned 32-bit word holding it.
  const int L = a.seq_lens[b];
  constexpr int kMaxHeadsPerWave = (kMaxG + W - 1) / W;
  const int esz = __builtin_amdgcn_readfirstlane(a.q_dtype == DT_F32 ? 4 : (a.q_dtype == DT_E4M3 ? 1 : 2));
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(a.q, a.num_seqs * a.hq * kHeadDim * esz);
  uint32_t qword[kMaxHeadsPerWave][2];
  int qshift[kMaxHeadsPerWave][2];
#pragma unroll
  for (int k = 0; k < kMaxHeadsPerWave; ++k) {
    const int g = min(wave + k * W, G - 1);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int byte = (((b * a.hq + kvh * G + g) * kHeadDim) + lane + 64 * e) * esz;
      qword[k][e] = __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, byte & ~3, 0, 0);
      qshift[k][e] = 8 * (byte & 3);
    }
  }
  const int pw0 = p_begin + wave;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int bt_idx = pw0 + W * lane;
  const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(bt, a.max_pages * 4);
  const int pid_vec = (int)__builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, lane * W < span ? 4 * bt_idx : kOutOfRange, 0, 0);

  // Fused step: the workgroup that holds the sequence's last page appends the new token there;
  // the wave that streams that page (pages are dealt round-robin) takes both the K and the V
  // vector (their words load here; every wave issues the loads, out of range where it does not
  // append).
  const int n_pages = (L + kPage - 1) / kPage;
  const int last_pg = n_pages - 1;
  const int app_slot = (L - 1) & (kPage - 1);
  const bool app_wg = a.append && last_pg >= p_begin && last_pg < p_begin + span;
  const bool app_wave = app_wg && (last_pg - p_begin) % W == wave;
  uint32_t nword[2][2];  // [K|V][element lane | lane + 64]
  int nshift[2];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    // an empty range when this wave does not append: nothing can be read whatever the offset
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(which ? a.vnew : a.knew, app_wave ? a.num_seqs * a.hkv * kHeadDim * 2 : 0);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int byte = ((b * a.hkv + kvh) * kHeadDim + lane + 64 * e) * 2;
      nword[which][e] = __builtin_amdgcn_raw_buffer_load_b32(r, app_wave ? (byte & ~3) : kOutOfRange, 0, 0);
      nshift[e] = 8 * (byte & 3);
    }
  }
  const int app_pid_w = (int)__builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, app_wg ? 4 * last_pg : kOutOfRange, 0, 0);
  __builtin_amdgcn_sched_barrier(0);  // all of the above issues before anything waits
  // converted here, before the page loads are issued: the wait for the block-table entries
  // covers these words, and none of the page loads has to complete before the query math
  float qv[kMaxHeadsPerWave][2];
#pragma unroll
  for (int k = 0; k < kMaxHeadsPerWave; ++k)
#pragma unroll
    for (int e = 0; e < 2; ++e) qv[k][e] = raw_to_f32(qword[k][e] >> qshift[k][e], a.q_dtype) * a.q_scale;
  __builtin_amdgcn_sched_barrier(0);

  if (p_begin >= n_pages) return;  // uniform over the workgroup
  const int p_end = min(p_begin + span, n_pages);
  // runs of this unit (fixed splits: lengths beyond the host hint are cut off at the grid, so
  // that every counted run exists)
  const int pieces = a.plan.balanced ? pieces_cut : min((n_pages + span - 1) / span, a.plan.nsplit);

  // ---- 1. this wave's pages; start the first loads before the query math ----
  const int npw = max(0, (p_end - pw0 + W - 1) / W);  // <= 64 (span <= 64 W)
  const uint8_t* pool_h = a.pool + (int64_t)kvh * kPageHeadBytes;
  const int64_t page_stride = (int64_t)a.hkv * kPageHeadBytes;
  auto page_base = [&](int i) {
    // uniform by construction; readfirstlane makes that explicit so the buffer descriptor stays in
    // scalar registers
    const uint64_t addr = (uint64_t)(pool_h + (int64_t)__builtin_amdgcn_readlane(pid_vec, min(i, 63)) * page_stride);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
  };
  const int koff = 64 * n + 16 * jg, voff = kVCodesOff + 16 * lane, poff = 4 * n, qoff = 16 * jg;
  constexpr int NB = D + 1;  // register buffers: D pages in flight plus the one being processed
  PageData<PF> st[NB];
#pragma unroll
  for (int d = 0; d < D; ++d) st[d] = load_page<PF>(page_base(d), d < npw, koff, voff, poff, qoff);

  // ---- 2. q' = R_b (q_scale q) in registers, then 24-bit fixed point q' ~= delta_g * Q,
  //         stored as three int8 limbs in the A-tile byte order ----
#pragma unroll
  for (int k = 0; k < kMaxHeadsPerWave; ++k) {
    const int g = wave + k * W;
    if (g < G) {
      float v0 = qv[k][0], v1 = qv[k][1];
      rotate_wave(v0, v1, a.had_block, a.quat, a.quat_full, lane);
      if constexpr (FMT == 2) {
        mxfp8_limbs(v0, v1, g, lane, sm.q8, sm.q8s);
        continue;
      }
      if constexpr (FMT == 1) {
        // fp16 high/low parts; channel (4jg + kk) + 32q + 16e sits at element 2q + e = ch >> 4
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ch = lane + 64 * e;
          const float v = e ? v1 : v0;
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (float)hi);
          sm.qh[0][g][ch & 3][(ch >> 2) & 3][ch >> 4] = hi;
          sm.qh[1][g][ch & 3][(ch >> 2) & 3][ch >> 4] = lo;
        }
        continue;
      }
      float qs;
      const float w_mid = q_limbs(v0, v1, &sm.qlimb[0][g][0][0][0], (int)sizeof(sm.qlimb[0]), lane, &qs);
      if (lane == 0) {
        sm.qdelta[g] = w_mid;
        sm.qsum[g] = qs;  // sum of the q' actually used
      }
    }
  }
  if (lane == 0) sm.prog[wave] = 0;
  __syncthreads();

  // ---- 2b. fused step, after the barrier so that no other wave waits for it (its own first pages
  //          are in flight meanwhile): the appending wave rotates and quantizes the new K and V
  //          vectors exactly as the append path defines them, stages their rows in LDS for the
  //          substitution into its last page, and stores them into the page ----
  uint32_t app_word = 0, app_byte = 0, app_param[2] = {0u, 0u};
  if (app_wave) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      float x0 = raw_to_f32(nword[which][0] >> nshift[0], a.kv_dtype);
      float x1 = raw_to_f32(nword[which][1] >> nshift[1], a.kv_dtype);
      rotate_wave(x0, x1, a.had_block, a.quat, a.quat_full, lane);
      uint32_t c0, c1, prm;
      if constexpr (FMT == 0) {
        const float lo = -wave_max(-fminf(x0, x1)), hi = wave_max(fmaxf(x0, x1));
        const uint32_t s_bits = f32_to_f16_bits((hi - lo) * (1.0f / 15.0f));
        const uint32_t z_bits = f32_to_f16_bits(lo);
        const float sf = f16_bits_to_f32(s_bits), zf = f16_bits_to_f32(z_bits);
        const float r15 = sf > 0.0f ? __builtin_amdgcn_rcpf(15.0f * sf) : 0.0f;
        c0 = __float_as_uint(fmaf(__builtin_amdgcn_fmed3f((x0 - zf) * r15, 0.0f, 1.0f), 15.0f, 12582912.0f)) & 15u;
        c1 = __float_as_uint(fmaf(__builtin_amdgcn_fmed3f((x1 - zf) * r15, 0.0f, 1.0f), 15.0f, 12582912.0f)) & 15u;
        prm = s_bits | (z_bits << 16);
      } else {
        // UE8M0 exponent per 32 channels: lanes 0-31 / 32-63 hold groups 0 / 1 (x0) and 2 / 3 (x1)
        float m0 = row_max16(fabsf(x0)), m1 = row_max16(fabsf(x1));
        m0 = fmaxf(m0, xor_lane<16>(m0, lane_id()));
        m1 = fmaxf(m1, xor_lane<16>(m1, lane_id()));
        const int e0 = min(max((int)((__float_as_uint(m0) >> 23) & 255u) - 2, 0), 254);
        const int e1 = min(max((int)((__float_as_uint(m1) >> 23) & 255u) - 2, 0), 254);
        c0 = e2m1_code(ldexpf(x0, 127 - e0));
        c1 = e2m1_code(ldexpf(x1, 127 - e1));
        prm = (uint32_t)__builtin_amdgcn_readlane(e0, 0) | ((uint32_t)__builtin_amdgcn_readlane(e0, 32) << 8) |
              ((uint32_t)__builtin_amdgcn_readlane(e1, 0) << 16) | ((uint32_t)__builtin_amdgcn_readlane(e1, 32) << 24);
      }
      app_param[which] = prm;
      sm.acode[which][lane] = (uint8_t)c0;
      sm.acode[which][lane + 64] = (uint8_t)c1;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // row byte 4a+q holds channels a+32q (low nibble) and a+32q+16 (high nibble)
      const int ra = lane >> 2, rq = lane & 3;
      const uint32_t byte = (uint32_t)sm.acode[which][ra + 32 * rq] | ((uint32_t)sm.acode[which][ra + 32 * rq + 16] << 4);
      ((uint8_t*)sm.arow[which])[lane] = (uint8_t)byte;
      if (lane == 0) sm.aparam[which] = prm;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (which == 0) app_word = sm.arow[0][lane & 15];
      else app_byte = byte;
    }
  }
  {
    // every wave issues the four stores; out of range unless it appends
    const int app_pid = __builtin_amdgcn_readfirstlane(app_pid_w);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(a.pool + (int64_t)kvh * kPageHeadBytes + (int64_t)app_pid * page_stride,
                                               kPageHeadBytes);
    const int kw = (app_wave && lane < 16) ? 64 * app_slot + 4 * lane : kOutOfRange;
    const int vb = app_wave ? kVCodesOff + 256 * (app_slot >> 2) + 4 * lane + (app_slot & 3) : kOutOfRange;
    const int pk = (app_wave && lane == 0) ? kKParamsOff + 4 * app_slot : kOutOfRange;
    const int pv = (app_wave && lane == 0) ? kVParamsOff + 4 * app_slot : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(app_word, r, kw, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)app_byte, r, vb, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(app_param[0], r, pk, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(app_param[1], r, pv, 0, 0);
  }


  const int ga = n >> 1;   // A-tile row 2g+limb -> head of this lane's A row (HPL 2)
  const int limb = n & 1;  // 0: high limb / high fp16 part, 1: low
  // p.V A-tile rows in use (p~ parts of an existing head), and the heads of this lane's score
  // and accumulator rows: h0 (and h0 + 1 with two heads per lane group)
  const bool a_row_used = HPL == 1 ? ((n & 3) < 2 && (n >> 2) < G) : ga < G;
  const int h0 = HPL == 1 ? jg : 2 * jg;
  const bool has0 = h0 < G, has1 = HPL == 2 && h0 + 1 < G;
  const float c2 = a.sm_scale_log2;
  i32x4 qa[4];
  f16x8 qh[4];
  i32x8 qa8[2];
  int qsa[2];
  float alpha0 = 0.f, beta0 = 0.f, alpha1 = 0.f, beta1 = 0.f;
  if constexpr (FMT == 0) {
    q_tiles_i4<HPL>([&](int l, int g, int a2) { return *(const i32x4*)&sm.qlimb[l][g][a2][jg][0]; }, G, n, qa);
    alpha0 = has0 ? sm.qdelta[h0] * c2 : 0.0f;
    beta0 = has0 ? sm.qsum[h0] * c2 : 0.0f;
    alpha1 = has1 ? sm.qdelta[h0 + 1] * c2 : 0.0f;
    beta1 = has1 ? sm.qsum[h0 + 1] * c2 : 0.0f;
  } else if constexpr (FMT == 1) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qh[kk] = a_row_used ? *(const f16x8*)&sm.qh[limb][ga][kk][jg][0] : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  } else {
    mxfp8_a_tiles(sm.q8, sm.q8s, a_row_used, limb, n, jg, qa8, qsa);
  }

  // ---- 3. stream this wave's pages ----
  WaveState s;
  s.m0 = s.m1 = kNegBig;
  s.l0 = s.l1 = s.pz0 = s.pz1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // scaled MXFP4 path: the p.V tiles and the masked scores of the current 4-page group
  static_assert(FMT != 2 || NB == 4, "the scaled path takes its pages in groups of four");
  ScaledAcc sacc;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc.c[g][i] = 0.0f;
  float xs0[4], xs1[4];
  const int valid0 = L - pw0 * kPage;
  const int late_bias = (a.plan.balanced && 2 * block_id_x() >= a.num_seqs * a.hkv * a.plan.nsplit) ? 1 : 0;
  for (int i0 = 0; i0 < npw; i0 += NB) {
    // The waves of a workgroup hold equal shares of the pages, but the issue arbiter favours
    // older waves, which would finish first and leave the last pages to fewer waves (fewer loads
    // in flight).  8 waves: waves w and w ^ 4 share a SIMD (a workgroup's waves go to the CU's
    // four SIMDs in turn); each publishes its progress in LDS and the one ahead of its SIMD-mate
    // yields the issue slots, so the pair keep pace page group by page group.  Otherwise a
    // wave's priority falls as it progresses, so the waves that are behind get the issue slots.
    if constexpr (W == 8) {
      // The volatile accesses go through a generic pointer, i.e. flat instructions, whose wait
      // also drains this wave's page loads in flight once per group of pages.  Measured: LDS
      // atomics in their place (ds_write / ds_read, no drain) made the llama step ~2% slower.
      if (lane == 0) *(volatile int*)&sm.prog[wave] = i0;
      const int mate = __builtin_amdgcn_readfirstlane(*(volatile const int*)&sm.prog[wave ^ 4]);
      if (i0 > mate) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(3);
    } else if constexpr (FMT != 1) {
      // Balanced plan (two workgroups per CU): the second half of the grid shares the CUs' SIMDs
      // with the first half, whose older waves win the ties; it takes one level more at equal
      // progress.  The MXFP4 fp16-tile decode (three workgroups per CU) runs without it: 3%
      // faster measured on one box (199.6-200.5 against 205.8-206.7 us).
      const int progress = 4 * i0 - late_bias * npw;  // compared with 3 npw, 2 npw, npw
      if (progress < npw) __builtin_amdgcn_s_setprio(3);
      else if (progress < 2 * npw) __builtin_amdgcn_s_setprio(2);
      else if (progress < 3 * npw) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (FMT == 1 && NB % 2 == 0) {
      // MXFP4 pages in pairs (process_pages_mx2): the pair's first load goes out before it, into
      // the buffer freed by the previous pair's second page, and its second load after it, into
      // the buffer of the pair's first page; the loads and their order are those of the
      // one-page loop below
#pragma unroll
      for (int d = 0; d < NB; d += 2) {
        const int i = i0 + d;
        st[(d + D) % NB] = load_page<PF>(page_base(i + D), i + D < npw, koff, voff, poff, qoff);
        if (i < npw) {
          const bool has_b = i + 1 < npw;  // a page past the wave's last holds zeros: masked whole
          if (app_wg && pw0 + W * i == last_pg) patch_appended<PF>(st[d], sm.arow, sm.aparam, app_slot, n, jg);
          if (app_wg && has_b && pw0 + W * (i + 1) == last_pg)
            patch_appended<PF>(st[d + 1], sm.arow, sm.aparam, app_slot, n, jg);
          process_pages_mx2(st[d], st[d + 1], valid0 - i * W * kPage, has_b ? valid0 - (i + 1) * W * kPage : 0, s,
                            qh, c2, has0, has1, n, jg, a_row_used, sm.ptile[wave], a.e8_shift);
        }
        st[(d + 1 + D) % NB] = load_page<PF>(page_base(i + 1 + D), i + 1 + D < npw, koff, voff, poff, qoff);
      }
      continue;
    }
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      const int i = i0 + d;
      // page i sits in buffer d; page i + D goes to the buffer freed by page i - 1
      st[(d + D) % NB] = load_page<PF>(page_base(i + D), i + D < npw, koff, voff, poff, qoff);
      if (i < npw) {
        if (app_wg && pw0 + W * i == last_pg) patch_appended<PF>(st[d], sm.arow, sm.aparam, app_slot, n, jg);
        if constexpr (FMT == 0)
          process_page<HPL>(st[d], valid0 - i * W * kPage, valid0 - i * W * kPage, s, qa, alpha0, beta0, alpha1, beta1,
                       has0, has1, n, jg, a_row_used, sm.ptile[wave][0]);
        else if constexpr (FMT == 1)
          process_page_mx(st[d], valid0 - i * W * kPage, valid0 - i * W * kPage, valid0 - i * W * kPage, s, qh, c2,
                          has0, has1, n, jg, a_row_used, sm.ptile[wave][0], a.e8_shift);
        else
          scaled_stage_page(st[d], valid0 - i * W * kPage, qa8, qsa, c2, n, jg, d, sm.wb[wave].st, xs0[d], xs1[d]);
      } else if constexpr (FMT == 2) {
        xs0[d] = xs1[d] = -INFINITY;
      }
      if constexpr (FMT == 2) {
        if (d == NB - 1) scaled_flush(xs0, xs1, s, sacc, sm.wb[wave].st, G, has0, has1, n, jg, lane);
      }
    }
  }

  // ---- 4. wave partial -> LDS ----
  const float l0 = row_sum16(s.l0), l1 = row_sum16(s.l1);
  const float pz0 = row_sum16(s.pz0), pz1 = row_sum16(s.pz1);
  if constexpr (FMT == 2) {
    // tile register 4a + t of lane half b: head 2a + b, limb t, channel 32g + lane % 32
    const int bh = lane >> 5, col = lane & 31;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int h = 2 * a4 + bh;
      if (h < G) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          sm.wb[wave].wo[h][32 * g + col] = sacc.c[g][4 * a4] + sacc.c[g][4 * a4 + 1] + sacc.c[g][4 * a4 + 2];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4 && FMT != 2; ++q) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = n + 32 * q + 16 * e;
      const f32x4 v = s.acc[2 * q + e];
      // INT4: undo the subnormal encoding (2^24, or 2^24/16 for the high nibbles); MXFP4: none
      const float sc = FMT != 0 ? 1.0f : (e ? 1048576.0f : 16777216.0f);
      if (has0) sm.wb[wave].wo[h0][ch] = sc * (v[0] + v[1]) + pz0;
      if (has1) sm.wb[wave].wo[h0 + 1][ch] = sc * (v[2] + v[3]) + pz1;
    }
  }
  if (n == 0) {
    if (has0) { sm.wm[wave][h0] = s.m0; sm.wl[wave][h0] = l0; }
    if (has1) { sm.wm[wave][h0 + 1] = s.m1; sm.wl[wave][h0 + 1] = l1; }
  }
  __syncthreads();

  // ---- 5. merge the waves (wave w handles heads w, w+W, ...); finish, or write the split partial ----
  for (int g = wave; g < G; g += W) {
    float M = sm.wm[0][g];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm.wm[w][g]);
    float O0 = 0.f, O1 = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm.wm[w][g] - M);  // exponent <= 0
      O0 = fmaf(f, sm.wb[w].wo[g][lane], O0);
      O1 = fmaf(f, sm.wb[w].wo[g][lane + 64], O1);
      Ls = fmaf(f, sm.wl[w][g], Ls);
    }
    if (pieces == 1) {
      const float il = __builtin_amdgcn_rcpf(Ls);  // Ls >= 1: 1 ulp
      store_head(a, O0 * il, O1 * il, b, kvh * G + g, lane);
    } else {
      float* po = a.part_o + (slot * G + g) * kHeadDim;
      st_coherent(po + lane, O0);
      st_coherent(po + lane + 64, O1);
      if (lane == 0) {
        st_coherent(a.part_ml + (slot * G + g) * 2 + 0, M);
        st_coherent(a.part_ml + (slot * G + g) * 2 + 1, Ls);
      }
    }
  }
  if (pieces == 1) return;

  // ---- 6. the unit's last run to finish merges all of its runs' partials ----
  // Counting wraps at the unit's number of runs, so the counter is back at zero after the last.
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __builtin_amdgcn_atomic_inc32(a.counters + (b * a.hkv + kvh), (uint32_t)(pieces - 1),
                                                        __ATOMIC_RELAXED, "agent");
    sm.last = done == (uint32_t)(pieces - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  merge_runs(a, unit_s0, pieces, b, kvh, wave, W);
}

DecodePlan plan_decode(int num_seqs, int hkv, int max_seq_len) {
  DecodePlan plan;
  const int max_pg = (max_seq_len + kPage - 1) / kPage;
  const int64_t units = (int64_t)num_seqs * hkv;
  // One (sequence, kv head) per CU (at most 256 units of at most 512 pages): 8-wave workgroups,
  // no split.  More units or longer sequences than that: 4-wave workgroups over 256-page splits,
  // three of which share a CU, so that one workgroup's start and end latency overlap another's
  // streaming.  Narrow batches (fewer than 256 units) with enough pages to fill the chip (at
  // least 64 per CU at the longest length): the balanced cut, 4-wave workgroups, two per CU, two
  // pages in flight per wave; slots = 512 minus one per unit (the most the cut can add by rounding
  // up per unit), so that the pieces fit two workgroups per CU.  Smaller narrow batches: fixed
  // 128-page splits, halved until the grid has 512 workgroups (the cut would cost one more
  // dependent load, of seq_lens, before a workgroup knows its pages).  Measured on the decode
  // workloads of the benchmark.
  int W, P;
  bool balanced = false;
  if (units >= 256 && units * ((max_pg + 511) / 512) <= 256) {
    W = 8;
    P = 512;
  } else if (units >= 256) {
    W = 4;
    P = 256;
  } else {
    W = 4;
    P = 128;
    while (P > 16 && units * ((max_pg + P - 1) / P) < 512) P /= 2;
    balanced = units * max_pg >= 256 * 64;
  }
  // tuning overrides (read on every call, so a sweep can change them between calls)
  const char* ew = getenv("KVQ_DECODE_WAVES");
  const char* ep = getenv("KVQ_DECODE_PAGES_PER_SPLIT");
  const char* ed = getenv("KVQ_DECODE_DEPTH");
  const char* eb = getenv("KVQ_DECODE_BALANCED");
  const char* es = getenv("KVQ_DECODE_SLOTS");
  const char* em = getenv("KVQ_DECODE_MIN_PIECE");
  const int env_w = ew ? atoi(ew) : 0, env_p = ep ? atoi(ep) : 0, env_d = ed ? atoi(ed) : 0;
  if (env_w) W = env_w;
  if (env_p) P = env_p;
  if (eb) balanced = atoi(eb) != 0;
  if (W != 4 && W != 8) W = 8;
  // the cut runs one thread per sequence and counts pages in 32 bits
  if (balanced && (max_pg <= 0 || num_seqs > 64 * W || num_seqs > 256 || (int64_t)num_seqs * max_pg >= (1 << 30)))
    balanced = false;
  int D = env_d ? env_d : (balanced ? 2 : 3);
  if (D != 2 && D != 3 && D != 4) D = 3;
  if (P > 64 * W) P = 64 * W;
  if (P < 1) P = 1;
  plan.waves = W;
  plan.depth = D;
  plan.balanced = balanced ? 1 : 0;
  plan.slots = 0;
  plan.min_piece = 0;
  if (balanced) {
    int64_t S = es ? atoll(es) : 512 - units;
    int mp = em ? atoi(em) : 16;
    mp = mp < 1 ? 1 : (mp > 64 * W ? 64 * W : mp);
    // a piece holds at most 64 W pages (one block-table entry per lane of each wave): enough slots
    // that ceil(total / slots) stays within that for any lengths up to max_seq_len (the grid then
    // rounded up to whole rounds of 256 workgroups)
    const int64_t need = (units * max_pg + 64 * W - 1) / (64 * W);
    if (S < need) S = (need + units + 255) / 256 * 256 - units;
    if (S < 1) S = 1;
    plan.slots = (int32_t)S;
    plan.min_piece = mp;
    plan.pages_per_split = 64 * W;
    plan.nsplit = (int32_t)((S + units + units - 1) / units);
    return plan;
  }
  plan.pages_per_split = P;
  plan.nsplit = max_pg > 0 ? (max_pg + P - 1) / P : 1;
  return plan;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: [counters][part_ml][part_o], each part 256-byte aligned.  The counter region has
// the same size (room for kCounterUnits units) for every call with at most that many units, so
// such calls share one layout and a call never finds another call's partials where it expects
// zeroed counters.

static size_t counter_bytes(size_t units) { return align256(4 * (units > kCounterUnits ? units : kCounterUnits)); }

size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int hkv, int group) {
  if (plan.nsplit <= 1) return 0;
  const size_t units = (size_t)num_seqs * hkv;
  const size_t slots = units * plan.nsplit;
  return counter_bytes(units) + align256(slots * group * 2 * 4) + slots * group * kHeadDim * 4;
}

void carve_workspace(void* ws, const DecodePlan& plan, int num_seqs, int hkv, int group, float** part_ml,
                     float** part_o, uint32_t** counters) {
  const size_t units = (size_t)num_seqs * hkv;
  const size_t slots = units * plan.nsplit;
  uint8_t* p = (uint8_t*)ws;
  *counters = (uint32_t*)p;
  p += counter_bytes(units);
  *part_ml = (float*)p;
  p += align256(slots * group * 2 * 4);
  *part_o = (float*)p;
}

hipError_t launch_decode(const DecodeParams& p, int variant, hipStream_t stream) {
  const int fmt = variant;
  const int64_t units = (int64_t)p.num_seqs * p.hkv;
  const dim3 grid((unsigned)(units * p.plan.nsplit));
  // INT4 with at most 4 query heads per kv head: one head per lane group
  const int hpl = (fmt == 0 && p.group <= 4) ? 1 : 2;
  // the scaled MXFP4 path takes its pages in groups of four: three in flight plus one
  const int depth = fmt == 2 ? 3 : p.plan.depth;
#define KVQ_DECODE_CASE(F, WV, DV, H)                                                            \
  if (fmt == F && p.plan.waves == WV && depth == DV && hpl == H) {                             \
    hipLaunchKernelGGL((decode_kernel<F, WV, DV, H>), grid, dim3(WV * 64), 0, stream, p);       \
  } else
  KVQ_DECODE_CASE(0, 4, 2, 1) KVQ_DECODE_CASE(0, 4, 3, 1) KVQ_DECODE_CASE(0, 4, 4, 1)
  KVQ_DECODE_CASE(0, 8, 2, 1) KVQ_DECODE_CASE(0, 8, 3, 1) KVQ_DECODE_CASE(0, 8, 4, 1)
  KVQ_DECODE_CASE(0, 4, 2, 2) KVQ_DECODE_CASE(0, 4, 3, 2) KVQ_DECODE_CASE(0, 4, 4, 2)
  KVQ_DECODE_CASE(0, 8, 2, 2) KVQ_DECODE_CASE(0, 8, 3, 2) KVQ_DECODE_CASE(0, 8, 4, 2)
  KVQ_DECODE_CASE(1, 4, 2, 2) KVQ_DECODE_CASE(1, 4, 3, 2) KVQ_DECODE_CASE(1, 4, 4, 2)
  KVQ_DECODE_CASE(1, 8, 2, 2) KVQ_DECODE_CASE(1, 8, 3, 2) KVQ_DECODE_CASE(1, 8, 4, 2)
  KVQ_DECODE_CASE(2, 4, 3, 2) KVQ_DECODE_CASE(2, 8, 3, 2) { return hipErrorInvalidValue; }
#undef KVQ_DECODE_CASE
  return hipGetLastError();
}

}  // namespace kvq
