// kvq_prefill_attn: chunked-prefill attention over the rotated 4-bit paged cache (UltraQuant
// article, section on what it showed: prefixes stay resident in the 4-bit cache, so a new turn
// attends over them instead of re-running their prefill; SAW-INT4 summary, "Summary": attention
// served straight from the paged 4-bit cache).
//
// The chunk of sequence b is its last n_b positions, already appended (kvq_append); chunk token
// j sits at position p_j = seq_lens[b] - n_b + j and attends positions 0 .. p_j.
//
// A workgroup (W waves) owns (sequence, kv head, tile of W * floor(8 RS/G) chunk tokens).  Wave w
// takes RS sets of 8 rows: its floor(8 RS/G) chunk tokens times the G query heads of the kv head
// (where G does not divide 8 RS, the last rows of the sets belong to no token and stay idle).  Each wave
// streams every page its rows attend; per page it unpacks the K and V codes once (the
// row-independent half of the per-page step that decode uses, kvq_attn.h) and runs the scores,
// online softmax and p.V of each row set against them: a set's 8 rows fill the 8 row pairs of the
// matrix-core tiles, and each row pair carries its own causal limit.  The waves
// of a workgroup read the same pages close together in time, so the caches serve all but the
// first read of each page; the sequence's block-table entries are staged in LDS once per
// workgroup.  Query rotation and the final rotation back run for the 8 rows of a wave at once.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

using namespace attn;

constexpr int kSetRows = 8;           // rows (chunk token x query head) per row set
constexpr int kMaxTablePages = 8192;  // staged block-table entries: positions < 131072

// Per wave: the query operands (prologue) and the output rows (epilogue) share one slice; a wave
// only overwrites its own operands, which it has read into registers before its page loop.
template <int RS>
struct PrefillWaveSmem {
  union {
    struct {
      union {
        uint8_t qlimb[3][kSetRows * RS][2][4][16];  // INT4: q' limbs, as in decode
        _Float16 qh[2][kSetRows * RS][4][4][8];     // MXFP4: q' fp16 high/low parts
      };
      float qdelta[kSetRows * RS];
      float qsum[kSetRows * RS];
    } q;
    float wo[kSetRows * RS][kHeadDim];
  };
  _Float16 ptile[RS][2 * kSetRows][kPage];
};

template <int W, int RS>
struct PrefillSmem {
  PrefillWaveSmem<RS> w[W];
  int32_t table[kMaxTablePages];
};

}  // namespace

template <int FMT, int W, int D, int RS>
__global__ __launch_bounds__(W * 64) void prefill_kernel(PrefillParams a) {
  constexpr int kRows = kSetRows * RS;  // rows per wave
  __shared__ PrefillSmem<W, RS> sm;
  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  PrefillWaveSmem<RS>& ws = sm.w[wave];
  const int n = lane & 15, jg = lane >> 4;
  const int G = a.group;
  const int tpw = kRows / G;  // chunk tokens per wave
  const int rows_used = tpw * G;  // rows past it (G = 3, 5, 6, 7) belong to no token of this wave
  const int units = a.num_seqs * a.hkv;
  const int tile = block_id_x() / units, unit = block_id_x() % units;  // tile-major order
  const int kvh = unit % a.hkv, b = unit / a.hkv;

  const int qbeg = a.cu_q[b], nq = a.cu_q[b + 1] - qbeg;
  const int L = a.seq_lens[b];
  const int t0 = tile * W * tpw;  // first chunk token of the tile
  if (t0 >= nq) return;           // uniform over the workgroup
  const int pos0 = L - nq;        // position of chunk token 0
  const int n_pages_tile = (pos0 + min(t0 + W * tpw, nq) - 1) / kPage + 1;
  const int tw0 = t0 + wave * tpw;  // first chunk token of this wave
  const bool wave_live = tw0 < nq;
  const int npw = wave_live ? (pos0 + min(tw0 + tpw, nq) - 1) / kPage + 1 : 0;

  // ---- 0. the query words of this wave's rows (row r: token tw0 + r/G, head r%G; rows past the
  //         chunk load its last token and are ignored), and the tile's block-table entries ----
  const int esz = __builtin_amdgcn_readfirstlane(a.q_dtype == DT_F32 ? 4 : (a.q_dtype == DT_E4M3 ? 1 : 2));
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(a.q, a.num_tokens * a.hq * kHeadDim * esz);
  uint32_t qword[kRows][2];
  int qshift[kRows][2];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int t = min(tw0 + r / G, nq - 1);
    const int row = (qbeg + t) * a.hq + kvh * G + r % G;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int byte = (row * kHeadDim + lane + 64 * e) * esz;
      qword[r][e] = __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, byte & ~3, 0, 0);
      qshift[r][e] = 8 * (byte & 3);
    }
  }
  // one 4-byte load per entry (entries past the tile's pages read as zero), all in flight at once
  constexpr int kTableLoads = kMaxTablePages / (W * 64);
  uint32_t tw[kTableLoads];
  {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(a.block_table + (int64_t)b * a.max_pages, n_pages_tile * 4);
#pragma unroll
    for (int k = 0; k < kTableLoads; ++k) tw[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (k * W * 64 + tid) * 4, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < kTableLoads; ++k) sm.table[k * W * 64 + tid] = (int32_t)tw[k];

  // ---- 1. q' = R (q_scale q) for the wave's rows, then the decode's operand encodings ----
  {
    float v0[kRows], v1[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      v0[r] = raw_to_f32(qword[r][0] >> qshift[r][0], a.q_dtype) * a.q_scale;
      v1[r] = raw_to_f32(qword[r][1] >> qshift[r][1], a.q_dtype) * a.q_scale;
    }
    rotate_rows<kRows>(v0, v1, a.had_block, a.quat, a.quat_full, lane, false);
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if constexpr (FMT == 1) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ch = lane + 64 * e;
          const float v = e ? v1[r] : v0[r];
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (float)hi);
          ws.q.qh[0][r][ch & 3][(ch >> 2) & 3][ch >> 4] = hi;
          ws.q.qh[1][r][ch & 3][(ch >> 2) & 3][ch >> 4] = lo;
        }
      } else {
        float qs;
        const float w_mid = q_limbs(v0[r], v1[r], &ws.q.qlimb[0][r][0][0][0], (int)sizeof(ws.q.qlimb[0]), lane, &qs);
        if (lane == 0) {
          ws.q.qdelta[r] = w_mid;
          ws.q.qsum[r] = qs;
        }
      }
    }
  }
  __syncthreads();  // block-table entries and query operands staged

  // Row set k holds rows 8k .. 8k+7; A-tile row 2g+limb of set k is row 8k + g.
  const int ga = n >> 1, limb = n & 1;
  const float c2 = a.sm_scale_log2;
  i32x4 qa[RS][4];
  f16x8 qh[RS][4];
  float alpha0[RS], beta0[RS], alpha1[RS], beta1[RS];
  bool a_row_used[RS], has0[RS], has1[RS];
  int lim0[RS], lim1[RS];  // tokens of page i that rows x0 / x1 attend: lim - 16 i
#pragma unroll
  for (int k = 0; k < RS; ++k) {
    const int rbase = kSetRows * k;
    a_row_used[k] = rbase + ga < rows_used && tw0 + (rbase + ga) / G < nq;
    const int t_row0 = tw0 + (rbase + 2 * jg) / G, t_row1 = tw0 + (rbase + 2 * jg + 1) / G;
    has0[k] = rbase + 2 * jg < rows_used && t_row0 < nq;
    has1[k] = rbase + 2 * jg + 1 < rows_used && t_row1 < nq;
    lim0[k] = pos0 + t_row0 + 1;
    lim1[k] = pos0 + t_row1 + 1;
    alpha0[k] = beta0[k] = alpha1[k] = beta1[k] = 0.0f;
    if constexpr (FMT == 0) {
      // a set's 8 rows fill the tile's 8 row pairs, so the lo limbs take the second tile (only
      // row pair ga is read)
      q_tiles_i4<2>([&](int l, int g, int a2) {
        return a_row_used[k] ? *(const i32x4*)&ws.q.qlimb[l][rbase + g][a2][jg][0] : i32x4{0, 0, 0, 0};
      }, kSetRows, n, qa[k]);
      alpha0[k] = has0[k] ? ws.q.qdelta[rbase + 2 * jg] * c2 : 0.0f;
      beta0[k] = has0[k] ? ws.q.qsum[rbase + 2 * jg] * c2 : 0.0f;
      alpha1[k] = has1[k] ? ws.q.qdelta[rbase + 2 * jg + 1] * c2 : 0.0f;
      beta1[k] = has1[k] ? ws.q.qsum[rbase + 2 * jg + 1] * c2 : 0.0f;
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qh[k][kk] = a_row_used[k] ? *(const f16x8*)&ws.q.qh[limb][rbase + ga][kk][jg][0]
                                  : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // ---- 2. stream pages 0 .. npw-1 (the positions this wave's rows attend) ----
  const uint8_t* pool_h = a.pool + (int64_t)kvh * kPageHeadBytes;
  const int64_t page_stride = (int64_t)a.hkv * kPageHeadBytes;
  auto page_base = [&](int i) {
    const int id = sm.table[min(i, kMaxTablePages - 1)];
    const uint64_t addr = (uint64_t)(pool_h + (int64_t)id * page_stride);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
  };
  const int koff = 64 * n + 16 * jg, voff = kVCodesOff + 16 * lane, poff = 4 * n, qoff = 16 * jg;
  constexpr int NB = D + 1;
  PageData<FMT> st[NB];
#pragma unroll
  for (int d = 0; d < D; ++d) st[d] = load_page<FMT>(page_base(d), d < npw, koff, voff, poff, qoff);
  WaveState s[RS];
#pragma unroll
  for (int k = 0; k < RS; ++k) {
    s[k].m0 = s[k].m1 = kNegBig;
    s[k].l0 = s[k].l1 = s[k].pz0 = s[k].pz1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s[k].acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i0 = 0; i0 < npw; i0 += NB) {
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      const int i = i0 + d;
      st[(d + D) % NB] = load_page<FMT>(page_base(i + D), i + D < npw, koff, voff, poff, qoff);
      if (i < npw) {
        if constexpr (FMT == 0) {
          const PageI4 u = unpack_i4(st[d], L - i * kPage, n);
#pragma unroll
          for (int k = 0; k < RS; ++k)
            rows_i4(u, lim0[k] - i * kPage, lim1[k] - i * kPage, s[k], qa[k], alpha0[k], beta0[k], alpha1[k],
                    beta1[k], has0[k], has1[k], n, jg, a_row_used[k], ws.ptile[k]);
        } else {
          const KTileMx kt = unpack_k_mx(st[d]);
          const VTileMx vt = unpack_v_mx(st[d], L - i * kPage, jg);
#pragma unroll
          for (int k = 0; k < RS; ++k)
            softmax_pv_mx(vt, scores_mx(kt, qh[k]), lim0[k] - i * kPage, lim1[k] - i * kPage, s[k], c2, has0[k],
                          has1[k], n, jg, a_row_used[k], ws.ptile[k]);
        }
      }
    }
  }

  // ---- 3. normalise the rows, rotate them back, store ----
#pragma unroll
  for (int k = 0; k < RS; ++k) {
    const float l0 = row_sum16(s[k].l0), l1 = row_sum16(s[k].l1);
    const float pz0 = row_sum16(s[k].pz0), pz1 = row_sum16(s[k].pz1);
    const float il0 = has0[k] ? 1.0f / l0 : 0.0f, il1 = has1[k] ? 1.0f / l1 : 0.0f;
    const int rbase = kSetRows * k;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int ch = n + 32 * q + 16 * e;
        const f32x4 v = s[k].acc[2 * q + e];
        const float sc = FMT == 1 ? 1.0f : (e ? 1048576.0f : 16777216.0f);
        ws.wo[rbase + 2 * jg][ch] = (sc * (v[0] + v[1]) + pz0) * il0;
        ws.wo[rbase + 2 * jg + 1][ch] = (sc * (v[2] + v[3]) + pz1) * il1;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float o0[kRows], o1[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    o0[r] = ws.wo[r][lane];
    o1[r] = ws.wo[r][lane + 64];
  }
  if (!a.out_rotated) rotate_rows<kRows>(o0, o1, a.had_block, a.quat, a.quat_full, lane, true);
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int t = tw0 + r / G;
    if (r < rows_used && t < nq) {
      const int64_t base = ((int64_t)(qbeg + t) * a.hq + kvh * G + r % G) * kHeadDim;
      store_elem(a.out, base + lane, a.out_dtype, o0[r]);
      store_elem(a.out, base + lane + 64, a.out_dtype, o1[r]);
    }
  }
}

namespace {
constexpr int kPrefillWaves = 4;
constexpr int kPrefillDepth = 3;
constexpr int kPrefillSets = 2;  // row sets per wave: 16 rows share each page's unpack
}  // namespace

int prefill_tokens_per_tile(int group) { return kPrefillWaves * (kSetRows * kPrefillSets / group); }

hipError_t launch_prefill(const PrefillParams& p, int fmt, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.hkv * p.tiles));
  if (fmt == 0)
    hipLaunchKernelGGL((prefill_kernel<0, kPrefillWaves, kPrefillDepth, kPrefillSets>), grid, dim3(kPrefillWaves * 64),
                       0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<1, kPrefillWaves, kPrefillDepth, kPrefillSets>), grid, dim3(kPrefillWaves * 64),
                       0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
