// kvq_prefill_attn: chunked-prefill attention over the rotated 4-bit paged cache (UltraQuant
// article, section on what it showed: prefixes stay resident in the 4-bit cache, so a new turn
// attends over them instead of re-running their prefill; SAW-INT4 summary, "Summary": attention
// served straight from the paged 4-bit cache).
//
// The chunk of sequence b is its last n_b positions, already appended (kvq_append); chunk token
// j sits at position p_j = seq_lens[b] - n_b + j and attends positions 0 .. p_j.
//
// A workgroup (8 waves) owns (sequence, kv head, tile of chunk tokens); each wave owns 32 rows
// (chunk token x query head: floor(32/G) tokens times the G query heads of the kv head; rows past
// that, for G = 3, 5, 6, 7, belong to no token).  The workgroup walks the keys in blocks of 32
// (two pages).  Each block is staged once into LDS for all eight waves, dequantized there, and every
// wave runs its 32 rows against it on the 32x32 matrix cores:
//   S^T = K Q^T   v_mfma_f32_32x32x16_f16, A = the block's keys (INT4: the exact codes c as the
//                 fp16 subnormals c 2^-24; MXFP4: the e2m1 values times their UE8M0 scales, exact in
//                 fp16), B = q'' = sm_scale log2(e) R q as an fp16 high and a low part (two MFMAs
//                 into one accumulator, ~22 bits of q'');  INT4 then takes
//                 S - m = (2^24 scale_k) acc + (zero_k sum(q'') - m) per key (m: the row's
//                 reference maximum, folded into the same two fmas).  MXFP4: S = acc.
//                 The output leaves lane l with row l%32 and 16 keys of the block in registers, so
//                 the row maximum is an in-lane reduction plus one 32-lane swap.
//   online softmax in the log2 domain, the reference maximum moved only by more than 2^8;
//   O^T += V^T P^T  v_mfma_f32_32x32x16_f16, A = V^ transposed in LDS (INT4: fp16(scale c + zero),
//                 MXFP4: exact), B = p in fp16 straight from the score registers: the keys are taken
//                 in the order the score layout gives them (bits 2 and 3 of the key swapped), and V^
//                 is laid out in LDS in that same order.
// The pages of the block after next load into registers while a block is computed and the next
// one staged; each page id is loaded one step before its page.  Both parts of q'' stay in
// registers (they pass through LDS once, into the B-operand order).  Query rotation and the final
// rotation back run in fp32 in registers, 16 rows of a wave at a time, through LDS.
#include "kvq_attn.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

using namespace attn;

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWaves = 8;
constexpr int kSub = 512 / (kWaves * 64);  // staging parts per thread (a block is 512 parts)
constexpr int kRows = 32;                  // rows per wave: the MFMA's 32 columns
constexpr int kBlk = 32;                   // keys per step: two pages
constexpr int kKPitch = kHeadDim + 8;      // fp16 per key row of the staged K (16-byte pad)
constexpr int kVPitch = kBlk + 8;          // fp16 per channel row of the staged V^T

// K slot s of a staged key row holds channel (s / 8) + 16 (s % 8): code row word a carries channel
// a + 16 i in nibble i, so a word unpacks to 8 consecutive slots.
__device__ __forceinline__ int k_slot(int ch) { return 8 * (ch & 15) + (ch >> 4); }
// Position of key k (0..31) in the matrix-core k order of the p.V contraction: bits 2 and 3 swapped.
__device__ __forceinline__ int v_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Every row pitch is a multiple of 16 bytes, so the operand reads are single 16-byte LDS loads.
struct alignas(16) Stage {
  alignas(16) _Float16 k[kBlk][kKPitch];       // keys of the block (slot order above)
  alignas(16) _Float16 vt[kHeadDim][kVPitch];  // V^ transposed: [channel][v_pos(key)]
  alignas(16) float ks[kBlk];                  // INT4: 2^24 scale of each key (0 past the sequence)
  alignas(16) float kz[kBlk];                  // INT4: zero of each key (0 past the sequence)
};

struct alignas(16) PrefillSmem {
  union alignas(16) {
    Stage st[2];
    alignas(16) _Float16 qst[kWaves][kRows / 2][kHeadDim];    // prologue: q'' high parts of 16 rows per wave
    alignas(16) float orow[kWaves][kRows / 2][kHeadDim + 4];  // epilogue: 16 output rows per wave
  } u;
  alignas(16) _Float16 qlo[kWaves][kRows][kKPitch];  // prologue: q'' low parts [row][slot], B-operand order
};

// The global words one thread stages per block: one K code row word, one V code word, the V
// parameter words of the V word's four slots and the K parameter word of the K word's slot.
struct BlockRegs {
  uint32_t kc, vc;
  u32x4 vp;
  uint32_t kp;
};

}  // namespace

template <int FMT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    PrefillParams a) {
  __shared__ PrefillSmem sm;
  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int tpw = kRows / G;       // chunk tokens per wave
  const int rows_used = tpw * G;   // rows past it belong to no token
  const int units = a.num_seqs * a.hkv;
  const int tile = block_id_x() / units, unit = block_id_x() % units;  // tile-major order
  const int kvh = unit % a.hkv, b = unit / a.hkv;

  const int qbeg = a.cu_q[b], nq = a.cu_q[b + 1] - qbeg;
  const int L = a.seq_lens[b];
  const int t0 = tile * kWaves * tpw;  // first chunk token of the tile
  if (t0 >= nq) return;                // uniform over the workgroup
  const int pos0 = L - nq;             // position of chunk token 0
  const int last_pos = pos0 + min(t0 + kWaves * tpw, nq) - 1;
  const int n_pages_tile = last_pos / kPage + 1;
  const int nblk = last_pos / kBlk + 1;
  const int tw0 = t0 + wave * tpw;     // first chunk token of this wave

  // this lane's row (column of the score tile) and the last position it attends
  const int col = lane & 31, half = lane >> 5;
  const int row_pos = pos0 + min(tw0 + col / G, nq - 1);
  const int wave_min_pos = pos0 + min(tw0, nq - 1);

  // ---- 1. q'' = sm_scale log2(e) R (q_scale q) for the wave's 32 rows, as fp16 high and low
  //         parts in the B-operand order (16 rows at a time through LDS); row r is token
  //         tw0 + r/G, query head r%G; rows that belong to no token are zero ----
  const float c2 = a.sm_scale_log2;
  f16x8 qh[8], ql[8];
  float qsum = 0.0f;  // sum of the q'' actually used (INT4 zero points)
  {
    const int esz = __builtin_amdgcn_readfirstlane(a.q_dtype == DT_F32 ? 4 : (a.q_dtype == DT_E4M3 ? 1 : 2));
    const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(a.q, a.num_tokens * a.hq * kHeadDim * esz);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float v0[kRows / 2], v1[kRows / 2];
#pragma unroll
      for (int rr = 0; rr < kRows / 2; ++rr) {
        const int r = 16 * p + rr;
        const bool live = r < rows_used && tw0 + r / G < nq;
        const int t = min(tw0 + r / G, nq - 1);
        const int row = (qbeg + t) * a.hq + kvh * G + r % G;
        float x[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int byte = (row * kHeadDim + lane + 64 * e) * esz;
          const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, live ? (byte & ~3) : kOutOfRange, 0, 0);
          x[e] = raw_to_f32(w >> (8 * (byte & 3)), a.q_dtype) * a.q_scale;
        }
        v0[rr] = x[0];
        v1[rr] = x[1];
      }
      rotate_rows<kRows / 2>(v0, v1, a.had_block, a.quat, a.quat_full, lane, false);
      if (p == 1) __syncthreads();  // every wave has taken its first half's operands
#pragma unroll
      for (int rr = 0; rr < kRows / 2; ++rr) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ch = lane + 64 * e;
          const float v = (e ? v1[rr] : v0[rr]) * c2;
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (float)hi);
          sm.u.qst[wave][rr][k_slot(ch)] = hi;
          sm.qlo[wave][16 * p + rr][k_slot(ch)] = lo;
        }
      }
      __syncthreads();
      // lanes whose row lies in this half take their high parts: MFMA kb reads slots 16 kb + 8 half ..
      if ((col >> 4) == p) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) qh[kb] = *(const f16x8*)&sm.u.qst[wave][col & 15][16 * kb + 8 * half];
      }
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      ql[kb] = *(const f16x8*)&sm.qlo[wave][col][16 * kb + 8 * half];
#pragma unroll
      for (int j = 0; j < 8; ++j) qsum += (float)qh[kb][j] + (float)ql[kb][j];
    }
    qsum += xor_lane<32>(qsum, lane);
  }
  __syncthreads();  // the stage buffers may now be overwritten

  // ---- 2. staging: a block is 512 parts, part u (page u / 256 of the block) one K code row word
  //         and one V code word with their parameter words; thread t takes parts t + 256 k ----
  const int su = tid & 255;
  auto spage_of = [&](int k) { return kSub == 2 ? k : __builtin_amdgcn_readfirstlane(tid >> 8); };
  const int s_tok = su >> 4;      // K: slot of the K word (16 threads per slot)
  const int s_kw = su & 15;       // K: code row word a
  const int s_q = su >> 6;        // V: quad of slots 4 s_q .. 4 s_q + 3
  // V: row byte j (one V word); consecutive threads take channels j/4 next to each other, so
  // their V^T rows (80 bytes apart) fall on different LDS banks
  const int s_vj = 4 * (su & 15) + ((su >> 4) & 3);
  const uint8_t* pool_h = a.pool + (int64_t)kvh * kPageHeadBytes;
  const int64_t page_stride = (int64_t)a.hkv * kPageHeadBytes;
  // this wave's page of block blk (its id loads a step before the page; past the tile: id 0 and
  // out-of-range page loads)
  const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(a.block_table + (int64_t)b * a.max_pages, n_pages_tile * 4);
  auto load_id1 = [&](int blk, int k) {
    return __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, 4 * (2 * blk + spage_of(k)), 0, 0);
  };
  // A page past the tile gets an empty buffer range: its loads return zeros.  The offsets never
  // change, so every block issues the same loads and the memory-counter waits stay exact.
  const int off_kc = 64 * s_tok + 4 * s_kw, off_vc = kVCodesOff + 256 * s_q + 4 * s_vj;
  const int off_vp = kVParamsOff + 16 * s_q, off_kp = kKParamsOff + 4 * s_tok;
  auto load_block1 = [&](int blk, uint32_t id, BlockRegs& r, int spage) {
    const int pg = 2 * blk + spage;
    const bool live = blk < nblk && pg < n_pages_tile;
    const int pid = __builtin_amdgcn_readfirstlane((int)id);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(pool_h + (int64_t)pid * page_stride, live ? kPageHeadBytes : 0);
    r.kc = __builtin_amdgcn_raw_buffer_load_b32(rs, off_kc, 0, 0);
    r.vc = __builtin_amdgcn_raw_buffer_load_b32(rs, off_vc, 0, 0);
    r.vp = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off_vp, 0, 0));
    r.kp = __builtin_amdgcn_raw_buffer_load_b32(rs, off_kp, 0, 0);
  };
  auto store_block1 = [&](int blk, const BlockRegs& r, Stage& st, int spage) {
    const int kbase = 16 * spage;  // first key of this part's page in the block
    // ---- K: code row word a of slot s_tok -> slots 8a .. 8a+7 ----
    {
      const int key = kbase + s_tok;
      const uint32_t x = r.kc;
      uint32_t o[4];
      if constexpr (FMT == 0) {
        // the codes as fp16 subnormals c 2^-24: nibble i of the word goes to slot 8a + i
        const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        o[0] = perm(hi, lo, 0x0C040C00u);
        o[1] = perm(hi, lo, 0x0C050C01u);
        o[2] = perm(hi, lo, 0x0C060C02u);
        o[3] = perm(hi, lo, 0x0C070C03u);
      } else {
        // byte q holds channel group q: its two e2m1 codes times 2^(E_q - 127)
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __builtin_bit_cast(uint32_t, cvt_fp4(x, ue8m0_scale(r.kp, 8 * q, a.e8_shift), q));
      }
      *(u32x4*)&st.k[key][8 * s_kw] = u32x4{o[0], o[1], o[2], o[3]};
      if constexpr (FMT == 0) {
        if (s_kw == 0) {
          const bool valid = blk * kBlk + key < L;
          st.ks[key] = valid ? f16_bits_to_f32(r.kp & 0xFFFFu) * 16777216.0f : 0.0f;
          st.kz[key] = valid ? f16_bits_to_f32(r.kp >> 16) : 0.0f;
        }
      }
    }
    // ---- V: the word is row byte j = s_vj of slots 4 s_q + r (byte r), with channel
    //      j/4 + 32 (j%4) in its low nibble and that + 16 in its high nibble ----
    {
      const int key0 = kbase + 4 * s_q;
      const int vp0 = v_pos(key0);  // the quad's four keys sit at vp0 .. vp0 + 3
      const int j = s_vj;
      const int ch = (j >> 2) + 32 * (j & 3);
      const uint32_t x = r.vc;
      if constexpr (FMT == 0) {
        // in packed fp16, tokens (0, 2) and (1, 3) of the quad per register: the codes c become
        // exact fp16 values as (1024 + c) - 1024, and one packed fma rounds s c + z to fp16 once
        uint32_t par[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) par[rr] = blk * kBlk + key0 + rr < L ? r.vp[rr] : 0u;  // past L: V = 0
        typedef __attribute__((ext_vector_type(2))) _Float16 h2;
        const h2 s02 = __builtin_bit_cast(h2, perm(par[2], par[0], 0x05040100u));
        const h2 z02 = __builtin_bit_cast(h2, perm(par[2], par[0], 0x07060302u));
        const h2 s13 = __builtin_bit_cast(h2, perm(par[3], par[1], 0x05040100u));
        const h2 z13 = __builtin_bit_cast(h2, perm(par[3], par[1], 0x07060302u));
        const h2 k1024 = __builtin_bit_cast(h2, 0x64006400u);
        const uint32_t M = 0x000F000Fu, B = 0x64006400u;
        const h2 clo02 = __builtin_bit_cast(h2, (x & M) | B) - k1024;
        const h2 clo13 = __builtin_bit_cast(h2, ((x >> 8) & M) | B) - k1024;
        const h2 chi02 = __builtin_bit_cast(h2, ((x >> 4) & M) | B) - k1024;
        const h2 chi13 = __builtin_bit_cast(h2, ((x >> 12) & M) | B) - k1024;
        const uint32_t vlo02 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(clo02, s02, z02));
        const uint32_t vlo13 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(clo13, s13, z13));
        const uint32_t vhi02 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(chi02, s02, z02));
        const uint32_t vhi13 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(chi13, s13, z13));
        // back to token order 0, 1, 2, 3
        *(u32x2*)&st.vt[ch][vp0] = u32x2{perm(vlo13, vlo02, 0x05040100u), perm(vlo13, vlo02, 0x07060302u)};
        *(u32x2*)&st.vt[ch + 16][vp0] = u32x2{perm(vhi13, vhi02, 0x05040100u), perm(vhi13, vhi02, 0x07060302u)};
      } else {
        _Float16 vlo[4], vhi[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool valid = blk * kBlk + key0 + rr < L;  // slots past the sequence: V taken as 0
          const float sc = valid ? ue8m0_scale(r.vp[rr], 8 * (j & 3), a.e8_shift) : 0.0f;
          const f16x2 hv = cvt_fp4(x, sc, rr);
          vlo[rr] = hv[0];
          vhi[rr] = hv[1];
        }
        *(f16x4*)&st.vt[ch][vp0] = f16x4{vlo[0], vlo[1], vlo[2], vlo[3]};
        *(f16x4*)&st.vt[ch + 16][vp0] = f16x4{vhi[0], vhi[1], vhi[2], vhi[3]};
      }
    }
  };

  struct Ids { uint32_t v[kSub]; };
  struct Regs { BlockRegs r[kSub]; };
  auto load_id = [&](int blk) {
    Ids i;
#pragma unroll
    for (int k = 0; k < kSub; ++k) i.v[k] = load_id1(blk, k);
    return i;
  };
  auto load_block = [&](int blk, const Ids& id, Regs& r) {
#pragma unroll
    for (int k = 0; k < kSub; ++k) load_block1(blk, id.v[k], r.r[k], spage_of(k));
  };
  auto store_block = [&](int blk, const Regs& r, Stage& st) {
#pragma unroll
    for (int k = 0; k < kSub; ++k) store_block1(blk, r.r[k], st, spage_of(k));
  };

  // ---- 3. the key blocks ----
  f32x16 o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[ct][i] = 0.0f;
  // m: the row's reference maximum (log2 domain); set from the first block, then moved only when
  // a score exceeds it by more than 2^8 (any reference gives the same softmax, and p <= 2^8 keeps
  // fp16 p and the fp32 sums in range)
  float m = 0.0f, l = 0.0f;

  auto compute = [&](int blk, const Stage& st) {
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
    // the operands of step kb + 2 are read while step kb multiplies (three register sets), so the
    // LDS latency stays off the matrix cores' chain
    f16x8 ka[3];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ka[kb] = *(const f16x8*)&st.k[col][16 * kb + 8 * half];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if (kb + 2 < 8) ka[(kb + 2) % 3] = *(const f16x8*)&st.k[col][16 * (kb + 2) + 8 * half];
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[kb % 3], qh[kb], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[kb % 3], ql[kb], s, 0, 0, 0);
    }
    // The softmax below is one dependent chain that the next products wait for; while a wave runs
    // it, it takes the issue slots ahead of its SIMD-mate's products and staging (measured: INT4
    // 1.97-1.98 -> 1.93-1.96 ms, MXFP4 1.84 -> 1.79 ms; raising the products instead, or the
    // staging as well, was slower).
    __builtin_amdgcn_s_setprio(1);
    // register i holds key 8 (i/4) + 4 half + i%4 of the block, for row `col`; d[i] = S - m
    f32x16 d;
    if constexpr (FMT == 0) {
      f32x4 ks4[4], kz4[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        ks4[g4] = *(const f32x4*)&st.ks[8 * g4 + 4 * half];
        kz4[g4] = *(const f32x4*)&st.kz[8 * g4 + 4 * half];
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int r = 0; r < 4; ++r) d[4 * g4 + r] = fmaf(ks4[g4][r], s[4 * g4 + r], fmaf(kz4[g4][r], qsum, -m));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) d[i] = s[i] - m;
    }
    if (blk * kBlk + kBlk - 1 > wave_min_pos) {  // some key of the block lies past some row's position
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key_pos = blk * kBlk + 8 * (i >> 2) + 4 * half + (i & 3);
        d[i] = key_pos <= row_pos ? d[i] : -INFINITY;
      }
    }
    float mb = d[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mb = fmaxf(mb, d[i]);
    mb = fmaxf(mb, xor_lane<32>(mb, lane));
    if (blk == 0 || __any(mb > 8.0f)) {
      // the first block sets m (every row attends position 0); later, m moves up by mb
      const float delta = blk == 0 ? mb : fmaxf(mb, 0.0f);
      const float f = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[ct][i] *= f;
      l *= f;
      m += delta;
#pragma unroll
      for (int i = 0; i < 16; ++i) d[i] -= delta;
    }
    // p in fp16 (round to nearest even, two per conversion); l sums those same fp16 weights
    // exactly (dot products with ones, accumulated in fp32)
    f16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const f16x2 h = __builtin_convertvector(
          (f32x2){__builtin_amdgcn_exp2f(d[i]), __builtin_amdgcn_exp2f(d[i + 1])}, f16x2);
      l = __builtin_amdgcn_fdot2(h, (f16x2){(_Float16)1.0f, (_Float16)1.0f}, l, false);
      pb[i >> 3][i & 7] = h[0];
      pb[i >> 3][(i & 7) + 1] = h[1];
    }
    f16x8 va[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) va[t] = *(const f16x8*)&st.vt[32 * (t >> 1) + col][16 * (t & 1) + 8 * half];
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[t], pb[t & 1], o[t >> 1], 0, 0, 0);
  };

  // Block blk + 2 loads while block blk is computed and block blk + 1 is staged: two register
  // sets, the loop body unrolled by two so that both stay statically addressed.
  Regs rg[2];
  Ids id0 = load_id(0), id1 = load_id(1);
  load_block(0, id0, rg[0]);
  id0 = load_id(2);
  load_block(1, id1, rg[1]);
  id1 = load_id(3);
  store_block(0, rg[0], sm.u.st[0]);
  __syncthreads();
  // blocks in pairs: an odd count gets one more block, past the tile, whose keys every row masks
  for (int blk = 0; blk < nblk; blk += 2) {
    load_block(blk + 2, id0, rg[0]);
    id0 = load_id(blk + 4);
    compute(blk, sm.u.st[0]);
    store_block(blk + 1, rg[1], sm.u.st[1]);
    __syncthreads();
    load_block(blk + 3, id1, rg[1]);
    id1 = load_id(blk + 5);
    compute(blk + 1, sm.u.st[1]);
    store_block(blk + 2, rg[0], sm.u.st[0]);
    __syncthreads();
  }

  // ---- 4. normalise, rotate back and store, 16 rows of the wave at a time ----
  l += xor_lane<32>(l, lane);
  const float il = 1.0f / l;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if ((col >> 4) == p) {
      // register i of channel tile ct holds channel 32 ct + 8 (i/4) + 4 half + i%4 of row col
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)&sm.u.orow[wave][col & 15][32 * ct + 8 * g4 + 4 * half] =
              f32x4{o[ct][4 * g4] * il, o[ct][4 * g4 + 1] * il, o[ct][4 * g4 + 2] * il, o[ct][4 * g4 + 3] * il};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float x0[kRows / 2], x1[kRows / 2];
#pragma unroll
    for (int rr = 0; rr < kRows / 2; ++rr) {
      x0[rr] = sm.u.orow[wave][rr][lane];
      x1[rr] = sm.u.orow[wave][rr][lane + 64];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (!a.out_rotated) rotate_rows<kRows / 2>(x0, x1, a.had_block, a.quat, a.quat_full, lane, true);
#pragma unroll
    for (int rr = 0; rr < kRows / 2; ++rr) {
      const int r = 16 * p + rr;
      const int t = tw0 + r / G;
      if (r < rows_used && t < nq) {
        const int64_t base = ((int64_t)(qbeg + t) * a.hq + kvh * G + r % G) * kHeadDim;
        store_elem(a.out, base + lane, a.out_dtype, x0[rr]);
        store_elem(a.out, base + lane + 64, a.out_dtype, x1[rr]);
      }
    }
  }
}

int prefill_tokens_per_tile(int group) { return kWaves * (kRows / group); }

hipError_t launch_prefill(const PrefillParams& p, int fmt, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.num_seqs * p.hkv * p.tiles));
  if (fmt == 0)
    hipLaunchKernelGGL(prefill_kernel<0>, grid, dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
