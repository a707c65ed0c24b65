// Forward chunk attention, bf16 inputs, fp32 accumulation, CDNA4 (gfx950).
//
// Computes, for one Q chunk against one KV chunk, the partial softmax
// attention O and its per-row log-sum-exp (natural log), the quantities a ring
// step merges (nougat.kr, "MaxText long-context training: KV parallelism",
// section "헤드를 나누거나, KV를 돌리거나": partial compute, then merge),
// under the causal mask on global positions and the document mask of packed
// input (siliconandsystems.com, "Llama 3 parallelism", section on the four
// parallelisms).
//
// Work decomposition
//   * one work-group = 8 waves, two per SIMD; each wave owns 32 query rows of
//     one query head.  With grouped-query attention the waves take 4 query
//     heads that read the same KV head x 2 row blocks (or 2 heads x 4, or
//     1 head x 8), so every K/V tile staged in LDS feeds 8 waves.  Two waves
//     per SIMD let one wave's softmax VALU work, LDS waits and tile loads run
//     while the other issues MFMAs (a wave's registers, 256, hold its Q rows,
//     O accumulators and scores without spilling).
//   * keys stream through LDS in tiles of 64 rows, double-buffered, copied
//     with direct-to-LDS loads issued one tile ahead (tile_io.h).
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K tile is the A operand
//     (ds_read_b128), the wave's Q rows are the B operand (in VGPRs for the
//     whole kernel).  Each lane holds one query column and 16 key rows of the
//     32x32 accumulator.
//   * O^T += V^T P^T: P^T goes from the S^T accumulator straight into the B
//     operand; V^T is read with the LDS transpose read ds_read_b64_tr_b16.
//   * Softmax reference point.  Each row's exponent offset m is fixed at the
//     max of the first tile in which the row has an allowed key, and never
//     moves: P = exp2((s - m) c) may exceed 1 for later keys, and the result
//     O = sum P v / sum P, LSE = m + ln sum P is the same.  No running max, no
//     rescaling of the accumulators, no per-tile max in the common path.  A
//     tile whose row sum exceeds 2^64 (a score more than ~44 above m, in
//     natural-log units) flags the work-group, which then redoes its rows
//     with the exact online softmax (running max, rescale), so any input is
//     handled; for ordinary inputs the flag never fires.
//   * fully masked tiles (causal or document) are skipped; the element mask is
//     evaluated only on partial tiles and on the ragged last tile.
//   * work-groups run heavy-first (later query tiles have more causal work),
//     spread so that every XCD gets the same mix (common.h, xcd_work).
#include "common.h"
#include "kernels.h"
#include "tile_io.h"

namespace cp {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BK = 64;      // keys per tile
constexpr int NQB = 1;      // 32-row query blocks per wave
constexpr int QW = 32 * NQB; // query rows per wave
constexpr int NWV = 8;      // waves per work-group (two per SIMD)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float ROWSUM_LIMIT = 18446744073709551616.0f;   // 2^64

__device__ inline void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D>
struct FwdState {
  bf16x8 qf[NQB][D / 16];
  f32x16 oacc[NQB][D / 32];
  float moff[NQB];
  float mrow[NQB];
  float lrow[NQB];
  int32_t lim[NQB];
  int32_t qdoc[NQB];
};

// Scores of a 64-key tile: S^T[kb][qb] = K (keys kb*32..) Q^T (queries qb*32..)
template <int D>
__device__ inline void fwd_scores(const FwdState<D>& st, const RowReader<D>& rr, uint32_t Kt, f32x16 (&s)[2][NQB]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bf16x8 ka = rr.at(Kt, kb, 0);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
      s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.qf[qb][0], f32x16{}, 0, 0, 0);
  }
#pragma unroll
  for (int kd = 1; kd < D / 16; ++kd) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = rr.at(Kt, kb, kd);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.qf[qb][kd], s[kb][qb], 0, 0, 0);
    }
  }
}

// Element mask of a partial or ragged tile.  Positions increase along local
// order, so "key position <= query position" is "key index < lim".
template <int D>
__device__ inline void fwd_mask(const FwdState<D>& st, f32x16 (&s)[2][NQB], uint32_t Dt, int32_t kb0,
                                bool docs, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
      const int32_t kidx = kb0 + kk;
      const int32_t kd_ = lds_ld4i(Dt + 4 * kk);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const bool ok = (kidx < st.lim[qb]) & (!docs | (kd_ == st.qdoc[qb]));
        s[kb][qb][r] = ok ? s[kb][qb][r] : -INFINITY;
      }
    }
}

// Row max of a tile's scores per query column (both lane halves combined).
__device__ inline void fwd_tile_max(const f32x16 (&s)[2][NQB], float (&mx)[NQB]) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float m0 = fmaxf(s[0][qb][0], s[0][qb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m0 = fmaxf(m0, fmaxf(s[0][qb][r], s[0][qb][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) m0 = fmaxf(m0, fmaxf(s[1][qb][r], s[1][qb][r + 1]));
    mx[qb] = fmaxf(m0, __shfl_xor(m0, 32));
  }
}

// P = exp2(s c - m c), row sums, and O^T += V^T P^T.  Returns this lane's
// largest tile row-sum share (for the overflow check).
template <int D>
__device__ inline float fwd_accumulate(FwdState<D>& st, const TrReader<D>& tr, uint32_t Vt,
                                       const f32x16 (&s)[2][NQB], float c) {
  float tsum[NQB] = {};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 pf[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][t * 8 + i], c, st.moff[qb]));
          tsum[qb] += p;
          pf[qb][t][i] = (__bf16)p;
        }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 va = tr.at(Vt, kb * 32 + 16 * t, db);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          st.oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb][t], st.oacc[qb][db], 0, 0, 0);
      }
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) { st.lrow[qb] += tsum[qb]; mx = fmaxf(mx, tsum[qb]); }
  return mx;
}

// ---- software-pipelined tile (full tiles, reference point set) -------------
// Per 64-key tile: S0 = QK(keys 0..31); then S1 = QK(keys 32..63) beside
// exp(S0); then O += V0 P0 beside exp(S1); then O += V1 P1.  The stages are
// independent, so the compiler interleaves each stage's MFMAs with the other
// half's softmax VALU work; the second wave on the SIMD fills what remains.

template <int D>
__device__ inline void qk_half(const FwdState<D>& st, const RowReader<D>& rr, uint32_t Kt, int kb, f32x16 (&s)[NQB]) {
  bf16x8 ka[D / 16];
#pragma unroll
  for (int kd = 0; kd < D / 16; ++kd) ka[kd] = rr.at(Kt, kb, kd);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], st.qf[qb][0], f32x16{}, 0, 0, 0);
#pragma unroll
  for (int kd = 1; kd < D / 16; ++kd)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kd], st.qf[qb][kd], s[qb], 0, 0, 0);
}

template <int D>
__device__ inline void exp_half(const FwdState<D>& st, const f32x16 (&s)[NQB], bf16x8 (&pf)[NQB][2], float (&tsum)[NQB],
                                float c) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][t * 8 + i], c, st.moff[qb]));
        tsum[qb] += p;
        pf[qb][t][i] = (__bf16)p;
      }
}

template <int D>
__device__ inline void pv_half(FwdState<D>& st, const TrReader<D>& tr, uint32_t Vt, int kb, const bf16x8 (&pf)[NQB][2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 va = tr.at(Vt, kb * 32 + 16 * t, db);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        st.oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb][t], st.oacc[qb][db], 0, 0, 0);
    }
  }
}


// Element mask of one 32-key half (keys kh0.. of the tile).
template <int D>
__device__ inline void mask_half(const FwdState<D>& st, f32x16 (&s)[NQB], uint32_t Dt, int32_t kb0, int kh0,
                                 bool docs, int hh) {
  asm volatile("; partial tile" ::: "memory");   // keeps the caller's branch real (no if-conversion)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kk = kh0 + (r >> 2) * 8 + hh * 4 + (r & 3);
    const int32_t kidx = kb0 + kk;
    const int32_t kd_ = lds_ld4i(Dt + 4 * kk);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const bool ok = (kidx < st.lim[qb]) & (!docs | (kd_ == st.qdoc[qb]));
      s[qb][r] = ok ? s[qb][r] : -INFINITY;
    }
  }
}

// Rows that have no reference point yet take the max of this half's scores
// (their accumulators and sums are still zero, so nothing is rescaled).
template <int D>
__device__ inline void init_half(FwdState<D>& st, const f32x16 (&s)[NQB], float c) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float m0 = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m0 = fmaxf(m0, fmaxf(s[qb][r], s[qb][r + 1]));
    m0 = fmaxf(m0, __shfl_xor(m0, 32));
    if (st.mrow[qb] == -INFINITY && m0 != -INFINITY) {
      st.mrow[qb] = m0;
      st.moff[qb] = -m0 * c;
    }
  }
}

template <int D>
__device__ inline bool unset_row(const FwdState<D>& st) {
  bool u = false;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) u |= st.mrow[qb] == -INFINITY;
  return u;
}

// One 64-key tile, one code path for all tiles (the same registers carry the
// accumulators throughout): partial tiles insert the mask and tiles with
// unset reference points insert the init between the pipeline stages.
template <int D>
__device__ inline float fwd_tile_piped(FwdState<D>& st, const RowReader<D>& rr, const TrReader<D>& tr, uint32_t Kt,
                                       uint32_t Vt, uint32_t Dt, int32_t kb0, bool full, bool docs, float c, int lane) {
  const int hh = lane >> 5;
  f32x16 s0[NQB], s1[NQB];
  bf16x8 p0[NQB][2], p1[NQB][2];
  float tsum[NQB] = {};
  qk_half<D>(st, rr, Kt, 0, s0);
  if (!full) mask_half<D>(st, s0, Dt, kb0, 0, docs, hh);
  if (__any(unset_row(st))) init_half<D>(st, s0, c);
  qk_half<D>(st, rr, Kt, 1, s1);
  exp_half<D>(st, s0, p0, tsum, c);
  
  keep_live(p0);   // P0 must be computed here, next to QK1, not sunk past the branches below
  if (!full) mask_half<D>(st, s1, Dt, kb0, 32, docs, hh);
  if (__any(unset_row(st))) init_half<D>(st, s1, c);
  pv_half<D>(st, tr, Vt, 0, p0);
  exp_half<D>(st, s1, p1, tsum, c);
  
  pv_half<D>(st, tr, Vt, 1, p1);
  float mx = 0.f;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) { st.lrow[qb] += tsum[qb]; mx = fmaxf(mx, tsum[qb]); }
  return mx;
}

// Exact online softmax for one tile (the fallback path): running max and
// rescaling of the accumulators whenever the max rises.
template <int D>
__device__ inline void fwd_tile_exact(FwdState<D>& st, const TrReader<D>& tr, uint32_t Vt, f32x16 (&s)[2][NQB], float c) {
  float mx[NQB];
  fwd_tile_max(s, mx);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float mn = fmaxf(st.mrow[qb], mx[qb]);
    if (mn > st.mrow[qb]) {
      const float alpha = (st.mrow[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((st.mrow[qb] - mn) * c);
      st.lrow[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) st.oacc[qb][db] *= alpha;
      st.mrow[qb] = mn;
      st.moff[qb] = -mn * c;
    }
  }
  fwd_accumulate<D>(st, tr, Vt, s, c);
}

template <int D>
__global__ __launch_bounds__(64 * NWV, 1) void fwd_bf16_kernel(FwdParams a) {
  // LDS arena: K and V tiles and the keys' doc ids, double-buffered.
  constexpr uint32_t TB = BK * D * 2, RW = BK * 4;     // bytes of one K or V tile, of one doc-id row
  constexpr uint32_t K0 = 0, K1 = TB, V0 = 2 * TB, V1 = 3 * TB, X0 = 4 * TB, X1 = X0 + RW;
  __shared__ __attribute__((aligned(16))) char smem[X1 + RW];
  __shared__ int32_t overflow_flag;
  const uint32_t S0 = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int lq = lane & 31, hh = lane >> 5;

  int32_t grp, hidx;
  if (!xcd_work(blockIdx.x, a.hq / a.heads_per_wg, a.nqt, grp, hidx)) return;
  const int32_t qt = a.nqt - 1 - hidx;                 // heavy first
  const int hpw = a.heads_per_wg;
  const int groups_per_kv = a.G / hpw;
  const int kvh = grp / groups_per_kv;
  const int head = kvh * a.G + (grp % groups_per_kv) * hpw + (wave % hpw);
  const int qblk = wave / hpw;

  const SpanD qs = a.qs, ks = a.ks;
  const int32_t Lq = span_len(qs), Lk = span_len(ks);
  const bool causal = a.causal != 0;
  const bool docs = qs.doc != nullptr;
  const int32_t wg_q0 = qt * QW * a.qblocks_per_wg;
  const int32_t wg_q1 = min(Lq, wg_q0 + QW * a.qblocks_per_wg);
  const int32_t q0 = wg_q0 + qblk * QW;
  const bool wave_live = q0 < Lq;
  const int32_t q1 = min(Lq, q0 + QW);

  // ---- key range of the work-group ------------------------------------
  int32_t klo = 0, khi = Lk;
  if (causal) khi = span_count_le(ks, span_pos(qs, wg_q1 - 1));
  if (docs) {
    klo = wave_lower_bound(ks.doc, Lk, qs.doc[wg_q0]);
    khi = min(khi, wave_lower_bound(ks.doc, Lk, qs.doc[wg_q1 - 1] + 1));
  }
  const int32_t kt0 = klo / BK;
  const int32_t kt1 = khi > klo ? (khi + BK - 1) / BK : kt0;

  const __bf16* kbase = a.k + (int64_t)kvh * D;
  const __bf16* vbase = a.v + (int64_t)kvh * D;
  const TileLoader<D, BK, NWV> ldr(a.kv_stride * 2, wave, lane);
  auto issue = [&](int32_t kt, uint32_t Kd, uint32_t Vd, uint32_t Dd) {
    if (kt * BK + BK <= Lk) {   // whole tile: precomputed lane offsets
      const int64_t boff = (int64_t)kt * BK * a.kv_stride;
      ldr.load(Kd, (const char*)(kbase + boff));
      ldr.load(Vd, (const char*)(vbase + boff));
    } else {                     // ragged last tile: rows clamped
      tile_load_lds<D, BK, NWV>(Kd, kbase, a.kv_stride, kt * BK, Lk, wave, lane);
      tile_load_lds<D, BK, NWV>(Vd, vbase, a.kv_stride, kt * BK, Lk, wave, lane);
    }
    if (docs && wave == 0) {
      const int32_t row = min(kt * BK + lane, Lk - 1);
      row_load_lds(ks.doc, row, Dd);
    }
  };
  if (kt0 < kt1) issue(kt0, S0 + K0, S0 + V0, S0 + X0);
  if (tid == 0) overflow_flag = 0;

  // ---- this wave's Q rows as MFMA B operands ----------------------------
  FwdState<D> st;
  auto reset = [&]() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) st.oacc[qb][db] = f32x16{};
      st.mrow[qb] = -INFINITY;
      st.moff[qb] = 0.f;
      st.lrow[qb] = 0.f;
    }
  };
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int32_t row = min(q0 + qb * 32 + lq, Lq - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (int64_t)row * a.q_stride + (int64_t)head * D + hh * 8);
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) st.qf[qb][kd] = src[kd * 2];
    st.lim[qb] = causal ? min(Lk, span_count_le(ks, span_pos(qs, row))) : Lk;
    st.qdoc[qb] = docs ? qs.doc[row] : 0;
  }
  reset();
  const float c = a.scale_log2;              // scale * log2(e)

  // wave-uniform bounds for classifying tiles: keys [0, lim_lo) are visible to
  // every row of the wave, keys >= lim_hi to none; doc ids of the first and
  // last row
  const int32_t lim_lo = causal ? min(Lk, span_count_le(ks, span_pos(qs, q0 < Lq ? q0 : Lq - 1))) : Lk;
  const int32_t lim_hi = causal ? min(Lk, span_count_le(ks, span_pos(qs, q1 - 1))) : Lk;
  const int32_t qd_lo = docs ? qs.doc[q0 < Lq ? q0 : Lq - 1] : 0;
  const int32_t qd_hi = docs ? qs.doc[q1 - 1] : 0;

  auto classify = [&](int32_t kt, uint32_t Dc, bool& live, bool& full) {
    const int32_t kb0 = kt * BK, kb1 = min(Lk, kb0 + BK);
    live = wave_live && kb0 < lim_hi;
    full = kb1 - kb0 == BK && kb1 <= lim_lo;
    if (docs) {
      const int32_t kd_lo = lds_ld4i(Dc), kd_hi = lds_ld4i(Dc + 4 * (kb1 - kb0 - 1));
      live = live && kd_hi >= qd_lo && kd_lo <= qd_hi;
      full = full && qd_lo == qd_hi && kd_lo == kd_hi && kd_lo == qd_lo;
    }
    // wave-uniform by construction; make it scalar so the branches are too
    live = __builtin_amdgcn_readfirstlane((int)live) != 0;
    full = __builtin_amdgcn_readfirstlane((int)full) != 0;
  };

  const RowReader<D> rr(lane);
  const TrReader<D> tr(lane);

  wait_vm0();
  __syncthreads();

  // ---- main loop: fixed reference point, accumulators touched by MFMA only --
  float worst = 0.f;   // largest tile row-sum share seen by this lane
  auto tile = [&](int32_t kt, uint32_t Kc, uint32_t Vc, uint32_t Dc, uint32_t Kn, uint32_t Vn, uint32_t Dn) {
    if (kt + 1 < kt1) issue(kt + 1, Kn, Vn, Dn);
    bool live, full;
    classify(kt, Dc, live, full);
    if (live) worst = fmaxf(worst, fwd_tile_piped<D>(st, rr, tr, Kc, Vc, Dc, kt * BK, full, docs, c, lane));
    wait_vm0();
    __syncthreads();
  };
  for (int32_t kt = kt0; kt < kt1; kt += 2) {
    tile(kt, S0 + K0, S0 + V0, S0 + X0, S0 + K1, S0 + V1, S0 + X1);
    if (kt + 1 < kt1) tile(kt + 1, S0 + K1, S0 + V1, S0 + X1, S0 + K0, S0 + V0, S0 + X0);
  }

  // ---- fallback: a row sum grew past 2^64 -> redo with the exact algorithm --
  if (__any(!(worst <= ROWSUM_LIMIT)) && lane == 0) atomicOr(&overflow_flag, 1);
  __syncthreads();
  if (overflow_flag != 0) {
    asm volatile("; exact fallback" ::: "memory");
    reset();
    if (kt0 < kt1) issue(kt0, S0 + K0, S0 + V0, S0 + X0);
    wait_vm0();
    __syncthreads();
    auto tile_exact = [&](int32_t kt, uint32_t Kc, uint32_t Vc, uint32_t Dc, uint32_t Kn, uint32_t Vn, uint32_t Dn) {
      if (kt + 1 < kt1) issue(kt + 1, Kn, Vn, Dn);
      bool live, full;
      classify(kt, Dc, live, full);
      if (live) {
        f32x16 s[2][NQB];
        fwd_scores<D>(st, rr, Kc, s);
        if (!full) fwd_mask<D>(st, s, Dc, kt * BK, docs, hh);
        fwd_tile_exact<D>(st, tr, Vc, s, c);
      }
      wait_vm0();
      __syncthreads();
    };
    for (int32_t kt = kt0; kt < kt1; kt += 2) {
      tile_exact(kt, S0 + K0, S0 + V0, S0 + X0, S0 + K1, S0 + V1, S0 + X1);
      if (kt + 1 < kt1) tile_exact(kt + 1, S0 + K1, S0 + V1, S0 + X1, S0 + K0, S0 + V0, S0 + X0);
    }
  }

  // ---- epilogue -----------------------------------------------------------
  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float ltot = st.lrow[qb] + __shfl_xor(st.lrow[qb], 32);
    const int32_t row = q0 + qb * 32 + lq;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (row < Lq) {
      const float lse = ltot > 0.f ? (st.mrow[qb] * c + __builtin_amdgcn_logf(ltot)) * LN2 : -INFINITY;
      float* lse_p = a.lse + (int64_t)head * a.lse_ld + row;
      // merge into a running (O, LSE) (nougat.kr MaxText page, section on
      // splitting heads or rotating the KV: a step's partial result is merged
      // into the running one): L = ln(e^La + e^Lb), weights e^(La-L), e^(Lb-L)
      // in fp64, -inf the identity.
      float w_acc = 0.f, w_new = 1.f, lse_out = lse;
      if (a.merge) {
        const double la = *lse_p, lb = lse;
        const double m = la > lb ? la : lb;
        if (m == -INFINITY) {
          w_new = 0.f;
        } else {
          const double L = m + log(exp(la - m) + exp(lb - m));
          w_acc = (float)exp(la - L);
          w_new = (float)exp(lb - L);
          lse_out = (float)L;
        }
      }
      if (hh == 0) *lse_p = lse_out;
      const int64_t obase = ((int64_t)row * a.hq + head) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + j * 8 + hh * 4;
          const float sc = inv * w_new;
          f32x4 v4 = {st.oacc[qb][db][4 * j] * sc, st.oacc[qb][db][4 * j + 1] * sc,
                      st.oacc[qb][db][4 * j + 2] * sc, st.oacc[qb][db][4 * j + 3] * sc};
          if (a.merge) {
            const f32x4 acc = *(const f32x4*)((const float*)a.o + obase + d);
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = fmaf(w_acc, acc[i], v4[i]);
          }
          if (a.o_f32) {
            *(f32x4*)((float*)a.o + obase + d) = v4;
          } else {
            const bf16x4 b4 = {(__bf16)v4[0], (__bf16)v4[1], (__bf16)v4[2], (__bf16)v4[3]};
            *(bf16x4*)((__bf16*)a.o + obase + d) = b4;
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  FwdParams a = p;
  const int32_t Lq = span_len(a.qs);
  a.heads_per_wg = a.G >= 4 ? 4 : a.G;
  a.qblocks_per_wg = NWV / a.heads_per_wg;
  a.nqt = (Lq + QW * a.qblocks_per_wg - 1) / (QW * a.qblocks_per_wg);
  a.scale_log2 = a.scale * LOG2E;
  const int32_t ngroups = a.hq / a.heads_per_wg;
  a.n_work = a.nqt * ngroups;
  if (a.n_work == 0) return hipSuccess;
  const int32_t grid = xcd_grid(ngroups, a.nqt);
  if (a.d == 128) {
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(64 * NWV), 0, stream, a);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(64 * NWV), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cp
