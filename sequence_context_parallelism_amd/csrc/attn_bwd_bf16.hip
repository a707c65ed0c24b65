// Backward chunk attention, bf16 inputs, fp32 accumulation, CDNA4 (gfx950).
//
// Given the final (merged) row LSE and Delta = rowsum(dO * O), adds this
// chunk pair's contribution to dQ, dK and dV: the gradient of the masked
// softmax attention whose forward is in attn_fwd_bf16.hip.  The pages do not
// describe the backward; it is the derivative of that definition, with P
// recomputed from the saved LSE (the recompute-in-backward idea behind
// activation checkpointing, siliconandsystems.com "Llama 3 parallelism",
// section on long context changing more than the attention cost).
//
// Two kernels, neither with atomics (deterministic):
//   dkdv (KV-outer): a work-group of 8 waves (two per SIMD) owns 128 keys of
//     one KV head and streams 64-row tiles of Q and dO for every query head
//     of the GQA group through LDS (direct-to-LDS loads, double-buffered).
//     The work-group's K and V rows stay resident in LDS.  Wave w takes keys
//     32(w % 4) .. +31 (their dK^T, dV^T accumulators in VGPRs) against query
//     rows 32(w / 4) .. +31 of each tile.  Per tile: S = Q K^T,
//     dP = dO V^T - Delta (row reads of both operands; the dP accumulator
//     starts at -Delta), P = exp2(S c + nl) with nl = -LSE log2 e, dS = P dP,
//     then dV^T += dO^T P and dK^T += Q^T dS (A operands read with the LDS
//     transpose read; P and dS go from the accumulator layout straight into
//     the B operand).  4 MFMA products per (query, key) pair.  The two waves
//     of a key block sum their partial dK, dV through LDS at the end; the
//     softmax scale of dK is applied once, there.
//   dq (Q-outer): a work-group of 8 waves (two per SIMD) owns 64 query rows
//     of 4 query heads sharing a KV head, 32 rows of one head per wave (like
//     the forward), and streams 64-key tiles of K and V.  Per tile:
//     S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, dQ^T += K^T dS^T.  3 MFMA products
//     per pair (S and dP are recomputed rather than exchanged).
// With two waves per SIMD each wave's exp/dS VALU work runs beside the other
// wave's MFMAs.  Masked entries get S = -inf before the exponential, so P = 0;
// fully masked tiles are skipped and element masks run only on partial or
// ragged tiles.  Heavy-first orders: ascending keys for dkdv, descending
// queries for dq.  Inside a dkdv work-group the query tiles run from the last
// one down.
#include "common.h"
#include "kernels.h"
#include "tile_io.h"

namespace cp {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BQ = 64;     // query rows per tile (dkdv) / per wave (dq)
constexpr int BKW = 32;    // keys per wave (dkdv)
constexpr int BKG = 128;   // keys per work-group (dkdv)
constexpr int BK = 64;     // keys per tile (dq)
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ inline f32x4 lds_f4(uint32_t a) { return *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)a; }
__device__ inline float lds_ldf(uint32_t a) { return *(const __attribute__((address_space(3))) float*)(uintptr_t)a; }
__device__ inline void lds_stf(uint32_t a, float x) { *(__attribute__((address_space(3))) float*)(uintptr_t)a = x; }

// -LSE * log2(e); an empty row (LSE = -inf) maps to -inf, so that
// exp2(S c + nl) = 0 for it whatever S is.
__device__ inline float neg_lse2(float lse) { return lse == -INFINITY ? -INFINITY : -lse * LOG2E; }

// ============================== dK, dV ======================================

// K rows sit this many bytes after the V rows in LDS (one 128-key tile)
template <int D>
constexpr uint32_t KV_GAP = 128 * D * 2;

template <int D>
struct KvState {
  f32x16 dka[D / 32], dva[D / 32]; // dK^T (unscaled), dV^T accumulators [d block]
  int32_t qlim;                    // queries [qlim, ..) see this lane's key causally
  int32_t kdoc;
  bool kvalid;
};

// Element mask of block qb: S = -inf where the lane's key is not visible.
template <int D>
__device__ inline void dkdv_mask(const KvState<D>& st, f32x16& s, uint32_t QDt, int32_t qa0, int qb,
                                 int32_t Lq, bool docs, int hh) {
  asm volatile("; partial tile" ::: "memory");   // keeps the caller's branch real (no if-conversion)
  int qbase = qb * 32 + hh * 4;
  asm volatile("" : "+v"(qbase));   // recomputed here, not hoisted out of the tile loop
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = qbase + (r >> 2) * 8 + (r & 3);
    const int32_t qidx = qa0 + qr;
    const bool ok = st.kvalid & (qidx < Lq) & (qidx >= st.qlim) & (!docs | (lds_ld4i(QDt + 4 * qr) == st.kdoc));
    s[r] = ok ? s[r] : -INFINITY;
  }
}

// The wave's 32 keys against the 32-query block qb of the tile (rows
// 32 qb .. 32 qb + 31): S and dP - Delta (accumulator element r: key = the
// lane's key, query row qb*32 + 8(r/4) + 4hh + r%4; the dP accumulator starts
// at -Delta), P = exp2(S c + nl), dS = P dP, then dV^T += dO^T P and
// dK^T += Q^T dS over that block's two 16-query slots.  rq and tq carry the
// block's row offset in their lane bases; vb is the lane's address in the
// wave's V rows (its K rows KV_GAP bytes on), so the tile offsets and the
// per-step offsets fold into the LDS instructions' immediates.
//
// Explicit software pipeline (scheduling walls keep the order): operand
// reads run two MFMAs ahead through a two-entry register ring, and slot 1's
// P/dS VALU work is spread over slot 0's gradient MFMAs.  The wave raises its
// issue priority for its two MFMA stretches and drops it for the mask and
// slot 0's P/dS, so the SIMD's other wave, if it is in a VALU stretch, yields
// the issue slots to the MFMAs, and its own VALU work fills the gaps.
template <int D>
__device__ inline void dkdv_block(KvState<D>& st, const RowReader<D>& rq, const TrReader<D>& tq, uint32_t Qt,
                                  uint32_t Ot, uint32_t vb, uint32_t Nl, uint32_t NDt, uint32_t QDt, int32_t qa0,
                                  int qb, int32_t Lq, bool mask, bool docs, float c, int lane) {
  constexpr int NKD = D / 16, NDB = D / 32;
  const int hh = lane >> 5;
  f32x16 s, dp;
  {
    f32x16 init;   // -Delta of the element's query row
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 d4 = lds_f4(NDt + 4 * (qb * 32 + j * 8 + hh * 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) init[j * 4 + i] = d4[i];
    }
    bf16x8 ra[2], ro[2], rv[2], rk[2];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ra[k] = rq.at(Qt, 0, k);
      ro[k] = rq.at(Ot, 0, k);
      rv[k] = lds_ld16(vb ^ (uint32_t)(k << 5));
      rk[k] = lds_ld16((vb ^ (uint32_t)(k << 5)) + KV_GAP<D>);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[kd & 1], rk[kd & 1], kd ? s : f32x16{}, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ro[kd & 1], rv[kd & 1], kd ? dp : init, 0, 0, 0);
      if (kd + 2 < NKD) {
        ra[kd & 1] = rq.at(Qt, 0, kd + 2);
        ro[kd & 1] = rq.at(Ot, 0, kd + 2);
        rv[kd & 1] = lds_ld16(vb ^ (uint32_t)((kd + 2) << 5));
        rk[kd & 1] = lds_ld16((vb ^ (uint32_t)((kd + 2) << 5)) + KV_GAP<D>);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (mask) dkdv_mask<D>(st, s, QDt, qa0, qb, Lq, docs, hh);
  __builtin_amdgcn_sched_barrier(0);

  // gradient operands of MFMA pair m (slot m / NDB, d block m % NDB)
  bf16x8 go[2], gq[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    go[m] = tq.at(Ot, 16 * (m / NDB), m % NDB);
    gq[m] = tq.at(Qt, 16 * (m / NDB), m % NDB);
  }
  bf16x8 pf[2], dsf[2];
  auto pds = [&](int r, const f32x4& n4) {
    const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, n4[r & 3]));
    pf[r >> 3][r & 7] = (__bf16)p;
    dsf[r >> 3][r & 7] = (__bf16)(p * dp[r]);
  };
  {
    const f32x4 n0 = lds_f4(Nl + 4 * (qb * 32 + 0 * 8 + hh * 4));
    const f32x4 n1 = lds_f4(Nl + 4 * (qb * 32 + 1 * 8 + hh * 4));
#pragma unroll
    for (int r = 0; r < 4; ++r) pds(r, n0);
#pragma unroll
    for (int r = 4; r < 8; ++r) pds(r, n1);
  }
  const f32x4 n2 = lds_f4(Nl + 4 * (qb * 32 + 2 * 8 + hh * 4));
  const f32x4 n3 = lds_f4(Nl + 4 * (qb * 32 + 3 * 8 + hh * 4));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  constexpr int PER = 8 / NDB;   // slot-1 elements per slot-0 MFMA pair
#pragma unroll
  for (int m = 0; m < 2 * NDB; ++m) {
    const int u = m / NDB, db = m % NDB;
    st.dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(go[m & 1], pf[u], st.dva[db], 0, 0, 0);
    st.dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gq[m & 1], dsf[u], st.dka[db], 0, 0, 0);
    if (m + 2 < 2 * NDB) {
      go[m & 1] = tq.at(Ot, 16 * ((m + 2) / NDB), (m + 2) % NDB);
      gq[m & 1] = tq.at(Qt, 16 * ((m + 2) / NDB), (m + 2) % NDB);
    }
    if (m < NDB) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int r = 8 + m * PER + e;
        pds(r, r < 12 ? n2 : n3);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

__device__ inline void lds_st4(uint32_t a, const f32x4& x) {
  *(__attribute__((address_space(3))) f32x4*)(uintptr_t)a = x;
}

// Park a 32-key x D accumulator set (accumulator layout) at LDS address P, or
// add the parked one into it: lane-contiguous 16-byte groups.
template <int D>
__device__ inline void park_acc(uint32_t P, const f32x16 (&acc)[D / 32], int lane) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lds_st4(P + ((db * 4 + j) * 64 + lane) * 16,
              f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]});
}
template <int D>
__device__ inline void unpark_add(uint32_t P, f32x16 (&acc)[D / 32], int lane) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = lds_f4(P + ((db * 4 + j) * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][4 * j + i] += x[i];
    }
}

// dst[key row, d] += mul * acc, or = with `store` (accumulator layout:
// d = db*32 + 8j + 4hh + i)
template <int D>
__device__ inline void add_rows(float* dst, const f32x16 (&acc)[D / 32], float mul, int hh, bool store) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4* p = (f32x4*)(dst + db * 32 + j * 8 + hh * 4);
      f32x4 o = store ? f32x4{} : *p;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] += mul * acc[db][4 * j + i];
      *p = o;
    }
}

constexpr int KNW = 8;   // waves per dkdv work-group: 4 key blocks x 2 query halves

template <int D>
__global__ __launch_bounds__(64 * KNW, 1) void dkdv_bf16_kernel(BwdParams a) {
  // LDS arena: Q and dO tiles (double-buffered), then per-row LSE (as
  // -LSE log2 e), -Delta and doc ids, each double-buffered, then the work-
  // group's V rows and K rows (read as MFMA B operands).  After the tile loop
  // the tile area holds the parked partial accumulators (4 x 32 keys x D
  // floats = as many bytes as the four tiles).
  constexpr uint32_t TB = BQ * D * 2, RW = BQ * 4;
  constexpr uint32_t Q0 = 0, Q1 = TB, O0 = 2 * TB, O1 = 3 * TB;
  constexpr uint32_t L0 = 4 * TB, L1 = L0 + RW, N0 = L1 + RW, N1 = N0 + RW, X0 = N1 + RW, X1 = X0 + RW;
  constexpr uint32_t VT = X1 + RW;   // V rows, then K rows KV_GAP bytes on
  static_assert(4 * BKW * D * 4 <= 4 * TB, "parked accumulators must fit in the tile area");
  static_assert(VT % 16 == 0, "V tile alignment");
  static_assert(KV_GAP<D> == BKG * D * 2, "K rows follow the V rows");
  __shared__ __attribute__((aligned(16))) char smem[VT + 2 * BKG * D * 2];
  const uint32_t S0 = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int kb = wave & 3, qh = wave >> 2;                      // key block, query half
  const int lq = lane & 31, hh = lane >> 5;

  int32_t kvh, kt;                                      // ascending kt = heavy first
  if (!xcd_work(blockIdx.x, a.hkv, a.nkt, kvh, kt)) return;

  const SpanD qs = a.qs, ks = a.ks;
  const int32_t Lq = span_len(qs), Lk = span_len(ks);
  const bool causal = a.causal != 0;
  const bool docs = qs.doc != nullptr;
  const int32_t k0 = kt * BKG, k1 = min(Lk, k0 + BKG);
  const int32_t wk0 = k0 + kb * BKW, wk1 = min(Lk, wk0 + BKW);
  const bool wave_has_keys = wk0 < Lk;

  // ---- query range of the work-group ------------------------------------
  int32_t qlo = 0, qhi = Lq;
  if (causal) qlo = span_count_lt(qs, span_pos(ks, k0));
  if (docs) {
    qlo = max(qlo, wave_lower_bound(qs.doc, Lq, ks.doc[k0]));
    qhi = min(qhi, wave_lower_bound(qs.doc, Lq, ks.doc[k1 - 1] + 1));
  }
  const int32_t qt0 = qlo / BQ;
  const int32_t qt1 = qhi > qlo ? (qhi + BQ - 1) / BQ : qt0;
  const int G = a.G;
  const int nitems = (qt1 - qt0) * G;

  // Item `it` = (query tile, head), query tiles in DESCENDING order: the
  // work-groups resident on one XCD hold different key blocks of the same KV
  // head, so starting them all at the last query tile has them read the same
  // Q/dO tiles at about the same time (L2 hits instead of HBM re-reads).
  // Q, dO tiles and the rows' LSE, Delta (and doc ids) of item `it`.  The
  // wave that loaded the LSE (Delta) row converts it in LDS once its loads
  // have landed (prepare): nl = -LSE log2 e, and -Delta.
  const TileLoader<D, BQ, KNW> ldq(a.q_stride * 2, wave, lane), ldo((int64_t)a.hq * D * 2, wave, lane);
  // The next item to issue, kept as running byte pointers (wave-uniform, in
  // SGPRs) that move by constant steps: one head on, or back to the group's
  // first head and one query tile down.  No division or 64-bit multiply per
  // item.
  struct Cursor {
    int32_t qt, g;
    const char *q, *o;
    const float *l, *d;
  };
  Cursor nx{qt1 - 1, 0,
            (const char*)(a.q + (int64_t)(qt1 - 1) * BQ * a.q_stride + (int64_t)kvh * G * D),
            (const char*)(a.dout + ((int64_t)(qt1 - 1) * BQ * a.hq + (int64_t)kvh * G) * D),
            a.lse + (int64_t)kvh * G * a.lse_ld, a.delta + (int64_t)kvh * G * a.lse_ld};
  const int64_t q_back = (int64_t)BQ * a.q_stride * 2 + (int64_t)G * D * 2;    // bytes
  const int64_t o_back = ((int64_t)BQ * a.hq + G) * D * 2;
  const int64_t l_back = (int64_t)G * a.lse_ld;                                // floats
  auto advance = [&](Cursor& c) {
    c.q += D * 2;
    c.o += D * 2;
    c.l += a.lse_ld;
    c.d += a.lse_ld;
    if (++c.g == G) {
      c.g = 0;
      --c.qt;
      c.q -= q_back;
      c.o -= o_back;
      c.l -= l_back;
      c.d -= l_back;
    }
  };
  auto issue = [&](const Cursor& c, uint32_t Qd, uint32_t Od, uint32_t Ld, uint32_t Dd, uint32_t Xd) {
    if (c.qt * BQ + BQ <= Lq) {   // whole tile: precomputed lane offsets
      ldq.load(Qd, c.q);
      ldo.load(Od, c.o);
    } else {                      // ragged last tile: rows clamped
      const int head = kvh * G + c.g;
      tile_load_lds<D, BQ, KNW>(Qd, a.q + (int64_t)head * D, a.q_stride, c.qt * BQ, Lq, wave, lane);
      tile_load_lds<D, BQ, KNW>(Od, a.dout + (int64_t)head * D, (int64_t)a.hq * D, c.qt * BQ, Lq, wave, lane);
    }
    const int32_t row = min(c.qt * BQ + lane, Lq - 1);
    if (wave == 0)
      row_load_lds(c.l, row, Ld);
    else if (wave == 1)
      row_load_lds(c.d, row, Dd);
    else if (wave == 2 && docs)
      row_load_lds(qs.doc, row, Xd);
  };
  auto prepare = [&](uint32_t Ld, uint32_t Dd) {
    if (wave == 0) lds_stf(Ld + 4 * lane, neg_lse2(lds_ldf(Ld + 4 * lane)));
    else if (wave == 1) lds_stf(Dd + 4 * lane, -lds_ldf(Dd + 4 * lane));
  };
  if (nitems > 0) {
    // the work-group's V rows (rows past Lk clamped: their keys are masked)
    if (k0 + BKG <= Lk) {
      const TileLoader<D, BKG, KNW> ldv(a.kv_stride * 2, wave, lane);
      ldv.load(S0 + VT, (const char*)(a.v + (int64_t)k0 * a.kv_stride + (int64_t)kvh * D));
      ldv.load(S0 + VT + KV_GAP<D>, (const char*)(a.k + (int64_t)k0 * a.kv_stride + (int64_t)kvh * D));
    } else {
      tile_load_lds<D, BKG, KNW>(S0 + VT, a.v + (int64_t)kvh * D, a.kv_stride, k0, Lk, wave, lane);
      tile_load_lds<D, BKG, KNW>(S0 + VT + KV_GAP<D>, a.k + (int64_t)kvh * D, a.kv_stride, k0, Lk, wave, lane);
    }
    issue(nx, S0 + Q0, S0 + O0, S0 + L0, S0 + N0, S0 + X0);
    advance(nx);
  }
  const uint32_t Vw = S0 + VT + kb * (BKW * D * 2);   // this wave's 32 V rows

  KvState<D> st;
  {
    const int32_t mykey = min(wk0 + lq, Lk - 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) { st.dka[db] = f32x16{}; st.dva[db] = f32x16{}; }
    st.qlim = causal ? span_count_lt(qs, span_pos(ks, mykey)) : 0;
    st.kdoc = docs ? ks.doc[mykey] : 0;
    st.kvalid = wk0 + lq < Lk;
  }
  // wave-uniform bounds: queries >= q_all see all of the wave's keys, queries
  // < q_none see none of them (causally)
  const int32_t wlast = wave_has_keys ? wk1 - 1 : Lk - 1;
  const int32_t q_none = causal ? span_count_lt(qs, span_pos(ks, wave_has_keys ? wk0 : Lk - 1)) : 0;
  const int32_t q_all = causal ? span_count_lt(qs, span_pos(ks, wlast)) : 0;
  const int32_t kd_lo = docs ? ks.doc[wave_has_keys ? wk0 : Lk - 1] : 0;
  const int32_t kd_hi = docs ? ks.doc[wlast] : 0;
  const float c = a.scale * LOG2E;

  // lane bases with this wave's query half (rows 32 qh ..) and V rows folded
  // in; the XOR-ed chunk and d-block steps act on bits the offsets leave clear
  RowReader<D> rq(lane);
  TrReader<D> tq(lane);
  const uint32_t vb = Vw + rq.base;
  rq.base += (uint32_t)(qh * 32 * 2 * D);
  tq.b0 += (uint32_t)(qh * 32 * 2 * D);
  tq.b1 += (uint32_t)(qh * 32 * 2 * D);

  wait_vm0();
  if (nitems > 0) prepare(S0 + L0, S0 + N0);
  __syncthreads();

  int32_t cur_qt = qt1 - 1, cur_g = 0;   // the item being computed
  auto step = [&](int it, uint32_t Qc, uint32_t Oc, uint32_t Lc, uint32_t Dc, uint32_t Xc, uint32_t Qn,
                  uint32_t On, uint32_t Ln, uint32_t Dn, uint32_t Xn) {
    if (it + 1 < nitems) {
      issue(nx, Qn, On, Ln, Dn, Xn);
      advance(nx);
    }
    const int32_t qa0 = cur_qt * BQ;
    if (++cur_g == G) { cur_g = 0; --cur_qt; }
    const int32_t wq0 = qa0 + 32 * qh, wq1 = min(Lq, wq0 + 32);   // this wave's query rows
    bool live = wave_has_keys && wq0 < Lq && wq1 - 1 >= q_none;
    bool full = wq1 - wq0 == 32 && wq0 >= q_all && wk1 - wk0 == BKW;
    if (docs) {   // both reads stay inside the 64-row buffer (qa0 < Lq)
      const int32_t qd_lo = lds_ld4i(Xc + 4 * min(32 * qh, Lq - 1 - qa0)), qd_hi = lds_ld4i(Xc + 4 * (wq1 - 1 - qa0));
      live = live && kd_hi >= qd_lo && kd_lo <= qd_hi;
      full = full && qd_lo == qd_hi && kd_lo == kd_hi && kd_lo == qd_lo;
    }
    live = __builtin_amdgcn_readfirstlane((int)live) != 0;   // wave-uniform: scalar branches
    full = __builtin_amdgcn_readfirstlane((int)full) != 0;
    if (live) dkdv_block<D>(st, rq, tq, Qc, Oc, vb, Lc, Dc, Xc, qa0, qh, Lq, !full, docs, c, lane);
    wait_vm0();
    if (it + 1 < nitems) prepare(Ln, Dn);
    __syncthreads();
  };
  for (int it = 0; it < nitems; it += 2) {
    step(it, S0 + Q0, S0 + O0, S0 + L0, S0 + N0, S0 + X0, S0 + Q1, S0 + O1, S0 + L1, S0 + N1, S0 + X1);
    if (it + 1 < nitems)
      step(it + 1, S0 + Q1, S0 + O1, S0 + L1, S0 + N1, S0 + X1, S0 + Q0, S0 + O0, S0 + L0, S0 + N0, S0 + X0);
  }

  // ---- sum the two query halves; dK (scaled here), dV: exclusive to this
  // work-group, read-modify-write.  The second-half wave of key block kb
  // parks its dK^T, the first-half wave adds it and writes dK; then the
  // roles swap for dV.  The loop ended with a barrier: the arena is free.
  const uint32_t P = S0 + kb * (BKW * D * 4);
  const bool writer = st.kvalid && wave_has_keys;
  float* const krow = a.dk + ((int64_t)(wk0 + lq) * a.hkv + kvh) * D;
  float* const vrow = a.dv + ((int64_t)(wk0 + lq) * a.hkv + kvh) * D;
  if (qh == 1) park_acc<D>(P, st.dka, lane);
  __syncthreads();
  if (qh == 0) {
    unpark_add<D>(P, st.dka, lane);
    if (writer) add_rows<D>(krow, st.dka, a.scale, hh, a.store != 0);
  }
  __syncthreads();
  if (qh == 0) park_acc<D>(P, st.dva, lane);
  __syncthreads();
  if (qh == 1) {
    unpark_add<D>(P, st.dva, lane);
    if (writer) add_rows<D>(vrow, st.dva, 1.0f, hh, a.store != 0);
  }
}

// ================================= dQ =======================================

constexpr int DQB = 1;     // 32-row query blocks per wave (dq)
constexpr int DQW = 32 * DQB;
constexpr int DNW = 8;     // waves per work-group (dq), two per SIMD

template <int D>
struct QState {
  bf16x8 qf[DQB][D / 16];   // B operands: the wave's query rows
  bf16x8 of[DQB][D / 16];   // B operands: their dO rows
  f32x16 acc[DQB][D / 32];  // dQ^T accumulators (unscaled) [query block][d block]
  float nl[DQB];            // -LSE * log2(e) of the lane's query column
  float dl[DQB];            // Delta of the lane's query column
  int32_t lim[DQB];         // keys [0, lim) are causally visible (and < Lk)
  int32_t qdoc[DQB];
};

// S^T accumulator element r of the 32-key half starting at key kh0 of the
// tile: query = the lane's column, key = kh0 + 8(r/4) + 4hh + r%4.  Masked
// entries get -inf.
template <int D>
__device__ inline void dq_mask(const QState<D>& st, f32x16& s, uint32_t Dt, int32_t kb0, int kh0, bool docs,
                               int hh) {
  asm volatile("; partial tile" ::: "memory");   // keeps the caller's branch real (no if-conversion)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kk = kh0 + (r >> 2) * 8 + hh * 4 + (r & 3);
    const int32_t kd_ = lds_ld4i(Dt + 4 * kk);
    const bool ok = (kb0 + kk < st.lim[0]) & (!docs | (kd_ == st.qdoc[0]));
    s[r] = ok ? s[r] : -INFINITY;
  }
}

// One 64-key tile for one wave as an explicit software pipeline (scheduling
// walls keep the order): S^T, dP^T of key half 0; those of half 1 beside
// half 0's dS^T; dQ^T += K^T dS^T of half 0 beside half 1's dS^T; then half
// 1's.  Operand reads run two MFMAs ahead through two-entry register rings.
// dS^T = P^T (dP^T - Delta) with P^T = exp2(S^T c + nl) goes from the
// accumulator layout straight into the B operand of the dQ^T product.
template <int D>
__device__ inline void dq_tile(QState<D>& st, const RowReader<D>& rr, const TrReader<D>& tr, uint32_t Kt,
                               uint32_t Vt, uint32_t Dt, int32_t kb0, bool mask, bool docs, float c, int lane) {
  static_assert(DQB == 1, "one 32-row query block per wave");
  constexpr int NKD = D / 16, NDB = D / 32, NG = 2 * NDB;   // d steps; d blocks; dQ MFMAs per half
  const int hh = lane >> 5;
  f32x16 s0, dp0, s1, dp1;
  bf16x8 ds0[2], ds1[2];
  bf16x8 rk[2], rv[2];   // K, V row operands (S^T, dP^T)
  bf16x8 ga[2];          // K^T operands (dQ^T)
  auto ds_elem = [&](const f32x16& s, const f32x16& dp, bf16x8 (&dsf)[2], int r) {
    const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, st.nl[0]));
    dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - st.dl[0]));
  };
  // step j of the tile's 2*NKD S/dP steps: key half j / NKD, d step j % NKD
  auto ld_row = [&](int j) {
    rk[j & 1] = rr.at(Kt, j / NKD, j % NKD);
    rv[j & 1] = rr.at(Vt, j / NKD, j % NKD);
  };
  // dQ MFMA g of the tile's 2*NG: key half g / NG, 16-key slot (g % NG) / NDB, d block g % NDB
  auto ld_tr = [&](int g) { ga[g & 1] = tr.at(Kt, 32 * (g / NG) + 16 * ((g % NG) / NDB), g % NDB); };

  ld_row(0);
  ld_row(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {   // half 0
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rk[kd & 1], st.qf[0][kd], kd ? s0 : f32x16{}, 0, 0, 0);
    dp0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rv[kd & 1], st.of[0][kd], kd ? dp0 : f32x16{}, 0, 0, 0);
    ld_row(kd + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (mask) dq_mask<D>(st, s0, Dt, kb0, 0, docs, hh);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {   // half 1 beside half 0's dS
    const int j = NKD + kd;
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rk[j & 1], st.qf[0][kd], kd ? s1 : f32x16{}, 0, 0, 0);
    dp1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rv[j & 1], st.of[0][kd], kd ? dp1 : f32x16{}, 0, 0, 0);
    if (j + 2 < 2 * NKD) ld_row(j + 2);
    else ld_tr(j + 2 - 2 * NKD);
#pragma unroll
    for (int e = 0; e < 16 / NKD; ++e) ds_elem(s0, dp0, ds0, kd * (16 / NKD) + e);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (mask) dq_mask<D>(st, s1, Dt, kb0, 32, docs, hh);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < 2 * NG; ++g) {   // dQ of half 0 beside half 1's dS, then half 1
    const int t = (g % NG) / NDB, db = g % NDB;
    st.acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[g & 1], g < NG ? ds0[t] : ds1[t], st.acc[0][db], 0,
                                                            0, 0);
    if (g + 2 < 2 * NG) ld_tr(g + 2);
    if (g < NG) {
#pragma unroll
      for (int e = 0; e < 16 / NG; ++e) ds_elem(s1, dp1, ds1, g * (16 / NG) + e);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__global__ __launch_bounds__(64 * DNW, 1) void dq_bf16_kernel(BwdParams a) {
  // LDS arena: K and V tiles and the keys' doc ids, double-buffered.
  constexpr uint32_t TB = BK * D * 2, RW = BK * 4;
  constexpr uint32_t K0 = 0, K1 = TB, V0 = 2 * TB, V1 = 3 * TB, X0 = 4 * TB, X1 = X0 + RW;
  __shared__ __attribute__((aligned(16))) char smem[X1 + RW];
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
  const int32_t wg_q0 = qt * DQW * a.qblocks_per_wg;
  const int32_t wg_q1 = min(Lq, wg_q0 + DQW * a.qblocks_per_wg);
  const int32_t q0 = wg_q0 + qblk * DQW;
  const bool wave_live = q0 < Lq;
  const int32_t q1 = min(Lq, q0 + DQW);

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
  const TileLoader<D, BK, DNW> ldr(a.kv_stride * 2, wave, lane);
  auto issue = [&](int32_t t, uint32_t Kd, uint32_t Vd, uint32_t Xd) {
    if (t * BK + BK <= Lk) {   // whole tile: precomputed lane offsets
      const int64_t boff = (int64_t)t * BK * a.kv_stride;
      ldr.load(Kd, (const char*)(kbase + boff));
      ldr.load(Vd, (const char*)(vbase + boff));
    } else {                   // ragged last tile: rows clamped
      tile_load_lds<D, BK, DNW>(Kd, kbase, a.kv_stride, t * BK, Lk, wave, lane);
      tile_load_lds<D, BK, DNW>(Vd, vbase, a.kv_stride, t * BK, Lk, wave, lane);
    }
    if (docs && wave == 0) {
      const int32_t row = min(t * BK + lane, Lk - 1);
      row_load_lds(ks.doc, row, Xd);
    }
  };
  if (kt0 < kt1) issue(kt0, S0 + K0, S0 + V0, S0 + X0);

  QState<D> st;
#pragma unroll
  for (int qb = 0; qb < DQB; ++qb) {
    const int32_t row = min(q0 + qb * 32 + lq, Lq - 1);
    const bf16x8* qsrc = (const bf16x8*)(a.q + (int64_t)row * a.q_stride + (int64_t)head * D + hh * 8);
    const bf16x8* osrc = (const bf16x8*)(a.dout + ((int64_t)row * a.hq + head) * D + hh * 8);
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      st.qf[qb][kd] = qsrc[kd * 2];
      st.of[qb][kd] = osrc[kd * 2];
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.acc[qb][db] = f32x16{};
    st.nl[qb] = neg_lse2(a.lse[(int64_t)head * a.lse_ld + row]);
    st.dl[qb] = a.delta[(int64_t)head * a.lse_ld + row];
    st.lim[qb] = causal ? min(Lk, span_count_le(ks, span_pos(qs, row))) : Lk;
    st.qdoc[qb] = docs ? qs.doc[row] : 0;
  }
  const int32_t lim_lo = causal ? min(Lk, span_count_le(ks, span_pos(qs, q0 < Lq ? q0 : Lq - 1))) : Lk;
  const int32_t lim_hi = causal ? min(Lk, span_count_le(ks, span_pos(qs, q1 - 1))) : Lk;
  const int32_t qd_lo = docs ? qs.doc[q0 < Lq ? q0 : Lq - 1] : 0;
  const int32_t qd_hi = docs ? qs.doc[q1 - 1] : 0;
  const float c = a.scale * LOG2E;

  const RowReader<D> rr(lane);
  const TrReader<D> tr(lane);

  wait_vm0();
  __syncthreads();

  auto step = [&](int32_t t, uint32_t Kc, uint32_t Vc, uint32_t Xc, uint32_t Kn, uint32_t Vn, uint32_t Xn) {
    if (t + 1 < kt1) issue(t + 1, Kn, Vn, Xn);
    const int32_t kb0 = t * BK, kb1 = min(Lk, kb0 + BK);
    bool live = wave_live && kb0 < lim_hi;
    bool full = kb1 - kb0 == BK && kb1 <= lim_lo;
    if (docs) {
      const int32_t kd_lo = lds_ld4i(Xc), kd_hi = lds_ld4i(Xc + 4 * (kb1 - kb0 - 1));
      live = live && kd_hi >= qd_lo && kd_lo <= qd_hi;
      full = full && qd_lo == qd_hi && kd_lo == kd_hi && kd_lo == qd_lo;
    }
    live = __builtin_amdgcn_readfirstlane((int)live) != 0;   // wave-uniform: scalar branches
    full = __builtin_amdgcn_readfirstlane((int)full) != 0;
    if (live) dq_tile<D>(st, rr, tr, Kc, Vc, Xc, kb0, !full, docs, c, lane);
    wait_vm0();
    __syncthreads();
  };
  for (int32_t t = kt0; t < kt1; t += 2) {
    step(t, S0 + K0, S0 + V0, S0 + X0, S0 + K1, S0 + V1, S0 + X1);
    if (t + 1 < kt1) step(t + 1, S0 + K1, S0 + V1, S0 + X1, S0 + K0, S0 + V0, S0 + X0);
  }

  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < DQB; ++qb) {
    const int32_t row = q0 + qb * 32 + lq;
    if (row < Lq) {
      float* dst = a.dq + ((int64_t)row * a.hq + head) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4* p = (f32x4*)(dst + db * 32 + j * 8 + hh * 4);
          f32x4 v = a.store ? f32x4{} : *p;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += a.scale * st.acc[qb][db][4 * j + i];
          *p = v;
        }
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16_dkdv(const BwdParams& p, hipStream_t stream) {
  if (span_len(p.qs) == 0 || span_len(p.ks) == 0) return hipSuccess;
  BwdParams a = p;
  a.nkt = (span_len(a.ks) + BKG - 1) / BKG;
  a.n_work = a.nkt * a.hkv;
  const int32_t grid = xcd_grid(a.hkv, a.nkt);
  if (a.d == 128) hipLaunchKernelGGL(dkdv_bf16_kernel<128>, dim3(grid), dim3(64 * KNW), 0, stream, a);
  else hipLaunchKernelGGL(dkdv_bf16_kernel<64>, dim3(grid), dim3(64 * KNW), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16_dq(const BwdParams& p, hipStream_t stream) {
  if (span_len(p.qs) == 0 || span_len(p.ks) == 0) return hipSuccess;
  BwdParams b = p;
  b.heads_per_wg = b.G >= 4 ? 4 : b.G;
  b.qblocks_per_wg = DNW / b.heads_per_wg;
  b.nqt = (span_len(b.qs) + DQW * b.qblocks_per_wg - 1) / (DQW * b.qblocks_per_wg);
  b.n_work = b.nqt * (b.hq / b.heads_per_wg);
  const int32_t grid = xcd_grid(b.hq / b.heads_per_wg, b.nqt);
  if (b.d == 128) hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3(grid), dim3(64 * DNW), 0, stream, b);
  else hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3(grid), dim3(64 * DNW), 0, stream, b);
  return hipGetLastError();
}

// dQ first: the two kernels are independent, and whatever runs after the
// backward (the next step's forward) then starts behind the dK/dV kernel,
// which draws less power than the dQ kernel and leaves the shader clock
// higher (measured on the 64K Ulysses share: 34.29-34.34 -> 33.91-33.93 ms per
// forward + backward step on one box).
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  hipError_t e = launch_bwd_bf16_dq(p, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_bf16_dkdv(p, stream);
}

}  // namespace cp
