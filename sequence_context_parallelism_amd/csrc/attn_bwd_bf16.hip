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
//     one KV head and streams 64-row items (query tile, query head) of Q, dO
//     and the row arrays through LDS (direct-to-LDS loads, three buffers).
//     The two waves of a SIMD own the same 32 keys and split the products:
//     one holds the K rows in VGPRs and computes S = Q K^T,
//     P = exp2(S c + nl) (nl = -LSE log2 e) and dV^T += dO^T P; the other
//     holds the V rows and computes dP = dO V^T - Delta (accumulator started
//     at -Delta), dS = P dP with P passed through LDS, and dK^T += Q^T dS.
//     4 MFMA products per (query, key) pair, each wave reading one operand
//     per MFMA from LDS (row reads, or the LDS transpose read for the
//     gradient products' A operands).  The softmax scale of dK is applied
//     once, at the end.  Key tiles kt and nkt-1-kt run as partners on one
//     XCD, the first walking its query tiles from the last, the second from
//     the first (dkdv_work in common.h), so that the work-groups of an XCD
//     share the Q/dO tiles they copy through its L2.
//   dq (Q-outer): a work-group of 8 waves (two per SIMD) owns 64 query rows
//     of 4 query heads sharing a KV head, 32 rows of one head per wave (like
//     the forward), and streams 64-key tiles of K and V.  Per tile:
//     S^T = K Q^T, dP^T = V dO^T, P^T, dS^T, dQ^T += K^T dS^T.  3 MFMA products
//     per pair (S and dP are recomputed rather than exchanged).
// With two waves per SIMD each wave's exp/dS VALU work runs beside the other
// wave's MFMAs.  Masked entries get S = -inf before the exponential, so P = 0;
// fully masked tiles are skipped and element masks run only on partial or
// ragged tiles.  The dq work-groups run heavy-first (descending queries).
#include <type_traits>

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
//
// The work-group owns 128 keys of one KV head and streams 64-row items
// (query tile, query head) through LDS, triple-buffered.  Each SIMD holds 32
// of the keys and its two waves split the four products of the item's two
// 32-row blocks between them:
//   wave "P" (waves 0-3): S = Q K^T with the wave's K rows in VGPRs,
//     P = exp2(S c + nl), dV^T += dO^T P;  P goes to its partner through LDS;
//   wave "dS" (waves 4-7): dP = dO V^T - Delta with the wave's V rows in
//     VGPRs, dS = P dP, dK^T += Q^T dS.
// Each wave reads one 1 KiB operand from LDS per MFMA (the other is in
// registers) and keeps one set of accumulators (dV^T or dK^T) for all rows,
// so the end needs no exchange between waves.  Interval k (between two
// work-group barriers) runs item k's score products and item k-1's gradient
// products: P and dP of item k-1 are carried in registers across one
// barrier, the Q/dO tiles of items k-1 and k are resident while item k+1's
// copy lands.  Both 32-row blocks of an item are always computed (their two
// accumulator chains interleave); a block with no allowed entry gets P = 0
// from the element mask, and an item with none is skipped whole.

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

constexpr int KNW = 8;   // waves per dkdv work-group: 4 key blocks x 2 roles

template <int D>
struct KvState {
  bf16x8 kv[D / 16];   // this wave's K (P wave) or V (dS wave) rows: MFMA B operands, lane = key
  f32x16 acc[D / 32];  // dV^T (P wave) or dK^T (dS wave, unscaled)
  f32x16 sc[2];        // P wave: S of the item's two blocks; dS wave: dP - Delta
  bf16x8 pb[2][2];     // P wave: P of the two blocks (B operand layout), kept for the gradient
  int32_t qlim, kdoc;
  bool kvalid;
};

// Scores of both 32-row blocks of the item in tile Tt, their accumulator
// chains interleaved: S (P wave: A = Q rows) or dP (dS wave: A = dO rows,
// accumulators from -Delta at NDt).
template <int D, bool DS>
__device__ inline void kv_scores(KvState<D>& st, const RowLanes<D>& rq, uint32_t Tt, uint32_t NDt, int hh) {
  constexpr int NKD = D / 16;
  if constexpr (DS) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 d4 = lds_f4(NDt + 4 * (qb * 32 + j * 8 + hh * 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) st.sc[qb][j * 4 + i] = d4[i];
      }
  }
  bf16x8 r0[2], r1[2];
  r0[0] = rq.at(Tt, 0, 0);
  r1[0] = rq.at(Tt, 1, 0);
  r0[1] = rq.at(Tt, 0, 1);
  r1[1] = rq.at(Tt, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {
    st.sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[kd & 1], st.kv[kd], (DS || kd) ? st.sc[0] : f32x16{}, 0, 0, 0);
    st.sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[kd & 1], st.kv[kd], (DS || kd) ? st.sc[1] : f32x16{}, 0, 0, 0);
    if (kd + 2 < NKD) {
      r0[kd & 1] = rq.at(Tt, 0, kd + 2);
      r1[kd & 1] = rq.at(Tt, 1, kd + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Element mask of block qb: S = -inf where the lane's key is not visible.
template <int D>
__device__ inline void kv_mask(const KvState<D>& st, f32x16& s, uint32_t QDt, int32_t qa0, int qb, int32_t Lq,
                               bool docs, int hh) {
  asm volatile("; partial tile" ::: "memory");   // keeps the caller's branch real (no if-conversion)
  int qbase = qb * 32 + hh * 4;
  asm volatile("" : "+v"(qbase));
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = qbase + (r >> 2) * 8 + (r & 3);
    const int32_t qidx = qa0 + qr;
    const bool ok = st.kvalid & (qidx < Lq) & (qidx >= st.qlim) & (!docs | (lds_ld4i(QDt + 4 * qr) == st.kdoc));
    s[r] = ok ? s[r] : -INFINITY;
  }
}

// P wave: P = exp2(S c + nl) of both blocks into st.pb and the exchange area.
template <int D>
__device__ inline void kv_p(KvState<D>& st, uint32_t Nl, float c, int hh, uint32_t Xc) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 n4 = lds_f4(Nl + 4 * (qb * 32 + j * 8 + hh * 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = j * 4 + i;
        st.pb[qb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(st.sc[qb][r], c, n4[i]));
      }
    }
    *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(Xc + qb * 2048u) = st.pb[qb][0];
    *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(Xc + qb * 2048u + 1024u) = st.pb[qb][1];
  }
}

// Gradient products of both blocks of the item in tile At: dV^T += dO^T P
// (P wave, g = st.pb) or dK^T += Q^T dS (dS wave, dS formed here from the
// partner's P at Xp and st.sc; block 1's dS is formed between block 0's MFMAs).
template <int D, bool DS>
__device__ inline void kv_grad(KvState<D>& st, const TrLanes<D>& tq, uint32_t At, uint32_t Xp) {
  constexpr int NDB = D / 32, NM = 2 * NDB, PER = 16 / NM;
  bf16x8 g0[2], g1[2], p1[2];
  if constexpr (DS) {
    bf16x8 p0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      p0[h] = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(Xp + h * 1024u);
      p1[h] = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(Xp + 2048u + h * 1024u);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) g0[r >> 3][r & 7] = (__bf16)((float)p0[r >> 3][r & 7] * st.sc[0][r]);
  } else {
    g0[0] = st.pb[0][0];
    g0[1] = st.pb[0][1];
    g1[0] = st.pb[1][0];
    g1[1] = st.pb[1][1];
  }
  bf16x8 ga[2];
  ga[0] = tq.at(At, 0, 0);
  ga[1] = tq.at(At, 16 * (1 / NDB), 1 % NDB);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 2 * NM; ++m) {
    const int qb = m / NM, mm = m % NM, u = mm / NDB, db = mm % NDB;
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[m & 1], qb ? g1[u] : g0[u], st.acc[db], 0, 0, 0);
    if (m + 2 < 2 * NM) {
      const int n = m + 2, nqb = n / NM, nm = n % NM;
      ga[m & 1] = tq.at(At, 32 * nqb + 16 * (nm / NDB), nm % NDB);
    }
    if constexpr (DS) {
      if (m < NM) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int r = m * PER + e;
          g1[r >> 3][r & 7] = (__bf16)((float)p1[r >> 3][r & 7] * st.sc[1][r]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

constexpr int SNB = 3;   // Q/dO tile buffers (dkdv)

template <int D>
__global__ __launch_bounds__(64 * KNW, 1) void dkdv_bf16_kernel(BwdParams a) {
  // LDS arena: SNB Q tiles, SNB dO tiles, then SNB sets of per-row arrays
  // (-LSE log2 e, -Delta, doc ids), then the P exchange area: [SNB buffers]
  // [4 SIMD pairs][2 blocks][2 halves] x 64 lanes x 16 bytes.  Item k uses
  // set k % SNB of each, so a loop unrolled SNB times addresses them all
  // with constant offsets.
  constexpr uint32_t TB = BQ * D * 2, RW = BQ * 4;
  constexpr uint32_t QB0 = 0, OB0 = SNB * TB, RB0 = 2 * SNB * TB;
  constexpr uint32_t XB0 = RB0 + SNB * 3 * RW;
  constexpr uint32_t XSZ = SNB * 4 * 2 * 2 * 1024;
  static_assert(XB0 % 16 == 0, "exchange alignment");
  __shared__ __attribute__((aligned(16))) char smem[XB0 + XSZ];
  const uint32_t S0 = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & 3;                 // 32-key block of the work-group's 128
  const bool is_ds = (wave >> 2) != 0;     // wave-uniform role
  const int lq = lane & 31, hh = lane >> 5;

  // one key tile of one KV head; dir: the order of its query tiles
  int32_t kvh, kt, dir = -1;
  if (a.pair) {
    if (!dkdv_work(blockIdx.x, a.hkv, a.nkt, kvh, kt, dir)) return;
  } else if (!xcd_work(blockIdx.x, a.hkv, a.nkt, kvh, kt)) {
    return;
  }

  const SpanD qs = a.qs, ks = a.ks;
  const int32_t Lq = span_len(qs), Lk = span_len(ks);
  const bool causal = a.causal != 0;
  const bool docs = qs.doc != nullptr;
  const int G = a.G;
  const TileLoader<D, BQ, KNW> ldq(a.q_stride * 2, wave, lane), ldo((int64_t)a.hq * D * 2, wave, lane);
  const float c = a.scale * LOG2E;
  // lane parts of the row and transposed reads, for the Q tiles (from the arena
  // start) and the dO tiles (from their region's start): each role reads one
  // kind of tile row-wise and the other transposed
  const RowLanes<D> rq(RowReader<D>(lane), S0 + QB0), rqo(RowReader<D>(lane), S0 + OB0);
  const TrLanes<D> tq(TrReader<D>(lane), S0 + QB0), tqo(TrReader<D>(lane), S0 + OB0);
  // this lane's 16-byte slot in the exchange area of pair kb: + buf * 16384 + qb * 2048 (+ 1024 half 1)
  const uint32_t Xl = S0 + XB0 + (uint32_t)kb * 4096u + (uint32_t)lane * 16u;

  const int32_t k0 = kt * BKG, k1 = min(Lk, k0 + BKG);
  const int32_t wk0 = k0 + kb * BKW, wk1 = min(Lk, wk0 + BKW);
  const bool wave_has_keys = wk0 < Lk;

  int32_t qlo = 0, qhi = Lq;
  if (causal) qlo = span_count_lt(qs, span_pos(ks, k0));
  if (docs) {
    qlo = max(qlo, wave_lower_bound(qs.doc, Lq, ks.doc[k0]));
    qhi = min(qhi, wave_lower_bound(qs.doc, Lq, ks.doc[k1 - 1] + 1));
  }
  const int32_t qt0 = qlo / BQ;
  const int32_t qt1 = qhi > qlo ? (qhi + BQ - 1) / BQ : qt0;
  const int nitems = (qt1 - qt0) * G;
  const int32_t qfirst = dir < 0 ? qt1 - 1 : qt0;

  // the next item to issue, as running byte pointers: heads of a query tile
  // in turn, then the next tile in direction dir
  struct Cursor {
    int32_t qt, g;
    const char *q, *o;
    const float *l, *d;
  };
  Cursor nx{qfirst, 0,
            (const char*)(a.q + (int64_t)qfirst * BQ * a.q_stride + (int64_t)kvh * G * D),
            (const char*)(a.dout + ((int64_t)qfirst * BQ * a.hq + (int64_t)kvh * G) * D),
            a.lse + (int64_t)kvh * G * a.lse_ld, a.delta + (int64_t)kvh * G * a.lse_ld};
  const int64_t q_wrap = (int64_t)dir * BQ * a.q_stride * 2 - (int64_t)G * D * 2;
  const int64_t o_wrap = (int64_t)dir * BQ * a.hq * D * 2 - (int64_t)G * D * 2;
  const int64_t l_back = (int64_t)G * a.lse_ld;
  auto advance = [&](Cursor& cu) {
    cu.q += D * 2;
    cu.o += D * 2;
    cu.l += a.lse_ld;
    cu.d += a.lse_ld;
    if (++cu.g == G) {
      cu.g = 0;
      cu.qt += dir;
      cu.q += q_wrap;
      cu.o += o_wrap;
      cu.l -= l_back;
      cu.d -= l_back;
    }
  };
  // item copies into tile buffer and row set tb (0..SNB-1)
  auto issue = [&](const Cursor& cu, int tb) {
    const uint32_t Qd = S0 + QB0 + tb * TB, Od = S0 + OB0 + tb * TB, R = S0 + RB0 + tb * 3 * RW;
    const bool whole = cu.qt * BQ + BQ <= Lq;
    if (whole) {
      ldq.load(Qd, cu.q);
      ldo.load(Od, cu.o);
    } else {
      const int head = kvh * G + cu.g;
      tile_load_lds<D, BQ, KNW>(Qd, a.q + (int64_t)head * D, a.q_stride, cu.qt * BQ, Lq, wave, lane);
      tile_load_lds<D, BQ, KNW>(Od, a.dout + (int64_t)head * D, (int64_t)a.hq * D, cu.qt * BQ, Lq, wave, lane);
    }
    // row arrays: 16 bytes per lane for a whole tile, rows clamped otherwise
    const int32_t row = min(cu.qt * BQ + lane, Lq - 1);
    auto rows = [&](const void* base, uint32_t dst) {
      if (whole) row64_load_lds(base, cu.qt * BQ, dst, lane);
      else row_load_lds(base, row, dst);
    };
    if (wave == 0)
      rows(cu.l, R);
    else if (wave == 1)
      rows(cu.d, R + RW);
    else if (wave == 2 && docs)
      rows(qs.doc, R + 2 * RW);
  };
  auto prepare = [&](int tb) {   // -LSE log2 e and -Delta, in place
    const uint32_t R = S0 + RB0 + tb * 3 * RW;
    if (wave == 0) lds_stf(R + 4 * lane, neg_lse2(lds_ldf(R + 4 * lane)));
    else if (wave == 1) lds_stf(R + RW + 4 * lane, -lds_ldf(R + RW + 4 * lane));
  };

  // this wave's 32 K (P wave) or V (dS wave) rows as B operands (lane =
  // key, 8 consecutive d per k step); rows past Lk clamped (their keys are
  // masked)
  KvState<D> st;
  {
    const int32_t mykey = min(wk0 + lq, Lk - 1);
    const bf16x8* src = (const bf16x8*)((is_ds ? a.v : a.k) + (int64_t)mykey * a.kv_stride + (int64_t)kvh * D +
                                        hh * 8);
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) st.kv[kd] = src[kd * 2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.acc[db] = f32x16{};
    st.qlim = causal ? span_count_lt(qs, span_pos(ks, mykey)) : 0;
    st.kdoc = docs ? ks.doc[mykey] : 0;
    st.kvalid = wk0 + lq < Lk;
  }
  // queries < q_none see none of the wave's keys, queries >= q_all every
  // one (causally); doc ids of its first and last key
  const int32_t wlast = wave_has_keys ? wk1 - 1 : Lk - 1;
  const int32_t q_none = causal ? span_count_lt(qs, span_pos(ks, wave_has_keys ? wk0 : Lk - 1)) : 0;
  const int32_t q_all = causal ? span_count_lt(qs, span_pos(ks, wlast)) : 0;
  const int32_t kd_lo = docs ? ks.doc[wave_has_keys ? wk0 : Lk - 1] : 0;
  const int32_t kd_hi = docs ? ks.doc[wlast] : 0;

  if (nitems > 0) {
    issue(nx, 0);
    advance(nx);
  }
  wait_vm0();
  if (nitems > 0) prepare(0);
  __syncthreads();

  // item starting at row qa0 (rows of set tb): does the wave have any
  // allowed entry in it, and is every entry of both its blocks allowed
  auto classify = [&](int32_t qa0, int tb, bool& live, bool& full) {
    const int32_t wq0 = qa0, wq1 = min(Lq, qa0 + BQ);
    live = wave_has_keys && wq1 - 1 >= q_none;
    full = wq1 - wq0 == BQ && wq0 >= q_all && wk1 - wk0 == BKW;
    if (docs) {
      const uint32_t Xr = S0 + RB0 + tb * 3 * RW + 2 * RW;
      const int32_t qd_lo = lds_ld4i(Xr), qd_hi = lds_ld4i(Xr + 4 * (wq1 - 1 - qa0));
      live = live && kd_hi >= qd_lo && kd_lo <= qd_hi;
      full = full && qd_lo == qd_hi && kd_lo == kd_hi && kd_lo == qd_lo;
    }
    live = __builtin_amdgcn_readfirstlane((int)live) != 0;
    full = __builtin_amdgcn_readfirstlane((int)full) != 0;
  };

  // The two roles run separate copies of the item loop (same barriers,
  // same copies), so that each copy's registers hold only its own carried
  // state: P of the previous item (P wave) or its dP (dS wave).  The loop
  // is unrolled SNB times: interval k uses buffer set k % SNB, a constant
  // in each copy of the body.
  auto run = [&](auto role) {
    constexpr bool DS = decltype(role)::value;
    bool prev_live = false;            // the previous item (its gradient runs this interval)
    int32_t cur_qt = qfirst, cur_g = 0;
    auto body = [&](int k, auto phase) {
      constexpr int tb = decltype(phase)::value, tbp = (tb + SNB - 1) % SNB, tbn = (tb + 1) % SNB;
      if (k + 1 < nitems) {
        issue(nx, tbn);
        advance(nx);
      }
      const uint32_t R = S0 + RB0 + tb * 3 * RW;
      const uint32_t Xprev = Xl + (uint32_t)tbp * 16384u, Xcur = Xl + (uint32_t)tb * 16384u;
      bool live = false, full = true;
      int32_t qa0 = 0;
      if (k < nitems) {
        qa0 = cur_qt * BQ;
        if (++cur_g == G) {
          cur_g = 0;
          cur_qt += dir;
        }
      }
      if constexpr (DS) {
        // dS wave: dS and dK of item k-1 (P from the partner), then dP of item k
        if (prev_live) kv_grad<D, true>(st, tq, tbp * TB, Xprev);
        if (k < nitems) {
          classify(qa0, tb, live, full);
          if (live) kv_scores<D, true>(st, rqo, tb * TB, R + RW, hh);
        }
      } else {
        // P wave: dV of item k-1, then S and P of item k
        if (prev_live) kv_grad<D, false>(st, tqo, tbp * TB, 0);
        if (k < nitems) {
          classify(qa0, tb, live, full);
          if (live) {
            kv_scores<D, false>(st, rq, tb * TB, 0, hh);
            if (!full) {
              kv_mask<D>(st, st.sc[0], R + 2 * RW, qa0, 0, Lq, docs, hh);
              kv_mask<D>(st, st.sc[1], R + 2 * RW, qa0, 1, Lq, docs, hh);
            }
            kv_p<D>(st, R, c, hh, Xcur);
          }
        }
      }
      prev_live = live;
      wait_vm0();
      if (k + 1 < nitems) prepare(tbn);
      __syncthreads();
    };
    for (int k = 0; k <= nitems; k += SNB) {
      static_assert(SNB == 3, "the unrolled body below assumes three buffer sets");
      body(k, std::integral_constant<int, 0>{});
      if (k + 1 > nitems) break;
      body(k + 1, std::integral_constant<int, 1>{});
      if (k + 2 > nitems) break;
      body(k + 2, std::integral_constant<int, 2>{});
    }
  };
  if (is_ds) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});

  if (st.kvalid && wave_has_keys) {
    float* const dst = (is_ds ? a.dk : a.dv) + ((int64_t)(wk0 + lq) * a.hkv + kvh) * D;
    add_rows<D>(dst, st.acc, is_ds ? a.scale : 1.0f, hh, a.store != 0);
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
  // Partner key tiles pay off when a key tile's work falls linearly with its
  // index: a causal pair of spans whose key positions reach into the query
  // positions.  With document masks, or with every key before every query
  // (all key tiles equally heavy), the heavy-first order shares the copied
  // tiles as well and measured faster.
  const SpanD& qs = a.qs;
  const SpanD& ks = a.ks;
  a.pair = a.causal && qs.doc == nullptr && span_pos(ks, span_len(ks) - 1) >= span_pos(qs, 0);
  const int32_t grid = a.pair ? dkdv_grid(a.hkv, a.nkt) : xcd_grid(a.hkv, a.nkt);
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
