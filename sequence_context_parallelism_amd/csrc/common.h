// Device-side helpers shared by the attention kernels of libcpattn: chunk
// position runs, the tile classification that drives tile skipping, wave-wide
// searches over document ids, and the XCD-aware work-group remap.
//
// A chunk of tokens ("span") is up to two runs of global positions: local
// token t < l0 sits at p0 + t, local token t >= l0 at p1 + (t - l0), with
// p1 >= p0 + l0, so positions increase along local order (a zigzag shard is
// exactly two such runs).  Document ids, when present, are per local token and
// non-decreasing along local order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cp {

struct SpanD {
  int64_t p0, p1;
  int32_t l0, l1;
  const int32_t* doc;
};

enum : int { TILE_SKIP = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };

__host__ __device__ inline int32_t span_len(const SpanD& s) { return s.l0 + s.l1; }

__host__ __device__ inline int64_t span_pos(const SpanD& s, int32_t t) {
  return t < s.l0 ? s.p0 + t : s.p1 + (int64_t)(t - s.l0);
}

// Number of local tokens whose position is <= x.
__host__ __device__ inline int32_t span_count_le(const SpanD& s, int64_t x) {
  int64_t n0 = x - s.p0 + 1, n1 = x - s.p1 + 1;
  n0 = n0 < 0 ? 0 : (n0 > s.l0 ? s.l0 : n0);
  n1 = n1 < 0 ? 0 : (n1 > s.l1 ? s.l1 : n1);
  return n1 > 0 ? s.l0 + (int32_t)n1 : (int32_t)n0;
}

// Number of local tokens whose position is < x.
__host__ __device__ inline int32_t span_count_lt(const SpanD& s, int64_t x) {
  return span_count_le(s, x - 1);
}

// Class of a block whose queries and keys each lie inside one run (contiguous
// positions).  For contiguous runs with monotone doc ids this is exact: SKIP
// iff no entry is allowed, FULL iff every entry is allowed.
__device__ inline int run_block_class(int64_t qlo, int64_t qhi, int64_t klo, int64_t khi,
                                      int32_t dq0, int32_t dq1, int32_t dk0, int32_t dk1,
                                      bool causal, bool docs) {
  if (causal && klo > qhi) return TILE_SKIP;
  if (docs && (dk1 < dq0 || dk0 > dq1)) return TILE_SKIP;
  bool full = (!causal || khi <= qlo) && (!docs || (dq0 == dq1 && dk0 == dk1 && dq0 == dk0));
  return full ? TILE_FULL : TILE_PARTIAL;
}

// Class of the block of local queries [a0, a1) x local keys [b0, b1) (both
// non-empty, inside their spans).  Each range is split at its run boundary and
// the up-to-four run blocks are combined, which keeps the result exact.
__device__ inline int block_class(const SpanD& qs, int32_t a0, int32_t a1, const SpanD& ks,
                                  int32_t b0, int32_t b1, bool causal) {
  const bool docs = qs.doc != nullptr;
  int32_t qa[2][2], kb[2][2];
  int nq = 0, nk = 0;
  if (a0 < qs.l0) { qa[nq][0] = a0; qa[nq][1] = a1 < qs.l0 ? a1 : qs.l0; ++nq; }
  if (a1 > qs.l0) { qa[nq][0] = a0 > qs.l0 ? a0 : qs.l0; qa[nq][1] = a1; ++nq; }
  if (b0 < ks.l0) { kb[nk][0] = b0; kb[nk][1] = b1 < ks.l0 ? b1 : ks.l0; ++nk; }
  if (b1 > ks.l0) { kb[nk][0] = b0 > ks.l0 ? b0 : ks.l0; kb[nk][1] = b1; ++nk; }
  bool any_live = false, all_full = true;
  for (int x = 0; x < nq; ++x) {
    int32_t i0 = qa[x][0], i1 = qa[x][1] - 1;
    int64_t qlo = span_pos(qs, i0), qhi = span_pos(qs, i1);
    int32_t dq0 = docs ? qs.doc[i0] : 0, dq1 = docs ? qs.doc[i1] : 0;
    for (int y = 0; y < nk; ++y) {
      int32_t j0 = kb[y][0], j1 = kb[y][1] - 1;
      int64_t klo = span_pos(ks, j0), khi = span_pos(ks, j1);
      int32_t dk0 = docs ? ks.doc[j0] : 0, dk1 = docs ? ks.doc[j1] : 0;
      int c = run_block_class(qlo, qhi, klo, khi, dq0, dq1, dk0, dk1, causal, docs);
      any_live |= (c != TILE_SKIP);
      all_full &= (c == TILE_FULL);
    }
  }
  return !any_live ? TILE_SKIP : (all_full ? TILE_FULL : TILE_PARTIAL);
}

// First index i in [0, n) with doc[i] >= x (n if none), for a non-decreasing
// doc array.  Must be called by a whole wave with wave-uniform arguments; each
// round narrows the interval 64-fold with one load per lane.
__device__ inline int32_t wave_lower_bound(const int32_t* doc, int32_t n, int32_t x) {
  const int lane = threadIdx.x & 63;
  int32_t lo = 0, hi = n;   // answer in [lo, hi]
  while (hi - lo >= 64) {
    int32_t step = (hi - lo + 63) / 64;
    int32_t idx = lo + lane * step;
    bool ge = idx >= hi ? true : (doc[idx] >= x);
    uint64_t m = __ballot(ge);
    if (m == 0) {            // every probe < x: answer after the last probe
      lo = lo + 63 * step + 1;
    } else {
      int f = __ffsll((unsigned long long)m) - 1;   // first probe >= x
      int32_t nhi = lo + f * step;
      nhi = nhi < hi ? nhi : hi;
      if (f > 0) lo = lo + (f - 1) * step + 1;
      hi = nhi;
    }
  }
  int32_t idx = lo + lane;
  bool ge = idx >= hi ? true : (doc[idx] >= x);
  uint64_t m = __ballot(ge);
  int f = __ffsll((unsigned long long)m) - 1;
  int32_t r = lo + f;
  return r < hi ? r : hi;
}

// XCD-aware, load-balanced work order.  Work-groups are dispatched in
// blockIdx order, round-robin over the 8 XCDs (blockIdx b runs on XCD b % 8).
// A kernel's work is `ngroups` independent groups (the items of a group share
// one KV head, hence that XCD's L2) of `nidx` items each, item 0 the heaviest.
// The map gives every XCD the same mix of heavy and light items and keeps a
// group's items on as few XCDs as possible:
//   * 8 % ngroups == 0: group = xcd % ngroups, and the 8/ngroups XCDs of a
//     group take its items round-robin, heaviest first;
//   * ngroups % 8 == 0: XCD x takes groups x, x+8, ..., heaviest items first;
//   * otherwise: items in heaviest-first order, groups interleaved.
// Returns false for a padding block (no item).
__device__ inline bool xcd_work(int32_t b, int32_t ngroups, int32_t nidx, int32_t& group, int32_t& idx) {
  const int32_t xcd = b & 7, slot = b >> 3;
  if ((8 % ngroups) == 0) {
    const int32_t per = 8 / ngroups;
    group = xcd % ngroups;
    idx = slot * per + xcd / ngroups;
    return idx < nidx;
  }
  if ((ngroups % 8) == 0) {
    const int32_t m = ngroups / 8;
    group = xcd + 8 * (slot % m);
    idx = slot / m;
    return idx < nidx;
  }
  group = b % ngroups;
  idx = b / ngroups;
  return idx < nidx;
}

__host__ inline int32_t xcd_grid(int32_t ngroups, int32_t nidx) {
  int64_t n;
  if ((8 % ngroups) == 0) n = 8 * (((int64_t)nidx + 8 / ngroups - 1) / (8 / ngroups));
  else if ((ngroups % 8) == 0) n = (int64_t)ngroups * nidx;
  else n = (((int64_t)ngroups * nidx + 7) / 8) * 8;
  return (int32_t)n;
}

__host__ inline int32_t round_up8(int32_t n) { return (n + 7) & ~7; }

// Work order of a KV-outer kernel whose items are the `nkt` key tiles of
// `ngroups` KV heads, each running over the query tiles that see it (causal:
// key tile kt sees nkt - kt of them, in units of its width).  Key tiles kt
// and nkt-1-kt are partners: one XCD runs the first members of DKDV_COHORT
// pairs at once, walking their query tiles last to first (dir = -1), and
// then the second members in the reverse order of the first members'
// finishing, walking first to last (dir = +1).  On a causal share a pair's
// two parts together take the same time for every pair, and at any moment
// the cohort's work-groups stand on one of two query tiles, so the tiles
// they copy are shared through the XCD's L2.  Group placement follows
// xcd_work.  Returns false for a padding block.
constexpr int32_t DKDV_COHORT = 32;   // work-groups one XCD holds at once (one per CU)

__host__ __device__ inline int32_t dkdv_pair_slots(int32_t npairs) {
  return 2 * DKDV_COHORT * ((npairs + DKDV_COHORT - 1) / DKDV_COHORT);
}

__host__ __device__ inline bool dkdv_work(int32_t b, int32_t ngroups, int32_t nkt, int32_t& group, int32_t& kt, int32_t& dir) {
  const int32_t xcd = b & 7, slot = b >> 3;
  const int32_t np = (nkt + 1) / 2;
  int32_t first, stride, lslot;   // this XCD's pairs of `group`: first, first + stride, ...
  if ((8 % ngroups) == 0) {
    const int32_t per = 8 / ngroups;
    group = xcd % ngroups;
    first = xcd / ngroups;
    stride = per;
    lslot = slot;
  } else if ((ngroups % 8) == 0) {
    const int32_t spg = dkdv_pair_slots(np);
    group = xcd + 8 * (slot / spg);
    first = 0;
    stride = 1;
    lslot = slot % spg;
  } else {   // no pairing: key tiles in order, groups interleaved
    group = b % ngroups;
    kt = b / ngroups;
    dir = -1;
    return kt < nkt;
  }
  const int32_t round = lslot / DKDV_COHORT, u = lslot % DKDV_COHORT;
  const bool second = (round & 1) != 0;
  const int32_t i = (round >> 1) * DKDV_COHORT + (second ? DKDV_COHORT - 1 - u : u);
  const int32_t p = first + stride * i;
  if (p >= np) return false;
  kt = second ? nkt - 1 - p : p;
  dir = second ? 1 : -1;
  return !(second && kt == p);   // an odd count's middle tile has no partner
}

__host__ inline int32_t dkdv_grid(int32_t ngroups, int32_t nkt) {
  const int32_t np = (nkt + 1) / 2;
  int64_t n;
  if ((8 % ngroups) == 0) n = 8 * (int64_t)dkdv_pair_slots((np + 8 / ngroups - 1) / (8 / ngroups));
  else if ((ngroups % 8) == 0) n = (int64_t)ngroups * dkdv_pair_slots(np);
  else n = (((int64_t)ngroups * nkt + 7) / 8) * 8;
  return (int32_t)n;
}

}  // namespace cp
