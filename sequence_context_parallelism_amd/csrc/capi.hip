// Host side of libcpattn: argument validation, the C-ABI entry points declared
// in include/cpattn.h, and the ring / Ulysses drivers that sequence the
// kernels on the caller's stream.  No allocation happens here: every buffer,
// including scratch, belongs to the caller.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "cpattn.h"
#include "kernels.h"

using namespace cp;

namespace {

thread_local std::string g_last_error;

cp_status fail(cp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cp_status ok() {
  g_last_error.clear();
  return CP_OK;
}

cp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elt_size(cp_dtype t) { return t == CP_F32 ? 4 : 2; }

bool valid_dtype(cp_dtype t) { return t == CP_BF16 || t == CP_F32; }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Per-row arrays (LSE, Delta, doc ids) are read through 32-bit byte offsets
// (4 bytes per token) and token tiles through 32-bit offsets from the tile's
// first token (128 tokens at most); both stay below 2^31.
constexpr int32_t kMaxTokens = 1 << 29;
constexpr int64_t kMaxStrideBytes = int64_t(1) << 24;

cp_status check_shape(const cp_shape* sh) {
  if (!sh) return fail(CP_ERR_ARG, "shape is NULL");
  if (sh->hq <= 0 || sh->hkv <= 0) return fail(CP_ERR_ARG, "hq=%d and hkv=%d must be positive", sh->hq, sh->hkv);
  if (sh->hq % sh->hkv != 0) return fail(CP_ERR_ARG, "hq=%d is not a multiple of hkv=%d", sh->hq, sh->hkv);
  const int g = sh->hq / sh->hkv;
  if ((g & (g - 1)) != 0 || g > 64)
    return fail(CP_ERR_UNSUPPORTED, "group size hq/hkv=%d must be a power of two <= 64", g);
  if (sh->d != 64 && sh->d != 128) return fail(CP_ERR_UNSUPPORTED, "head dim d=%d not in {64, 128}", sh->d);
  if (!valid_dtype(sh->dtype)) return fail(CP_ERR_ARG, "unknown dtype %d", (int)sh->dtype);
  if (!(sh->scale > 0.f) || sh->scale != sh->scale) return fail(CP_ERR_ARG, "scale must be positive and finite");
  if (sh->causal != 0 && sh->causal != 1) return fail(CP_ERR_ARG, "causal must be 0 or 1");
  if (sh->flags & ~CP_CHECK_DOCS) return fail(CP_ERR_ARG, "unknown flag bits 0x%x", (unsigned)sh->flags);
  const size_t esz = elt_size(sh->dtype);
  if (sh->q_stride < (int64_t)sh->hq * sh->d) return fail(CP_ERR_ARG, "q_stride %lld < hq*d", (long long)sh->q_stride);
  if (sh->kv_stride < (int64_t)sh->hkv * sh->d) return fail(CP_ERR_ARG, "kv_stride %lld < hkv*d", (long long)sh->kv_stride);
  if ((sh->q_stride * esz) % 16 || (sh->kv_stride * esz) % 16)
    return fail(CP_ERR_ALIGN, "token strides must be multiples of 16 bytes");
  // tiles of up to 128 tokens are copied through 32-bit byte offsets from the
  // tile's first token, bounded by 2^31 - 1
  if (sh->q_stride * (int64_t)esz > kMaxStrideBytes || sh->kv_stride * (int64_t)esz > kMaxStrideBytes)
    return fail(CP_ERR_UNSUPPORTED, "token strides above %lld bytes are not supported", (long long)kMaxStrideBytes);
  return CP_OK;
}

cp_status check_span(const cp_span& s, const char* name) {
  if (s.len[0] < 0 || s.len[1] < 0) return fail(CP_ERR_ARG, "%s: negative length", name);
  if ((int64_t)s.len[0] + s.len[1] > kMaxTokens)
    return fail(CP_ERR_UNSUPPORTED, "%s: more than %d tokens", name, kMaxTokens);
  if (s.len[1] > 0 && s.pos[1] < s.pos[0] + s.len[0])
    return fail(CP_ERR_ARG, "%s: second run must start at or after the end of the first", name);
  return CP_OK;
}

SpanD to_dev(const cp_span& s) { return SpanD{s.pos[0], s.pos[1], s.len[0], s.len[1], s.doc}; }

int32_t span_total(const cp_span& s) { return s.len[0] + s.len[1]; }

cp_span run_span(int64_t p0, int32_t l0, int64_t p1, int32_t l1, const int32_t* doc) {
  cp_span s;
  s.pos[0] = p0; s.pos[1] = p1; s.len[0] = l0; s.len[1] = l1; s.doc = doc;
  return s;
}

// ---- unchecked launchers shared by the entry points and the drivers ----
// merge: (o fp32, lse) already hold a running result and this chunk's is
// merged into it in the kernel's epilogue (bf16 inputs only).
hipError_t run_fwd(const cp_shape* sh, const void* q, const cp_span& qs, const void* k, const void* v,
                   const cp_span& ks, void* o, cp_dtype o_dtype, float* lse, int64_t lse_ld,
                   hipStream_t st, bool merge = false) {
  FwdParams p{};
  p.q = (const __bf16*)q; p.k = (const __bf16*)k; p.v = (const __bf16*)v;
  p.qf = (const float*)q; p.kf = (const float*)k; p.vf = (const float*)v;
  p.q_stride = sh->q_stride; p.kv_stride = sh->kv_stride;
  p.qs = to_dev(qs); p.ks = to_dev(ks);
  p.hq = sh->hq; p.hkv = sh->hkv; p.G = sh->hq / sh->hkv; p.d = sh->d;
  p.scale = sh->scale; p.causal = sh->causal;
  p.o = o; p.o_f32 = o_dtype == CP_F32; p.lse = lse; p.lse_ld = lse_ld;
  p.merge = merge ? 1 : 0;
  return sh->dtype == CP_F32 ? launch_fwd_f32(p, st) : launch_fwd_bf16(p, st);
}

enum BwdPart { BWD_ALL, BWD_DKDV, BWD_DQ };

// With `store` the gradients are written instead of added to: for a call
// whose pairs are all the pairs of these rows.  The bf16 kernels store
// directly (no zero-fill, no read of the old values); for fp32 the outputs
// are zero-filled and the kernels accumulate.
hipError_t run_bwd(const cp_shape* sh, const void* q, const cp_span& qs, const void* k, const void* v,
                   const cp_span& ks, const void* dout, const float* lse, const float* delta,
                   int64_t lse_ld, float* dq, float* dk, float* dv, hipStream_t st, BwdPart part = BWD_ALL,
                   bool store = false) {
  const int64_t Lq = (int64_t)qs.len[0] + qs.len[1], Lk = (int64_t)ks.len[0] + ks.len[1];
  if (store && sh->dtype == CP_F32) {    // the fp32 kernels only accumulate: zero the outputs first
    hipError_t e = hipSuccess;
    if (part != BWD_DKDV) e = launch_fill_zero(Lq * sh->hq * sh->d, dq, st);
    if (e == hipSuccess && part != BWD_DQ) e = launch_fill_zero(Lk * sh->hkv * sh->d, dk, st);
    if (e == hipSuccess && part != BWD_DQ) e = launch_fill_zero(Lk * sh->hkv * sh->d, dv, st);
    if (e != hipSuccess) return e;
    store = false;
  }
  if (store && (Lq == 0 || Lk == 0)) {   // no pairs: the written gradients are zeros
    hipError_t e = hipSuccess;
    if (Lk == 0 && part != BWD_DKDV) e = launch_fill_zero(Lq * sh->hq * sh->d, dq, st);
    if (e == hipSuccess && Lq == 0 && part != BWD_DQ) e = launch_fill_zero(Lk * sh->hkv * sh->d, dk, st);
    if (e == hipSuccess && Lq == 0 && part != BWD_DQ) e = launch_fill_zero(Lk * sh->hkv * sh->d, dv, st);
    return e;
  }
  BwdParams p{};
  p.q = (const __bf16*)q; p.k = (const __bf16*)k; p.v = (const __bf16*)v; p.dout = (const __bf16*)dout;
  p.qf = (const float*)q; p.kf = (const float*)k; p.vf = (const float*)v; p.doutf = (const float*)dout;
  p.q_stride = sh->q_stride; p.kv_stride = sh->kv_stride;
  p.qs = to_dev(qs); p.ks = to_dev(ks);
  p.hq = sh->hq; p.hkv = sh->hkv; p.G = sh->hq / sh->hkv; p.d = sh->d;
  p.scale = sh->scale; p.causal = sh->causal;
  p.lse = lse; p.delta = delta; p.lse_ld = lse_ld;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.store = store ? 1 : 0;
  const bool f32 = sh->dtype == CP_F32;
  switch (part) {
    case BWD_DKDV: return f32 ? launch_bwd_f32_dkdv(p, st) : launch_bwd_bf16_dkdv(p, st);
    case BWD_DQ: return f32 ? launch_bwd_f32_dq(p, st) : launch_bwd_bf16_dq(p, st);
    default: return f32 ? launch_bwd_f32(p, st) : launch_bwd_bf16(p, st);
  }
}

#define CP_TRY_HIP(expr, what)                 \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_status(e_, what); \
  } while (0)

#define CP_TRY(expr)                           \
  do {                                         \
    cp_status s_ = (expr);                     \
    if (s_ != CP_OK) return s_;                \
  } while (0)

cp_status check_docs(const cp_span& a, const cp_span& b) {
  if ((a.doc == nullptr) != (b.doc == nullptr))
    return fail(CP_ERR_DOCS, "doc ids must be given for both the query and the key span, or neither");
  return CP_OK;
}

// Document ids must be >= 0 and non-decreasing in the order given (the mask
// compares ids of equal value, and the kernels' tile classification reads a
// tile's id range from its first and last token).
cp_status validate_ids(const int32_t* h, int64_t n, const char* what) {
  for (int64_t i = 0; i < n; ++i) {
    if (h[i] < 0) return fail(CP_ERR_DOCS, "%s: doc id %d at index %lld is negative", what, h[i], (long long)i);
    if (i > 0 && h[i] < h[i - 1])
      return fail(CP_ERR_DOCS, "%s: doc ids decrease at index %lld (%d after %d)", what, (long long)i, h[i],
                  h[i - 1]);
  }
  return CP_OK;
}

// A host copy of n device doc ids, taken on `st` (waits for the stream).
cp_status fetch_ids(const int32_t* dev, int64_t n, hipStream_t st, std::vector<int32_t>& out) {
  out.assign((size_t)n, 0);
  if (n == 0) return CP_OK;
  CP_TRY_HIP(hipMemcpyAsync(out.data(), dev, (size_t)n * 4, hipMemcpyDeviceToHost, st), "doc id copy");
  CP_TRY_HIP(hipStreamSynchronize(st), "doc id copy");
  return CP_OK;
}

bool checking_docs(const cp_shape* sh) { return (sh->flags & CP_CHECK_DOCS) != 0; }

// CP_CHECK_DOCS for a chunk call: each span's ids in local order (which is
// global order: positions increase along a span).
cp_status check_span_ids(const cp_shape* sh, const cp_span& s, const char* name, hipStream_t st) {
  if (!checking_docs(sh) || !s.doc) return CP_OK;
  std::vector<int32_t> h;
  CP_TRY(fetch_ids(s.doc, span_total(s), st, h));
  return validate_ids(h.data(), (int64_t)h.size(), name);
}

// CP_CHECK_DOCS for a whole sequence held in global order.
cp_status check_seq_ids(const cp_shape* sh, const int32_t* doc, int64_t S, hipStream_t st) {
  if (!checking_docs(sh) || !doc) return CP_OK;
  std::vector<int32_t> h;
  CP_TRY(fetch_ids(doc, S, st, h));
  return validate_ids(h.data(), S, "doc");
}

cp_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(CP_ERR_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(CP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return CP_OK;
}

struct RingLayout {
  size_t acc_o, part_o, part_lse, delta, total;
};

RingLayout ring_layout(const cp_shape* sh, int64_t n, cp_dtype o_dtype, bool backward) {
  RingLayout L{};
  const size_t obytes = align256((size_t)n * sh->hq * sh->d * 4);
  const size_t lbytes = align256((size_t)n * sh->hq * 4);
  size_t off = 0;
  L.acc_o = off; if (o_dtype == CP_BF16) off += obytes;
  L.part_o = off; off += obytes;
  L.part_lse = off; off += lbytes;
  L.delta = off; if (backward) off += lbytes;
  L.total = off;
  return L;
}

// The zigzag assignment as a chunk table: rank r holds chunks r and 2P-1-r.
std::vector<int32_t> zigzag_pairs(int32_t P) {
  std::vector<int32_t> t(2 * (size_t)P);
  for (int32_t r = 0; r < P; ++r) {
    t[2 * r] = r;
    t[2 * r + 1] = 2 * P - 1 - r;
  }
  return t;
}

// A two-chunks-per-rank assignment: chunks[2r] < chunks[2r+1], every chunk
// 0..2P-1 exactly once.
cp_status check_pairs(const int32_t* chunks, int32_t P) {
  if (!chunks) return fail(CP_ERR_ARG, "chunks is NULL");
  std::vector<char> seen(2 * (size_t)P, 0);
  for (int32_t r = 0; r < P; ++r) {
    const int32_t a = chunks[2 * r], b = chunks[2 * r + 1];
    if (a < 0 || b >= 2 * P || a >= b)
      return fail(CP_ERR_ARG, "rank %d: chunks (%d, %d) must satisfy 0 <= a < b < 2P=%d", r, a, b, 2 * P);
    if (seen[a] || seen[b]) return fail(CP_ERR_ARG, "rank %d: a chunk is assigned twice", r);
    seen[a] = seen[b] = 1;
  }
  return CP_OK;
}

// CP_CHECK_DOCS for a ring: the ids come in sharded order; put them back in
// global order under the chunk table and check that order.
cp_status check_ring_ids(const cp_shape* sh, const int32_t* doc, int64_t S, int32_t P, const int32_t* pairs,
                         hipStream_t st) {
  if (!checking_docs(sh) || !doc) return CP_OK;
  std::vector<int32_t> h, g((size_t)S);
  CP_TRY(fetch_ids(doc, S, st, h));
  const int64_t c = S / (2 * P), n = 2 * c;
  for (int32_t r = 0; r < P; ++r)
    for (int half = 0; half < 2; ++half)
      std::copy(h.begin() + r * n + half * c, h.begin() + r * n + (half + 1) * c,
                g.begin() + (int64_t)pairs[2 * r + half] * c);
  return validate_ids(g.data(), S, "doc (global order)");
}

cp_status check_ring_args(const cp_shape* sh, int64_t S, int32_t P, int32_t rank) {
  CP_TRY(check_shape(sh));
  if (P < 1) return fail(CP_ERR_ARG, "P=%d must be >= 1", P);
  if (S <= 0 || S % (2 * (int64_t)P) != 0) return fail(CP_ERR_ARG, "S=%lld must be a positive multiple of 2P=%d", (long long)S, 2 * P);
  if (S > kMaxTokens) return fail(CP_ERR_UNSUPPORTED, "S=%lld above %d tokens", (long long)S, kMaxTokens);
  if (rank < -1 || rank >= P) return fail(CP_ERR_ARG, "rank=%d out of [-1, P)", rank);
  return CP_OK;
}

// Emulated ring traffic (one rank): the KV shard each step reads arrives in a
// double-buffered receive area through a copy on a second stream, issued one
// step ahead; in the backward, each step's finished dK/dV shard leaves through
// a copy into a send area.  Events order the copies against the compute.
struct RingOverlap {
  hipStream_t cs;
  char* recv[2];         // compact K rows then V rows of one shard, [n, hkv, d]
  float* send;           // dK rows then dV rows of one shard, fp32 [n, hkv, d]
};

struct OverlapLayout {
  size_t recv0, recv1, send, total;
};

OverlapLayout overlap_layout(const cp_shape* sh, int64_t n, bool backward, size_t base) {
  OverlapLayout L{};
  const size_t kv = align256((size_t)2 * n * sh->hkv * sh->d * elt_size(sh->dtype));
  L.recv0 = base;
  L.recv1 = L.recv0 + kv;
  L.send = L.recv1 + kv;
  L.total = L.send + (backward ? align256((size_t)2 * n * sh->hkv * sh->d * 4) : 0);
  return L;
}

// Events of one call (timing off), released when the call returns; a pending
// event is freed by the runtime once it completes.
struct EventSet {
  std::vector<hipEvent_t> e;
  ~EventSet() {
    for (hipEvent_t x : e) (void)hipEventDestroy(x);
  }
  hipError_t make(size_t count) {
    e.assign(count, nullptr);
    for (size_t i = 0; i < count; ++i) {
      hipError_t r = hipEventCreateWithFlags(&e[i], hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

// Argument checks shared by the ring entry points.
cp_status ring_args(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const void* q, const void* k,
                    const void* v, void* o, cp_dtype o_dtype, float* lse, const void* dout, float* dq, float* dk,
                    float* dv) {
  CP_TRY(check_ring_args(sh, S, P, rank));
  if (!valid_dtype(o_dtype)) return fail(CP_ERR_ARG, "unknown o_dtype");
  CP_TRY(check_ptr(q, "q"));
  CP_TRY(check_ptr(k, "k"));
  CP_TRY(check_ptr(v, "v"));
  CP_TRY(check_ptr(o, "o"));
  if (!lse) return fail(CP_ERR_ARG, "lse is NULL");
  if (dout != nullptr) {
    CP_TRY(check_ptr(dout, "dout"));
    CP_TRY(check_ptr(dq, "dq"));
    CP_TRY(check_ptr(dk, "dk"));
    CP_TRY(check_ptr(dv, "dv"));
  }
  return CP_OK;
}

cp_status check_workspace(const void* workspace, size_t ws_bytes, size_t need) {
  if (need == 0) return CP_OK;
  if (!workspace) return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes required", need);
  if (ws_bytes < need) return fail(CP_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(CP_ERR_ALIGN, "workspace must be 256-byte aligned");
  return CP_OK;
}

}  // namespace

extern "C" {

int32_t cp_abi_version(void) { return CP_ABI_VERSION; }

const char* cp_last_error(void) { return g_last_error.c_str(); }

cp_status cp_attn_chunk_fwd(const cp_shape* sh, const void* q, cp_span qs, const void* k, const void* v,
                            cp_span ks, void* o, cp_dtype o_dtype, float* lse, void* stream) {
  CP_TRY(check_shape(sh));
  CP_TRY(check_span(qs, "qs"));
  CP_TRY(check_span(ks, "ks"));
  CP_TRY(check_docs(qs, ks));
  if (!valid_dtype(o_dtype)) return fail(CP_ERR_ARG, "unknown o_dtype");
  const int32_t Lq = span_total(qs), Lk = span_total(ks);
  if (Lq == 0) return ok();
  CP_TRY(check_ptr(q, "q"));
  CP_TRY(check_ptr(o, "o"));
  CP_TRY(check_ptr(lse, "lse"));
  if (Lk > 0) { CP_TRY(check_ptr(k, "k")); CP_TRY(check_ptr(v, "v")); }
  CP_TRY(check_span_ids(sh, qs, "qs.doc", (hipStream_t)stream));
  CP_TRY(check_span_ids(sh, ks, "ks.doc", (hipStream_t)stream));
  CP_TRY_HIP(run_fwd(sh, q, qs, k, v, ks, o, o_dtype, lse, Lq, (hipStream_t)stream), "cp_attn_chunk_fwd");
  return ok();
}

cp_status cp_lse_merge(int64_t rows, int32_t h, int32_t d, float* o_acc, float* lse_acc, const float* o_part,
                       const float* lse_part, void* stream) {
  if (rows < 0 || h <= 0) return fail(CP_ERR_ARG, "rows=%lld, h=%d", (long long)rows, h);
  if (d != 64 && d != 128) return fail(CP_ERR_UNSUPPORTED, "d=%d not in {64, 128}", d);
  if (rows == 0) return ok();
  CP_TRY(check_ptr(o_acc, "o_acc"));
  CP_TRY(check_ptr(o_part, "o_part"));
  if (!lse_acc || !lse_part) return fail(CP_ERR_ARG, "lse pointer is NULL");
  CP_TRY_HIP(launch_lse_merge(rows, h, d, o_acc, lse_acc, rows, o_part, lse_part, rows, (hipStream_t)stream),
             "cp_lse_merge");
  return ok();
}

cp_status cp_attn_delta(int64_t rows, int32_t h, int32_t d, const void* o, cp_dtype o_dtype, const void* dout,
                        cp_dtype dout_dtype, float* delta, void* stream) {
  if (rows < 0 || h <= 0) return fail(CP_ERR_ARG, "rows=%lld, h=%d", (long long)rows, h);
  if (d != 64 && d != 128) return fail(CP_ERR_UNSUPPORTED, "d=%d not in {64, 128}", d);
  if (!valid_dtype(o_dtype) || !valid_dtype(dout_dtype)) return fail(CP_ERR_ARG, "unknown dtype");
  if (rows == 0) return ok();
  CP_TRY(check_ptr(o, "o"));
  CP_TRY(check_ptr(dout, "dout"));
  if (!delta) return fail(CP_ERR_ARG, "delta is NULL");
  CP_TRY_HIP(launch_delta(rows, h, d, o, o_dtype == CP_F32, dout, dout_dtype == CP_F32, delta, rows,
                          (hipStream_t)stream), "cp_attn_delta");
  return ok();
}

static cp_status chunk_bwd(const cp_shape* sh, const void* q, cp_span qs, const void* k, const void* v,
                           cp_span ks, const void* dout, const float* lse, const float* delta, float* dq,
                           float* dk, float* dv, void* stream, BwdPart part, const char* name) {
  CP_TRY(check_shape(sh));
  CP_TRY(check_span(qs, "qs"));
  CP_TRY(check_span(ks, "ks"));
  CP_TRY(check_docs(qs, ks));
  const int32_t Lq = span_total(qs), Lk = span_total(ks);
  if (Lq == 0 || Lk == 0) return ok();
  CP_TRY(check_ptr(q, "q"));
  CP_TRY(check_ptr(k, "k"));
  CP_TRY(check_ptr(v, "v"));
  CP_TRY(check_ptr(dout, "dout"));
  if (part != BWD_DKDV) CP_TRY(check_ptr(dq, "dq"));
  if (part != BWD_DQ) {
    CP_TRY(check_ptr(dk, "dk"));
    CP_TRY(check_ptr(dv, "dv"));
  }
  if (!lse || !delta) return fail(CP_ERR_ARG, "lse or delta is NULL");
  CP_TRY(check_span_ids(sh, qs, "qs.doc", (hipStream_t)stream));
  CP_TRY(check_span_ids(sh, ks, "ks.doc", (hipStream_t)stream));
  CP_TRY_HIP(run_bwd(sh, q, qs, k, v, ks, dout, lse, delta, Lq, dq, dk, dv, (hipStream_t)stream, part), name);
  return ok();
}

cp_status cp_attn_chunk_bwd(const cp_shape* sh, const void* q, cp_span qs, const void* k, const void* v,
                            cp_span ks, const void* dout, const float* lse, const float* delta, float* dq,
                            float* dk, float* dv, void* stream) {
  return chunk_bwd(sh, q, qs, k, v, ks, dout, lse, delta, dq, dk, dv, stream, BWD_ALL, "cp_attn_chunk_bwd");
}

cp_status cp_attn_chunk_bwd_dkdv(const cp_shape* sh, const void* q, cp_span qs, const void* k, const void* v,
                                 cp_span ks, const void* dout, const float* lse, const float* delta, float* dk,
                                 float* dv, void* stream) {
  return chunk_bwd(sh, q, qs, k, v, ks, dout, lse, delta, nullptr, dk, dv, stream, BWD_DKDV,
                   "cp_attn_chunk_bwd_dkdv");
}

cp_status cp_attn_chunk_bwd_dq(const cp_shape* sh, const void* q, cp_span qs, const void* k, const void* v,
                               cp_span ks, const void* dout, const float* lse, const float* delta, float* dq,
                               void* stream) {
  return chunk_bwd(sh, q, qs, k, v, ks, dout, lse, delta, dq, nullptr, nullptr, stream, BWD_DQ,
                   "cp_attn_chunk_bwd_dq");
}

cp_status cp_zigzag_layout(int64_t S, int32_t P, int32_t rank, int64_t pos0[2], int32_t len[2]) {
  if (!pos0 || !len) return fail(CP_ERR_ARG, "output pointer is NULL");
  if (P < 1 || S <= 0 || S % (2 * (int64_t)P) != 0 || rank < 0 || rank >= P)
    return fail(CP_ERR_ARG, "need P >= 1, S > 0 divisible by 2P and 0 <= rank < P (S=%lld P=%d rank=%d)",
                (long long)S, P, rank);
  const int64_t c = S / (2 * P);
  if (c > INT32_MAX) return fail(CP_ERR_ARG, "chunk too long");
  pos0[0] = rank * c;
  pos0[1] = (2 * (int64_t)P - 1 - rank) * c;
  len[0] = (int32_t)c;
  len[1] = (int32_t)c;
  return ok();
}

cp_status cp_ring_schedule(int64_t S, int32_t P, int32_t rank, int32_t step, int32_t* src_rank, int8_t kind[4]) {
  if (!src_rank || !kind) return fail(CP_ERR_ARG, "output pointer is NULL");
  int64_t pos0[2];
  int32_t len[2];
  CP_TRY(cp_zigzag_layout(S, P, rank, pos0, len));
  if (step < 0 || step >= P) return fail(CP_ERR_ARG, "step=%d out of [0, P)", step);
  const int32_t src = ((rank - step) % P + P) % P;
  const int32_t qc[2] = {rank, 2 * P - 1 - rank};
  const int32_t kc[2] = {src, 2 * P - 1 - src};
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) kind[a * 2 + b] = kc[b] > qc[a] ? 0 : (kc[b] == qc[a] ? 1 : 2);
  *src_rank = src;
  return ok();
}

size_t cp_ring_workspace_bytes(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, cp_dtype o_dtype,
                               int32_t backward) {
  if (check_ring_args(sh, S, P, rank) != CP_OK || !valid_dtype(o_dtype)) return 0;
  return ring_layout(sh, S / P, o_dtype, backward != 0).total;
}

}  // extern "C"

namespace {

// The ring driver.  Rank r holds chunks pairs[2r] < pairs[2r+1] (each of
// S/(2P) tokens; the zigzag table, or a document-balanced one), so every
// shard is a two-run span.  With `ov` (a single rank, no per-step capture)
// the steps read their KV shard from the receive area (see RingOverlap).
cp_status ring_drive(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const int32_t* pairs, const void* q,
                     const void* k, const void* v, const int32_t* doc, void* o, cp_dtype o_dtype, float* lse,
                     const void* dout, float* dq, float* dk, float* dv, float* step_o, float* step_lse, char* ws,
                     hipStream_t st, const RingOverlap* ov) {
  const bool backward = dout != nullptr;
  const int64_t n = S / P;                       // rows per rank = 2c
  const int32_t c = (int32_t)(S / (2 * P));
  const RingLayout lay = ring_layout(sh, n, o_dtype, backward);
  float* acc_o_ws = (float*)(ws + lay.acc_o);
  float* part_o = (float*)(ws + lay.part_o);
  float* part_lse = (float*)(ws + lay.part_lse);
  float* dlt = (float*)(ws + lay.delta);

  const size_t in_esz = elt_size(sh->dtype), o_esz = elt_size(o_dtype);
  const int64_t orow = (int64_t)sh->hq * sh->d;          // elements per output row
  const int64_t kvrow = (int64_t)sh->hkv * sh->d;

  if (backward) {
    const int64_t dq_rows = rank < 0 ? S : n;
    CP_TRY_HIP(launch_fill_zero(dq_rows * orow, dq, st), "zero dq");
    CP_TRY_HIP(launch_fill_zero(S * kvrow, dk, st), "zero dk");
    CP_TRY_HIP(launch_fill_zero(S * kvrow, dv, st), "zero dv");
  }

  // emulated traffic: events [0] start, [1] forward end, [2] end; then per
  // pass (forward, backward) P "shard received" and P "step computed" events;
  // then P "step's dK/dV computed" events of the backward
  EventSet ev;
  cp_shape shc = *sh;                                     // receive rows are compact
  shc.kv_stride = kvrow;
  const size_t shard_b = (size_t)n * kvrow * in_esz;     // K (or V) rows of one shard
  if (ov) {
    CP_TRY_HIP(ev.make(3 + 5 * (size_t)P), "ring events");
    CP_TRY_HIP(hipEventRecord(ev.e[0], st), "ring event");
    CP_TRY_HIP(hipStreamWaitEvent(ov->cs, ev.e[0], 0), "ring wait");   // earlier readers of the areas
  }
  auto ev_ready = [&](int pass, int32_t s) { return ev.e[3 + (size_t)pass * 2 * P + s]; };
  auto ev_done = [&](int pass, int32_t s) { return ev.e[3 + (size_t)pass * 2 * P + P + s]; };
  auto ev_dkdv = [&](int32_t s) { return ev.e[3 + 4 * (size_t)P + s]; };
  // Before step s computes: the shard of step s + 1 into recv[(s + 1) & 1],
  // once step s - 1 (its last reader) is done.
  auto prefetch = [&](int pass, int32_t r, int32_t s) -> hipError_t {
    if (!ov || s + 1 >= P) return hipSuccess;
    hipError_t e = hipSuccess;
    if (s >= 2) e = hipStreamWaitEvent(ov->cs, ev_done(pass, s - 1), 0);
    const int32_t j = ((r - (s + 1)) % P + P) % P;
    char* dst = ov->recv[(s + 1) & 1];
    const size_t pitch = (size_t)sh->kv_stride * in_esz, width = (size_t)kvrow * in_esz;
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(dst, width, (const char*)k + (size_t)j * n * pitch, pitch, width, n,
                           hipMemcpyDeviceToDevice, ov->cs);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(dst + shard_b, width, (const char*)v + (size_t)j * n * pitch, pitch, width, n,
                           hipMemcpyDeviceToDevice, ov->cs);
    if (e == hipSuccess) e = hipEventRecord(ev_ready(pass, s + 1), ov->cs);
    return e;
  };
  // The KV operands of step s: in place for s = 0 (the rank's own shard) or
  // without emulation, else the receive area once its copy has landed.
  auto step_kv = [&](int pass, int32_t s, int32_t j, const char*& kj, const char*& vj,
                     const cp_shape*& shs) -> hipError_t {
    shs = sh;
    kj = (const char*)k + (size_t)j * n * sh->kv_stride * in_esz;
    vj = (const char*)v + (size_t)j * n * sh->kv_stride * in_esz;
    if (!ov || s == 0) return hipSuccess;
    shs = &shc;
    kj = ov->recv[s & 1];
    vj = ov->recv[s & 1] + shard_b;
    return hipStreamWaitEvent(st, ev_ready(pass, s), 0);
  };

  const int32_t r0 = rank < 0 ? 0 : rank, r1 = rank < 0 ? P : rank + 1;
  for (int32_t r = r0; r < r1; ++r) {
    const int64_t out_row0 = rank < 0 ? (int64_t)r * n : 0;       // row offset into o / dq
    const char* qr = (const char*)q + (size_t)r * n * sh->q_stride * in_esz;
    const cp_span qs = run_span((int64_t)pairs[2 * r] * c, c, (int64_t)pairs[2 * r + 1] * c, c,
                                doc ? doc + r * n : nullptr);
    char* o_r = (char*)o + (size_t)out_row0 * orow * o_esz;
    float* lse_r = lse + (rank < 0 ? (size_t)r * sh->hq * n : 0);
    float* acc_o = o_dtype == CP_F32 ? (float*)o_r : acc_o_ws;

    for (int32_t s = 0; s < P; ++s) {
      const int32_t j = ((r - s) % P + P) % P;
      const char *kj, *vj;
      const cp_shape* shs;
      CP_TRY_HIP(prefetch(0, r, s), "ring receive copy");
      CP_TRY_HIP(step_kv(0, s, j, kj, vj, shs), "ring wait");
      const cp_span ks = run_span((int64_t)pairs[2 * j] * c, c, (int64_t)pairs[2 * j + 1] * c, c,
                                  doc ? doc + j * n : nullptr);
      // bf16 steps after the first merge into the running result in the
      // forward kernel's epilogue (no partial round trip through HBM)
      if (s > 0 && !step_o && sh->dtype == CP_BF16) {
        CP_TRY_HIP(run_fwd(shs, qr, qs, kj, vj, ks, acc_o, CP_F32, lse_r, n, st, true), "ring forward step");
        if (ov) CP_TRY_HIP(hipEventRecord(ev_done(0, s), st), "ring event");
        continue;
      }
      float* so = step_o ? step_o + (size_t)s * n * orow : (s == 0 ? acc_o : part_o);
      float* sl = step_lse ? step_lse + (size_t)s * sh->hq * n : (s == 0 ? lse_r : part_lse);
      CP_TRY_HIP(run_fwd(shs, qr, qs, kj, vj, ks, so, CP_F32, sl, n, st), "ring forward step");
      if (ov) CP_TRY_HIP(hipEventRecord(ev_done(0, s), st), "ring event");
      if (s == 0) {
        if (step_o) {
          CP_TRY_HIP(launch_copy_f32(n * orow, so, acc_o, st), "ring copy");
          CP_TRY_HIP(launch_copy_f32(n * sh->hq, sl, lse_r, st), "ring copy");
        }
      } else {
        CP_TRY_HIP(launch_lse_merge(n, sh->hq, sh->d, acc_o, lse_r, n, so, sl, n, st), "ring merge");
      }
    }
    if (o_dtype == CP_BF16) CP_TRY_HIP(launch_f32_to_bf16(n * orow, acc_o, (__bf16*)o_r, st), "ring convert");
    if (ov) {   // the backward pass refills the receive areas after the forward's last reads
      CP_TRY_HIP(hipEventRecord(ev.e[1], st), "ring event");
      CP_TRY_HIP(hipStreamWaitEvent(ov->cs, ev.e[1], 0), "ring wait");
    }

    if (backward) {
      const char* dout_r = (const char*)dout + (size_t)out_row0 * orow * in_esz;
      float* dq_r = dq + (size_t)out_row0 * orow;
      CP_TRY_HIP(launch_delta(n, sh->hq, sh->d, o_r, o_dtype == CP_F32, dout_r, sh->dtype == CP_F32, dlt, n, st),
                 "ring delta");
      for (int32_t s = 0; s < P; ++s) {
        const int32_t j = ((r - s) % P + P) % P;
        const char *kj, *vj;
        const cp_shape* shs;
        CP_TRY_HIP(prefetch(1, r, s), "ring receive copy");
        CP_TRY_HIP(step_kv(1, s, j, kj, vj, shs), "ring wait");
        const cp_span ks = run_span((int64_t)pairs[2 * j] * c, c, (int64_t)pairs[2 * j + 1] * c, c,
                                    doc ? doc + j * n : nullptr);
        float* dkj = dk + (size_t)j * n * kvrow;
        float* dvj = dv + (size_t)j * n * kvrow;
        if (!ov) {
          CP_TRY_HIP(run_bwd(shs, qr, qs, kj, vj, ks, dout_r, lse_r, dlt, n, dq_r, dkj, dvj, st),
                     "ring backward step");
        } else {   // dK/dV first: the step's dK/dV shard leaves for its owner while dQ runs
          const size_t gb = (size_t)n * kvrow * 4;
          CP_TRY_HIP(run_bwd(shs, qr, qs, kj, vj, ks, dout_r, lse_r, dlt, n, dq_r, dkj, dvj, st, BWD_DKDV),
                     "ring backward step (dK/dV)");
          CP_TRY_HIP(hipEventRecord(ev_dkdv(s), st), "ring event");
          CP_TRY_HIP(hipStreamWaitEvent(ov->cs, ev_dkdv(s), 0), "ring wait");
          CP_TRY_HIP(hipMemcpyAsync(ov->send, dkj, gb, hipMemcpyDeviceToDevice, ov->cs), "ring send copy");
          CP_TRY_HIP(hipMemcpyAsync((char*)ov->send + gb, dvj, gb, hipMemcpyDeviceToDevice, ov->cs), "ring send copy");
          CP_TRY_HIP(run_bwd(shs, qr, qs, kj, vj, ks, dout_r, lse_r, dlt, n, dq_r, dkj, dvj, st, BWD_DQ),
                     "ring backward step (dQ)");
          // the step's last reader of its receive area
          CP_TRY_HIP(hipEventRecord(ev_done(1, s), st), "ring event");
        }
      }
    }
  }
  if (ov) {   // the call's completion on `stream` covers the copies too
    CP_TRY_HIP(hipEventRecord(ev.e[2], ov->cs), "ring event");
    CP_TRY_HIP(hipStreamWaitEvent(st, ev.e[2], 0), "ring wait");
  }
  return ok();
}

}  // namespace

extern "C" {

cp_status cp_ring_emulate(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const void* q, const void* k,
                          const void* v, const int32_t* doc, void* o, cp_dtype o_dtype, float* lse,
                          const void* dout, float* dq, float* dk, float* dv, float* step_o, float* step_lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  CP_TRY(ring_args(sh, S, P, rank, q, k, v, o, o_dtype, lse, dout, dq, dk, dv));
  if ((step_o == nullptr) != (step_lse == nullptr))
    return fail(CP_ERR_ARG, "step_o and step_lse must both be given or both be NULL");
  if (step_o && rank < 0) return fail(CP_ERR_ARG, "per-step capture needs a single rank");
  if (step_o) CP_TRY(check_ptr(step_o, "step_o"));
  CP_TRY(check_workspace(workspace, ws_bytes, ring_layout(sh, S / P, o_dtype, dout != nullptr).total));
  const std::vector<int32_t> pairs = zigzag_pairs(P);
  CP_TRY(check_ring_ids(sh, doc, S, P, pairs.data(), (hipStream_t)stream));
  return ring_drive(sh, S, P, rank, pairs.data(), q, k, v, doc, o, o_dtype, lse, dout, dq, dk, dv, step_o,
                    step_lse, (char*)workspace, (hipStream_t)stream, nullptr);
}

cp_status cp_ring_emulate_layout(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const int32_t* chunks,
                                 const void* q, const void* k, const void* v, const int32_t* doc, void* o,
                                 cp_dtype o_dtype, float* lse, const void* dout, float* dq, float* dk, float* dv,
                                 void* workspace, size_t ws_bytes, void* stream) {
  CP_TRY(ring_args(sh, S, P, rank, q, k, v, o, o_dtype, lse, dout, dq, dk, dv));
  CP_TRY(check_pairs(chunks, P));
  CP_TRY(check_workspace(workspace, ws_bytes, ring_layout(sh, S / P, o_dtype, dout != nullptr).total));
  const std::vector<int32_t> pairs(chunks, chunks + 2 * (size_t)P);     // the host table, copied once
  CP_TRY(check_ring_ids(sh, doc, S, P, pairs.data(), (hipStream_t)stream));
  return ring_drive(sh, S, P, rank, pairs.data(), q, k, v, doc, o, o_dtype, lse, dout, dq, dk, dv, nullptr,
                    nullptr, (char*)workspace, (hipStream_t)stream, nullptr);
}

size_t cp_ring_overlap_workspace_bytes(const cp_shape* sh, int64_t S, int32_t P, cp_dtype o_dtype, int32_t backward) {
  if (check_ring_args(sh, S, P, 0) != CP_OK || !valid_dtype(o_dtype)) return 0;
  const int64_t n = S / P;
  const size_t base = align256(ring_layout(sh, n, o_dtype, backward != 0).total);
  return overlap_layout(sh, n, backward != 0, base).total;
}

cp_status cp_ring_emulate_overlap(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const void* q,
                                  const void* k, const void* v, const int32_t* doc, void* o, cp_dtype o_dtype,
                                  float* lse, const void* dout, float* dq, float* dk, float* dv, void* workspace,
                                  size_t ws_bytes, void* stream, void* copy_stream) {
  CP_TRY(ring_args(sh, S, P, rank, q, k, v, o, o_dtype, lse, dout, dq, dk, dv));
  if (rank < 0) return fail(CP_ERR_ARG, "the traffic emulation runs one rank (rank >= 0)");
  if (copy_stream == stream) return fail(CP_ERR_ARG, "copy_stream must differ from stream");
  const bool backward = dout != nullptr;
  const int64_t n = S / P;
  const size_t base = align256(ring_layout(sh, n, o_dtype, backward).total);
  const OverlapLayout L = overlap_layout(sh, n, backward, base);
  CP_TRY(check_workspace(workspace, ws_bytes, L.total));
  char* ws = (char*)workspace;
  RingOverlap ov{(hipStream_t)copy_stream, {ws + L.recv0, ws + L.recv1}, (float*)(ws + L.send)};
  const std::vector<int32_t> pairs = zigzag_pairs(P);
  CP_TRY(check_ring_ids(sh, doc, S, P, pairs.data(), (hipStream_t)stream));
  return ring_drive(sh, S, P, rank, pairs.data(), q, k, v, doc, o, o_dtype, lse, dout, dq, dk, dv, nullptr,
                    nullptr, ws, (hipStream_t)stream, &ov);
}

size_t cp_ulysses_workspace_bytes(const cp_shape* sh, int64_t S, int32_t sp, int32_t backward) {
  if (check_shape(sh) != CP_OK || S <= 0 || sp < 1 || sh->hq % sp || sh->hkv % sp) return 0;
  return backward ? align256((size_t)(sh->hq / sp) * S * 4) : 0;
}

}  // extern "C"

namespace {

// Arguments of a Ulysses share, apart from its scratch.
cp_status ulysses_args(const cp_shape* sh_full, int64_t S, int32_t sp, int32_t sp_rank, const void* q,
                       const void* k, const void* v, void* o, cp_dtype o_dtype, float* lse, const void* dout,
                       float* dq, float* dk, float* dv) {
  CP_TRY(check_shape(sh_full));
  if (S <= 0) return fail(CP_ERR_ARG, "S=%lld out of range", (long long)S);
  if (S > kMaxTokens) return fail(CP_ERR_UNSUPPORTED, "S=%lld above %d tokens", (long long)S, kMaxTokens);
  if (sp < 1 || sp_rank < 0 || sp_rank >= sp) return fail(CP_ERR_ARG, "sp=%d, sp_rank=%d", sp, sp_rank);
  if (sh_full->hq % sp || sh_full->hkv % sp)
    return fail(CP_ERR_ARG, "sp=%d must divide hq=%d and hkv=%d (KV heads bound the Ulysses degree)", sp,
                sh_full->hq, sh_full->hkv);
  if (!valid_dtype(o_dtype)) return fail(CP_ERR_ARG, "unknown o_dtype");
  CP_TRY(check_ptr(q, "q"));
  CP_TRY(check_ptr(k, "k"));
  CP_TRY(check_ptr(v, "v"));
  CP_TRY(check_ptr(o, "o"));
  if (!lse) return fail(CP_ERR_ARG, "lse is NULL");
  const bool backward = dout != nullptr;
  if (backward) {
    CP_TRY(check_ptr(dout, "dout"));
    CP_TRY(check_ptr(dq, "dq"));
    CP_TRY(check_ptr(dk, "dk"));
    CP_TRY(check_ptr(dv, "dv"));
  }
  return CP_OK;
}

// The share's kernels on `st`; dlt: scratch of (hq/sp)*S fp32 for Delta
// (backward only).
cp_status ulysses_drive(const cp_shape* sh_full, int64_t S, int32_t sp, int32_t sp_rank, const void* q,
                        const void* k, const void* v, const int32_t* doc, void* o, cp_dtype o_dtype, float* lse,
                        const void* dout, float* dq, float* dk, float* dv, float* dlt, hipStream_t st) {
  const bool backward = dout != nullptr;
  cp_shape sh = *sh_full;
  sh.hq = sh_full->hq / sp;
  sh.hkv = sh_full->hkv / sp;
  const size_t esz = elt_size(sh.dtype);
  const char* qs_ptr = (const char*)q + (size_t)sp_rank * sh.hq * sh.d * esz;
  const char* ks_ptr = (const char*)k + (size_t)sp_rank * sh.hkv * sh.d * esz;
  const char* vs_ptr = (const char*)v + (size_t)sp_rank * sh.hkv * sh.d * esz;
  if (!aligned16(qs_ptr) || !aligned16(ks_ptr)) return fail(CP_ERR_ALIGN, "head slice not 16-byte aligned");
  const cp_span span = run_span(0, (int32_t)S, S, 0, doc);
  CP_TRY(check_seq_ids(sh_full, doc, S, st));
  CP_TRY_HIP(run_fwd(&sh, qs_ptr, span, ks_ptr, vs_ptr, span, o, o_dtype, lse, S, st), "ulysses forward");
  if (backward) {
    // one chunk holds every pair: the gradients are written, not added to
    // (run_bwd zero-fills first where the kernels only accumulate)
    CP_TRY_HIP(launch_delta(S, sh.hq, sh.d, o, o_dtype == CP_F32, dout, sh.dtype == CP_F32, dlt, S, st),
               "ulysses delta");
    CP_TRY_HIP(run_bwd(&sh, qs_ptr, span, ks_ptr, vs_ptr, span, dout, lse, dlt, S, dq, dk, dv, st, BWD_ALL, true),
               "ulysses backward");
  }
  return ok();
}

}  // namespace

// Scratch of cp_ulysses_share_noalloc: the backward's Delta rows live in a
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` only names the symbol; its device address on the current GPU is
// looked up once per device (hipGetSymbolAddress) and only that address is
// handed to kernels.
constexpr size_t kNoallocScratchBytes = CP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, resolved on the first
// call per device and kept.
cp_status scratch_address(void** out) {
  int dev = -1;
  CP_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CP_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    CP_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
    if (!p) return fail(CP_ERR_HIP, "scratch address: null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status cp_ulysses_share(const cp_shape* sh_full, int64_t S, int32_t sp, int32_t sp_rank, const void* q,
                           const void* k, const void* v, const int32_t* doc, void* o, cp_dtype o_dtype, float* lse,
                           const void* dout, float* dq, float* dk, float* dv, void* workspace, size_t ws_bytes,
                           void* stream) {
  CP_TRY(ulysses_args(sh_full, S, sp, sp_rank, q, k, v, o, o_dtype, lse, dout, dq, dk, dv));
  if (dout) {
    const size_t need = cp_ulysses_workspace_bytes(sh_full, S, sp, 1);
    if (!workspace || ws_bytes < need) return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(CP_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  return ulysses_drive(sh_full, S, sp, sp_rank, q, k, v, doc, o, o_dtype, lse, dout, dq, dk, dv, (float*)workspace,
                       (hipStream_t)stream);
}

cp_status cp_ulysses_share_noalloc(const cp_shape* sh_full, int64_t S, int32_t sp, int32_t sp_rank, const void* q,
                                   const void* k, const void* v, const int32_t* doc, void* o, cp_dtype o_dtype,
                                   float* lse, const void* dout, float* dq, float* dk, float* dv, void* stream) {
  CP_TRY(ulysses_args(sh_full, S, sp, sp_rank, q, k, v, o, o_dtype, lse, dout, dq, dk, dv));
  if (sh_full->flags & CP_CHECK_DOCS)
    return fail(CP_ERR_ARG, "CP_CHECK_DOCS copies ids to the host and waits; check them with cp_check_docs first");
  float* dlt = nullptr;
  if (dout) {
    const size_t need = cp_ulysses_workspace_bytes(sh_full, S, sp, 1);
    if (need > kNoallocScratchBytes)
      return fail(CP_ERR_WORKSPACE, "Delta needs %zu bytes, above the %zu-byte built-in scratch", need,
                  kNoallocScratchBytes);
    void* p = nullptr;
    CP_TRY(scratch_address(&p));
    dlt = (float*)p;
  }
  return ulysses_drive(sh_full, S, sp, sp_rank, q, k, v, doc, o, o_dtype, lse, dout, dq, dk, dv, dlt,
                       (hipStream_t)stream);
}

static cp_status check_a2a(int64_t S, int32_t h, int32_t d, int32_t elt_bytes, int32_t sp, int32_t rank,
                           const void* a, const void* b, int64_t stride) {
  if (S <= 0 || S > INT32_MAX) return fail(CP_ERR_ARG, "S=%lld out of range", (long long)S);
  if (h <= 0 || d <= 0) return fail(CP_ERR_ARG, "h=%d, d=%d must be positive", h, d);
  if (elt_bytes != 2 && elt_bytes != 4) return fail(CP_ERR_ARG, "elt_bytes=%d not in {2, 4}", elt_bytes);
  if (sp < 1 || rank < 0 || rank >= sp) return fail(CP_ERR_ARG, "sp=%d, rank=%d", sp, rank);
  if (S % sp != 0) return fail(CP_ERR_ARG, "S=%lld is not a multiple of sp=%d (equal token shards)", (long long)S, sp);
  if (h % sp != 0 && sp % h != 0) return fail(CP_ERR_ARG, "h=%d and sp=%d: one must divide the other", h, sp);
  if (((int64_t)d * elt_bytes) % 16 != 0) return fail(CP_ERR_ALIGN, "a head row (d * elt_bytes) must be a multiple of 16 bytes");
  if (stride < (int64_t)h * d) return fail(CP_ERR_ARG, "token stride %lld < h*d", (long long)stride);
  if ((stride * elt_bytes) % 16 != 0) return fail(CP_ERR_ALIGN, "token stride must be a multiple of 16 bytes");
  CP_TRY(check_ptr(a, "input"));
  CP_TRY(check_ptr(b, "output"));
  return ok();
}

cp_status cp_a2a_tokens_to_heads(int64_t S, int32_t h, int32_t d, int32_t elt_bytes, int32_t sp, int32_t rank,
                                 const void* x, int64_t x_stride, void* y, void* stream) {
  CP_TRY(check_a2a(S, h, d, elt_bytes, sp, rank, x, y, x_stride));
  // heads rank `rank` receives: its slice, or (sp > h) the one KV head its
  // query heads read, shared with the other sp/h ranks of its group
  const int32_t h_out = h >= sp ? h / sp : 1;
  const int32_t h0 = h >= sp ? rank * (h / sp) : (int32_t)((int64_t)rank * h / sp);
  const int64_t head_b = (int64_t)d * elt_bytes;
  CP_TRY_HIP(launch_rows_copy(S, (int32_t)(h_out * head_b), (const char*)x + h0 * head_b, x_stride * elt_bytes, y,
                              h_out * head_b, (hipStream_t)stream),
             "all-to-all (tokens to heads)");
  return ok();
}

cp_status cp_a2a_heads_to_tokens(int64_t S, int32_t h, int32_t d, int32_t elt_bytes, int32_t sp, int32_t rank,
                                 const void* o, void* z, int64_t z_stride, void* stream) {
  CP_TRY(check_a2a(S, h, d, elt_bytes, sp, rank, o, z, z_stride));
  if (h % sp != 0) return fail(CP_ERR_ARG, "h=%d must be a multiple of sp=%d for the output exchange", h, sp);
  const int32_t h_in = h / sp;
  const int64_t head_b = (int64_t)d * elt_bytes;
  CP_TRY_HIP(launch_rows_copy(S, (int32_t)(h_in * head_b), o, h_in * head_b, (char*)z + (int64_t)rank * h_in * head_b,
                              z_stride * elt_bytes, (hipStream_t)stream),
             "all-to-all (heads to tokens)");
  return ok();
}

size_t cp_allgather_workspace_bytes(const cp_shape* sh, int64_t S, int32_t P, int32_t has_doc, int32_t backward) {
  if (check_ring_args(sh, S, P, 0) != CP_OK) return 0;
  const int64_t n = S / P;
  return align256((size_t)n * 4 * (has_doc ? 1 : 0)) + (backward ? align256((size_t)n * sh->hq * 4) : 0);
}

cp_status cp_allgather_share(const cp_shape* sh, int64_t S, int32_t P, int32_t rank, const void* q, const void* k,
                             const void* v, const int32_t* doc, void* o, cp_dtype o_dtype, float* lse,
                             const void* dout, float* dq, float* dk, float* dv, void* workspace, size_t ws_bytes,
                             void* stream) {
  CP_TRY(check_ring_args(sh, S, P, rank));
  if (rank < 0) return fail(CP_ERR_ARG, "rank=%d: one rank's share", rank);
  if (!valid_dtype(o_dtype)) return fail(CP_ERR_ARG, "unknown o_dtype");
  CP_TRY(check_ptr(q, "q"));
  CP_TRY(check_ptr(k, "k"));
  CP_TRY(check_ptr(v, "v"));
  CP_TRY(check_ptr(o, "o"));
  if (!lse) return fail(CP_ERR_ARG, "lse is NULL");
  const bool backward = dout != nullptr;
  if (backward) {
    CP_TRY(check_ptr(dout, "dout"));
    CP_TRY(check_ptr(dq, "dq"));
    CP_TRY(check_ptr(dk, "dk"));
    CP_TRY(check_ptr(dv, "dv"));
  }
  const size_t need = cp_allgather_workspace_bytes(sh, S, P, doc != nullptr, backward);
  if (need > 0) {
    if (!workspace || ws_bytes < need) return fail(CP_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(CP_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  hipStream_t st = (hipStream_t)stream;
  CP_TRY(check_seq_ids(sh, doc, S, st));
  const int64_t n = S / P;
  const int32_t c = (int32_t)(S / (2 * P));
  char* ws = (char*)workspace;
  // the rank's doc ids in local order (its two zigzag chunks), gathered from
  // the global array
  int32_t* qdoc = nullptr;
  if (doc) {
    qdoc = (int32_t*)ws;
    CP_TRY_HIP(hipMemcpyAsync(qdoc, doc + (int64_t)rank * c, (size_t)c * 4, hipMemcpyDeviceToDevice, st), "doc copy");
    CP_TRY_HIP(hipMemcpyAsync(qdoc + c, doc + (int64_t)(2 * P - 1 - rank) * c, (size_t)c * 4, hipMemcpyDeviceToDevice, st),
               "doc copy");
  }
  float* dlt = (float*)(ws + align256((size_t)n * 4 * (doc ? 1 : 0)));
  const cp_span qs = run_span((int64_t)rank * c, c, (int64_t)(2 * P - 1 - rank) * c, c, qdoc);
  const cp_span ks = run_span(0, (int32_t)S, S, 0, doc);
  CP_TRY_HIP(run_fwd(sh, q, qs, k, v, ks, o, o_dtype, lse, n, st), "all-gather forward");
  if (backward) {
    // one call holds every pair: the gradients are written (see cp_ulysses_share)
    CP_TRY_HIP(launch_delta(n, sh->hq, sh->d, o, o_dtype == CP_F32, dout, sh->dtype == CP_F32, dlt, n, st),
               "all-gather delta");
    CP_TRY_HIP(run_bwd(sh, q, qs, k, v, ks, dout, lse, dlt, n, dq, dk, dv, st, BWD_ALL, true),
               "all-gather backward");
  }
  return ok();
}

cp_status cp_check_docs(const int32_t* doc, int64_t n, int32_t on_host, void* stream) {
  if (n < 0) return fail(CP_ERR_ARG, "n=%lld is negative", (long long)n);
  if (n == 0) return ok();
  if (!doc) return fail(CP_ERR_ARG, "doc is NULL");
  if (on_host) {
    CP_TRY(validate_ids(doc, n, "doc"));
    return ok();
  }
  std::vector<int32_t> h;
  CP_TRY(fetch_ids(doc, n, (hipStream_t)stream, h));
  CP_TRY(validate_ids(h.data(), n, "doc"));
  return ok();
}

cp_status cp_chunk_work(int64_t S, int32_t P, const int32_t* doc, int64_t* work) {
  if (!work) return fail(CP_ERR_ARG, "work is NULL");
  if (P < 1 || S <= 0 || S % (2 * (int64_t)P) != 0)
    return fail(CP_ERR_ARG, "need P >= 1 and S > 0 divisible by 2P (S=%lld P=%d)", (long long)S, P);
  const int64_t c = S / (2 * P);
  // a query at position i sees the keys of its document up to itself
  int64_t doc_start = 0;
  for (int32_t ch = 0; ch < 2 * P; ++ch) work[ch] = 0;
  for (int64_t i = 0; i < S; ++i) {
    if (doc) {
      if (doc[i] < 0 || (i > 0 && doc[i] < doc[i - 1])) return fail(CP_ERR_DOCS, "doc ids must be >= 0 and non-decreasing");
      if (i > 0 && doc[i] != doc[i - 1]) doc_start = i;
    }
    work[i / c] += i - doc_start + 1;
  }
  return ok();
}

cp_status cp_balanced_pairs(int64_t S, int32_t P, const int32_t* doc, int32_t* chunks, int64_t* rank_work) {
  if (!chunks || !rank_work) return fail(CP_ERR_ARG, "output pointer is NULL");
  std::vector<int64_t> w(2 * (size_t)(P > 0 ? P : 1));
  CP_TRY(cp_chunk_work(S, P, doc, w.data()));
  // two chunks per rank, minimising the largest sum: pair the k-th lightest
  // chunk with the k-th heaviest (ties broken by position)
  std::vector<int32_t> order(2 * P);
  for (int32_t i = 0; i < 2 * P; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return w[x] < w[y]; });
  for (int32_t r = 0; r < P; ++r) {
    int32_t a = order[r], b = order[2 * P - 1 - r];
    if (a > b) std::swap(a, b);
    chunks[2 * r] = a;
    chunks[2 * r + 1] = b;
    rank_work[r] = w[a] + w[b];
  }
  return ok();
}

cp_status cp_tile_map(const cp_shape* sh, cp_span qs, cp_span ks, int32_t bq, int32_t bk, int8_t* out,
                      void* stream) {
  CP_TRY(check_shape(sh));
  CP_TRY(check_span(qs, "qs"));
  CP_TRY(check_span(ks, "ks"));
  CP_TRY(check_docs(qs, ks));
  if (bq <= 0 || bk <= 0) return fail(CP_ERR_ARG, "tile sizes must be positive");
  if (span_total(qs) == 0 || span_total(ks) == 0) return ok();
  if (!out) return fail(CP_ERR_ARG, "out is NULL");
  CP_TRY(check_span_ids(sh, qs, "qs.doc", (hipStream_t)stream));
  CP_TRY(check_span_ids(sh, ks, "ks.doc", (hipStream_t)stream));
  CP_TRY_HIP(launch_tile_map(to_dev(qs), to_dev(ks), sh->causal, bq, bk, out, (hipStream_t)stream),
             "cp_tile_map");
  return ok();
}

}  // extern "C"
