// fp32 chunk attention, forward and backward: the precision path.
//
// Same operation as the bf16 kernels (masked softmax attention of a Q chunk
// against a KV chunk, partial O and natural-log LSE, and the closed-form
// backward from the final LSE and Delta), computed with fp64 dot products,
// exponentials and accumulators so that fp32 inputs reach fp32-rounding
// accuracy in O and LSE.  One wave per (row, head): in the key (or query)
// loop the 64 lanes take 64 keys (queries) each, and for the d-dimensional
// accumulations the lanes take the d columns.  This path is for accuracy,
// not throughput.
#include "common.h"
#include "kernels.h"

namespace cp {
namespace {

// Allowed-key interval of one query row: keys outside [klo, khi) are masked;
// inside, the exact per-pair mask still applies.
__device__ inline void key_interval(const SpanD& qs, const SpanD& ks, int32_t qrow, bool causal,
                                    int32_t& klo, int32_t& khi) {
  const int32_t Lk = span_len(ks);
  klo = 0;
  khi = causal ? span_count_le(ks, span_pos(qs, qrow)) : Lk;
  if (qs.doc) {
    klo = wave_lower_bound(ks.doc, Lk, qs.doc[qrow]);
    khi = min(khi, wave_lower_bound(ks.doc, Lk, qs.doc[qrow] + 1));
  }
}

__device__ inline bool pair_ok(const SpanD& qs, const SpanD& ks, int32_t i, int32_t j, bool causal) {
  if (causal && span_pos(ks, j) > span_pos(qs, i)) return false;
  if (qs.doc && qs.doc[i] != ks.doc[j]) return false;
  return true;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline double wave_max(double x) {
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
__device__ inline double wave_sum(double x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams a) {
  constexpr int PER = (D + 63) / 64;
  __shared__ double qsh[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int32_t Lq = span_len(a.qs);
  if (item >= (int64_t)Lq * a.hq) return;          // wave-uniform
  const int32_t i = (int32_t)(item / a.hq);
  const int h = (int)(item % a.hq);
  const int g = h / a.G;
  const bool causal = a.causal != 0;
  for (int e = lane; e < D; e += 64) qsh[wave][e] = a.qf[(int64_t)i * a.q_stride + (int64_t)h * D + e];
  wave_sync();
  int32_t klo, khi;
  key_interval(a.qs, a.ks, i, causal, klo, khi);

  double m = -INFINITY, l = 0.0;
  double o[PER];
  for (int x = 0; x < PER; ++x) o[x] = 0.0;
  for (int32_t j0 = klo; j0 < khi; j0 += 64) {
    const int32_t j = j0 + lane;
    double s = -INFINITY;
    if (j < khi && pair_ok(a.qs, a.ks, i, j, causal)) {
      const float* kr = a.kf + (int64_t)j * a.kv_stride + (int64_t)g * D;
      double acc = 0.0;
      for (int e = 0; e < D; ++e) acc = fma(qsh[wave][e], (double)kr[e], acc);
      s = acc * (double)a.scale;
    }
    const double cm = wave_max(s);
    if (cm == -INFINITY) continue;
    const double mn = fmax(m, cm);
    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
    const double p = (s == -INFINITY) ? 0.0 : exp(s - mn);
    l = l * alpha + wave_sum(p);
    for (int x = 0; x < PER; ++x) o[x] *= alpha;
    const int32_t nk = min(64, khi - j0);
    for (int t = 0; t < nk; ++t) {
      const double pt = __shfl(p, t);
      if (pt == 0.0) continue;
      const float* vr = a.vf + (int64_t)(j0 + t) * a.kv_stride + (int64_t)g * D;
      for (int x = 0; x < PER; ++x) {
        const int e = lane + 64 * x;
        if (e < D) o[x] = fma(pt, (double)vr[e], o[x]);
      }
    }
    m = mn;
  }
  const bool live = l > 0.0;
  if (lane == 0) a.lse[(int64_t)h * a.lse_ld + i] = live ? (float)(m + log(l)) : -INFINITY;
  const int64_t ob = ((int64_t)i * a.hq + h) * D;
  for (int x = 0; x < PER; ++x) {
    const int e = lane + 64 * x;
    if (e < D) {
      const double val = live ? o[x] / l : 0.0;
      if (a.o_f32) ((float*)a.o)[ob + e] = (float)val;
      else ((__bf16*)a.o)[ob + e] = (__bf16)(float)val;
    }
  }
}

// dQ rows: one wave per (query row, head)
template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(BwdParams a) {
  constexpr int PER = (D + 63) / 64;
  __shared__ double qsh[4][D];
  __shared__ double osh[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int32_t Lq = span_len(a.qs);
  if (item >= (int64_t)Lq * a.hq) return;
  const int32_t i = (int32_t)(item / a.hq);
  const int h = (int)(item % a.hq);
  const int g = h / a.G;
  const bool causal = a.causal != 0;
  for (int e = lane; e < D; e += 64) {
    qsh[wave][e] = a.qf[(int64_t)i * a.q_stride + (int64_t)h * D + e];
    osh[wave][e] = a.doutf[((int64_t)i * a.hq + h) * D + e];
  }
  wave_sync();
  const float lse = a.lse[(int64_t)h * a.lse_ld + i];
  if (lse == -INFINITY) return;
  const double dl = a.delta[(int64_t)h * a.lse_ld + i];
  int32_t klo, khi;
  key_interval(a.qs, a.ks, i, causal, klo, khi);
  double dq[PER];
  for (int x = 0; x < PER; ++x) dq[x] = 0.0;
  for (int32_t j0 = klo; j0 < khi; j0 += 64) {
    const int32_t j = j0 + lane;
    double ds = 0.0;
    if (j < khi && pair_ok(a.qs, a.ks, i, j, causal)) {
      const float* kr = a.kf + (int64_t)j * a.kv_stride + (int64_t)g * D;
      const float* vr = a.vf + (int64_t)j * a.kv_stride + (int64_t)g * D;
      double s = 0.0, dp = 0.0;
      for (int e = 0; e < D; ++e) {
        s = fma(qsh[wave][e], (double)kr[e], s);
        dp = fma(osh[wave][e], (double)vr[e], dp);
      }
      const double p = exp(s * (double)a.scale - (double)lse);
      ds = p * (dp - dl);
    }
    const int32_t nk = min(64, khi - j0);
    for (int t = 0; t < nk; ++t) {
      const double dst = __shfl(ds, t);
      if (dst == 0.0) continue;
      const float* kr = a.kf + (int64_t)(j0 + t) * a.kv_stride + (int64_t)g * D;
      for (int x = 0; x < PER; ++x) {
        const int e = lane + 64 * x;
        if (e < D) dq[x] = fma(dst, (double)kr[e], dq[x]);
      }
    }
  }
  float* out = a.dq + ((int64_t)i * a.hq + h) * D;
  for (int x = 0; x < PER; ++x) {
    const int e = lane + 64 * x;
    if (e < D) out[e] += (float)(dq[x] * (double)a.scale);
  }
}

// dK, dV rows: one wave per (key row, KV head), summing over the group's heads
template <int D>
__global__ __launch_bounds__(256) void dkv_f32_kernel(BwdParams a) {
  constexpr int PER = (D + 63) / 64;
  __shared__ double ksh[4][D];
  __shared__ double vsh[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int32_t Lq = span_len(a.qs), Lk = span_len(a.ks);
  if (item >= (int64_t)Lk * a.hkv) return;
  const int32_t j = (int32_t)(item / a.hkv);
  const int g = (int)(item % a.hkv);
  const bool causal = a.causal != 0;
  for (int e = lane; e < D; e += 64) {
    ksh[wave][e] = a.kf[(int64_t)j * a.kv_stride + (int64_t)g * D + e];
    vsh[wave][e] = a.vf[(int64_t)j * a.kv_stride + (int64_t)g * D + e];
  }
  wave_sync();
  int32_t qlo = causal ? span_count_lt(a.qs, span_pos(a.ks, j)) : 0, qhi = Lq;
  if (a.qs.doc) {
    qlo = max(qlo, wave_lower_bound(a.qs.doc, Lq, a.ks.doc[j]));
    qhi = min(qhi, wave_lower_bound(a.qs.doc, Lq, a.ks.doc[j] + 1));
  }
  double dk[PER], dv[PER];
  for (int x = 0; x < PER; ++x) dk[x] = dv[x] = 0.0;
  for (int hg = 0; hg < a.G; ++hg) {
    const int h = g * a.G + hg;
    for (int32_t i0 = qlo; i0 < qhi; i0 += 64) {
      const int32_t i = i0 + lane;
      double p = 0.0, ds = 0.0;
      if (i < qhi && pair_ok(a.qs, a.ks, i, j, causal)) {
        const float lse = a.lse[(int64_t)h * a.lse_ld + i];
        if (lse != -INFINITY) {
          const float* qr = a.qf + (int64_t)i * a.q_stride + (int64_t)h * D;
          const float* orow = a.doutf + ((int64_t)i * a.hq + h) * D;
          double s = 0.0, dp = 0.0;
          for (int e = 0; e < D; ++e) {
            s = fma((double)qr[e], ksh[wave][e], s);
            dp = fma((double)orow[e], vsh[wave][e], dp);
          }
          p = exp(s * (double)a.scale - (double)lse);
          ds = p * (dp - (double)a.delta[(int64_t)h * a.lse_ld + i]);
        }
      }
      const int32_t nq = min(64, qhi - i0);
      for (int t = 0; t < nq; ++t) {
        const double pt = __shfl(p, t), dst = __shfl(ds, t);
        if (pt == 0.0 && dst == 0.0) continue;
        const float* qr = a.qf + (int64_t)(i0 + t) * a.q_stride + (int64_t)h * D;
        const float* orow = a.doutf + ((int64_t)(i0 + t) * a.hq + h) * D;
        for (int x = 0; x < PER; ++x) {
          const int e = lane + 64 * x;
          if (e < D) {
            dv[x] = fma(pt, (double)orow[e], dv[x]);
            dk[x] = fma(dst, (double)qr[e], dk[x]);
          }
        }
      }
    }
  }
  float* okp = a.dk + ((int64_t)j * a.hkv + g) * D;
  float* ovp = a.dv + ((int64_t)j * a.hkv + g) * D;
  for (int x = 0; x < PER; ++x) {
    const int e = lane + 64 * x;
    if (e < D) {
      okp[e] += (float)(dk[x] * (double)a.scale);
      ovp[e] += (float)dv[x];
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& a, hipStream_t stream) {
  const int64_t items = (int64_t)span_len(a.qs) * a.hq;
  if (items == 0) return hipSuccess;
  const unsigned grid = (unsigned)((items + 3) / 4);
  if (a.d == 128) hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32_dq(const BwdParams& a, hipStream_t stream) {
  const int64_t qitems = (int64_t)span_len(a.qs) * a.hq;
  if (qitems == 0 || span_len(a.ks) == 0) return hipSuccess;
  const dim3 grid((unsigned)((qitems + 3) / 4));
  if (a.d == 128) hipLaunchKernelGGL(dq_f32_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(dq_f32_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32_dkdv(const BwdParams& a, hipStream_t stream) {
  const int64_t kitems = (int64_t)span_len(a.ks) * a.hkv;
  if (kitems == 0 || span_len(a.qs) == 0) return hipSuccess;
  const dim3 grid((unsigned)((kitems + 3) / 4));
  if (a.d == 128) hipLaunchKernelGGL(dkv_f32_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(dkv_f32_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdParams& a, hipStream_t stream) {
  hipError_t e = launch_bwd_f32_dq(a, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_f32_dkdv(a, stream);
}

}  // namespace cp
