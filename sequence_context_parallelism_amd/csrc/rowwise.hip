// Streaming (HBM-bound) kernels of libcpattn: the exact LSE merge of two
// partial results, the backward's Delta = rowsum(dO * O), dtype conversion,
// zero fill, copy, and the debug dump of the tile classification.
//
// The merge is the combination step of a ring rank (nougat.kr, "MaxText
// long-context training: KV parallelism", section "헤드를 나누거나, KV를
// 돌리거나": each step's partial result is merged into the running one).
// Each (row, head) is handled by d/4 consecutive lanes, one 16-byte piece of
// O per lane, so every access is a coalesced 16-byte vector; the merge weights
// are computed once per (row, head) in fp64, 64 pairs at a time across the
// lanes of a wave, and passed to the lanes that stream the pair's row.
#include "common.h"
#include "kernels.h"

namespace cp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each wave merges 64 consecutive (row, head) pairs.  First every lane
// computes the two weights and the new LSE of one pair in fp64 (64 pairs in
// parallel); then the wave streams the pairs' O rows, 64 / SEG pairs per step
// (SEG = d/4 lanes per pair, one 16-byte piece of O each, so every access is
// a coalesced 16-byte vector), each lane taking its pair's weights from the
// lane that computed them.
template <int SEG>   // lanes per (row, head) = d / 4
__global__ __launch_bounds__(256) void merge_kernel(int64_t rows, int h, float* __restrict__ o_acc,
                                                    float* __restrict__ lse_acc, int64_t acc_ld,
                                                    const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int64_t part_ld) {
  constexpr int PER_STEP = 64 / SEG;            // pairs streamed per step
  const int lane = threadIdx.x & 63;
  const int64_t n = rows * h;
  const int64_t rh0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;   // the wave's first pair
  if (rh0 >= n) return;                          // wave-uniform
  // ---- weights of pair rh0 + lane -------------------------------------
  double ca = 0.0, cb = 0.0;
  {
    const int64_t rh = rh0 + lane;
    if (rh < n) {
      const int64_t r = rh / h;
      const int hd = (int)(rh % h);
      const double la = lse_acc[(int64_t)hd * acc_ld + r];
      const double lb = lse_part[(int64_t)hd * part_ld + r];
      const double m = fmax(la, lb);
      float lnew = -INFINITY;
      if (m != -INFINITY) {
        const double L = m + log(exp(la - m) + exp(lb - m));
        ca = exp(la - L);
        cb = exp(lb - L);
        lnew = (float)L;
      }
      lse_acc[(int64_t)hd * acc_ld + r] = lnew;
    }
  }
  // ---- stream the O rows ------------------------------------------------
  const int sub = lane / SEG, piece = lane % SEG;
#pragma unroll 8
  for (int step = 0; step < SEG; ++step) {
    const int j = step * PER_STEP + sub;         // pair index within the wave's 64
    const float fa = (float)__shfl(ca, j), fb = (float)__shfl(cb, j);
    const int64_t rh = rh0 + j;
    if (rh < n) {
      f32x4* pa = (f32x4*)(o_acc + rh * (SEG * 4)) + piece;
      // the partial is read once: a non-temporal load keeps it from displacing
      // the accumulator in the caches (0.166 -> 0.128 ms at 65,536 x 8 x 128)
      const f32x4 pb = __builtin_nontemporal_load((const f32x4*)(o_part + rh * (SEG * 4)) + piece);
      f32x4 x = *pa;
      x[0] = fa * x[0] + fb * pb[0];
      x[1] = fa * x[1] + fb * pb[1];
      x[2] = fa * x[2] + fb * pb[2];
      x[3] = fa * x[3] + fb * pb[3];
      *pa = x;
    }
  }
}

template <int SEG, typename TO, typename TD>
__global__ __launch_bounds__(256) void delta_kernel(int64_t rows, int h, const TO* __restrict__ o,
                                                    const TD* __restrict__ dout, float* __restrict__ delta,
                                                    int64_t ld) {
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gt / SEG;
  const int piece = (int)(gt % SEG);
  const bool in = rh < rows * h;
  float acc = 0.f;
  if (in) {
    const int64_t base = rh * (SEG * 4) + piece * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += (float)o[base + i] * (float)dout[base + i];
  }
#pragma unroll
  for (int off = SEG / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (in && piece == 0) delta[(int64_t)(rh % h) * ld + rh / h] = acc;
}

// The same for bf16 O and dO with 16-byte loads: SEG = d / 8 lanes per
// (row, head), 8 elements each.
template <int SEG>
__global__ __launch_bounds__(256) void delta_bf16_kernel(int64_t rows, int h, const __bf16* __restrict__ o,
                                                         const __bf16* __restrict__ dout, float* __restrict__ delta,
                                                         int64_t ld) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gt / SEG;
  const int piece = (int)(gt % SEG);
  const bool in = rh < rows * h;
  float acc = 0.f;
  if (in) {
    const int64_t base = rh * (SEG * 8) + piece * 8;
    const bf16x8 a = *(const bf16x8*)(o + base);
    const bf16x8 b = *(const bf16x8*)(dout + base);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
  }
#pragma unroll
  for (int off = SEG / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (in && piece == 0) delta[(int64_t)(rh % h) * ld + rh / h] = acc;
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(int64_t n, const float* __restrict__ src,
                                                          __bf16* __restrict__ dst) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const f32x4 x = *(const f32x4*)(src + i);
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *(bf16x4*)(dst + i) = y;
  } else {
    for (int64_t j = i; j < n; ++j) dst[j] = (__bf16)src[j];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int64_t n, float* __restrict__ dst) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *(f32x4*)(dst + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t j = i; j < n; ++j) dst[j] = 0.f;
  }
}

__global__ __launch_bounds__(256) void copy_f32_kernel(int64_t n, const float* __restrict__ src,
                                                       float* __restrict__ dst) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *(f32x4*)(dst + i) = *(const f32x4*)(src + i);
  } else {
    for (int64_t j = i; j < n; ++j) dst[j] = src[j];
  }
}

__global__ __launch_bounds__(256) void tile_map_kernel(SpanD qs, SpanD ks, int causal, int bq, int bk,
                                                       int32_t nqt, int32_t nkt, int8_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)nqt * nkt) return;
  const int32_t a = (int32_t)(t / nkt), b = (int32_t)(t % nkt);
  const int32_t a0 = a * bq, a1 = min(span_len(qs), a0 + bq);
  const int32_t b0 = b * bk, b1 = min(span_len(ks), b0 + bk);
  out[t] = (int8_t)block_class(qs, a0, a1, ks, b0, b1, causal != 0);
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int h, int d, float* o_acc, float* lse_acc, int64_t acc_ld,
                            const float* o_part, const float* lse_part, int64_t part_ld,
                            hipStream_t stream) {
  const int64_t rh = rows * h;
  if (rh == 0) return hipSuccess;
  const int seg = d / 4;
  const unsigned grid = blocks_for(rh);          // one lane per pair in the weight phase: 64 pairs per wave
  switch (seg) {
    case 32: hipLaunchKernelGGL(merge_kernel<32>, dim3(grid), dim3(256), 0, stream, rows, h, o_acc, lse_acc, acc_ld, o_part, lse_part, part_ld); break;
    case 16: hipLaunchKernelGGL(merge_kernel<16>, dim3(grid), dim3(256), 0, stream, rows, h, o_acc, lse_acc, acc_ld, o_part, lse_part, part_ld); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int SEG>
static hipError_t delta_dispatch(int64_t rows, int h, const void* o, int o_f32, const void* dout,
                                 int dout_f32, float* delta, int64_t ld, hipStream_t stream) {
  const unsigned grid = blocks_for(rows * h * SEG);
  if (o_f32 && dout_f32)
    hipLaunchKernelGGL((delta_kernel<SEG, float, float>), dim3(grid), dim3(256), 0, stream, rows, h, (const float*)o, (const float*)dout, delta, ld);
  else if (o_f32)
    hipLaunchKernelGGL((delta_kernel<SEG, float, __bf16>), dim3(grid), dim3(256), 0, stream, rows, h, (const float*)o, (const __bf16*)dout, delta, ld);
  else if (dout_f32)
    hipLaunchKernelGGL((delta_kernel<SEG, __bf16, float>), dim3(grid), dim3(256), 0, stream, rows, h, (const __bf16*)o, (const float*)dout, delta, ld);
  else
    hipLaunchKernelGGL((delta_bf16_kernel<SEG / 2>), dim3(blocks_for(rows * h * (SEG / 2))), dim3(256), 0, stream, rows, h,
                       (const __bf16*)o, (const __bf16*)dout, delta, ld);
  return hipGetLastError();
}

hipError_t launch_delta(int64_t rows, int h, int d, const void* o, int o_f32, const void* dout,
                        int dout_f32, float* delta, int64_t delta_ld, hipStream_t stream) {
  if (rows * h == 0) return hipSuccess;
  switch (d / 4) {
    case 32: return delta_dispatch<32>(rows, h, o, o_f32, dout, dout_f32, delta, delta_ld, stream);
    case 16: return delta_dispatch<16>(rows, h, o, o_f32, dout, dout_f32, delta, delta_ld, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_f32_to_bf16(int64_t n, const float* src, __bf16* dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks_for((n + 3) / 4)), dim3(256), 0, stream, n, src, dst);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int64_t n, float* dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for((n + 3) / 4)), dim3(256), 0, stream, n, dst);
  return hipGetLastError();
}

hipError_t launch_copy_f32(int64_t n, const float* src, float* dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks_for((n + 3) / 4)), dim3(256), 0, stream, n, src, dst);
  return hipGetLastError();
}

hipError_t launch_tile_map(SpanD qs, SpanD ks, int causal, int bq, int bk, int8_t* out,
                           hipStream_t stream) {
  const int32_t nqt = (span_len(qs) + bq - 1) / bq, nkt = (span_len(ks) + bk - 1) / bk;
  const int64_t n = (int64_t)nqt * nkt;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_map_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, qs, ks, causal, bq, bk, nqt, nkt, out);
  return hipGetLastError();
}

}  // namespace cp
