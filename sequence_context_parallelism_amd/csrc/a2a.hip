// Emulated Ulysses all-to-all on one GPU: the token-split <-> head-split
// exchange of a sequence-parallel attention layer (aionda.blog, "Ulysses
// sequence parallelism for long-context training", section 현황; nougat.kr,
// "MaxText long-context training: KV parallelism", diagram text, A2A).
//
// With every rank's token shard resident in one token-major tensor
// [S, h, d], what rank r holds after the forward exchange is, for every
// token, the heads of its slice; the backward (output) exchange writes a
// rank's head slice back into the token-split tensor.  Both are copies of
// 16-byte chunks, bound by HBM bandwidth: one thread per chunk, loads and
// stores of 16 bytes, consecutive threads on consecutive chunks of a row.
#include "kernels.h"

namespace cp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// dst row s (dst_stride bytes apart) = chunks [0, row_chunks) of
// src + s * src_stride + src_off bytes.  Strides and offsets are multiples of 16.
__global__ __launch_bounds__(256) void rows_copy_kernel(int64_t rows, int32_t row_chunks, const char* __restrict__ src,
                                                        int64_t src_stride, char* __restrict__ dst,
                                                        int64_t dst_stride) {
  const int64_t total = rows * row_chunks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t s = i / row_chunks;
    const int32_t c = (int32_t)(i - s * row_chunks);
    const u32x4 v = *(const u32x4*)(src + s * src_stride + (int64_t)c * 16);
    *(u32x4*)(dst + s * dst_stride + (int64_t)c * 16) = v;
  }
}

}  // namespace

hipError_t launch_rows_copy(int64_t rows, int32_t row_bytes, const void* src, int64_t src_stride_b, void* dst,
                            int64_t dst_stride_b, hipStream_t stream) {
  const int32_t row_chunks = row_bytes / 16;
  const int64_t total = rows * row_chunks;
  if (total == 0) return hipSuccess;
  // enough work-groups to fill all CUs several times, each looping over chunks
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 256 * 32 ? want : 256 * 32);
  hipLaunchKernelGGL(rows_copy_kernel, dim3(grid), dim3(256), 0, stream, rows, row_chunks, (const char*)src,
                     src_stride_b, (char*)dst, dst_stride_b);
  return hipGetLastError();
}

}  // namespace cp
