// Internal launch interface between the C-ABI host code (capi.hip) and the
// kernels of libcpattn.  Not installed; the public interface is cpattn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace cp {

struct FwdParams {
  const __bf16* q;           // bf16 path inputs
  const __bf16* k;
  const __bf16* v;
  const float* qf;           // fp32 path inputs
  const float* kf;
  const float* vf;
  int64_t q_stride, kv_stride;   // elements between tokens
  SpanD qs, ks;
  int hq, hkv, G, d;
  float scale;
  int causal;
  void* o;                   // [Lq, hq, d] contiguous
  int o_f32;                 // 1: fp32 O, 0: bf16 O
  float* lse;                // [hq, lse_ld]
  int64_t lse_ld;
  int merge;                 // 1 (bf16 path, fp32 O): (o, lse) hold a running result; merge into it
  // filled in by the launcher
  int heads_per_wg, qblocks_per_wg, nqt, n_work;
  float scale_log2;
};

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;        // [Lq, hq, d] contiguous
  const float* qf;
  const float* kf;
  const float* vf;
  const float* doutf;
  int64_t q_stride, kv_stride;
  SpanD qs, ks;
  int hq, hkv, G, d;
  float scale;
  int causal;
  const float* lse;          // final LSE   [hq, lse_ld]
  const float* delta;        // final Delta [hq, lse_ld]
  int64_t lse_ld;
  float* dq;                 // [Lq, hq, d]  += (or = with store)
  float* dk;                 // [Lk, hkv, d] += (or = with store)
  float* dv;                 // [Lk, hkv, d] += (or = with store)
  int store;                 // bf16 path: 1 = write the gradients (the call's pairs are all of them), 0 = add
  // filled in by the launcher
  int nkt, n_work;
  int pair;                  // dK/dV work order: partner key tiles (dkdv_work) or heavy-first (xcd_work)
  int heads_per_wg, qblocks_per_wg, nqt;
};

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);       // dq then dkdv
hipError_t launch_bwd_bf16_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16_dq(const BwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream);        // dq then dkdv
hipError_t launch_bwd_f32_dkdv(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f32_dq(const BwdParams& p, hipStream_t stream);

// acc <- acc (+) part, exact LSE-weighted combination; rows x h row-heads
hipError_t launch_lse_merge(int64_t rows, int h, int d, float* o_acc, float* lse_acc, int64_t acc_ld,
                            const float* o_part, const float* lse_part, int64_t part_ld,
                            hipStream_t stream);
// delta[h, r] = sum_e dout[r, h, e] * o[r, h, e]
hipError_t launch_delta(int64_t rows, int h, int d, const void* o, int o_f32, const void* dout,
                        int dout_f32, float* delta, int64_t delta_ld, hipStream_t stream);
hipError_t launch_f32_to_bf16(int64_t n, const float* src, __bf16* dst, hipStream_t stream);
hipError_t launch_fill_zero(int64_t n, float* dst, hipStream_t stream);
hipError_t launch_copy_f32(int64_t n, const float* src, float* dst, hipStream_t stream);
// dst row s = the first row_bytes of src row s (row_bytes and both strides
// multiples of 16; pointers 16-byte aligned)
hipError_t launch_rows_copy(int64_t rows, int32_t row_bytes, const void* src, int64_t src_stride_b, void* dst,
                            int64_t dst_stride_b, hipStream_t stream);
hipError_t launch_tile_map(SpanD qs, SpanD ks, int causal, int bq, int bk, int8_t* out,
                           hipStream_t stream);

}  // namespace cp
