// Backward chunk attention, bf16 inputs, fp32 accumulation, CDNA4 (gfx950).
//
// Given the final (merged) row LSE and Delta = rowsum(dO * O), accumulates
// this chunk pair's contribution to dQ, dK and dV: the gradient of the masked
// softmax attention whose forward is in attn_fwd_bf16.hip.  The pages do not
// describe the backward; it is the derivative of that definition, with P
// recomputed from the saved LSE (the recompute-in-backward idea behind
// activation checkpointing, siliconandsystems.com "Llama 3 parallelism",
// section on long context changing more than the attention cost).
//
// Work decomposition (KV-outer)
//   * one work-group = 4 waves = 128 keys of one KV head; wave w owns 32 keys,
//     whose K and V rows it keeps in VGPRs as MFMA B operands and whose dK^T
//     and dV^T accumulators it keeps for the whole kernel.
//   * the group streams query tiles of 64 rows for every query head of the
//     GQA group; each tile of Q and dO is staged in LDS twice: row-major (the
//     A operand when contracting over d) and interleaved by 4 rows (the A
//     operand when contracting over queries).  The next tile's global loads
//     are issued before the current tile's MFMAs.
//   * per tile and wave: S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_bf16,
//     accumulator lane = key, 16 query rows), P = exp2(S*c - LSE2),
//     dS = scale * P * (dP - Delta); dV^T += dO^T P and dK^T += Q^T dS take P
//     and dS straight from the accumulator layout as B operands.
//   * dQ = dS K needs all 128 keys: dS goes through LDS and each wave computes
//     32 of the d columns, then adds them to the fp32 dQ with global atomics.
//   * fully masked tiles are skipped; element masks only on partial or ragged
//     tiles.  Heavy-first order: earlier keys are seen by more queries.
#include "common.h"
#include "kernels.h"

namespace cp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BQ = 64;    // query rows per tile
constexpr int BKW = 32;   // keys per wave
constexpr int BKG = 128;  // keys per work-group
constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct Lds {
  static constexpr int RST = D + 8;                  // padded row-major stride
  static constexpr int QR = 0;                        // Q row-major  [64][RST]
  static constexpr int DOR = QR + BQ * RST * 2;       // dO row-major [64][RST]
  static constexpr int QI = DOR + BQ * RST * 2;       // Q  [16][D][4]
  static constexpr int DOI = QI + BQ * D * 2;         // dO [16][D][4]
  static constexpr int DS = DOI + BQ * D * 2;         // dS [64][BKG + 8]
  static constexpr int DSST = BKG + 8;
  static constexpr int KI = DS + BQ * DSST * 2;       // K  [32][D][4]
  static constexpr int LSE = KI + BKG * D * 2;        // lse2 [64]
  static constexpr int DLT = LSE + BQ * 4;            // delta [64]
  static constexpr int QDOC = DLT + BQ * 4;           // query doc ids [64]
  static constexpr int TOTAL = QDOC + BQ * 4;
};

// interleave 4 rows x 8 dims (4 x 16-byte pieces) into 8 pieces of 4 rows
__device__ inline void store_interleaved(__bf16* dst, int D, int rg, int dg, const u32x4 r[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    u32x2 lo, hi;
    lo.x = __builtin_amdgcn_perm(r[1][m], r[0][m], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(r[3][m], r[2][m], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(r[1][m], r[0][m], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(r[3][m], r[2][m], 0x07060302u);
    int d0 = dg * 8 + 2 * m;
    *(u32x2*)(dst + ((rg * D) + d0) * 4) = lo;
    *(u32x2*)(dst + ((rg * D) + d0 + 1) * 4) = hi;
  }
}

__device__ inline bf16x8 read_interleaved(const __bf16* src, int D, int t, int hh, int d) {
  u32x2 lo = *(const u32x2*)(src + ((4 * t + hh) * D + d) * 4);
  u32x2 hi = *(const u32x2*)(src + ((4 * t + 2 + hh) * D + d) * 4);
  u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, v);
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(BwdParams a) {
  using L = Lds<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __bf16* Qr = (__bf16*)(smem + L::QR);
  __bf16* dOr = (__bf16*)(smem + L::DOR);
  __bf16* Qi = (__bf16*)(smem + L::QI);
  __bf16* dOi = (__bf16*)(smem + L::DOI);
  __bf16* dSl = (__bf16*)(smem + L::DS);
  __bf16* Ki = (__bf16*)(smem + L::KI);
  float* lse2 = (float*)(smem + L::LSE);
  float* dlt = (float*)(smem + L::DLT);
  int32_t* qdocl = (int32_t*)(smem + L::QDOC);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;

  const int32_t w = xcd_remap(blockIdx.x, gridDim.x);
  if (w >= a.n_work) return;
  const int kvh = w / a.nkt;
  const int32_t kt = w % a.nkt;                        // ascending = heavy first

  const SpanD qs = a.qs, ks = a.ks;
  const int32_t Lq = span_len(qs), Lk = span_len(ks);
  const bool causal = a.causal != 0;
  const bool docs = qs.doc != nullptr;
  const int32_t k0 = kt * BKG, k1 = min(Lk, k0 + BKG);
  const int32_t wk0 = k0 + wave * BKW, wk1 = min(Lk, wk0 + BKW);
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

  // ---- this wave's keys: K, V as B operands; K interleaved into LDS --------
  const int32_t mykey = min(wk0 + lq, Lk - 1);
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const bf16x8* ksrc = (const bf16x8*)(a.k + (int64_t)mykey * a.kv_stride + (int64_t)kvh * D + hh * 8);
    const bf16x8* vsrc = (const bf16x8*)(a.v + (int64_t)mykey * a.kv_stride + (int64_t)kvh * D + hh * 8);
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      kf[kd] = ksrc[kd * 2];
      vf[kd] = vsrc[kd * 2];
    }
  }
  const int64_t mykpos = span_pos(ks, mykey);
  const int32_t mykdoc = docs ? ks.doc[mykey] : 0;
  {
    constexpr int ITEMS = (BKG / 4) * (D / 8);
    for (int item = tid; item < ITEMS; item += 256) {
      int rg = item / (D / 8), dg = item % (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        int32_t row = min(k0 + rg * 4 + x, Lk - 1);
        r[x] = *(const u32x4*)(a.k + (int64_t)row * a.kv_stride + (int64_t)kvh * D + dg * 8);
      }
      store_interleaved(Ki, D, rg, dg, r);
    }
  }

  f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dva[db] = f32x16{}; dka[db] = f32x16{}; }

  // ---- staging of one (query tile, head) item ------------------------------
  constexpr int SITEMS = (BQ / 4) * (D / 8);           // 4 rows x 8 dims each
  constexpr int SI_PER_T = (SITEMS + 255) / 256;
  u32x4 qreg[SI_PER_T][4], oreg[SI_PER_T][4];
  float lreg = 0.f, dreg = 0.f;
  int32_t docreg = 0;
  const int nitems = (qt1 - qt0) * a.G;

  auto load_item = [&](int it) {
    const int32_t qt = qt0 + it / a.G;
    const int head = kvh * a.G + it % a.G;
    const int32_t base = qt * BQ;
#pragma unroll
    for (int i = 0; i < SI_PER_T; ++i) {
      int item = tid + i * 256;
      if (item < SITEMS) {
        int rg = item / (D / 8), dg = item % (D / 8);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          int32_t row = min(base + rg * 4 + x, Lq - 1);
          qreg[i][x] = *(const u32x4*)(a.q + (int64_t)row * a.q_stride + (int64_t)head * D + dg * 8);
          oreg[i][x] = *(const u32x4*)(a.dout + ((int64_t)row * a.hq + head) * D + dg * 8);
        }
      }
    }
    if (tid < BQ) {
      int32_t row = min(base + tid, Lq - 1);
      lreg = a.lse[(int64_t)head * a.lse_ld + row];
      dreg = a.delta[(int64_t)head * a.lse_ld + row];
      docreg = docs ? qs.doc[row] : 0;
    }
  };
  auto store_item = [&]() {
#pragma unroll
    for (int i = 0; i < SI_PER_T; ++i) {
      int item = tid + i * 256;
      if (item < SITEMS) {
        int rg = item / (D / 8), dg = item % (D / 8);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          *(u32x4*)(Qr + (rg * 4 + x) * L::RST + dg * 8) = qreg[i][x];
          *(u32x4*)(dOr + (rg * 4 + x) * L::RST + dg * 8) = oreg[i][x];
        }
        store_interleaved(Qi, D, rg, dg, qreg[i]);
        store_interleaved(dOi, D, rg, dg, oreg[i]);
      }
    }
    if (tid < BQ) {
      lse2[tid] = (lreg == -INFINITY) ? INFINITY : lreg * LOG2E;
      dlt[tid] = dreg;
      qdocl[tid] = docreg;
    }
  };

  if (nitems > 0) {
    load_item(0);
    store_item();
  }
  __syncthreads();

  const float c = a.scale * LOG2E;
  for (int it = 0; it < nitems; ++it) {
    const int32_t qt = qt0 + it / a.G;
    const int head = kvh * a.G + it % a.G;
    const int32_t qa0 = qt * BQ, qa1 = min(Lq, qa0 + BQ);
    if (it + 1 < nitems) load_item(it + 1);

    const int wg_cls = block_class(qs, qa0, qa1, ks, k0, k1, causal);
    const int cls = (wave_has_keys && wg_cls != TILE_SKIP)
                        ? block_class(qs, qa0, qa1, ks, wk0, wk1, causal) : TILE_SKIP;

    if (cls != TILE_SKIP) {
      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          bf16x8 qa = *(const bf16x8*)(Qr + (qb * 32 + lq) * L::RST + kd * 16 + hh * 8);
          bf16x8 oa = *(const bf16x8*)(dOr + (qb * 32 + lq) * L::RST + kd * 16 + hh * 8);
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kd], s[qb], 0, 0, 0);
          dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kd], dp[qb], 0, 0, 0);
        }
      }
      const bool need_mask = cls == TILE_PARTIAL || qa1 - qa0 < BQ || wk1 - wk0 < BKW;
      const bool key_ok = wk0 + lq < wk1;
      bf16x8 pf[4], dsf[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = qb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -lse2[qr]));
          if (need_mask) {
            const int32_t qidx = qa0 + qr;
            bool ok = key_ok && qidx < qa1 && (!causal || mykpos <= span_pos(qs, qidx)) &&
                      (!docs || qdocl[qr] == mykdoc);
            if (!ok) p = 0.f;
          }
          const float ds = p * (dp[qb][r] - dlt[qr]) * a.scale;
          const int t = qb * 2 + (r >> 3), sl = r & 7;
          pf[t][sl] = (__bf16)p;
          dsf[t][sl] = (__bf16)ds;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = db * 32 + lq;
          bf16x8 oa = read_interleaved(dOi, D, t, hh, d);
          bf16x8 qa = read_interleaved(Qi, D, t, hh, d);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pf[t], dva[db], 0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsf[t], dka[db], 0, 0, 0);
        }
      }
      // dS (bf16) to LDS, [query][key] row-major, for the dQ product
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int qr = t * 16 + (sl >> 2) * 8 + hh * 4 + (sl & 3);
          dSl[qr * L::DSST + wave * BKW + lq] = dsf[t][sl];
        }
    } else if (wg_cls != TILE_SKIP) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int qr = t * 16 + (sl >> 2) * 8 + hh * 4 + (sl & 3);
          dSl[qr * L::DSST + wave * BKW + lq] = (__bf16)0.f;
        }
    }
    __syncthreads();

    if (wg_cls != TILE_SKIP) {
      // dQ^T (32 d rows x 32 queries per block) = K^T dS^T over the 128 keys.
      // The (d block, query block) pairs are split over the 4 waves: D=128 has
      // 4 x 2 pairs (wave w: d block w, both query blocks), D=64 has 2 x 2
      // (wave w: d block w/2, query block w%2).
      constexpr int QBW = D / 64;                 // query blocks per wave
      const int dblk = D == 128 ? wave : (wave >> 1);
      const int qbb = D == 128 ? 0 : (wave & 1);
      f32x16 dq[QBW];
#pragma unroll
      for (int x = 0; x < QBW; ++x) dq[x] = f32x16{};
      const int d = dblk * 32 + lq;
#pragma unroll
      for (int t = 0; t < BKG / 16; ++t) {
        // natural slot order: slot s <-> key 16t + 8hh + s, for A and B alike
        u32x2 lo = *(const u32x2*)(Ki + ((4 * t + 2 * hh) * D + d) * 4);
        u32x2 hi = *(const u32x2*)(Ki + ((4 * t + 2 * hh + 1) * D + d) * 4);
        u32x4 kv = {lo.x, lo.y, hi.x, hi.y};
        bf16x8 ka = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
        for (int x = 0; x < QBW; ++x) {
          const int qb = qbb + x;
          bf16x8 db8 = *(const bf16x8*)(dSl + (qb * 32 + lq) * L::DSST + t * 16 + hh * 8);
          dq[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, db8, dq[x], 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < QBW; ++x) {
        const int32_t row = qa0 + (qbb + x) * 32 + lq;
        if (row < qa1) {
          float* dst = a.dq + ((int64_t)row * a.hq + head) * D + dblk * 32 + hh * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(dst + j * 8 + i, dq[x][4 * j + i]);
        }
      }
    }
    __syncthreads();
    if (it + 1 < nitems) {
      store_item();
      __syncthreads();
    }
  }

  // ---- dK, dV (exclusive to this work-group): read-modify-write -------------
  if (wave_has_keys && wk0 + lq < wk1) {
    const int64_t base = ((int64_t)(wk0 + lq) * a.hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + j * 8 + hh * 4;
        f32x4* pk = (f32x4*)(a.dk + base + d);
        f32x4* pv = (f32x4*)(a.dv + base + d);
        f32x4 ok = *pk, ov = *pv;
        ok[0] += dka[db][4 * j]; ok[1] += dka[db][4 * j + 1];
        ok[2] += dka[db][4 * j + 2]; ok[3] += dka[db][4 * j + 3];
        ov[0] += dva[db][4 * j]; ov[1] += dva[db][4 * j + 1];
        ov[2] += dva[db][4 * j + 2]; ov[3] += dva[db][4 * j + 3];
        *pk = ok;
        *pv = ov;
      }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  BwdParams a = p;
  const int32_t Lk = span_len(a.ks);
  a.nkt = (Lk + BKG - 1) / BKG;
  a.n_work = a.nkt * a.hkv;
  if (a.n_work == 0 || span_len(a.qs) == 0) return hipSuccess;
  const int32_t grid = round_up8(a.n_work);
  if (a.d == 128) {
    hipLaunchKernelGGL(bwd_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_bf16_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cp
