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
//   * one work-group = 4 waves; each wave owns 64 query rows of one query
//     head.  With grouped-query attention the 4 waves of a group take 4 query
//     heads that read the same KV head (or 2 heads x 2 row blocks, or 1 head x
//     4 row blocks), so every K/V tile staged in LDS feeds 4 waves.
//   * keys stream through LDS in tiles of 64, double-buffered: the next tile's
//     global loads are issued before the current tile's MFMAs.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K tile is the A operand
//     (read from LDS), the wave's Q rows are the B operand (held in VGPRs for
//     the whole kernel).  In the 32x32 accumulator each lane holds one query
//     column and 16 key rows, so the softmax row statistics need one cross-lane
//     exchange (lane ^ 32) per tile.
//   * O^T += V^T P^T: P^T goes from the S^T accumulator straight into the B
//     operand (no LDS round trip).  V is stored in LDS interleaved by groups of
//     4 keys ([key/4][d][4]) so the A operand of each lane is two 8-byte reads.
//   * fully masked tiles (causal or document) are skipped; the element mask is
//     evaluated only on partial tiles and on the ragged last tile.
//   * work-groups run heavy-first (later query tiles have more causal work),
//     remapped so each XCD works on a contiguous range of KV heads.
#include "common.h"
#include "kernels.h"

namespace cp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int BK = 64;      // keys per tile
constexpr int QW = 64;      // query rows per wave
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D>
struct Lds {
  static constexpr int KST = D + 8;                 // padded K row (elements)
  static constexpr int KBYTES = BK * KST * 2;
  static constexpr int VBYTES = BK * D * 2;
  static constexpr int STAGE = KBYTES + VBYTES + BK * 4;   // + key doc ids
  static constexpr int TOTAL = 2 * STAGE;
};

__device__ inline bf16x8 cvt8(const f32x16& s, int base, float c, float moff, float& sum) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float p = __builtin_amdgcn_exp2f(fmaf(s[base + i], c, moff));
    sum += p;
    r[i] = (__bf16)p;
  }
  return r;
}

template <int D>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(FwdParams a) {
  using L = Lds<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;

  const int32_t w = xcd_remap(blockIdx.x, gridDim.x);
  if (w >= a.n_work) return;
  const int32_t grp = w / a.nqt;
  const int32_t qt = a.nqt - 1 - (w % a.nqt);         // heavy first
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

  // ---- key range of the work-group -------------------------------------
  int32_t klo = 0, khi = Lk;
  if (causal) khi = span_count_le(ks, span_pos(qs, wg_q1 - 1));
  if (docs) {
    klo = wave_lower_bound(ks.doc, Lk, qs.doc[wg_q0]);
    int32_t hi2 = wave_lower_bound(ks.doc, Lk, qs.doc[wg_q1 - 1] + 1);
    khi = min(khi, hi2);
  }
  const int32_t kt0 = klo / BK;
  const int32_t kt1 = khi > klo ? (khi + BK - 1) / BK : kt0;

  // ---- this wave's Q rows as MFMA B operands ----------------------------
  bf16x8 qf[2][D / 16];
  int64_t qpos_l[2];
  int32_t qdoc_l[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int32_t row = min(q0 + qb * 32 + lq, Lq - 1);
    const bf16x8* src = (const bf16x8*)(a.q + (int64_t)row * a.q_stride + (int64_t)head * D + hh * 8);
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) qf[qb][kd] = src[kd * 2];
    qpos_l[qb] = span_pos(qs, row);
    qdoc_l[qb] = docs ? qs.doc[row] : 0;
  }

  f32x16 oacc[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  float mrow[2] = {-INFINITY, -INFINITY};   // running max of raw scores
  float lrow[2] = {0.f, 0.f};               // this lane's share of the row sum
  const float c = a.scale_log2;              // scale * log2(e)

  // ---- global -> register staging of one K/V tile -----------------------
  // K: 64 rows x D, 16-byte pieces, row-major into LDS (padded rows).
  // V: each thread takes 4 consecutive keys x 8 dims and writes 8 pieces of
  //    4 keys (8 bytes) into the [key/4][d][4] layout.
  constexpr int KPIECES = BK * D / 8;                 // 16-byte pieces per K tile
  constexpr int KP_PER_T = KPIECES / 256;             // 4 (D=128) or 2 (D=64)
  constexpr int VITEMS = (BK / 4) * (D / 8);          // (4 keys x 8 dims) items
  constexpr int VI_PER_T = (VITEMS + 255) / 256;      // 1
  u32x4 kreg[KP_PER_T];
  u32x4 vreg[VI_PER_T][4];
  int32_t dreg = 0;

  auto load_tile = [&](int32_t kt) {
    const int32_t base = kt * BK;
#pragma unroll
    for (int i = 0; i < KP_PER_T; ++i) {
      int piece = tid + i * 256;
      int key = piece / (D / 8), col = (piece % (D / 8)) * 8;
      int32_t row = min(base + key, Lk - 1);
      kreg[i] = *(const u32x4*)(a.k + (int64_t)row * a.kv_stride + (int64_t)kvh * D + col);
    }
#pragma unroll
    for (int i = 0; i < VI_PER_T; ++i) {
      int item = tid + i * 256;
      if (item < VITEMS) {
        int kg = item / (D / 8), dg = item % (D / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int32_t row = min(base + kg * 4 + r, Lk - 1);
          vreg[i][r] = *(const u32x4*)(a.v + (int64_t)row * a.kv_stride + (int64_t)kvh * D + dg * 8);
        }
      }
    }
    if (docs && tid < BK) dreg = ks.doc[min(base + tid, Lk - 1)];
  };
  auto store_tile = [&](int stage) {
    char* st = smem + stage * L::STAGE;
    __bf16* Ks = (__bf16*)st;
    __bf16* Vs = (__bf16*)(st + L::KBYTES);
    int32_t* Ds = (int32_t*)(st + L::KBYTES + L::VBYTES);
#pragma unroll
    for (int i = 0; i < KP_PER_T; ++i) {
      int piece = tid + i * 256;
      int key = piece / (D / 8), col = (piece % (D / 8)) * 8;
      *(u32x4*)(Ks + key * L::KST + col) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VI_PER_T; ++i) {
      int item = tid + i * 256;
      if (item < VITEMS) {
        int kg = item / (D / 8), dg = item % (D / 8);
#pragma unroll
        for (int m = 0; m < 4; ++m) {        // dword m holds dims 2m, 2m+1
          u32x2 lo, hi;
          lo.x = __builtin_amdgcn_perm(vreg[i][1][m], vreg[i][0][m], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(vreg[i][3][m], vreg[i][2][m], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(vreg[i][1][m], vreg[i][0][m], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(vreg[i][3][m], vreg[i][2][m], 0x07060302u);
          int d0 = dg * 8 + 2 * m;
          *(u32x2*)(Vs + ((kg * D) + d0) * 4) = lo;
          *(u32x2*)(Vs + ((kg * D) + d0 + 1) * 4) = hi;
        }
      }
    }
    if (docs && tid < BK) Ds[tid] = dreg;
  };

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();

  for (int32_t kt = kt0; kt < kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    if (kt + 1 < kt1) load_tile(kt + 1);

    const int32_t kb0 = kt * BK, kb1 = min(Lk, kb0 + BK);
    int cls = wave_live ? block_class(qs, q0, q1, ks, kb0, kb1, causal) : TILE_SKIP;
    if (cls != TILE_SKIP) {
      const char* st = smem + stage * L::STAGE;
      const __bf16* Ks = (const __bf16*)st;
      const __bf16* Vs = (const __bf16*)(st + L::KBYTES);
      const int32_t* Ds = (const int32_t*)(st + L::KBYTES + L::VBYTES);

      // S^T[kb][qb]: keys kb*32.. (rows) x queries qb*32.. (columns)
      f32x16 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < D / 16; ++kd) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 ka = *(const bf16x8*)(Ks + (kb * 32 + lq) * L::KST + kd * 16 + hh * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][kd], s[kb][qb], 0, 0, 0);
        }
      }

      if (cls == TILE_PARTIAL || kb1 - kb0 < BK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int kk = kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
            int32_t kidx = kb0 + kk;
            bool kin = kidx < kb1;
            int64_t kp = span_pos(ks, kidx);
            int32_t kd_ = docs ? Ds[kk] : 0;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              bool ok = kin && (!causal || kp <= qpos_l[qb]) && (!docs || kd_ == qdoc_l[qb]);
              if (!ok) s[kb][qb][r] = -INFINITY;
            }
          }
      }

      // online softmax per query column
      float mx[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m0 = s[0][qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m0 = fmaxf(m0, s[0][qb][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) m0 = fmaxf(m0, s[1][qb][r]);
        m0 = fmaxf(m0, __shfl_xor(m0, 32));
        mx[qb] = fmaxf(mrow[qb], m0);
      }
      const bool grow = (mx[0] > mrow[0]) || (mx[1] > mrow[1]);
      if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float alpha = (mx[qb] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((mrow[qb] - mx[qb]) * c);
          lrow[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
          mrow[qb] = mx[qb];
        }
      }
      bf16x8 pf[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float moff = (mrow[qb] == -INFINITY) ? 0.f : -mrow[qb] * c;
#pragma unroll
        for (int t = 0; t < 4; ++t) pf[qb][t] = cvt8(s[t >> 1][qb], (t & 1) * 8, c, moff, lrow[qb]);
      }

      // O^T[qb][db] += V^T (d rows db*32.., 16 keys per step) x P^T
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = db * 32 + lq;
          u32x2 lo = *(const u32x2*)(Vs + ((4 * t + hh) * D + d) * 4);
          u32x2 hi = *(const u32x2*)(Vs + ((4 * t + 2 + hh) * D + d) * 4);
          u32x4 av = {lo.x, lo.y, hi.x, hi.y};
          bf16x8 va = __builtin_bit_cast(bf16x8, av);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[qb][t], oacc[qb][db], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < kt1) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  if (!wave_live) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = lrow[qb] + __shfl_xor(lrow[qb], 32);
    const int32_t row = q0 + qb * 32 + lq;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (row < Lq) {
      if (hh == 0) {
        float lse = ltot > 0.f ? (mrow[qb] * c + __builtin_amdgcn_logf(ltot)) * LN2 : -INFINITY;
        a.lse[(int64_t)head * a.lse_ld + row] = lse;
      }
      const int64_t obase = ((int64_t)row * a.hq + head) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + j * 8 + hh * 4;
          f32x4 v4 = {oacc[qb][db][4 * j] * inv, oacc[qb][db][4 * j + 1] * inv,
                      oacc[qb][db][4 * j + 2] * inv, oacc[qb][db][4 * j + 3] * inv};
          if (a.o_f32) {
            *(f32x4*)((float*)a.o + obase + d) = v4;
          } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 b4 = {(__bf16)v4[0], (__bf16)v4[1], (__bf16)v4[2], (__bf16)v4[3]};
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
  a.qblocks_per_wg = 4 / a.heads_per_wg;
  a.nqt = (Lq + QW * a.qblocks_per_wg - 1) / (QW * a.qblocks_per_wg);
  a.scale_log2 = a.scale * LOG2E;
  const int32_t ngroups = a.hq / a.heads_per_wg;
  a.n_work = a.nqt * ngroups;
  if (a.n_work == 0) return hipSuccess;
  const int32_t grid = round_up8(a.n_work);
  if (a.d == 128) {
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cp
