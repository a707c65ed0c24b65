// LDS tile staging shared by the bf16 MFMA kernels (gfx950).
//
// A tile of R rows x D bf16 (row-major in HBM, `stride` elements between
// rows) is copied HBM -> LDS with direct-to-LDS loads (buffer_load ... lds,
// 16 bytes per lane; no VGPR round trip).  The LDS image keeps rows whole but
// permutes each row's 16-byte chunks by an XOR swizzle so that both access
// patterns the MFMA operands need are free of bank conflicts:
//   * row reads: 16 lanes each read one 16-byte chunk of 16 consecutive rows
//     (ds_read_b128, operand with the contraction along d);
//   * transposed reads: ds_read_b64_tr_b16, 32 lanes covering 4 consecutive
//     rows (aligned to 4) x 4 consecutive chunks (operand with the
//     contraction along rows).
// For d = 128 a row is 256 bytes, one full sweep of the 64 LDS banks, so the
// bank group (16 bytes) of chunk c of row r is its position c ^ f(r) with
// f(r) = 4 (r mod 4) + (r / 4 mod 4): a permutation of 0..15 over any 16
// aligned rows (row reads), and 4 (b ^ i) + (j ^ a) over rows 4a + i,
// chunks 4b + j (transposed reads) -- 16 distinct groups in both cases.
//
// ds_read_b64_tr_b16 (measured on gfx950): within each 16-lane group, if
// source lane s reads the 4 consecutive elements M[s][0..3] at its address,
// destination lane i receives M[4j + i/4][i%4] as element j (j = 0..3).  So
// when lane s of a group addresses row r0 + s/4, columns c0 + 4(s%4) .. +3,
// lane i receives column c0 + i of rows r0 .. r0 + 3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define CP_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define CP_LDS_AT(a) ((__attribute__((address_space(3))) void*)(uintptr_t)(a))

template <int D>
struct Swz {
  static constexpr int CHUNKS = D / 8;              // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  // chunk position of chunk c in row r
  __device__ static inline int pos(int r, int c) {
    if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((r >> 1) & 7);
  }
  // byte offset of element (r, col) for an 8-byte aligned col group
  __device__ static inline int off(int r, int col) {
    return r * ROW_BYTES + pos(r, col >> 3) * 16 + (col & 4) * 2;
  }
};

// Direct-to-LDS loads are buffer loads (buffer_load ... lds) through a raw
// buffer resource on a wave-uniform base, with a per-lane byte offset.  They
// are written as inline asm, so the compiler does not track them: it treats
// a tracked LDS DMA as a possible writer of any LDS that an LDS transpose read
// (ds_read_b64_tr_b16) touches, and waits for every load in flight
// (s_waitcnt vmcnt(0)) before the first such read after it, which stalls a
// wave mid-tile on the next tile's copy.  Every kernel here reads a copied
// tile only after its own s_waitcnt vmcnt(0) and a work-group barrier, which
// is what makes the copy visible; the asm has no output register (the data
// goes to LDS at M0 + 16 lane), and loads complete in issue order, so the
// compiler's own vmcnt waits for its tracked loads stay correct (an untracked
// load in flight only makes them wait longer).  The compiler's hazard checks
// do not look inside inline asm, so the asm brings its own wait states: the
// s_nop 4 covers the 5 that a VMEM instruction needs after a VALU write of an
// SGPR it reads (the resource descriptor may have just been reloaded from a
// spill lane with v_readlane) and the 1 that an LDS DMA needs after M0 is
// written.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// 16 bytes per lane at base + voff into LDS [lds + 16 lane, +16)
__device__ inline void buf_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
// One 4-byte element per lane: element `idx` of the array at `base` into LDS
// [lds + 4 lane, +4).
__device__ inline void row_load_lds(const void* base, int32_t idx, uint32_t lds) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"((uint32_t)idx * 4u), "s"(buf_rsrc(base)),
               "{m0}"(lds) : "memory");
}

// 64 consecutive 4-byte elements (256 bytes) at base + 4 idx0 into LDS
// [lds, +256): lanes 0..15 load 16 bytes each, the rest of the wave is masked
// off.  One instruction like row_load_lds, but a quarter of the lane-elements
// for the LDS DMA to write.  All 64 elements must be in bounds.
__device__ inline void row64_load_lds(const void* base, int32_t idx0, uint32_t lds, int lane) {
  if (lane < 16)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"((uint32_t)idx0 * 4u + (uint32_t)lane * 16u),
                 "s"(buf_rsrc(base)), "{m0}"(lds) : "memory");
}

// Issue the direct-to-LDS loads of an R x D tile at LDS address `dst` whose
// row i sits at src + i * stride (rows past `valid_rows` are clamped to
// valid_rows - 1, so every load is in bounds; callers mask those rows).  NW
// waves share the work; wave `wave` issues its share.
template <int D, int R, int NW>
__device__ inline void tile_load_lds(uint32_t dst, const __bf16* src, int64_t stride, int32_t row0,
                                     int32_t valid_rows, int wave, int lane) {
  constexpr int CHUNKS = D / 8;
  constexpr int TOTAL = R * CHUNKS;
  constexpr int PER_WAVE = TOTAL / (64 * NW);
  static_assert(TOTAL % (64 * NW) == 0, "tile must split evenly over the waves");
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src + (int64_t)row0 * stride);
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int slot0 = (wave * PER_WAVE + i) * 64;
    const int slot = slot0 + lane;
    const int r = slot / CHUNKS;
    const int cpos = slot % CHUNKS;
    int c = cpos;
    if constexpr (D == 128) c = cpos ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else c = cpos ^ ((r >> 1) & 7);
    int32_t row = row0 + r;
    row = row < valid_rows ? row : valid_rows - 1;
    buf_lds16(rs, dst + slot0 * 16, (uint32_t)((row - row0) * stride * 2 + c * 16));
  }
}

// Loads of R x D tiles whose rows are `stride_b` bytes apart, for wave
// `wave` of NW, with the per-lane byte offsets (row * stride + swizzled
// chunk) computed once: a tile's loads then cost one 64-bit add each.  Rows
// must all be valid (row0 + R <= valid rows); the ragged last tile goes
// through tile_load_lds, which clamps.
template <int D, int R, int NW>
struct TileLoader {
  static constexpr int CHUNKS = D / 8;
  static constexpr int PER_WAVE = R * CHUNKS / (64 * NW);
  static_assert(R * CHUNKS % (64 * NW) == 0, "tile must split evenly over the waves");
  uint32_t off[PER_WAVE];
  int wave;
  __device__ TileLoader(int64_t stride_b, int wave_uniform, int lane) : wave(wave_uniform) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int slot = (wave * PER_WAVE + i) * 64 + lane;
      const int r = slot / CHUNKS, cpos = slot % CHUNKS;
      int c;
      if constexpr (D == 128) c = cpos ^ (((r & 3) << 2) | ((r >> 2) & 3));
      else c = cpos ^ ((r >> 1) & 7);
      off[i] = (uint32_t)(r * stride_b + c * 16);
    }
  }
  // tile rows start at byte address `src` (wave-uniform); LDS tile at `dst`
  __device__ inline void load(uint32_t dst, const char* src) const {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) buf_lds16(rs, dst + (uint32_t)((wave * PER_WAVE + i) * 1024), off[i]);
  }
};

// Row read: 8 consecutive elements (16 bytes) of row r starting at column col
// (a multiple of 8).
template <int D>
__device__ inline bf16x8 lds_row8(const char* base, int r, int col) {
  return *(const bf16x8*)(base + r * Swz<D>::ROW_BYTES + Swz<D>::pos(r, col >> 3) * 16);
}

// Transposed read for a 16-lane group: this lane (s = lane % 16) addresses
// row r0 + s/4, columns c0 + 4(s%4); the lane i of the group receives
// column c0 + i of rows r0..r0+3.  r0 must be a multiple of 4, c0 of 16.
template <int D>
__device__ inline bf16x4 lds_tr4(const char* base, int r0, int c0, int s) {
  const int r = r0 + (s >> 2);
  const int col = c0 + 4 * (s & 3);
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + Swz<D>::off(r, col)));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- reads at 32-bit LDS addresses -----------------------------------------
// Kernels keep their tiles in one LDS arena and address them with uint32_t
// LDS addresses, so that a tile's base, a 32-row block and a 16-row step are
// compile-time constants the compiler folds into the instruction's offset
// field; only the swizzled lane part lives in VGPRs.  With the swizzle f(r)
// the lane part of every read is a fixed per-lane value XOR a small constant:
//   row read of row rb*32 + lq, chunk 2kd + hh:
//     rb*32*RB + (base ^ (kd << 5)),  base = lq*RB + ((hh ^ f(lq)) << 4)
//   transposed read of rows R + 8e + 4hh + s/4 (R a multiple of 16), columns
//   db*32 + 16cg + 4(s%4):
//     R*RB + (base_e ^ (db << 6))
// (RB = 2D bytes per row; f depends on r mod 16 only, and the XORed bits
// never overlap the row part.)
typedef __attribute__((address_space(3))) char lds_char;

__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_char*)p; }

__device__ inline bf16x8 lds_ld16(uint32_t a) { return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)a; }
__device__ inline u32x4 lds_ld16u(uint32_t a) { return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a; }
__device__ inline int32_t lds_ld4i(uint32_t a) { return *(const __attribute__((address_space(3))) int32_t*)(uintptr_t)a; }

template <int D>
__device__ inline int swz_f(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

// Row reads (operand with the contraction along d) of a [rows x D] tile.
template <int D>
struct RowReader {
  uint32_t base;
  __device__ explicit RowReader(int lane) {
    const int lq = lane & 31, hh = lane >> 5;
    base = (uint32_t)(lq * 2 * D + ((hh ^ swz_f<D>(lq)) << 4));
  }
  // 8 elements of row rb*32 + lq, columns kd*16 + 8hh .. +7
  __device__ inline bf16x8 at(uint32_t tile, int rb, int kd) const {
    return lds_ld16(tile + (uint32_t)(rb * 32 * 2 * D) + (base ^ (uint32_t)(kd << 5)));
  }
};

// Transposed reads (operand with the contraction along rows): for 16 rows
// R .. R+15 (R a multiple of 16) and the 32 columns of d block db, lane
// (s = lane % 16, cg = lane / 16 % 2, hh = lane / 32) receives column
// db*32 + 16cg + s of rows R + 4hh .. +3 (elements 0..3) and R + 8 + 4hh .. +3
// (elements 4..7): the A operand of a 32x32x16 MFMA whose K index runs over
// those 16 rows.
template <int D>
struct TrReader {
  uint32_t b0, b1;
  __device__ explicit TrReader(int lane) {
    const int s = lane & 15, cg = (lane >> 4) & 1, hh = lane >> 5;
    const int c0 = 16 * cg + 4 * (s & 3);
    const int r0 = 4 * hh + (s >> 2), r1 = 8 + r0;
    b0 = (uint32_t)(r0 * 2 * D + (((c0 >> 3) ^ swz_f<D>(r0)) << 4) + ((c0 & 4) << 1));
    b1 = (uint32_t)(r1 * 2 * D + (((c0 >> 3) ^ swz_f<D>(r1)) << 4) + ((c0 & 4) << 1));
  }
  __device__ inline bf16x8 at(uint32_t tile, int R, int db) const {
    const uint32_t t = tile + (uint32_t)(R * 2 * D);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(uintptr_t)(t + (b0 ^ (uint32_t)(db << 6))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(uintptr_t)(t + (b1 ^ (uint32_t)(db << 6))));
    return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
  }
};

// The same reads with every lane part precomputed once (one register per d
// step or d block) and kept opaque to the compiler, which would otherwise
// recompute the XORs in every tile of a loop whose registers are tight.
// `off` is added to every lane part (a tile region's start, so that the
// offsets left to the instruction stay below its 64 KiB field).
template <int D>
struct RowLanes {
  uint32_t a[D / 16];
  __device__ RowLanes(const RowReader<D>& r, uint32_t off) {
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd) {
      a[kd] = (r.base ^ (uint32_t)(kd << 5)) + off;
      asm volatile("" : "+v"(a[kd]));
    }
  }
  __device__ inline bf16x8 at(uint32_t tile, int rb, int kd) const {
    return lds_ld16(tile + (uint32_t)(rb * 32 * 2 * D) + a[kd]);
  }
};

template <int D>
struct TrLanes {
  uint32_t a0[D / 32], a1[D / 32];
  __device__ TrLanes(const TrReader<D>& r, uint32_t off) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      a0[db] = (r.b0 ^ (uint32_t)(db << 6)) + off;
      a1[db] = (r.b1 ^ (uint32_t)(db << 6)) + off;
      asm volatile("" : "+v"(a0[db]), "+v"(a1[db]));
    }
  }
  __device__ inline bf16x8 at(uint32_t tile, int R, int db) const {
    const uint32_t t = tile + (uint32_t)(R * 2 * D);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(t + a0[db]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)(t + a1[db]));
    return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
  }
};

// Pin values in place: an empty asm that reads them, so the compiler cannot
// sink their computation into a later block (which would undo an
// interleaving above it).
template <int A, int B>
__device__ inline void keep_live(const bf16x8 (&p)[A][B]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, p[a][b])));
}
template <int A>
__device__ inline void keep_live(const bf16x8 (&p)[A]) {
#pragma unroll
  for (int a = 0; a < A; ++a) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, p[a])));
}

}  // namespace cp
