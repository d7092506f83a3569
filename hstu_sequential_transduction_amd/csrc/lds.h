// Row-major bf16 tiles in LDS, filled by buffer->LDS DMA and read as MFMA
// operands either along rows (ds_read_b128) or down columns (the gfx950
// transpose read ds_read_b64_tr_b16), so no tile is ever stored transposed.
#pragma once

#include "common.h"

#define HSTU_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Tile rows hold D bf16 (2D bytes, no padding).  The 16-byte chunks of row r
// are XOR-permuted by swz(r), chosen so that
//  * 16 consecutive rows (aligned to 16) read at one logical chunk (one MFMA
//    operand row per lane, 16 lanes per 256-byte LDS cycle) land on 16
//    distinct 16-byte bank groups;
//  * 4 consecutive rows (aligned to 4) x one 64-byte piece (four chunks
//    aligned to four), what 32 lanes of a transpose read touch in one
//    cycle, land on four distinct 64-byte bank groups (so do the 32-byte
//    pieces of each 16-lane half).
// For D = 128 the row's chunk group of four is picked by r & 3 and the chunk
// within it by (r >> 2) & 3; for D = 64 (two rows per 256 bytes) the group
// by the row's parity and bit 0 of q = (r >> 1) & 7, the chunk by q >> 1.
template <int D>
struct SwzTile {
  static_assert(D == 32 || D == 64 || D == 128, "tile width");
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  HSTU_DEV static int swz(int r) {
    if constexpr (D == 128) {
      return ((r & 3) << 2) | ((r >> 2) & 3);
    } else if constexpr (D == 64) {
      const int q = (r >> 1) & 7;
      return ((q & 1) << 2) | (q >> 1);
    } else {
      return (r >> 2) & 3;
    }
  }
  // byte offset of logical 16-byte chunk c of row r
  HSTU_DEV static int off(int r, int c) { return r * ROW_BYTES + ((c ^ swz(r)) << 4); }
  static constexpr int bytes(int rows) { return rows * ROW_BYTES; }
};

// Operand whose M (or N) index runs along the lanes: row `row`, the eight
// columns [16 ch + 8 g, +8) that lane group g = lane/32 supplies to k-step ch.
template <int D>
HSTU_DEV bf16x8 lds_row8(const uint8_t* t, int row, int ch, int g) {
  return *reinterpret_cast<const bf16x8*>(t + SwzTile<D>::off(row, 2 * ch + g));
}

// B operand of a 32x32x16 MFMA whose k index runs down the tile rows: lane l
// takes column n0 + l%32 at rows k0 + 4g + {0..3} and k0 + 8 + 4g + {0..3}
// (g = l/32), the order in which a 32x32 accumulator reused as A operand
// holds its rows.  A transpose read hands lane 4a+c of each 16-lane group
// element c of the 8-byte pieces addressed by lanes a, a+4, a+8 and a+12 of
// that group, so source lane j addresses row k0 + 4g + j/4 (+8 for the upper
// half) at columns n0 + 16 (group & 1) + 4 (j & 3) .. +3.
template <int D>
HSTU_DEV bf16x8 lds_col8(const uint8_t* t, int k0, int n0, int lane) {
  const int j = lane & 15;
  const int r = k0 + 4 * (lane >> 5) + (j >> 2);
  const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int cb = (col & 7) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (HSTU_LDS bf16x4*)(t + SwzTile<D>::off(r, col >> 3) + cb));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (HSTU_LDS bf16x4*)(t + SwzTile<D>::off(r + 8, col >> 3) + cb));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Same, with the eight k rows in natural order k0 + 8g + {0..7}, for products
// whose other operand is read along rows with lds_row8.
template <int D>
HSTU_DEV bf16x8 lds_col8_nat(const uint8_t* t, int k0, int n0, int lane) {
  const int j = lane & 15;
  const int r = k0 + 8 * (lane >> 5) + (j >> 2);
  const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int cb = (col & 7) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (HSTU_LDS bf16x4*)(t + SwzTile<D>::off(r, col >> 3) + cb));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (HSTU_LDS bf16x4*)(t + SwzTile<D>::off(r + 4, col >> 3) + cb));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-major bf16 tile of D columns whose rows are padded to STRIDE bytes, so
// that neither read form needs a per-lane swizzle: every operand address is
// one per-lane base plus a compile-time offset.  With rows 16 * odd bytes apart
// (modulo the 256-byte bank cycle), 16 consecutive rows at one 16-byte chunk
// fall on 16 distinct bank groups (row reads); for tiles also read down columns
// (TR) the stride is chosen so that 4 consecutive rows x one 32-byte piece, what
// a 16-lane group of a transpose read touches, fall on distinct banks as well.
template <int D, bool TR>
struct PadTile {
  static_assert(D == 32 || D == 64 || D == 128, "tile width");
  static constexpr int STRIDE = D == 128 ? (TR ? 304 : 272) : D == 64 ? 144 : (TR ? 112 : 80);
  static constexpr int SPR = STRIDE / 16;  // 16-byte slots per row
  static constexpr int CPR = D / 8;        // of which hold data
  // whole KiB: the last DMA instruction fills a full KiB
  static constexpr int bytes(int rows) { return (rows * STRIDE + 1023) / 1024 * 1024; }
  HSTU_DEV static int off(int r, int c) { return r * STRIDE + c * 16; }
};

// PadTile operand reads: the same lane layouts as lds_row8 / lds_col8 /
// lds_col8_nat above.
template <int D, bool TR>
HSTU_DEV bf16x8 pad_row8(const uint8_t* t, int row, int ch, int g) {
  return *reinterpret_cast<const bf16x8*>(t + PadTile<D, TR>::off(row, 2 * ch + g));
}
template <int D>
HSTU_DEV bf16x8 pad_col8(const uint8_t* t, int k0, int n0, int lane) {
  constexpr int S = PadTile<D, true>::STRIDE;
  const int j = lane & 15;
  const int r = k0 + 4 * (lane >> 5) + (j >> 2);
  const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const uint8_t* p = t + r * S + col * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HSTU_LDS bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HSTU_LDS bf16x4*)(p + 8 * S));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int D>
HSTU_DEV bf16x8 pad_col8_nat(const uint8_t* t, int k0, int n0, int lane) {
  constexpr int S = PadTile<D, true>::STRIDE;
  const int j = lane & 15;
  const int r = k0 + 8 * (lane >> 5) + (j >> 2);
  const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const uint8_t* p = t + r * S + col * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HSTU_LDS bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((HSTU_LDS bf16x4*)(p + 4 * S));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Buffer resource over `bytes` bytes from `base` (word 3 of the gfx9 format:
// 32-bit raw addressing); loads at offsets past the range return zero.  The
// arguments must be wave-uniform; they are moved to scalar registers
// explicitly so that the descriptor never needs a per-lane loop.
HSTU_DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* sp = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(sp, 0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Start copying rows [r0, r0 + R) of a row-major bf16 matrix (row stride ld
// elements, D columns from `base`) into SwzTile<D> `t`; rows >= rlim arrive
// as zeros.  NW waves share the work.  One wave instruction fills 1 KiB of the
// tile, lane l's 16 bytes landing at byte 16 l, so each lane fetches the
// global chunk that the swizzle puts there.  Completion: dma_wait().
// `last_cols` (default: the whole row stride) bounds how many elements of the
// last valid row may be touched, so that a tile reaching past the right edge
// of a matrix never reads past the end of its allocation.  AUX is the loads'
// cache policy (0: default; 2: non-temporal, for data read exactly once, so
// that it does not push reused tiles out of the L2).
template <int D, int R, int NW, int AUX = 0>
HSTU_DEV void dma_tile(uint8_t* t, const bf16* base, int64_t ld, int r0, int rlim, int wave,
                       int lane, int last_cols = -1) {
  constexpr int NI = R * D * 2 / 1024;
  static_assert(NI * 1024 == R * D * 2, "tile must be a whole number of KiB");
  const int nrows = max(0, min(rlim - r0, R));
  const int lc_el = last_cols < 0 ? (int)ld : last_cols;
  const int nbytes = nrows > 0 ? ((nrows - 1) * (int)ld + lc_el) * 2 : 0;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(base + (int64_t)r0 * ld, nbytes);
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NW) {
    const int i = i0 + wave;
    if (NI % NW == 0 || i < NI) {
      const int p = i * 1024 + lane * 16;
      const int row = p / (2 * D);
      const int lc = ((p % (2 * D)) >> 4) ^ SwzTile<D>::swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (HSTU_LDS void*)(t + i * 1024), 16,
                                               row * (int)ld * 2 + lc * 16, 0, 0, AUX);
    }
  }
}

// dma_tile for a PadTile: slot s = 64 i + lane of wave instruction i lands at
// byte 16 s, i.e. row s / SPR, chunk s % SPR.  Padding slots (never read) are
// pointed past the buffer range, which returns zeros without a memory access.
template <int D, bool TR, int R, int NW>
HSTU_DEV void dma_pad_tile(uint8_t* t, const bf16* base, int64_t ld, int r0, int rlim, int wave,
                           int lane, int last_cols = -1) {
  using P = PadTile<D, TR>;
  constexpr int NI = P::bytes(R) / 1024;
  const int nrows = max(0, min(rlim - r0, R));
  const int lc_el = last_cols < 0 ? (int)ld : last_cols;
  const int nbytes = nrows > 0 ? ((nrows - 1) * (int)ld + lc_el) * 2 : 0;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(base + (int64_t)r0 * ld, nbytes);
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NW) {
    const int i = i0 + wave;
    if (NI % NW == 0 || i < NI) {
      const int sl = i * 64 + lane;
      const int row = sl / P::SPR;
      const int c = sl - row * P::SPR;
      const int off = c < P::CPR ? row * (int)ld * 2 + c * 16 : 0x7FFFFFF0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (HSTU_LDS void*)(t + i * 1024), 16, off, 0,
                                               0, 0);
    }
  }
}

// Start copying elements [r0, r0 + 64) of a 4-byte array (one wave); entries
// at or past rlim arrive as zeros.
HSTU_DEV void dma_words64(void* t, const void* base, int r0, int rlim, int lane) {
  const int nel = max(0, min(rlim - r0, 64));
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(reinterpret_cast<const uint32_t*>(base) + r0, nel * 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (HSTU_LDS void*)t, 4, lane * 4, 0, 0, 0);
}
// Same for an 8-byte array (two wave instructions).
HSTU_DEV void dma_dwords64(void* t, const void* base, int r0, int rlim, int lane) {
  const int nel = max(0, min(rlim - r0, 64));
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(reinterpret_cast<const uint64_t*>(base) + r0, nel * 8);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (HSTU_LDS void*)t, 4, lane * 4, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (HSTU_LDS void*)((uint8_t*)t + 256), 4,
                                           256 + lane * 4, 0, 0, 0);
}

// Wait for this wave's outstanding DMA (vmcnt(0); expcnt, lgkmcnt untouched).
HSTU_DEV void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }
