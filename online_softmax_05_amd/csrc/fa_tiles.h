// LDS tile machinery shared by the matrix-core kernels of the backward and
// the multi-query split-KV decode (gfx950): 64-row bf16 tiles loaded straight
// into LDS with a bank-spreading chunk swizzle, operand reads and transposed
// reads.  Kernels that include it live in an anonymous namespace of their own
// translation unit.
#pragma once

#include "fa_common.h"

namespace fa {
namespace tiles {

constexpr int kWaves = 4;
constexpr int kTile = 64;  // rows of every LDS tile (keys or queries)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS tile of kTile rows x D bf16, row-major, 16-byte chunk c of row r stored
// at chunk position c ^ swz(r % 8).  The swizzle was chosen by measuring LDS
// bank-conflict cycles: with it both the 128-bit operand reads (frag) and the
// transposed reads (tr) run conflict-free, 4 and 2 LDS cycles per
// instruction.  (Spreading the 16 rows of an operand read over 16 distinct
// 16-byte positions of a 256-byte bank period, an earlier choice, left half
// the operand-read cycles in conflicts.)
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 7) << 1) | ((row >> 2) & 1);
  return row & 7;
}

// W: the waves that load a tile together (kWaves unless a kernel says
// otherwise)
template <int D, int W = kWaves>
struct Tile {
  static constexpr int R = D / 8;   // 16-byte chunks per row
  static constexpr int ROW = R * 16;
  static constexpr int BYTES = kTile * ROW;
  static constexpr int IPW = kTile * R / 64 / W;  // 1 KiB direct loads per wave
  static_assert(IPW >= 1 && kTile * R % (64 * W) == 0, "tile shape");
};

// Per-lane address parts for one tile layout D.
template <int D, int W = kWaves>
struct TileAddr {
  int frag[D / 32];  // operand read (tile row 16blk + r16, dims 32t + 8g .. +7): + 16 blk ROW
  int tr[D / 16];    // transposed read of dim block db (tile rows 32kt + 16h + 4g + e): + (32kt + 16h) ROW
  int ld[Tile<D, W>::IPW];  // byte offset in the tile of each of this wave's direct loads

  __device__ __forceinline__ void init(int lane, int wave) {
    constexpr int ROW = Tile<D>::ROW;
    const int r16 = lane & 15, g = lane >> 4, e = (lane >> 2) & 3, r = lane & 3;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) frag[t] = r16 * ROW + 16 * ((4 * t + g) ^ swz<D>(r16));
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      tr[db] = (4 * g + e) * ROW + 16 * ((2 * db + (r >> 1)) ^ swz<D>(4 * g + e)) + 8 * (r & 1);
#pragma unroll
    for (int i = 0; i < Tile<D, W>::IPW; ++i) {
      const int slot = (wave * Tile<D, W>::IPW + i) * 64 + lane;
      const int row = slot / Tile<D>::R;
      ld[i] = 2 * (row * D + ((slot % Tile<D>::R) ^ swz<D>(row)) * 8);
    }
  }
};

// One head's rows of a tensor: base address and byte size, turned into a
// buffer resource at each load so that the hardware range check covers the
// head.  The byte size must fit in 31 bits (the callers' eligibility checks
// say so).
struct HeadBuf {
  const uint16_t* base;
  uint32_t bytes;
};
__device__ __forceinline__ HeadBuf head_buf(const uint16_t* base, uint32_t bytes) { return HeadBuf{base, bytes}; }

// Direct-to-LDS load (buffer_load_dwordx4 ... lds) of this wave's share of
// the tile whose first row is row0: one uniform byte offset per tile plus
// each lane's fixed offset (ld = TileAddr<D>::ld), no per-load address
// arithmetic.  Lanes past the
// end of the head fail the range check and write zeros (those rows are
// masked; zero rows add nothing to the products).  CPOL is the cache policy:
// 0, or kNonTemporal for data read once per call.
constexpr int kNonTemporal = 2;
template <int D, int CPOL = 0, int W = kWaves>
__device__ __forceinline__ void load_tile(const HeadBuf& b, int row0, const int* ld, lds_char* dst, int wave) {
  constexpr int IPW = Tile<D, W>::IPW;
#pragma unroll
  for (int i = 0; i < IPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)b.base, (short)0, (int)b.bytes, 0x00020000),
        (lds_void*)(dst + (wave * IPW + i) * 1024), 16, ld[i], row0 * D * 2, 0, CPOL);
}

// Largest tensor rows * D for which a head's bytes fit the buffer range.
__host__ __device__ constexpr bool head_fits(long long rows, int d) { return rows * d * 2 <= 0x7fffffffLL; }

__device__ __forceinline__ bf16x8 frag_read(const lds_char* p) { return *(const lds_bf16x8*)p; }

__device__ __forceinline__ bf16x8 tr_read(const lds_char* p, int row_bytes16) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + row_bytes16));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


}  // namespace tiles
}  // namespace fa
