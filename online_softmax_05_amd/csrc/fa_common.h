// Device-side helpers shared by the attention kernels (gfx950 only).
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//   [OA] "Reducing Memory Traffic with Output Accumulation in FlashAttention"
//
// All softmax arithmetic runs in the base-2 domain: a logit s is carried as
// t = s * log2(e), so exp(s - m) = exp2(t - m2) maps onto the hardware
// v_exp_f32, and lse = ln(2) * (m2 + log2(l)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) {
  // v_exp_f32; exp2(-inf) = 0, which is how masked logits drop out
  // ([VW] Step 7: a masked score contributes nothing).
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value held by the lane 32 positions away (lane ^ 32), combined with `op`:
// v_permlane32_swap returns {[lo, lo], [hi, hi]} for an input [lo, hi].
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// bf16 <-> f32 (round to nearest even on the way down: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Sum of the two bf16 values packed in w, added to acc in fp32
// (v_dot2c_f32_bf16 against the pair (1, 1): both products are exact).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Work-group -> (batch*head, tile) mapping: query tiles in the forward and
// dQ kernels, key tiles in the dK/dV kernel.
//
// Work-groups are handed to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2.  Renumbering so that XCD x works through a contiguous range of
// logical tiles keeps the tiles of a few (batch, head) blocks -- which re-read
// the same K/V (or Q/dO) -- on one L2.  Within the range the (batch, head)
// blocks go in pairs, the two blocks' tiles alternating, and with heavy_first
// each block's tiles come in descending order (heaviest first when a causal
// mask makes later query tiles longer).  Issuing one block's tiles after the
// other instead left the heaviest tiles of the range's last blocks starting
// when the rest were nearly done: a list-scheduling model of the causal
// 4x32x4096 prefill puts that tail at 10.6% of the launch, and pairs remove
// it while fewer blocks are in flight at once (at most 4 instead of 6).
// Groups of 4 blocks balance the measured launch further where a block's K/V
// is small and many blocks share an XCD (tile_group); where a block's K/V is
// large (long sequences) grouping only multiplies the HBM reads and blocks
// go one at a time.
struct TileCoord {
  int bh;
  int qt;
};
__device__ __forceinline__ int xcd_renumber(int pid, int total) {
  return (total & 7) == 0 ? (pid & 7) * (total >> 3) + (pid >> 3) : pid;
}
__device__ __forceinline__ TileCoord map_tile(int pid, int total, int n_qt, bool heavy_first, int group = 2) {
  const int lid = xcd_renumber(pid, total);
  const int n_bh = total / n_qt;
  const int gi = lid / (group * n_qt);  // group of blocks group*gi .. +group-1
  int r = lid - gi * group * n_qt;
  const int gsz = min(group, n_bh - gi * group);  // the last group may be smaller
  TileCoord c;
  c.bh = gi * group + r % gsz;
  r /= gsz;
  c.qt = heavy_first ? (n_qt - 1 - r) : r;
  return c;
}

// Group size for map_tile: 4 blocks when tile work grows along the tile
// axis (growing: a causal mask without a left window), at least 64 blocks
// share the launch (8 or more per XCD) and a block's K and V take at most
// 2 MiB; pairs for other blocks of at most 2 MiB; one block at a time above
// that.  Measured on the causal bf16 prefill 4x32x4096 (K and V 2 MiB per
// head): groups of 4 1.5% faster than pairs, dropout 3.7%.  Long context
// 1x16x16384 (8 MiB per head): groups of 4 30% slower than pairs, and pairs
// as fast as one block at a time but with twice the HBM reads (each block's
// K/V swept by half as many tiles at once).
__host__ __device__ __forceinline__ int tile_group(bool growing, int n_bh, long long kv_bytes) {
  if (kv_bytes > (2ll << 20)) return 1;
  return (growing && n_bh >= 64) ? 4 : 2;
}

// Division of x < 2^31 by a launch constant d >= 1 without a divide:
// floor(x / d) = floor(x * m / 2^s) with s = 31 + ceil(log2 d) and
// m = ceil(2^s / d) < 2^32, exact because m*d - 2^s < d <= 2^(s - 31)
// (the round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994).
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  return FastDiv{(uint32_t)(((1ull << (31 + l)) + d - 1) / d), 31 + l};
}
__device__ __forceinline__ int fast_div(int x, FastDiv d) { return (int)(((uint64_t)(uint32_t)x * d.m) >> d.s); }

// Four consecutive fp32 bias values of one row starting at key0, zero past
// nk or for an invalid row; vec: the row is 16-byte aligned and nk % 4 == 0.
__device__ __forceinline__ f32x4 load_bias4(const float* brow, int key0, int nk, bool vec, bool valid) {
  f32x4 w = {0.f, 0.f, 0.f, 0.f};
  if (!valid) return w;
  if (vec && key0 + 3 < nk) return *reinterpret_cast<const f32x4*>(brow + key0);
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = (key0 + j < nk) ? brow[key0 + j] : 0.f;
  return w;
}

__device__ __forceinline__ int clamp_klen(const int32_t* k_len, int b, int nk) {
  if (k_len == nullptr) return nk;
  int x = k_len[b];
  return x < 0 ? 0 : (x > nk ? nk : x);
}

}  // namespace fa
