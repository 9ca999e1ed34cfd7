// Dropout of attention probabilities with a counter-based random mask
// ([GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?",
// section 6: a training backward has to reproduce the forward's mask and
// scaling exactly).  The bits of element (b, h, i, j) are a pure function of
// the seed and the coordinates, so neither pass stores the mask.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011).  Ten rounds on a 4-word counter
// with a 2-word key; a round forms the 64-bit products of counter words 0 and
// 2 with two odd constants and recombines their halves with words 1, 3 and
// the key; the key advances by two Weyl increments between rounds.
//
// Mask layout (stated in include/fa.h): key = (seed lo, seed hi), counter =
// (i, j / 64, b*H + h, (j / 4) % 4); key index j uses byte j % 4 of output
// word (j / 16) % 4, and the element is kept iff that byte < keep_256.  A
// lane that owns the 16 keys 64t + 16kb + 4g + jj (kb, jj = 0..3) of one row
// -- the layout of the 16x16 accumulators -- needs exactly one call per
// 64-key tile: word kb, byte jj.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Philox4 {
  uint32_t x[4];
};

// BITOP3: each round's two three-way xors as one v_bitop3_b32 each (fewer
// instructions); false keeps two v_xor_b32 each, which a kernel at its
// register limit may schedule with fewer live values.
template <bool BITOP3 = true>
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t pa = (uint64_t)kMulA * c0;  // one v_mad_u64_u32 each
    const uint64_t pb = (uint64_t)kMulB * c2;
    uint32_t n0, n2;
    if (BITOP3) {  // truth table 0x96: a ^ b ^ c
      n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(pb >> 32), c1, k0, 0x96);
      n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(pa >> 32), c3, k1, 0x96);
    } else {
      n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
      n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
    }
    c1 = (uint32_t)pb;
    c3 = (uint32_t)pa;
    c0 = n0;
    c2 = n2;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  Philox4 out;
  out.x[0] = c0;
  out.x[1] = c1;
  out.x[2] = c2;
  out.x[3] = c3;
  return out;
}

// Dropout parameters as the kernels take them.  keep == 256 means no dropout.
struct DropoutSpec {
  uint32_t seed_lo, seed_hi;
  int keep;  // keep_256: number of byte values kept, 1..256
};

// The four random words of (row i, 64-key tile t, group g) of head bh.
template <bool BITOP3 = true>
__device__ __forceinline__ Philox4 dropout_words(const DropoutSpec& d, int i, int t, uint32_t bh, int g) {
  return philox4x32_10<BITOP3>((uint32_t)i, (uint32_t)t, bh, (uint32_t)g, d.seed_lo, d.seed_hi);
}

// Word w (0..3, any runtime value) of a generator output, without indexing
// a register array at run time.
__device__ __forceinline__ uint32_t philox_word(const Philox4& r, int w) {
  const uint32_t lo = (w & 1) ? r.x[1] : r.x[0];
  const uint32_t hi = (w & 1) ? r.x[3] : r.x[2];
  return (w & 2) ? hi : lo;
}

// Whether byte `jj` of word `w` keeps its element.
__device__ __forceinline__ bool dropout_keep(uint32_t w, int jj, int keep) {
  return (int)((w >> (8 * jj)) & 0xffu) < keep;
}

// Random byte of element (i, j) of head bh, straight from the layout (one
// generator call per element: for kernels whose lanes hold other patterns).
__device__ __forceinline__ bool dropout_keep_at(const DropoutSpec& d, int i, int j, uint32_t bh) {
  const Philox4 r = dropout_words(d, i, j >> 6, bh, (j >> 2) & 3);
  return dropout_keep(philox_word(r, (j >> 4) & 3), j & 3, d.keep);
}

}  // namespace fa
