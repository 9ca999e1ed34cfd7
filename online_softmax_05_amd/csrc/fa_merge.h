// Final merge of split-KV chunk states into one output row: each chunk's
// state (m_c, l_c, u_c) is rebased to the common maximum m and the states are
// added in ascending chunk order ([GS] "How Does FlashAttention Preserve
// Global Softmax Across Tiles?", section 4), then the row is divided once
// (section 5).  An empty chunk state (m = -inf, l = 0, u = 0) gets weight 0;
// a row whose states are all empty gets o = 0 and lse = -inf (section 6).
//
// One wave per row.  The chunk states are read with every load independent
// of the others: lanes take chunks for the maximum and the denominator, and
// each lane's value-sum loads are issued eight chunks at a time, the chunk
// weights coming from the lane that computed them (v_readlane), so a row
// costs a few memory latencies whatever its chunk count.
#pragma once

#include "fa_common.h"

namespace fa {

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Chunk c's state: m_c = ml[c * s_ml], l_c = ml[c * s_ml + 1], u_c[d] =
// u[c * s_u + d].  Writes store(u / l) to orow[0 .. dv) and, if lse_out is
// not null, the row's natural-log lse.  Called by all 64 lanes of a wave.
template <typename T, typename Store>
__device__ __forceinline__ void merge_chunk_states(const float* __restrict__ u, size_t s_u,
                                                   const float* __restrict__ ml, size_t s_ml, int n_c, int dv,
                                                   T* __restrict__ orow, float* __restrict__ lse_out, Store store) {
  const int lane = threadIdx.x & 63;
  // each lane's first chunk state, read once (most rows have at most 64
  // chunks; more are read again in the passes below)
  const float m0 = lane < n_c ? ml[lane * s_ml] : kNegInf;
  const float l0 = lane < n_c ? ml[lane * s_ml + 1] : 0.f;
  float mx = m0;
  for (int c = lane + 64; c < n_c; c += 64) mx = fmaxf(mx, ml[c * s_ml]);
  mx = wave_max64(mx);
  const float mu = (mx == kNegInf) ? 0.f : mx;
  const float w0 = fast_exp2(m0 - mu);  // weight of chunk `lane` (0 past n_c)
  float ls = w0 * l0;
  for (int c = lane + 64; c < n_c; c += 64) ls = fmaf(fast_exp2(ml[c * s_ml] - mu), ml[c * s_ml + 1], ls);
  const float l = wave_sum64(ls);
  const bool nonempty = l > 0.f;
  const float inv = nonempty ? 1.f / l : 0.f;
  // the dims go 64 at a time with every lane taking part (the chunk weights
  // are read from other lanes, which must have computed them)
  for (int d0 = 0; d0 < dv; d0 += 64) {
    const int d = d0 + lane;
    const bool act = d < dv;
    float acc = 0.f;
    for (int c0 = 0; c0 < n_c; c0 += 64) {
      const int cl = c0 + lane;
      const float wf = c0 == 0 ? w0 : (cl < n_c ? fast_exp2(ml[cl * s_ml] - mu) : 0.f);
      const int wl = __float_as_int(wf);  // weight of chunk c0 + lane
      const int cn = min(64, n_c - c0);
      const float* uc = u + (size_t)c0 * s_u + (act ? d : 0);
      int j = 0;
      for (; j + 8 <= cn; j += 8) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = act ? uc[(size_t)(j + e) * s_u] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(wl, j + e)), x[e], acc);
      }
      for (; j < cn; ++j) {
        const float x = act ? uc[(size_t)j * s_u] : 0.f;
        acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(wl, j)), x, acc);
      }
    }
    if (act) orow[d] = store(acc * inv);
  }
  if (lse_out != nullptr && lane == 0) *lse_out = nonempty ? (mx + fast_log2(l)) * kLn2 : kNegInf;
}

}  // namespace fa
