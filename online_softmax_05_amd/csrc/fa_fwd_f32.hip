// Exact attention forward, fp32 inputs and fp32 state, on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32): the same fused tile loop as the bf16
// kernel, without any rounding of P ([GS] section 5; [OA] "Completing the
// Output by Traversing Tiles").
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//   [OA] "Reducing Memory Traffic with Output Accumulation in FlashAttention"
//
// One work-group = 4 waves = 128 query rows; each wave owns 32 rows and
// computes S^T = K Q^T so that a lane holds one query and 16 of its keys per
// 32-key block (row reductions are in-lane plus one v_permlane32_swap, and
// the fp32 P^T accumulator register r is directly the B operand of the
// k-step "key 8(r/4) + 4*half + r%4" of O^T += V^T P^T).  With one key per
// lane half per k-step, V can stay row-major in LDS.  The tile is staged
// through a single LDS buffer: these shapes are small and this kernel
// favours plainness over overlap.
//
// Position masks (causal in either alignment, sliding windows) come as a
// visible key range [lo, end) per row whose ends grow with the row; the
// work-group visits only the key tiles that meet the union of its rows'
// ranges, and only tiles not inside every row's range of a wave are masked
// element by element ([GS] section 6).
//
// Dropout (optional): P is dropped with the counter-based mask of
// fa_dropout.h before the product with V; l sums the undropped P, and the
// epilogue multiplies by 256/keep.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_mask.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;

template <int DK, int DV, int BN>
struct TileF {
  static constexpr int KS = DK + 1;  // odd stride: the 32 rows a wave reads fall in distinct banks
  static constexpr int VS = DV;
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = BN * VS;
};

// 4 consecutive floats of a row, zero beyond d; vec: 16-byte aligned and d % 4 == 0
__device__ __forceinline__ f32x4 load_row4(const float* row, int d0, int d, bool vec) {
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  if (vec) {
    if (d0 < d) r = *reinterpret_cast<const f32x4*>(row + d0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (d0 + e < d) ? row[d0 + e] : 0.f;
  }
  return r;
}

template <int DK, int DV, int BN, bool BIAS>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, float* __restrict__ o,
    float* __restrict__ lse, int H, int Nq, int Nk, int dk, int dv, float scale_log2, KeyRange mr,
    DropoutSpec dsp, float drop_scale, int vec_q, int vec_k, int vec_v, int vec_bias, int n_qt) {
  using T = TileF<DK, DV, BN>;
  __shared__ __attribute__((aligned(16))) float smem[T::K_ELEMS + T::V_ELEMS];
  float* ks = smem;
  float* vs = smem + T::K_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, n_qt, mr.wr >= 0);
  const int b = tc.bh / H;
  const int q0 = tc.qt * kBM;
  const int klen = clamp_klen(k_len, b, Nk);
  const int qi = q0 + wave * 32 + col;
  const bool row_valid = qi < Nq;
  const size_t bh = (size_t)tc.bh;
  const float* qbh = q + bh * Nq * dk;
  const float* kbh = k + bh * Nk * dk;
  const float* vbh = v + bh * Nk * dv;

  // keys this row may see are [row_lo, row_end); tiles inside
  // [wave_max_lo, wave_min_end) need no per-element mask for this wave
  const int row_lo = key_lo(mr, qi);
  const int row_end = key_end(mr, qi, klen);
  const unsigned row_span = row_end > row_lo ? (unsigned)(row_end - row_lo) : 0u;
  const int wave_first = q0 + wave * 32;
  const int wave_max_lo = key_lo(mr, wave_first + 31);
  const int wave_min_end = key_end(mr, wave_first, klen);
  const int kbeg = key_lo(mr, q0);
  const int kend = key_end(mr, min(q0 + kBM, Nq) - 1, klen);
  const int t_begin = kbeg / BN;
  const int t_end = kend > kbeg ? (kend + BN - 1) / BN : t_begin;

  // Q^T fragment: k-step t holds dim 2t + half of row qi
  float qf[DK / 2];
  {
    const float* qrow = qbh + (size_t)(row_valid ? qi : 0) * dk;
#pragma unroll
    for (int t = 0; t < DK / 2; ++t) {
      const int d = 2 * t + hf;
      qf[t] = (row_valid && d < dk) ? qrow[d] : 0.f;
    }
  }

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;
  const float* brow = BIAS ? bias + (bh * Nq + (size_t)(row_valid ? qi : 0)) * Nk : nullptr;

  for (int it = t_begin; it < t_end; ++it) {
    const int n0 = it * BN;
    __syncthreads();  // the previous tile has been consumed by every wave
    for (int id = tid; id < BN * DK / 4; id += kThreads) {
      const int row = id / (DK / 4), c = id % (DK / 4);
      const int key = n0 + row;
      f32x4 w = (key < klen) ? load_row4(kbh + (size_t)key * dk, 4 * c, dk, vec_k != 0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[row * T::KS + 4 * c + e] = w[e];
    }
    for (int id = tid; id < BN * DV / 4; id += kThreads) {
      const int row = id / (DV / 4), c = id % (DV / 4);
      const int key = n0 + row;
      f32x4 w = (key < klen) ? load_row4(vbh + (size_t)key * dv, 4 * c, dv, vec_v != 0) : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(vs + row * T::VS + 4 * c) = w;
    }
    __syncthreads();

    // S^T = K Q^T
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll 8
      for (int t = 0; t < DK / 2; ++t) {
        const float a = ks[(kb * 32 + col) * T::KS + 2 * t + hf];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[t], s[kb], 0, 0, 0);
      }
    }

    // scale into the base-2 domain, then mask: one unsigned range test and
    // a select per element, under a wave-uniform branch (masking after the
    // scale keeps -inf for any sign of the scale)
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] *= scale_log2;
    if (n0 < wave_max_lo || n0 + BN > wave_min_end) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + kb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
          const bool vis = (unsigned)(key - row_lo) < row_span;
          s[kb][r] = vis ? s[kb][r] : kNegInf;
        }
    }
    // s[] keeps scale*log2e*(q.k) (or -inf); with a bias the biased logit
    // only feeds the maximum, and the exponent below re-adds the bias after
    // subtracting the maximum, so large bias values cancel before rounding
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) bv = load_bias4(brow, n0 + kb * 32 + 8 * i + 4 * hf, Nk, vec_bias != 0, row_valid);
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, BIAS ? s[kb][4 * i + j] + bv[j] * kLog2e : s[kb][4 * i + j]);
      }
    }
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) bv = load_bias4(brow, n0 + kb * 32 + 8 * i + 4 * hf, Nk, vec_bias != 0, row_valid);
        // dropout word of keys n0 + 32kb + 8i + 4hf .. +3 (all kept without dropout)
        uint32_t zw = 0u;
        if (dsp.keep < 256) {
          const int j0 = n0 + kb * 32 + 8 * i + 4 * hf;
          zw = philox_word(dropout_words(dsp, qi, j0 >> 6, (uint32_t)bh, (j0 >> 2) & 3), (j0 >> 4) & 3);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float off = BIAS ? fmaf(bv[j], kLog2e, -m_use) : -m_use;
          const float p = fast_exp2(s[kb][4 * i + j] + off);
          s[kb][4 * i + j] = dropout_keep(zw, j, dsp.keep) ? p : 0.f;
          psum += p;
        }
      }
    l_run = fmaf(alpha, l_run, psum);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }

    // O^T += V^T P^T, one key per lane half per k-step
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
          const float a = vs[key * T::VS + d * 32 + col];
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], oacc[d], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = half_swap_sum(l_run);
  if (!row_valid) return;
  const bool nonempty = l_tot > 0.f;
  const float inv = nonempty ? drop_scale / l_tot : 0.f;
  float* orow = o + (bh * Nq + qi) * (size_t)dv;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = d * 32 + 8 * i + 4 * hf;
      if (d0 >= dv) continue;
      f32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = oacc[d][4 * i + j] * inv;
      if (vec_v && d0 + 3 < dv) {
        *reinterpret_cast<f32x4*>(orow + d0) = w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (d0 + j < dv) orow[d0 + j] = w[j];
      }
    }
  }
  if (lse != nullptr && hf == 0)
    lse[bh * Nq + qi] = nonempty ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
}

template <int DK, int DV, int BN, bool BIAS>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long total = (long long)n_qt * a.H * a.B;
  const uintptr_t m16 = 15;
  const bool vec_q = (a.dk % 4 == 0) && (((uintptr_t)a.q & m16) == 0);
  const bool vec_k = (a.dk % 4 == 0) && (((uintptr_t)a.k & m16) == 0);
  const bool vec_v = (a.dv % 4 == 0) && (((uintptr_t)a.v & m16) == 0) && (((uintptr_t)a.o & m16) == 0);
  const bool vec_b = (a.Nk % 4 == 0) && (((uintptr_t)a.bias & m16) == 0);
  hipLaunchKernelGGL((fwd_f32_kernel<DK, DV, BN, BIAS>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, a.bias, a.k_len, (float*)a.o,
                     a.lse, a.H, a.Nq, a.Nk, a.dk, a.dv, a.scale * kLog2e, KeyRange{a.off, a.wl, a.wr},
                     DropoutSpec{a.seed_lo, a.seed_hi, a.keep_256}, 256.f / (float)a.keep_256, (int)vec_q, (int)vec_k,
                     (int)vec_v, (int)vec_b, n_qt);
  return hipGetLastError();
}

template <int DK, int DV, int BN>
hipError_t launch_b(const FwdArgs& a, hipStream_t s) {
  return a.bias ? launch_t<DK, DV, BN, true>(a, s) : launch_t<DK, DV, BN, false>(a, s);
}

template <int DK, int DV>
hipError_t launch_n(const FwdArgs& a, hipStream_t s) {
  switch (a.block_n) {
    case 32: return launch_b<DK, DV, 32>(a, s);
    case 128: return launch_b<DK, DV, 128>(a, s);
    default: return launch_b<DK, DV, 64>(a, s);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  const bool k64 = a.dk <= 64, v64 = a.dv <= 64;
  if (k64 && v64) return launch_n<64, 64>(a, s);
  if (k64) return launch_n<64, 128>(a, s);
  if (v64) return launch_n<128, 64>(a, s);
  return launch_n<128, 128>(a, s);
}

}  // namespace fa
