// Exact attention forward, bf16 inputs, fp32 state: the fused tile loop
// QK^T -> scale/bias/mask -> online softmax -> P.V -> one division
// ([GS] section 5; [OA] "Completing the Output by Traversing Tiles").
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//   [OA] "Reducing Memory Traffic with Output Accumulation in FlashAttention"
//
// Work decomposition (gfx950, 64-wide waves, v_mfma_f32_32x32x16_bf16)
// --------------------------------------------------------------------
// One work-group = 4 waves = 128 query rows of one (batch, head); each wave
// owns 32 rows and keeps their Q fragment in registers for the whole key
// loop ([OA] "Keeping Q While Processing the First K/V Tile").  K and V tiles
// of BN keys stream through LDS, double buffered: tile t+1 is fetched from
// HBM into registers while tile t is consumed.
//
// Each wave computes the TRANSPOSED score tile S^T = K Q^T (A = K from LDS,
// B = Q^T from registers).  In the 32x32 accumulator layout a lane then
// holds one query (lane % 32) and 16 of its keys, so
//   * the row maximum is an in-register max plus one v_permlane32_swap;
//   * the row sum never leaves the lane until the epilogue;
//   * the rescale factor alpha is a per-lane scalar;
//   * P^T is already laid out as the B operand of O^T += V^T P^T: the fp32
//     scores are only rounded to bf16, no data moves between lanes.
// The key order inside the V^T operand is permuted (in LDS) to match the
// order in which the accumulator hands keys to the lanes; a contraction
// does not care about the order of its summation index.
//
// Per row the state is (m, l, u) in the base-2 domain: m is the running
// maximum of t = s*log2(e), l the running denominator, u (= O^T in the
// accumulators) the unnormalised weighted value sum.  Both l and u are
// multiplied by alpha = exp2(m_old - m_new) whenever the maximum rises
// ([GS] section 4; [OA] "Rescaling Both Accumulators When the Maximum
// Increases"), and each row is divided once at the end ([GS] section 5).
// A row that has seen no allowed key keeps the empty state: its maximum is
// -inf, the exponent origin used is 0, every p is exp2(-inf) = 0 and
// alpha = 0 multiplies zeros, so exp(-inf - (-inf)) is never formed
// ([GS] section 6).
//
// Position masks (causal in either alignment, sliding windows) come as a
// visible key range [lo, end) per row whose ends grow with the row; the
// work-group visits only the key tiles that meet the union of its rows'
// ranges, and only tiles not inside every row's range of a wave are masked
// element by element ([GS] section 6).
//
// Dropout (optional): P is dropped with the counter-based mask of
// fa_dropout.h before the product with V; l sums the undropped P, and the
// epilogue multiplies by 256/keep.  A lane holds four 4-key groups of its
// row per 32 keys, one generator call each.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_mask.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per work-group
constexpr float kRebase = 8.f;    // lazy rebasing threshold (log2 units)

template <int DK, int DV, int BN>
struct Tile {
  static constexpr int KS = DK + 8;  // K row stride in LDS (elements): +16 B breaks bank aliasing
  static constexpr int VS = BN + 8;  // V^T row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = DV * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BN * DK / 8 / kThreads;          // 16-byte K chunks per thread
  static constexpr int V_TASKS = BN * DV / 32;                     // (4 keys x 8 dims) blocks
  static constexpr int V_PER_THREAD = (V_TASKS + kThreads - 1) / kThreads;
  static_assert(K_CHUNKS >= 1 && BN * DK / 8 % kThreads == 0, "K tile must split evenly");
};

// Position block of key group g (keys 4g..4g+3) inside a V^T row: swaps the
// two low bits of g so that the 8 keys a lane feeds to one MFMA k-step are
// contiguous (see the header comment).
__device__ __forceinline__ int vt_block(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

// 8 consecutive bf16 (16 bytes) of a row, zero beyond `d`; `vec` means the
// row start is 16-byte aligned and d is a multiple of 8.
__device__ __forceinline__ u32x4 load_row8(const uint16_t* row, int d0, int d, bool vec) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (vec) {
    if (d0 < d) r = *reinterpret_cast<const u32x4*>(row + d0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t lo = (d0 + e < d) ? row[d0 + e] : 0u;
      uint32_t hi = (d0 + e + 1 < d) ? row[d0 + e + 1] : 0u;
      r[e / 2] = lo | (hi << 16);
    }
  }
  return r;
}

template <int DK, int DV, int BN>
struct Prefetch {
  u32x4 k[Tile<DK, DV, BN>::K_CHUNKS];
  u32x4 v[Tile<DK, DV, BN>::V_PER_THREAD][4];
};

template <int DK, int DV, int BN>
__device__ __forceinline__ void fetch_tile(Prefetch<DK, DV, BN>& pf, const uint16_t* kbh, const uint16_t* vbh,
                                           int n0, int nk, int dk, int dv, bool vec_k, bool vec_v, int tid) {
  using T = Tile<DK, DV, BN>;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    int id = tid + i * kThreads;
    int row = id / (DK / 8), c = id % (DK / 8);
    int key = n0 + row;
    pf.k[i] = (key < nk) ? load_row8(kbh + (size_t)key * dk, c * 8, dk, vec_k) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < T::V_PER_THREAD; ++i) {
    int task = tid + i * kThreads;
    int g = task % (BN / 4), c = task / (BN / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int key = n0 + 4 * g + j;
      bool ok = (task < T::V_TASKS) && key < nk;
      pf.v[i][j] = ok ? load_row8(vbh + (size_t)key * dv, c * 8, dv, vec_v) : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int DK, int DV, int BN>
__device__ __forceinline__ void store_tile(const Prefetch<DK, DV, BN>& pf, uint16_t* buf, int tid) {
  using T = Tile<DK, DV, BN>;
  uint16_t* ks = buf;
  uint16_t* vt = buf + T::K_ELEMS;
#pragma unroll
  for (int i = 0; i < T::K_CHUNKS; ++i) {
    int id = tid + i * kThreads;
    int row = id / (DK / 8), c = id % (DK / 8);
    *reinterpret_cast<u32x4*>(ks + row * T::KS + c * 8) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < T::V_PER_THREAD; ++i) {
    int task = tid + i * kThreads;
    if (task < T::V_TASKS) {
      int g = task % (BN / 4), c = task / (BN / 4);
      int col = 4 * vt_block(g);
      // 4 keys x 8 dims -> 8 dims x 4 keys (bf16 halves regrouped with v_perm)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        u32x2 lo, hi;
        lo[0] = __builtin_amdgcn_perm(pf.v[i][1][p], pf.v[i][0][p], 0x05040100u);
        lo[1] = __builtin_amdgcn_perm(pf.v[i][3][p], pf.v[i][2][p], 0x05040100u);
        hi[0] = __builtin_amdgcn_perm(pf.v[i][1][p], pf.v[i][0][p], 0x07060302u);
        hi[1] = __builtin_amdgcn_perm(pf.v[i][3][p], pf.v[i][2][p], 0x07060302u);
        *reinterpret_cast<u32x2*>(vt + (c * 8 + 2 * p) * T::VS + col) = lo;
        *reinterpret_cast<u32x2*>(vt + (c * 8 + 2 * p + 1) * T::VS + col) = hi;
      }
    }
  }
}

template <int DK, int DV, int BN, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, uint16_t* __restrict__ o,
    float* __restrict__ lse, int H, int Nq, int Nk, int dk, int dv, float scale_log2, KeyRange mr,
    DropoutSpec dsp, float drop_scale, int vec_q, int vec_k, int vec_v, int vec_bias, int n_qt) {
  using T = Tile<DK, DV, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
  const int col = lane & 31;  // query row within the wave / MFMA column
  const int hf = lane >> 5;   // lane half

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, n_qt, mr.wr >= 0);
  const int b = tc.bh / H;
  const int q0 = tc.qt * kBM;
  const int klen = clamp_klen(k_len, b, Nk);
  const int qi = q0 + wave * 32 + col;  // this lane's query row (global)
  const bool row_valid = qi < Nq;

  const size_t bh = (size_t)tc.bh;
  const uint16_t* qbh = q + bh * Nq * dk;
  const uint16_t* kbh = k + bh * Nk * dk;
  const uint16_t* vbh = v + bh * Nk * dv;

  // keys this row may see are [row_lo, row_end) (empty when row_lo >=
  // row_end); tiles inside [wave_max_lo, wave_min_end) need no per-element
  // mask for this wave
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

  // Logit scale in the base-2 domain, made positive: a negative scale flips
  // the sign of Q instead (exact in bf16), and a zero scale is replaced by a
  // tiny positive one whose products with finite dot products round to 0 in
  // every exponent.
  const bool neg_scale = scale_log2 < 0.f;
  const float c = fmaxf(fabsf(scale_log2), 1e-30f);

  // Q^T fragment: B operand, k-step t holds dims 16t + 8*hf .. +7 of row qi
  bf16x8 qf[DK / 16];
  {
    const uint16_t* qrow = qbh + (size_t)(row_valid ? qi : 0) * dk;
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      u32x4 w = row_valid ? load_row8(qrow, 16 * t + 8 * hf, dk, vec_q != 0) : u32x4{0u, 0u, 0u, 0u};
      w[0] ^= flip; w[1] ^= flip; w[2] ^= flip; w[3] ^= flip;
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_run = kNegInf;  // running max (base 2), shared by both lane halves
  float l_run = 0.f;      // this lane half's part of the running denominator
  float lu_run = 0.f;     // the same over the bf16-rounded weights that multiply V

  Prefetch<DK, DV, BN> pf;
  if (t_begin < t_end) {
    fetch_tile<DK, DV, BN>(pf, kbh, vbh, t_begin * BN, klen, dk, dv, vec_k != 0, vec_v != 0, tid);
    store_tile<DK, DV, BN>(pf, smem + (t_begin & 1) * T::BUF, tid);
  }
  __syncthreads();

  const float* brow = BIAS ? bias + (bh * Nq + (size_t)(row_valid ? qi : 0)) * Nk : nullptr;

  for (int it = t_begin; it < t_end; ++it) {
    const int n0 = it * BN;
    const uint16_t* ks = smem + (it & 1) * T::BUF;
    const uint16_t* vt = ks + T::K_ELEMS;
    const bool has_next = it + 1 < t_end;
    if (has_next) fetch_tile<DK, DV, BN>(pf, kbh, vbh, n0 + BN, klen, dk, dv, vec_k != 0, vec_v != 0, tid);

    // ---- S^T = K Q^T for this wave's 32 rows and BN keys ----------------
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int t = 0; t < DK / 16; ++t) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + col) * T::KS + 16 * t + 8 * hf);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kb], 0, 0, 0);
      }
    }

    // ---- scale (+ bias) and mask, in the base-2 domain ---------------------
    // Accumulator register r of key block kb holds key n0 + 32kb + 8(r/4) +
    // 4hf + r%4.  Without a bias s[] keeps the raw dot products: the scale
    // c > 0 is folded into one FMA in the exponent and max(c s) = c max(s).
    // With a bias s[] keeps c s and the biased logit only feeds the maximum;
    // the exponent re-adds the bias after subtracting the maximum, so large
    // bias values cancel before rounding.
    //
    // The mask is one unsigned range test and a select per element, under a
    // wave-uniform branch: a short-circuit condition here was compiled into
    // per-element exec-mask diamonds that lost unmasked values.
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
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) bv = load_bias4(brow, n0 + kb * 32 + 8 * i + 4 * hf, Nk, vec_bias != 0, row_valid);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BIAS) {
            const float sc = s[kb][4 * i + j] * c;  // -inf stays -inf (c > 0)
            s[kb][4 * i + j] = sc;
            mx = fmaxf(mx, sc + bv[j] * kLog2e);
          } else {
            mx = fmaxf(mx, s[kb][4 * i + j]);
          }
        }
      }
    }
    if (!BIAS) mx *= c;

    // ---- running reference, rescale factor, exponentials -----------------
    // The reference m_run is moved only when this tile's maximum exceeds it
    // by more than kRebase (log2 units); in between, exponentials are taken
    // against the lagging reference and stay <= 2^kRebase.  Any common
    // origin gives the same o = u / l, so l and u stay exact; rebasing both
    // by alpha = exp2(m_old - m_new) when the reference moves keeps the state
    // consistent ([GS] section 4).  An empty row keeps m_run = -inf.
    mx = half_swap_max(mx);
    const bool grow = mx > m_run + kRebase;
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;  // 0 for the empty state
    m_run = m_new;
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;

    float psum = 0.f, usum = 0.f;
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      // dropout: bit r of km keeps accumulator slot r (key n0 + 32kb +
      // 8(r/4) + 4hf + r%4)
      uint32_t km = 0xffffu;
      if (dsp.keep < 256) {
        km = 0u;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int j0 = n0 + kb * 32 + 8 * i4 + 4 * hf;
          const uint32_t w = philox_word(dropout_words(dsp, qi, j0 >> 6, (uint32_t)bh, (j0 >> 2) & 3), (j0 >> 4) & 3);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) km |= dropout_keep(w, jj, dsp.keep) ? 1u << (4 * i4 + jj) : 0u;
        }
      }
      float xo[16];  // bias * log2e - m (bias path only)
      if (BIAS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 bv = load_bias4(brow, n0 + kb * 32 + 8 * i + 4 * hf, Nk, vec_bias != 0, row_valid);
#pragma unroll
          for (int j = 0; j < 4; ++j) xo[4 * i + j] = fmaf(bv[j], kLog2e, -m_use);
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r0 = 8 * t2 + e, r1 = r0 + 1;
          const float p0 = fast_exp2(BIAS ? s[kb][r0] + xo[r0] : fmaf(s[kb][r0], c, -m_use));
          const float p1 = fast_exp2(BIAS ? s[kb][r1] + xo[r1] : fmaf(s[kb][r1], c, -m_use));
          psum += p0 + p1;
          w[e / 2] = pack_bf16x2((km >> r0) & 1u ? p0 : 0.f, (km >> r1) & 1u ? p1 : 0.f);
          usum = add_bf16_pair(w[e / 2], usum);  // used only without dropout (then nothing is zeroed)
        }
        pb[kb * 2 + t2] = __builtin_bit_cast(bf16x8, w);
      }
    }
    l_run = fmaf(alpha, l_run, psum);
    lu_run = fmaf(alpha, lu_run, usum);

    // rescale u only when some row of the wave moved its reference
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
    }

    // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int ks16 = 0; ks16 < BN / 16; ++ks16) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (d * 32 + col) * T::VS + 16 * ks16 + 8 * hf);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks16], oacc[d], 0, 0, 0);
      }
    }

    if (has_next) store_tile<DK, DV, BN>(pf, smem + ((it + 1) & 1) * T::BUF, tid);
    __syncthreads();
  }

  // ---- epilogue: divide once; empty rows get o = 0, lse = -inf ------------
  const float l_tot = half_swap_sum(l_run);
  // without dropout O is divided by the sum of the bf16-rounded weights it
  // was built from (an exact weighted mean of V up to fp32 rounding); lse
  // and the dropout divisor use the unrounded sum
  const float l_used = half_swap_sum(lu_run);
  if (!row_valid) return;
  const bool nonempty = l_tot > 0.f;
  const float inv = nonempty ? drop_scale / (dsp.keep >= 256 ? l_used : l_tot) : 0.f;
  uint16_t* orow = o + (bh * Nq + qi) * (size_t)dv;
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = d * 32 + 8 * i + 4 * hf;  // dims d0 .. d0+3 of row qi
      if (d0 >= dv) continue;
      float x0 = oacc[d][4 * i + 0] * inv, x1 = oacc[d][4 * i + 1] * inv;
      float x2 = oacc[d][4 * i + 2] * inv, x3 = oacc[d][4 * i + 3] * inv;
      if (vec_v && d0 + 3 < dv) {
        u32x2 w;
        w[0] = pack_bf16x2(x0, x1);
        w[1] = pack_bf16x2(x2, x3);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      } else {
        float xs[4] = {x0, x1, x2, x3};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (d0 + j < dv) orow[d0 + j] = (uint16_t)(pack_bf16x2(xs[j], 0.f) & 0xffffu);
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
  const uintptr_t mask16 = 15;
  const bool vec_q = (a.dk % 8 == 0) && (((uintptr_t)a.q & mask16) == 0);
  const bool vec_k = (a.dk % 8 == 0) && (((uintptr_t)a.k & mask16) == 0);
  // V loads and O stores share one flag: both need dv % 8 == 0 and alignment
  const bool vec_v = (a.dv % 8 == 0) && (((uintptr_t)a.v & mask16) == 0) && (((uintptr_t)a.o & 7) == 0);
  const bool vec_b = (a.Nk % 4 == 0) && (((uintptr_t)a.bias & mask16) == 0);
  hipLaunchKernelGGL((fwd_bf16_kernel<DK, DV, BN, BIAS>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.bias, a.k_len,
                     (uint16_t*)a.o, a.lse, a.H, a.Nq, a.Nk, a.dk, a.dv, a.scale * kLog2e,
                     KeyRange{a.off, a.wl, a.wr}, DropoutSpec{a.seed_lo, a.seed_hi, a.keep_256},
                     256.f / (float)a.keep_256, (int)vec_q, (int)vec_k, (int)vec_v, (int)vec_b, n_qt);
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

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  const bool k64 = a.dk <= 64, v64 = a.dv <= 64;
  if (k64 && v64) return launch_n<64, 64>(a, s);
  if (k64) return launch_n<64, 128>(a, s);
  if (v64) return launch_n<128, 64>(a, s);
  return launch_n<128, 128>(a, s);
}

}  // namespace fa
