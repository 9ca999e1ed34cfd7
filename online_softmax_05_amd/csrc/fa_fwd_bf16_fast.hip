// Exact attention forward, bf16 inputs with head dims 64 or 128: the fast
// path of the fused tile loop QK^T -> scale/bias/mask -> online softmax ->
// P.V -> one division ([GS] section 5; [OA] "Completing the Output by
// Traversing Tiles").
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//   [OA] "Reducing Memory Traffic with Output Accumulation in FlashAttention"
//
// Layout and data movement (gfx950)
// ---------------------------------
// * One work-group = 4 waves = 128 query rows of one (batch, head); each wave
//   owns 32 rows (two 16-row blocks) and keeps their Q fragments in
//   registers for the whole key loop ([OA] "Keeping Q While Processing the
//   First K/V Tile").
// * Key tiles of 64 keys.  K and V tiles go from global memory straight into
//   LDS (global_load_lds_dwordx4: no staging registers, no LDS store
//   instructions), row-major, with the 16-byte chunks of row r stored at
//   chunk index c ^ (r & 7) so that the 16 rows one MFMA operand read
//   touches fall in distinct LDS banks.
// * The matrix products use v_mfma_f32_16x16x32_bf16.  Each wave computes
//   S^T = K Q^T: a lane of the 16x16 accumulator holds one query and four
//   consecutive keys, so the row maximum is an in-lane max plus two lane
//   swaps (v_permlane16_swap, v_permlane32_swap), and P^T is already the B
//   operand of O^T += V^T P^T after rounding to bf16.
// * The V^T operand is read with ds_read_b64_tr_b16: within each 16-lane
//   group, four lanes point at 8-byte pieces of four key rows and every lane
//   receives one dim of all four keys -- the transpose happens in the LDS
//   read, so V stays in its natural row-major order.
// * Software pipeline: K runs one tile ahead of V.  While the softmax of
//   tile t runs on the VALU, the MFMAs of S^T for tile t+1 are issued; the
//   loads of K_{t+2} and V_{t+1} are in flight during the whole iteration,
//   and one barrier per iteration publishes them.
//
// Online state per query row (base-2 domain): reference m (moved lazily,
// only when the tile maximum exceeds it by more than 8), denominator l and
// unnormalised value sum u = O^T accumulators; both l and u are rebased by
// alpha = exp2(m_old - m_new) whenever m moves ([GS] section 4), and each row
// is divided once at the end ([GS] section 5).  Rows with no allowed key keep
// m = -inf and produce o = 0, lse = -inf ([GS] section 6).
#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per work-group
constexpr int kBN = 64;           // keys per tile
constexpr float kRebase = 8.f;    // lazy rebasing threshold (log2 units)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(1))) void gbl_void;
typedef __attribute__((address_space(3))) void lds_void;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Tile of kBN rows x D bf16 in LDS: R 16-byte chunks per row, chunk c of row
// r at position c ^ (r & 7).
template <int D>
struct SwzTile {
  static constexpr int R = D / 8;
  static constexpr int BYTES = kBN * D * 2;
  static constexpr int INSTS = kBN * R / 64;            // 1 KiB wave-wide loads per tile
  static constexpr int INSTS_PER_WAVE = INSTS / kWaves;
  static_assert(R >= 8 && INSTS % kWaves == 0, "tile shape");
  __device__ static __forceinline__ int off(int row, int c) { return (row * R + (c ^ (row & 7))) * 16; }
};

// Issue the direct-to-LDS loads of one tile (this wave's share).  Rows past
// the last key re-read the last key row (finite values whose probabilities
// are zero), so no lane reads out of bounds.
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* gbh, int n0, int nk, lds_char* tile, int wave, int lane) {
  using T = SwzTile<D>;
#pragma unroll
  for (int i = 0; i < T::INSTS_PER_WAVE; ++i) {
    const int inst = wave * T::INSTS_PER_WAVE + i;
    const int slot = inst * 64 + lane;
    const int row = slot / T::R;
    const int c = (slot % T::R) ^ (row & 7);
    const int grow = min(n0 + row, nk - 1);
    const uint16_t* g = gbh + (size_t)grow * D + c * 8;
    __builtin_amdgcn_global_load_lds((gbl_void*)g, (lds_void*)(tile + inst * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// max / sum over the four lanes q, q+16, q+32, q+48 that share a query
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int DK>
struct QFrag {
  bf16x8 f[2][DK / 32];  // [query block][k-step]: dims 32t + 8g .. +7
};

// S^T (keys x queries) of one tile: s[kb][qb] is the 16x16 block of key
// block kb and query block qb; a lane holds keys 16kb + 4g + j of query
// 16qb + lane % 16.
template <int DK>
__device__ __forceinline__ void qk_tile(f32x4 (&s)[4][2], const QFrag<DK>& q, const lds_char* kt, int lane) {
  using T = SwzTile<DK>;
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DK / 32; ++t) {
      const bf16x8 a = *(const lds_bf16x8*)(kt + T::off(16 * kb + r16, 4 * t + g));
      s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q.f[0][t], s[kb][0], 0, 0, 0);
      s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q.f[1][t], s[kb][1], 0, 0, 0);
    }
  }
}

// O^T += V^T P^T for one tile: k-step T covers keys 32T .. 32T+31, slot s of
// lane group g holding key 32T + 16(s/4) + 4g + s%4.
template <int DV>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[DV / 16][2], const bf16x8 (&pb)[2][2], const lds_char* vt,
                                        int lane) {
  using T = SwzTile<DV>;
  const int g = lane >> 4, e = (lane >> 2) & 3, r = lane & 3;
#pragma unroll
  for (int db = 0; db < DV / 16; ++db) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4i16 lo, hi;
      {
        const int row = 32 * kt + 4 * g + e;
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vt + T::off(row, 2 * db + (r >> 1)) + 8 * (r & 1)));
        const int row2 = row + 16;
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(vt + T::off(row2, 2 * db + (r >> 1)) + 8 * (r & 1)));
      }
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[kt][0], o[db][0], 0, 0, 0);
      o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[kt][1], o[db][1], 0, 0, 0);
    }
  }
}

struct RowState {
  float m[2];  // reference maximum (base 2) per query block
  float l[2];  // this lane's share of the denominator
};

// Softmax of one tile in place: mask, running reference, exponentials, P in
// bf16, and the rescale factors.  Returns in alpha[qb] the factor the value
// sums must be multiplied by, and whether any row of the wave moved.
template <bool MASK, bool BIAS>
__device__ __forceinline__ bool softmax_tile(f32x4 (&s)[4][2], bf16x8 (&pb)[2][2], RowState& st, float (&alpha)[2],
                                             float c, int n0, const int (&row_end)[2], const float* const (&brow)[2],
                                             const bool (&rvalid)[2], int nk, bool vec_bias, int lane) {
  const int g = lane >> 4;
  float xo[2][4][4];  // bias path: the raw bias per element
  float mx[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float m = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key0 = n0 + 16 * kb + 4 * g;
      f32x4 bv = {0.f, 0.f, 0.f, 0.f};
      if (BIAS) bv = load_bias4(brow[qb], key0, nk, vec_bias, rvalid[qb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[kb][qb][j];
        if (MASK && key0 + j >= row_end[qb]) x = kNegInf;
        if (BIAS) {
          // keep c*s; the biased logit only feeds the maximum, and the
          // exponent adds bias*log2e - m in one rounding (large biases
          // cancel against the maximum before they are rounded)
          x *= c;
          xo[qb][kb][j] = bv[j];
          m = fmaxf(m, fmaf(bv[j], kLog2e, x));
        } else {
          m = fmaxf(m, x);
        }
        s[kb][qb][j] = x;
      }
    }
    mx[qb] = BIAS ? m : m * c;
  }
  bool any_grow = false;
  float m_use[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float tmax = quad_max(mx[qb]);
    const bool grow = tmax > st.m[qb] + kRebase;
    const float m_new = grow ? tmax : st.m[qb];
    alpha[qb] = grow ? fast_exp2(st.m[qb] - m_new) : 1.f;  // 0 for the empty state
    any_grow |= grow;
    st.m[qb] = m_new;
    m_use[qb] = (m_new == kNegInf) ? 0.f : m_new;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      u32x4 w;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * kt + h;
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float arg = BIAS ? s[kb][qb][j] + fmaf(xo[qb][kb][j], kLog2e, -m_use[qb])
                                 : fmaf(s[kb][qb][j], c, -m_use[qb]);
          p[j] = fast_exp2(arg);
        }
        psum += (p[0] + p[1]) + (p[2] + p[3]);
        w[2 * h] = cvt_pk_bf16(p[0], p[1]);
        w[2 * h + 1] = cvt_pk_bf16(p[2], p[3]);
      }
      pb[kt][qb] = __builtin_bit_cast(bf16x8, w);
    }
    st.l[qb] = fmaf(alpha[qb], st.l[qb], psum);
  }
  return __builtin_amdgcn_ballot_w64(any_grow) != 0;
}

template <int DK, int DV, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_fast_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, uint16_t* __restrict__ o,
    float* __restrict__ lse, int H, int Nq, int Nk, float scale_log2, int causal, int vec_bias, int n_qt) {
  __shared__ __attribute__((aligned(1024))) char kbuf0[SwzTile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[SwzTile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[SwzTile<DV>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[SwzTile<DV>::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, n_qt, causal != 0);
  const int b = tc.bh / H;
  const int q0 = tc.qt * kBM;
  const int klen = clamp_klen(k_len, b, Nk);
  const size_t bh = (size_t)tc.bh;
  const uint16_t* qbh = q + bh * Nq * DK;
  const uint16_t* kbh = k + bh * Nk * DK;
  const uint16_t* vbh = v + bh * Nk * DV;

  const int shift = Nk - Nq;
  int qrow[2], row_end[2];
  bool rvalid[2];
  const float* brow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = q0 + wave * 32 + qb * 16 + r16;
    rvalid[qb] = qrow[qb] < Nq;
    row_end[qb] = causal ? min(klen, qrow[qb] + shift + 1) : klen;
    brow[qb] = BIAS ? bias + (bh * Nq + (size_t)(rvalid[qb] ? qrow[qb] : 0)) * Nk : nullptr;
  }
  const int wave_first = q0 + wave * 32;
  const int wave_min_end = causal ? min(klen, wave_first + shift + 1) : klen;
  const int kend = visible_key_end(klen, causal != 0, min(q0 + kBM, Nq) - 1, Nq, Nk);
  const int n_tiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;

  // logit scale in the base-2 domain, made positive (a negative scale flips
  // the sign of Q, exactly; zero becomes a tiny positive value)
  const bool neg_scale = scale_log2 < 0.f;
  const float c = fmaxf(fabsf(scale_log2), 1e-30f);

  QFrag<DK> qf;
  {
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const uint16_t* qr = qbh + (size_t)(rvalid[qb] ? qrow[qb] : 0) * DK;
#pragma unroll
      for (int t = 0; t < DK / 32; ++t) {
        u32x4 w = rvalid[qb] ? *reinterpret_cast<const u32x4*>(qr + 32 * t + 8 * g) : u32x4{0u, 0u, 0u, 0u};
        w[0] ^= flip; w[1] ^= flip; w[2] ^= flip; w[3] ^= flip;
        qf.f[qb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  f32x4 oacc[DV / 16][2];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) {
    oacc[d][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    oacc[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  RowState st;
  st.m[0] = st.m[1] = kNegInf;
  st.l[0] = st.l[1] = 0.f;

  f32x4 s_cur[4][2];
  if (n_tiles > 0) {
    load_tile<DK>(kbh, 0, Nk, (lds_char*)kbuf0, wave, lane);
    load_tile<DV>(vbh, 0, Nk, (lds_char*)vbuf0, wave, lane);
    if (n_tiles > 1) load_tile<DK>(kbh, kBN, Nk, (lds_char*)kbuf1, wave, lane);
    wait_loads();
    __syncthreads();
    qk_tile<DK>(s_cur, qf, (const lds_char*)kbuf0, lane);
    __syncthreads();  // every wave has read K_0 before K_2 replaces it
  }

  // One pipelined iteration: loads of K_{t+2} and V_{t+1} in flight, S^T of
  // tile t+1 computed beside the softmax of tile t, then O += P_t V_t.
  auto iterate = [&](int t, lds_char* kdst, const lds_char* knext, const lds_char* vcur, lds_char* vdst) {
    const int n0 = t * kBN;
    if (t + 2 < n_tiles) load_tile<DK>(kbh, n0 + 2 * kBN, Nk, kdst, wave, lane);
    if (t + 1 < n_tiles) load_tile<DV>(vbh, n0 + kBN, Nk, vdst, wave, lane);
    f32x4 s_next[4][2];
    qk_tile<DK>(s_next, qf, knext, lane);  // garbage (never used) after the last tile
    bf16x8 pb[2][2];
    float alpha[2];
    bool grow;
    if (n0 + kBN > wave_min_end)
      grow = softmax_tile<true, BIAS>(s_cur, pb, st, alpha, c, n0, row_end, brow, rvalid, Nk, vec_bias != 0, lane);
    else
      grow = softmax_tile<false, BIAS>(s_cur, pb, st, alpha, c, n0, row_end, brow, rvalid, Nk, vec_bias != 0, lane);
    if (grow) {
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) {
        oacc[d][0] *= alpha[0];
        oacc[d][1] *= alpha[1];
      }
    }
    pv_tile<DV>(oacc, pb, vcur, lane);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s_cur[kb][0] = s_next[kb][0];
      s_cur[kb][1] = s_next[kb][1];
    }
    wait_loads();
    __syncthreads();
  };

  for (int t = 0; t < n_tiles; t += 2) {
    iterate(t, (lds_char*)kbuf0, (const lds_char*)kbuf1, (const lds_char*)vbuf0, (lds_char*)vbuf1);
    if (t + 1 < n_tiles)
      iterate(t + 1, (lds_char*)kbuf1, (const lds_char*)kbuf0, (const lds_char*)vbuf1, (lds_char*)vbuf0);
  }

  // ---- epilogue: divide once; empty rows get o = 0, lse = -inf ------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = quad_sum(st.l[qb]);
    if (!rvalid[qb]) continue;
    const bool nonempty = l_tot > 0.f;
    const float inv = nonempty ? 1.f / l_tot : 0.f;
    uint16_t* orow = o + (bh * Nq + qrow[qb]) * (size_t)DV;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      u32x2 w;
      w[0] = cvt_pk_bf16(oacc[d][qb][0] * inv, oacc[d][qb][1] * inv);
      w[1] = cvt_pk_bf16(oacc[d][qb][2] * inv, oacc[d][qb][3] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * d + 4 * g) = w;
    }
    if (lse != nullptr && g == 0)
      lse[bh * Nq + qrow[qb]] = nonempty ? (st.m[qb] + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <int DK, int DV, bool BIAS>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long total = (long long)n_qt * a.H * a.B;
  const bool vec_b = (a.Nk % 4 == 0) && (((uintptr_t)a.bias & 15) == 0);
  hipLaunchKernelGGL((fwd_bf16_fast_kernel<DK, DV, BIAS>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.bias, a.k_len,
                     (uint16_t*)a.o, a.lse, a.H, a.Nq, a.Nk, a.scale * kLog2e, a.causal, (int)vec_b, n_qt);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_b(const FwdArgs& a, hipStream_t s) {
  return a.bias ? launch_t<DK, DV, true>(a, s) : launch_t<DK, DV, false>(a, s);
}

}  // namespace

bool fwd_bf16_fast_eligible(const FwdArgs& a) {
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  return (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128) && a.Nk > 0 && aligned(a.q) &&
         aligned(a.k) && aligned(a.v) && aligned(a.o) && (a.block_n == 0 || a.block_n == kBN);
}

hipError_t launch_fwd_bf16_fast(const FwdArgs& a, hipStream_t s) {
  if (a.dk == 64 && a.dv == 64) return launch_b<64, 64>(a, s);
  if (a.dk == 64) return launch_b<64, 128>(a, s);
  if (a.dv == 64) return launch_b<128, 64>(a, s);
  return launch_b<128, 128>(a, s);
}

}  // namespace fa
