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
// * One work-group = 4 or 8 waves = 128 or 256 query rows of one (batch,
//   head) (the launch chooses); each wave owns 32 rows (two 16-row blocks)
//   and keeps their Q fragments in registers for the whole key loop ([OA]
//   "Keeping Q While Processing the First K/V Tile").
// * Key tiles of 64 keys.  K and V tiles go from global memory straight into
//   LDS (buffer_load_dwordx4 ... lds: no staging registers, no LDS store
//   instructions, a fixed per-lane offset and one uniform offset per tile,
//   the buffer's range check covering the last tile), row-major, with the
//   16-byte chunk c of row r stored at
//   chunk index c ^ f(r), with f chosen (by measuring LDS bank-conflict
//   cycles) so that both operand reads below run conflict-free.  Every
//   operand address is then a per-lane base (one per k-step for K, one per
//   16-dim block for V) plus a compile-time offset.
// * The matrix products use v_mfma_f32_16x16x32_bf16.  Each wave computes
//   S^T = K Q^T: a lane of the 16x16 accumulator holds one query and four
//   consecutive keys, so the row maximum is an in-lane max plus two lane
//   swaps (v_permlane16_swap, v_permlane32_swap), and P^T is already the B
//   operand of O^T += V^T P^T after rounding to bf16.
// * The V^T operand is read with ds_read_b64_tr_b16: within each 16-lane
//   group, four lanes point at 8-byte pieces of four key rows and every lane
//   receives one dim of all four keys -- the transpose happens in the LDS
//   read, so V stays in its natural row-major order.
// * Row sums of P are taken in fp32 before P is rounded to bf16 (a sum of
//   the rounded values on the matrix cores would leave ~1e-3 relative
//   error in l, and so in lse, on rows dominated by a few keys); O is
//   divided by a second fp32 sum, of the rounded weights that multiply V
//   (in eight-wave work-groups a product of P with a block of ones on the
//   matrix cores, in four-wave ones v_dot2 against ones on the vector ALU).
// * Double buffering: the loads of tile t+1 are in flight during the whole
//   of tile t, and one barrier per tile publishes them.  Two waves share
//   each SIMD (two 4-wave work-groups or one 8-wave work-group per CU), so
//   one wave's softmax (VALU) can overlap the other wave's matrix products.  Tiles that need no mask for
//   any row of the work-group run a variant without mask code, and so does
//   a wave whose 32 rows all see the whole of a masked tile.
// * Position masks (causal in either alignment, sliding windows) arrive as a
//   visible key range [lo, end) per row, both ends growing with the row
//   ([GS] section 6).  A work-group visits the key tiles that meet the union
//   of its rows' ranges: a masked run along the left window edge, unmasked
//   tiles inside every row's range, then a masked run along the right edge
//   (the causal diagonal, the key-length boundary).
// * Dropout (a separate instance): a lane's 16 keys of a row in a tile are
//   exactly the 16 bytes of one counter-based generator call (fa_dropout.h),
//   so each lane makes one call per query block and tile; dropped
//   probabilities are zeroed in the bf16 P operand only (l sums the
//   undropped ones) and the epilogue multiplies by 256/keep.
//
// Online state per query row (base-2 domain): reference m (moved lazily,
// only when the tile maximum exceeds it by more than 8), denominator l and
// unnormalised value sum u = O^T accumulators; both l and u are rebased by
// alpha = exp2(m_old - m_new) whenever m moves ([GS] section 4), and each row
// is divided once at the end ([GS] section 5).  Rows with no allowed key keep
// m = -inf and produce o = 0, lse = -inf ([GS] section 6).
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_mask.h"
#include "launch.h"

namespace fa {
namespace {

// W waves of 32 query rows per work-group: 4 (two work-groups per CU) or 8
// (one), chosen per launch
template <int W>
constexpr int threads_of() { return 64 * W; }
template <int W>
constexpr int rows_of() { return 32 * W; }  // query rows per work-group
constexpr int kBN = 64;           // keys per tile
constexpr float kRebase = 8.f;    // lazy rebasing threshold (log2 units)

// Pace LDS operand reads against the MFMAs that consume them (bounds the
// registers held by fragments in flight).
#ifndef FA_FAST_PACE
#define FA_FAST_PACE 1
#endif

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// max / sum over the four lanes q, q+16, q+32, q+48 that share a query.
// The max is med3(a, b, FLT_MAX) (a and b are finite or -inf): fmaxf would
// first quiet each operand that comes out of a lane swap (two more
// instructions per max), and a +inf bound folds back into fmaxf.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.402823466e38f); }
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Swizzle of the 16-byte chunk index inside a row of an LDS tile (depends on
// row % 8 only).  Chosen by measurement with the LDS bank-conflict counter:
// with it, both the 128-bit K-operand reads and the transposed V reads below
// run without bank-conflict cycles (4 and 2 LDS cycles per instruction).  An
// earlier choice that spread the 16 rows of a K read over 16 distinct 16-byte
// positions of a 256-byte bank period still spent half its LDS cycles in
// conflicts, so the LDS bank index on gfx950 is not the plain address modulo
// 256 bytes for these patterns.  D = 128: the upper three bits (the 32-byte
// pair of a transposed read) run over 0..7 across 8 consecutive rows.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 7) << 1) | ((row >> 2) & 1);
  return row & 7;
}

// Tile of kBN rows x D bf16 in LDS: R 16-byte chunks per row, chunk c of row
// r at chunk position c ^ swz<D>(r).
template <int D>
struct SwzTile {
  static constexpr int R = D / 8;
  static constexpr int ROW = R * 16;                 // bytes per row
  static constexpr int BYTES = kBN * ROW;
  static_assert(R >= 8 && kBN * R % (64 * 8) == 0, "tile shape");
};
// 1 KiB wave-wide direct loads per wave per tile, with W waves loading it
template <int D, int W>
constexpr int ipw() { return kBN * SwzTile<D>::R / 64 / W; }

// Per-lane parts of every address the kernel forms.
template <int DK, int DV, int W>
struct LaneAddr {
  int k[DK / 32];             // K fragment base per k-step
  int v[DV / 16];             // V^T transposed-read base per 16-dim block
  int kld[ipw<DK, W>()];  // byte offset in the tile (2 (row DK + 8 chunk)) of each direct K load
  int vld[ipw<DV, W>()];

  __device__ __forceinline__ void init(int lane, int wave) {
    const int r16 = lane & 15, g = lane >> 4, e = (lane >> 2) & 3, r = lane & 3;
    // K fragment (key block kb, k-step t): row 16kb + r16, chunk 4t + g
#pragma unroll
    for (int t = 0; t < DK / 32; ++t) k[t] = r16 * SwzTile<DK>::ROW + 16 * ((4 * t + g) ^ swz<DK>(r16));
    // V^T read (dim block db, key row 32kt + 16h + 4g + e, bytes 8(r & 1) of
    // chunk 2db + r/2); 32kt + 16h leaves row % 8 and so the swizzle alone
#pragma unroll
    for (int db = 0; db < DV / 16; ++db)
      v[db] = (4 * g + e) * SwzTile<DV>::ROW + 16 * ((2 * db + (r >> 1)) ^ swz<DV>(4 * g + e)) + 8 * (r & 1);
#pragma unroll
    for (int i = 0; i < ipw<DK, W>(); ++i) {
      const int slot = (wave * ipw<DK, W>() + i) * 64 + lane;
      const int row = slot / SwzTile<DK>::R;
      kld[i] = 2 * (row * DK + ((slot % SwzTile<DK>::R) ^ swz<DK>(row)) * 8);
    }
#pragma unroll
    for (int i = 0; i < ipw<DV, W>(); ++i) {
      const int slot = (wave * ipw<DV, W>() + i) * 64 + lane;
      const int row = slot / SwzTile<DV>::R;
      vld[i] = 2 * (row * DV + ((slot % SwzTile<DV>::R) ^ swz<DV>(row)) * 8);
    }
  }
};

// One head's K (or V): base address and byte size, turned into a buffer
// resource at each load so that the hardware range check covers the head.
struct HeadBuf {
  const uint16_t* base;
  uint32_t bytes;
};
__device__ __forceinline__ HeadBuf head_buf(const uint16_t* base, uint32_t bytes) { return HeadBuf{base, bytes}; }

// Direct-to-LDS loads (buffer_load_dwordx4 ... lds) of this wave's share of
// the tile whose first key row is row0: a uniform byte offset plus each
// lane's fixed offset in the tile, no per-load address arithmetic.  Lanes
// past the end of the head fail the range check and write zeros: those keys
// are masked (p = 0), and zero V rows add nothing.
template <int D, int IPW>
__device__ __forceinline__ void load_tile(const HeadBuf& b, int row0, const int* ld, lds_char* dst, int wave) {
#pragma unroll
  for (int i = 0; i < IPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)b.base, (short)0, (int)b.bytes, 0x00020000),
        (lds_void*)(dst + (wave * IPW + i) * 1024), 16, ld[i], row0 * D * 2, 0, 0);
}

template <int DK>
struct QFrag {
  bf16x8 f[2][DK / 32];  // [query block][k-step]: dims 32t + 8g .. +7
};

// 16 bytes of a head's Q at byte offset off; zeros at or past `bytes` (the
// hardware range check), so rows past Nq need no branch.
__device__ __forceinline__ u32x4 load_q16(const uint16_t* qbh, uint32_t bytes, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(
      __builtin_amdgcn_make_buffer_rsrc((void*)qbh, (short)0, (int)bytes, 0x00020000), off, 0, 0);
}

// S^T (keys x queries) of one tile: s[kb][qb] is the 16x16 block of key
// block kb and query block qb; a lane holds keys 16kb + 4g + j of query
// 16qb + lane % 16.
template <int DK, int DV, int W>
__device__ __forceinline__ void qk_tile(f32x4 (&s)[4][2], const QFrag<DK>& q, const lds_char* kt,
                                        const LaneAddr<DK, DV, W>& la) {
  constexpr int ROW = SwzTile<DK>::ROW;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // k-step outermost: consecutive MFMAs feed eight different accumulators,
  // so none waits on the result of the one issued just before it
#pragma unroll
  for (int t = 0; t < DK / 32; ++t) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8 a = *(const lds_bf16x8*)(kt + la.k[t] + 16 * kb * ROW);
      s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q.f[0][t], s[kb][0], 0, 0, 0);
      s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q.f[1][t], s[kb][1], 0, 0, 0);
    }
  }
#if FA_FAST_PACE
  // keep at most four K fragments in flight: four reads, then (2 MFMAs,
  // read); measured against two and eight ahead: 1-2% faster than either
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
  for (int i = 0; i < 4 * DK / 32; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    if (i + 4 < 4 * DK / 32) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
  }
#endif
}

struct RowState {
  float m[2];   // reference maximum (base 2) per query block
  float l[2];   // this lane's share (4 of the 64 keys of each tile) of the denominator
  float lu[2];  // the same share summed over the bf16-rounded weights that multiply V
};


// O^T += V^T P^T for one tile: k-step kt covers keys 32kt .. 32kt+31, slot
// s of lane group g holding key 32kt + 16(s/4) + 4g + s%4.
// With SUM, osum[qb] also accumulates the query block's sum of the rounded
// weights, as products with a block of ones (every entry of the 16x16 result
// is a query's sum).
template <int DK, int DV, int W, bool SUM>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[DV / 16][2], f32x4 (&osum)[2], const bf16x8 (&pb)[2][2],
                                        const lds_char* vt, const LaneAddr<DK, DV, W>& la) {
  constexpr int ROW = SwzTile<DV>::ROW;
  if (SUM) {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      osum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[kt][0], osum[0], 0, 0, 0);
      osum[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[kt][1], osum[1], 0, 0, 0);
    }
  }
  // k-step outermost: consecutive MFMAs feed different accumulators
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) {
      const lds_char* p = vt + la.v[db] + 32 * kt * ROW;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * ROW));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[kt][0], o[db][0], 0, 0, 0);
      o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[kt][1], o[db][1], 0, 0, 0);
    }
  }
#if FA_FAST_PACE
  // per V fragment: 2 transposed reads, 2 MFMAs, two fragments read ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
  for (int i = 0; i < DV / 8; ++i) {
    if (i + 2 < DV / 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
  }
#endif
}

// Softmax of one tile in place: mask, running reference, exponentials and P
// in bf16.  alpha[qb] receives the factor the value sums must be multiplied
// by; the return value says whether any row of the wave moved its reference.
// VSUM: also sum the rounded weights here (st.lu, v_dot2 against ones).
template <bool MASK, bool BIAS, bool DROP, bool VSUM>
__device__ __forceinline__ bool softmax_tile(f32x4 (&s)[4][2], bf16x8 (&pb)[2][2], RowState& st, float (&alpha)[2],
                                             float c, int n0, const int (&row_lo)[2],
                                             const unsigned (&row_span)[2], const float* const (&brow)[2],
                                             const bool (&rvalid)[2], int nk, bool vec_bias, int g,
                                             const Philox4 (&zw)[2], int keep) {
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
        if (MASK && (unsigned)(key0 + j - row_lo[qb]) >= row_span[qb]) x = kNegInf;
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
    float psum = 0.f, usum = 0.f;
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
        if (DROP) {
          // word kb of the query block's generator call: byte j keeps key 16kb + 4g + j
          const uint32_t zb = zw[qb].x[kb];
#pragma unroll
          for (int j = 0; j < 4; ++j) p[j] = dropout_keep(zb, j, keep) ? p[j] : 0.f;
        }
        w[2 * h] = cvt_pk_bf16(p[0], p[1]);
        w[2 * h + 1] = cvt_pk_bf16(p[2], p[3]);
        if (VSUM) usum = add_bf16_pair(w[2 * h + 1], add_bf16_pair(w[2 * h], usum));
      }
      pb[kt][qb] = __builtin_bit_cast(bf16x8, w);
    }
    st.l[qb] = fmaf(alpha[qb], st.l[qb], psum);
    if (VSUM) st.lu[qb] = fmaf(alpha[qb], st.lu[qb], usum);
  }
  return __builtin_amdgcn_ballot_w64(any_grow) != 0;
}

template <int DK, int DV, bool BIAS, bool DROP, int W>
struct FwdTile {
  // inputs of this work-group
  HeadBuf kbuf, vbuf;  // this head's K and V
  int nk, n_tiles;  // n_tiles: one past the last tile the work-group visits
  float c;
  int qrow0;    // global index of this lane's row in query block 0 (block 1: +16)
  int klen;     // keys of this sequence
  KeyRange mr;  // position masks; row ranges are rebuilt only for masked tiles
  DropoutSpec dsp;  // DROP only
  uint32_t bh;      // b*H + h, a dropout counter word
  bool rvalid[2];
  const float* brow[2];
  int vec_bias, g;
  // per-thread state
  LaneAddr<DK, DV, W> la;
  QFrag<DK> qf;
  f32x4 o[DV / 16][2];
  // Without dropout O is divided by the sum of the rounded weights that
  // multiply V.  Eight-wave work-groups take it on the matrix cores (osum,
  // 4 more products per tile), four-wave ones on the vector ALU (st.lu):
  // measured each way, 200 calls, the matrix cores were 1.5% faster on the
  // prefill and long context (eight waves) and 0.7% slower on the
  // sliding window (four).
  static constexpr bool MSUM = !DROP && W == 8;
  static constexpr bool VSUM = !DROP && W != 8;
  f32x4 osum[2];
  RowState st;
  int wfirst, wlast;  // this wave's first and last query row (wlast < wfirst: none)

  // One tile t (K_t and V_t in kcur / vcur) while tile t+1 loads into
  // knext / vnext: S^T, softmax, rescale, O += P V, then the barrier that
  // publishes tile t+1 and frees tile t's buffers.
  template <bool MASK>
  __device__ __forceinline__ void step(int t, int wave, const lds_char* kcur, const lds_char* vcur,
                                       lds_char* knext, lds_char* vnext) {
    const int n0 = t * kBN;
    // the next tile's K now, its V after the S^T products (measured: 0.6%
    // faster on the sliding-window prefill than both at the step's start)
    const bool more = t + 1 < n_tiles;
    if (more) load_tile_async<DK, ipw<DK, W>()>(kbuf, n0 + kBN, la.kld, knext, wave);
    // A masked tile that none of this wave's rows can see changes nothing
    // (all its P are zero, the reference stays): skip its products.  The
    // row ranges only grow with the row, so the first row's lowest key and
    // the last row's end bound them all.
    if (MASK) {
      const bool dead = wlast < wfirst || key_end(mr, wlast, klen) <= n0 || key_lo(mr, wfirst) >= n0 + kBN;
      if (__builtin_amdgcn_readfirstlane((int)dead)) {
        if (more) load_tile_async<DV, ipw<DV, W>()>(vbuf, n0 + kBN, la.vld, vnext, wave);
        wait_loads();
        __syncthreads();
        return;
      }
    }
    f32x4 s[4][2];
    qk_tile<DK, DV, W>(s, qf, kcur, la);
    if (more) load_tile_async<DV, ipw<DV, W>()>(vbuf, n0 + kBN, la.vld, vnext, wave);
    Philox4 zw[2];
    if (DROP) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) zw[qb] = dropout_words(dsp, qrow0 + 16 * qb, t, bh, g);
    }
    bf16x8 pb[2][2];
    float alpha[2];
    int row_lo[2] = {0, 0};
    unsigned row_span[2] = {0u, 0u};
    bool grow;
    // A tile that needs the mask for some row of the work-group may still
    // lie inside every range of this wave's rows (the wave's 32 rows span
    // 32 positions, the work-group's 128 or 256): then this wave takes it
    // unmasked.  Its last row has the largest lowest key, its first row the
    // smallest end.
    if (MASK && __builtin_amdgcn_readfirstlane(
                    (int)(key_lo(mr, wlast) <= n0 && key_end(mr, wfirst, klen) >= n0 + kBN))) {
      grow = softmax_tile<false, BIAS, DROP, VSUM>(s, pb, st, alpha, c, n0, row_lo, row_span, brow, rvalid, nk,
                                             vec_bias != 0, g, zw, dsp.keep);
    } else {
      if (MASK) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int lo = key_lo(mr, qrow0 + 16 * qb), end = key_end(mr, qrow0 + 16 * qb, klen);
          row_lo[qb] = lo;
          row_span[qb] = end > lo ? (unsigned)(end - lo) : 0u;
        }
      }
      grow = softmax_tile<MASK, BIAS, DROP, VSUM>(s, pb, st, alpha, c, n0, row_lo, row_span, brow, rvalid, nk,
                                            vec_bias != 0, g, zw, dsp.keep);
    }
    if (grow) {
#pragma unroll
      for (int d = 0; d < DV / 16; ++d) {
        o[d][0] *= alpha[0];
        o[d][1] *= alpha[1];
      }
      if (MSUM) {
        osum[0] *= alpha[0];
        osum[1] *= alpha[1];
      }
    }
    pv_tile<DK, DV, W, MSUM>(o, osum, pb, vcur, la);
    wait_loads();
    __syncthreads();
  }
};

// The grid's tile order (map_tile's grouped, heaviest-first order) with its
// divisions by launch constants precomputed: group * n_qt and H.
struct FwdMap {
  FastDiv by_gq, by_h;
  int n_qt, n_bh, group;  // group: 1, 2 or 4 blocks
};

// x / d and x % d for d in 1..4
__device__ __forceinline__ int div_small(int x, int d) {
  return d == 3 ? (int)(((uint64_t)(uint32_t)x * 0xAAAAAAABull) >> 33) : x >> (d >> 1);
}

__device__ __forceinline__ TileCoord fwd_tile(int pid, int total, const FwdMap& fm, bool heavy_first) {
  const int lid = xcd_renumber(pid, total);
  const int gi = fast_div(lid, fm.by_gq);
  const int r = lid - gi * fm.group * fm.n_qt;
  const int gsz = min(fm.group, fm.n_bh - gi * fm.group);  // the last group may be smaller
  const int qi = div_small(r, gsz);
  TileCoord c;
  c.bh = gi * fm.group + (r - qi * gsz);
  c.qt = heavy_first ? (fm.n_qt - 1 - qi) : qi;
  return c;
}

template <int DK, int DV, bool BIAS, bool DROP, int W>
__global__ __launch_bounds__(threads_of<W>(), 2) void fwd_bf16_fast_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, uint16_t* __restrict__ o,
    float* __restrict__ lse, int H, int Nq, int Nk, float scale_log2, KeyRange mr, DropoutSpec dsp,
    float drop_scale, int vec_bias, FwdMap fm) {
  __shared__ __attribute__((aligned(1024))) char kbuf0[SwzTile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[SwzTile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[SwzTile<DV>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[SwzTile<DV>::BYTES];
  lds_char* K0 = (lds_char*)kbuf0;
  lds_char* K1 = (lds_char*)kbuf1;
  lds_char* V0 = (lds_char*)vbuf0;
  lds_char* V1 = (lds_char*)vbuf1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS destinations stay scalar
  const int r16 = lane & 15, g = lane >> 4;

  const TileCoord tc = fwd_tile(blockIdx.x, gridDim.x, fm, mr.wr >= 0);
  const int qt = tc.qt;
  const int b = fast_div(tc.bh, fm.by_h);
  constexpr int kBM = rows_of<W>();
  const int q0 = qt * kBM;
  const size_t bh = (size_t)tc.bh;
  const uint16_t* qbh = q + bh * Nq * DK;

  // The K and V buffers end at the sequence's key length: rows at or past
  // it fail the hardware range check and arrive as zeros, so they are never
  // read from memory (a non-finite value stored there cannot reach P V
  // through a zero weight).  Without key lengths there is nothing to wait
  // for; with them the first tile waits for one scalar load.
  const int klen = clamp_klen(k_len, b, Nk);
  FwdTile<DK, DV, BIAS, DROP, W> ft;
  ft.dsp = dsp;
  ft.bh = (uint32_t)tc.bh;
  ft.kbuf = head_buf(k + bh * Nk * DK, (uint32_t)klen * DK * 2);
  ft.vbuf = head_buf(v + bh * Nk * DV, (uint32_t)klen * DV * 2);
  ft.nk = Nk;
  ft.vec_bias = vec_bias;
  ft.g = g;
  ft.la.init(lane, wave);

  // The first K/V tile and Q load together, before anything waits on
  // memory (other than the key length, when given): the start of a
  // work-group then costs one memory latency.  The first tile's rows begin
  // at the first row's lowest visible key, which the key length does not
  // move; a query tile left with no key tile ignores the loaded tile.
  const int t_begin = key_lo(mr, q0) / kBN;
  const bool t0_in = t_begin < (Nk + kBN - 1) / kBN;
  if (t0_in) {
    load_tile<DK, ipw<DK, W>()>(ft.kbuf, t_begin * kBN, ft.la.kld, K0, wave);
    load_tile<DV, ipw<DV, W>()>(ft.vbuf, t_begin * kBN, ft.la.vld, V0, wave);
  }
  u32x4 qw[2][DK / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint32_t row = (uint32_t)(q0 + wave * 32 + qb * 16 + r16);
#pragma unroll
    for (int t = 0; t < DK / 32; ++t)
      qw[qb][t] = load_q16(qbh, (uint32_t)Nq * DK * 2, (row * DK + 32 * t + 8 * g) * 2);
  }

  int qrow[2];
  ft.qrow0 = q0 + wave * 32 + r16;
  ft.wfirst = q0 + wave * 32;
  ft.wlast = min(ft.wfirst + 31, Nq - 1);
  ft.klen = klen;
  ft.mr = mr;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = q0 + wave * 32 + qb * 16 + r16;
    ft.rvalid[qb] = qrow[qb] < Nq;
    ft.brow[qb] = BIAS ? bias + (bh * Nq + (size_t)(ft.rvalid[qb] ? qrow[qb] : 0)) * Nk : nullptr;
  }
  // tiles [t_begin, t_end) meet some row's range; tiles [t_full, t_full_end)
  // lie inside every row's range (the last row has the largest lo, the first
  // row the smallest end)
  const int last_row = min(q0 + kBM, Nq) - 1;
  const int kbeg = key_lo(mr, q0);
  const int kend = key_end(mr, last_row, klen);
  const int t_end = kend > kbeg ? (kend + kBN - 1) / kBN : t_begin;
  ft.n_tiles = t_end;

  // logit scale in the base-2 domain, made positive (a negative scale flips
  // the sign of Q, exactly; zero becomes a tiny positive value)
  const bool neg_scale = scale_log2 < 0.f;
  ft.c = fmaxf(fabsf(scale_log2), 1e-30f);
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) {
    ft.o[d][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    ft.o[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  ft.st.m[0] = ft.st.m[1] = kNegInf;
  ft.st.l[0] = ft.st.l[1] = 0.f;
  ft.st.lu[0] = ft.st.lu[1] = 0.f;
  ft.osum[0] = ft.osum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_loads();
  __syncthreads();
  {
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int t = 0; t < DK / 32; ++t) {
        u32x4 w = qw[qb][t];
        w[0] ^= flip; w[1] ^= flip; w[2] ^= flip; w[3] ^= flip;
        ft.qf.f[qb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  if (t_begin < t_end) {
    // Tile t sits in buffer 0 or 1 by the parity of t - t_begin.  The
    // unmasked run starts at an even distance from t_begin (a tile moved
    // into the masked run is still computed correctly), so it always starts
    // in buffer 0.
    const int lo_last = key_lo(mr, last_row);
    const int end_first = key_end(mr, q0, klen);
    int t_full = min(max((lo_last + kBN - 1) / kBN, t_begin), t_end);
    t_full = min(t_full + ((t_full - t_begin) & 1), t_end);
    const int t_full_end = max(min(end_first / kBN, t_end), t_full);
    int t = t_begin;
    for (; t < t_full; ++t) {  // along the left window edge
      if ((t - t_begin) & 1)
        ft.template step<true>(t, wave, K1, V1, K0, V0);
      else
        ft.template step<true>(t, wave, K0, V0, K1, V1);
    }
    for (; t + 1 < t_full_end; t += 2) {
      ft.template step<false>(t, wave, K0, V0, K1, V1);
      ft.template step<false>(t + 1, wave, K1, V1, K0, V0);
    }
    if (t < t_full_end) {
      ft.template step<false>(t, wave, K0, V0, K1, V1);
      ++t;
    }
    for (; t < t_end; ++t) {  // the diagonal / right edge and the key-length boundary
      if ((t - t_begin) & 1)
        ft.template step<true>(t, wave, K1, V1, K0, V0);
      else
        ft.template step<true>(t, wave, K0, V0, K1, V1);
    }
  }

  // ---- epilogue: divide once; empty rows get o = 0, lse = -inf ------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = quad_sum(ft.st.l[qb]);
    // O is divided by the sum of the weights it was built from (the
    // bf16-rounded ones), so it is an exact weighted mean of the values up
    // to fp32 rounding: a row dominated by one key then returns that key's
    // value instead of carrying the key's own rounding (up to 2^-9 of |v|).
    // lse keeps the sum of the unrounded weights.  With dropout the
    // divisor stays the unrounded sum of the undropped weights.
    const float l_out = DROP ? l_tot : (decltype(ft)::MSUM ? ft.osum[qb][0] : quad_sum(ft.st.lu[qb]));
    if (!ft.rvalid[qb]) continue;
    const bool nonempty = l_tot > 0.f;
    const float inv = nonempty ? (DROP ? drop_scale : 1.f) / l_out : 0.f;
    uint16_t* orow = o + (bh * Nq + qrow[qb]) * (size_t)DV;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      u32x2 w;
      w[0] = cvt_pk_bf16(ft.o[d][qb][0] * inv, ft.o[d][qb][1] * inv);
      w[1] = cvt_pk_bf16(ft.o[d][qb][2] * inv, ft.o[d][qb][3] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * d + 4 * g) = w;
    }
    if (lse != nullptr && g == 0)
      lse[bh * Nq + qrow[qb]] = nonempty ? (ft.st.m[qb] + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

// The same loads written as inline assembly, for the tile loop.  With the
// builtin, the compiler's wait insertion could not tell the tile a step
// reads from the tile it loads for the next step: it waited for the next
// tile's K loads before the first read of the current K tile and for all
// loads before the first V read, so the loads overlapped little of the
// step.  The compiler does not see these loads at all; each step waits for
// them itself (wait_loads) before the barrier that publishes the tile.  M0
// (the LDS base of a direct load) is set inside the same statement; the
// kernel uses M0 for nothing else after its first tile.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is a reserved register; clobbering it is intended
template <int D, int IPW>
__device__ __forceinline__ void load_tile_async(const HeadBuf& b, int row0, const int* ld, lds_char* dst, int wave) {
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)b.base, (short)0, (int)b.bytes, 0x00020000);
  const uint32_t soff = (uint32_t)(row0 * D * 2);
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(dst + (wave * IPW + i) * 1024);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(ld[i]), "s"(rsrc), "s"(soff) : "memory", "m0");
  }
}
#pragma clang diagnostic pop

template <int DK, int DV, bool BIAS, bool DROP, int W>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + rows_of<W>() - 1) / rows_of<W>();
  const long long total = (long long)n_qt * a.H * a.B;
  FwdMap fm;
  fm.n_qt = n_qt;
  fm.n_bh = a.B * a.H;
  fm.group = tile_group(a.wl < 0 && a.wr >= 0, fm.n_bh, (long long)a.Nk * (DK + DV) * 2);
  fm.by_gq = make_fastdiv((uint32_t)(fm.group * n_qt));
  fm.by_h = make_fastdiv((uint32_t)a.H);
  const bool vec_b = (a.Nk % 4 == 0) && (((uintptr_t)a.bias & 15) == 0);
  hipLaunchKernelGGL((fwd_bf16_fast_kernel<DK, DV, BIAS, DROP, W>), dim3((unsigned)total), dim3(threads_of<W>()), 0,
                     stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.bias, a.k_len,
                     (uint16_t*)a.o, a.lse, a.H, a.Nq, a.Nk, a.scale * kLog2e, KeyRange{a.off, a.wl, a.wr},
                     DropoutSpec{a.seed_lo, a.seed_hi, a.keep_256}, 256.f / (float)a.keep_256, (int)vec_b, fm);
  return hipGetLastError();
}

// Eight waves (256 query rows, one work-group per CU) halve the K/V tile
// loads and LDS writes per FLOP but tie eight waves to each barrier.
// Measured against four (200 calls, same box): causal prefill 1.2% and long
// context 1.7% faster, the dropout prefill equal, the 1024-key sliding
// window 5% slower (its work-groups visit few tiles, so a work-group's start
// and its masked edge tiles weigh more).  Eight are used for launches
// without a left window, bias or dropout whose query tiles fill more than
// 128 rows and that still give at least two work-groups per CU.
template <int DK, int DV>
hipError_t launch_b(const FwdArgs& a, hipStream_t s) {
  if (a.keep_256 < 256)
    return a.bias ? launch_t<DK, DV, true, true, 4>(a, s) : launch_t<DK, DV, false, true, 4>(a, s);
  if (a.bias) return launch_t<DK, DV, true, false, 4>(a, s);
  const long long wg8 = (long long)((a.Nq + rows_of<8>() - 1) / rows_of<8>()) * a.B * a.H;
  if (a.wl < 0 && a.Nq > rows_of<4>() && wg8 >= 512) return launch_t<DK, DV, false, false, 8>(a, s);
  return launch_t<DK, DV, false, false, 4>(a, s);
}

}  // namespace

bool fwd_bf16_fast_eligible(const FwdArgs& a) {
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  // buffer loads address a head's K and V with 32-bit byte offsets
  // (Q too, up to the last query tile of at most 256 rows)
  const bool fits = (long long)a.Nk * (a.dk > a.dv ? a.dk : a.dv) * 2 <= 0x7fffffffLL &&
                    ((long long)a.Nq + rows_of<8>()) * a.dk * 2 <= 0x7fffffffLL;
  return (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128) && a.Nk > 0 && fits && aligned(a.q) &&
         aligned(a.k) && aligned(a.v) && aligned(a.o) && a.block_n == kBN;
}

hipError_t launch_fwd_bf16_fast(const FwdArgs& a, hipStream_t s) {
  if (a.dk == 64 && a.dv == 64) return launch_b<64, 64>(a, s);
  if (a.dk == 64) return launch_b<64, 128>(a, s);
  if (a.dv == 64) return launch_b<128, 64>(a, s);
  return launch_b<128, 128>(a, s);
}

}  // namespace fa
