// Attention backward by recomputation on the matrix cores: bf16 inputs, head
// dims 64 or 128 ([GS] section 7, "Why training need not save the full
// probability matrix"; [VW] Step 8, "Backward pass: the recompute trade").
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//
//   p_ij = exp(s_ij - L_i) on the allowed set, 0 elsewhere,  c_i = g_i . o_i
//   D_ij = p_ij (g_i . v_j - c_i)
//   dV = P^T G,   dK = scale D^T Q,   dQ = scale D K
//
// Two kernels, dQ first: it also forms c_i for its rows (each lane holds a
// quarter of a row of G and of O) and stores it for the dK/dV kernel that
// follows on the same stream.  Neither uses atomics, so the results are
// bitwise reproducible.
//
// dQ kernel: one work-group = 8 waves = 256 query rows of one (batch, head)
// (4 waves = 128 rows with a bias or dropout),
// 32 rows per wave (two 16-row blocks, so that every K or V fragment read
// from LDS feeds two products) with their Q and G rows held as MFMA
// operands.  Key tiles
// of 64 keys stream through LDS (direct-to-LDS loads, double buffered), and
// per tile each wave forms
//   S^T  = K Q^T     (v_mfma_f32_16x16x32_bf16; a lane holds 4 keys of one row)
//   dP^T = V G^T
//   D^T  = P^T o (dP^T - c)
//   dQ^T += K^T D^T  (K^T read transposed from LDS with ds_read_b64_tr_b16;
//                     D^T rounded to bf16 is directly the B operand)
// dK/dV kernel: one work-group = 8 waves = 128 keys (4 waves = 64 keys with
// a bias or dropout), 16 keys per wave with their K and V rows as MFMA
// operands; query tiles of 64 rows (Q, G, L, c) stream through LDS, and per
// tile each wave forms
//   S = Q K^T, dP = G V^T, P, D  (a lane holds 4 rows of one key)
//   dV^T += G^T P,  dK^T += Q^T D   (G^T, Q^T read transposed from LDS)
// P and D are rounded to bf16 only as matrix-core operands; every sum is
// fp32.
//
// Both grids are one-dimensional and XCD-aware (map_tile): the 8 XCDs each
// take a contiguous range of (batch*head, tile) work-groups, so the tiles of
// one head that run at the same time share an L2 and its re-read K/V (dQ) or
// Q/dO (dK/dV) tiles; the dQ kernel issues a head's causal tiles heaviest
// first.
//
// Position masks are the forward's visible key range [lo, end) per row
// (fa_mask.h); both kernels visit only tiles that meet some row's range and
// test elements only on edge tiles.  Dropout (a separate instance; [GS]
// section 6: the backward replays the forward's mask and scaling): with
// r = 256/keep and z the counter-based mask of fa_dropout.h, dV takes z r P
// and D = P o (z r dP - c).  In the dQ kernel a lane's 16 keys of a tile are
// one generator call; in the dK/dV kernel a lane holds one key of 16 rows,
// so each thread generates one call per query tile (row tid / 4, group
// tid % 4) into LDS, a tile ahead, and lanes read back the bytes they need.
#include <type_traits>

#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_mask.h"
#include "fa_tiles.h"
#include "launch.h"

namespace fa {
namespace {

using tiles::HeadBuf;
using tiles::head_buf;
using tiles::kTile;
using tiles::Tile;
using tiles::TileAddr;
using tiles::lds_char;
using tiles::cvt_pk_bf16;
using tiles::frag_read;
using tiles::load_tile;
using tiles::tr_read;
using tiles::wait_loads;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Operand rows held in registers: row `row` of a [*, D] bf16 tensor as the
// B operand of 16x16x32 products over D (dims 32t + 8g .. +7).
template <int D>
__device__ __forceinline__ void load_rows_b(bf16x8 (&f)[D / 32], const uint16_t* base, int row, bool valid, int g) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
    f[t] = valid ? *reinterpret_cast<const bf16x8*>(base + (size_t)row * D + 32 * t + 8 * g) : bf16x8{};
}

// Pack two 16x16 accumulator blocks (h = 0, 1) of fp32 values into the
// bf16 B operand of a 16x16x32 product whose 32-long k axis is the blocks'
// row axis: slot s of lane group g holds row 16(s/4) + 4g + s%4.
__device__ __forceinline__ bf16x8 pack_b(const f32x4& a, const f32x4& b) {
  u32x4 w;
  w[0] = cvt_pk_bf16(a[0], a[1]);
  w[1] = cvt_pk_bf16(a[2], a[3]);
  w[2] = cvt_pk_bf16(b[0], b[1]);
  w[3] = cvt_pk_bf16(b[2], b[3]);
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

template <int DK, int DV, bool BIAS, bool DROP, int W>
__global__ __launch_bounds__(64 * W, 2) void bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ cvec,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, uint16_t* __restrict__ dq, int H, int Nq,
    int Nk, float scale, KeyRange mr, DropoutSpec dsp, float drop_scale) {
  // separate arrays per buffer, each selected at compile time (the loop
  // below is unrolled by two), so the compiler sees that a tile load in
  // flight never writes the buffer being read and adds no wait for it
  __shared__ __attribute__((aligned(1024))) char kb0[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[Tile<DV>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[Tile<DV>::BYTES];
  lds_char* const K0 = (lds_char*)kb0;
  lds_char* const K1 = (lds_char*)kb1;
  lds_char* const V0 = (lds_char*)vb0;
  lds_char* const V1 = (lds_char*)vb1;

  constexpr int kDqRows = 32 * W;  // query rows per work-group (32 per wave)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int n_qt = (Nq + kDqRows - 1) / kDqRows;
  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, n_qt, mr.wr >= 0,
                                tile_group(mr.wl < 0 && mr.wr >= 0, (int)(gridDim.x / n_qt),
                                           (long long)Nk * (DK + DV) * 2));
  const size_t bh = (size_t)tc.bh;
  const int b = (int)(bh / H);
  const int q0 = tc.qt * kDqRows;
  const int klen = clamp_klen(k_len, b, Nk);

  TileAddr<DK, W> ka;
  TileAddr<DV, W> va;
  ka.init(lane, wave);
  va.init(lane, wave);
  // rows at or past the key length read as zeros (never from memory)
  const HeadBuf kh = head_buf(k + bh * Nk * DK, (uint32_t)klen * DK * 2);
  const HeadBuf vh = head_buf(v + bh * Nk * DV, (uint32_t)klen * DV * 2);
  const float c2 = scale * kLog2e;

  // Each wave holds 32 query rows as two 16-row blocks qb: every K or V
  // fragment read from LDS feeds both blocks' products.  Per block: the Q
  // and G rows as B operands, L log2 e, c, the visible key range.
  int row[2];
  bool rvalid[2], live[2];
  bf16x8 qf[2][DK / 32], gf[2][DV / 32];
  float l2[2], c_row[2];
  int row_lo[2];
  unsigned row_span[2];
  const float* brow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    row[qb] = q0 + 32 * wave + 16 * qb + r16;
    rvalid[qb] = row[qb] < Nq;
    load_rows_b<DK>(qf[qb], q + bh * Nq * DK, row[qb], rvalid[qb], g);
    load_rows_b<DV>(gf[qb], dout + bh * Nq * DV, row[qb], rvalid[qb], g);
    const float l_row = rvalid[qb] ? lse[bh * Nq + row[qb]] : kNegInf;
    live[qb] = l_row != kNegInf;  // rows without an allowed key contribute nothing
    l2[qb] = live[qb] ? l_row * kLog2e : 0.f;
    // c_i = g_i . o_i: this lane's quarter of the row (dims 32t + 8g .. +7),
    // then the four lanes r16, r16 + 16, r16 + 32, r16 + 48 of the row
    float cr = 0.f;
    {
      bf16x8 of[DV / 32];
      load_rows_b<DV>(of, o + bh * Nq * DV, row[qb], rvalid[qb], g);
#pragma unroll
      for (int t = 0; t < DV / 32; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) cr = fmaf((float)gf[qb][t][e], (float)of[t][e], cr);
      cr += __shfl_xor(cr, 16);
      cr += __shfl_xor(cr, 32);
      if (rvalid[qb] && g == 0) cvec[bh * Nq + row[qb]] = cr;
    }
    c_row[qb] = cr;
    // this row's visible keys [row_lo, row_lo + row_span) (none for a dead row)
    row_lo[qb] = key_lo(mr, row[qb]);
    const int end = live[qb] ? key_end(mr, row[qb], klen) : 0;
    row_span[qb] = end > row_lo[qb] ? (unsigned)(end - row_lo[qb]) : 0u;
    brow[qb] = BIAS ? bias + (bh * Nq + (size_t)(rvalid[qb] ? row[qb] : 0)) * Nk : nullptr;
  }

  f32x4 acc[2][DK / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int d = 0; d < DK / 16; ++d) acc[qb][d] = f32x4{0.f, 0.f, 0.f, 0.f};

  // key tiles that meet the union of the rows' ranges; tiles in
  // [t_full, t_full_end) lie inside every row's range and need no mask
  const int last_row = min(q0 + kDqRows, Nq) - 1;
  const int kbeg = key_lo(mr, q0);
  const int kend = key_end(mr, last_row, klen);
  const int t_begin = kbeg / kTile;
  const int t_end = kend > kbeg ? (kend + kTile - 1) / kTile : t_begin;
  const int t_full = (key_lo(mr, last_row) + kTile - 1) / kTile;
  const int t_full_end = key_end(mr, q0, klen) / kTile;
  // a wave with a row past Nq or without an allowed key masks every tile
  const bool wave_all_live = __builtin_amdgcn_ballot_w64(!(live[0] && live[1])) == 0;

  // key tile t (in kt, vt) while tile t + 1 loads into kn, vn
  auto tile = [&](auto mask_c, int t, const lds_char* kt, const lds_char* vt, lds_char* kn, lds_char* vn) {
    constexpr bool masked = decltype(mask_c)::value;
    wait_loads();
    __syncthreads();  // tile t visible; tile t-1's buffers free
    const int j0 = t * kTile;
    if (t + 1 < t_end) {
      load_tile<DK, 0, W>(kh, j0 + kTile, ka.ld, kn, wave);
      load_tile<DV, 0, W>(vh, j0 + kTile, va.ld, vn, wave);
    }
    // a masked tile that none of this wave's rows can see adds nothing to
    // dQ (all its P are zero): skip its products (the row ranges only grow
    // with the row, so the first row's lowest key and the last row's end
    // bound them all)
    if (masked) {
      const int wfirst = q0 + 32 * wave, wlast = min(wfirst + 31, Nq - 1);
      const bool dead = wlast < wfirst || key_end(mr, wlast, klen) <= j0 || key_lo(mr, wfirst) >= j0 + kTile;
      if (__builtin_amdgcn_readfirstlane((int)dead)) return;
    }
    // S^T and dP^T: key block kb, a lane holds keys 16kb + 4g + j of row[qb]
    f32x4 s[4][2], dp[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = dp[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < DK / 32; ++i) {
        const bf16x8 a = frag_read(kt + ka.frag[i] + 16 * kb * Tile<DK>::ROW);
        s[kb][0] = mfma(a, qf[0][i], s[kb][0]);
        s[kb][1] = mfma(a, qf[1][i], s[kb][1]);
      }
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) {
        const bf16x8 a = frag_read(vt + va.frag[i] + 16 * kb * Tile<DV>::ROW);
        dp[kb][0] = mfma(a, gf[0][i], dp[kb][0]);
        dp[kb][1] = mfma(a, gf[1][i], dp[kb][1]);
      }
    }
    // P^T and D^T = P^T o (dP^T - c)   (dropout: P^T o (z r dP^T - c)),
    // written over s
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      Philox4 zw;
      // plain xors here: with the fused form the d = 128 dropout instance
      // spills 16 registers
      if (DROP) zw = dropout_words<false>(dsp, row[qb], t, (uint32_t)bh, g);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key0 = j0 + 16 * kb + 4 * g;
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) bv = load_bias4(brow[qb], key0, Nk, false, rvalid[qb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float arg = fmaf(s[kb][qb][j], c2, -l2[qb]);
          if (BIAS) arg = fmaf(bv[j], kLog2e, arg);
          float p = fast_exp2(arg);
          if (masked && (unsigned)(key0 + j - row_lo[qb]) >= row_span[qb]) p = 0.f;
          const float d = dp[kb][qb][j];
          const float dpz = DROP ? (dropout_keep(zw.x[kb], j, dsp.keep) ? drop_scale * d : 0.f) : d;
          s[kb][qb][j] = p * (dpz - c_row[qb]);
        }
      }
    }
    // dQ^T += K^T D^T over the tile's two 32-key steps
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      const bf16x8 bop0 = pack_b(s[2 * kt2][0], s[2 * kt2 + 1][0]);
      const bf16x8 bop1 = pack_b(s[2 * kt2][1], s[2 * kt2 + 1][1]);
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        const bf16x8 a = tr_read(kt + ka.tr[db] + 32 * kt2 * Tile<DK>::ROW, 16 * Tile<DK>::ROW);
        acc[0][db] = mfma(a, bop0, acc[0][db]);
        acc[1][db] = mfma(a, bop1, acc[1][db]);
      }
    }
  };
  if (t_begin < t_end) {
    load_tile<DK, 0, W>(kh, t_begin * kTile, ka.ld, K0, wave);
    load_tile<DV, 0, W>(vh, t_begin * kTile, va.ld, V0, wave);
  }
  // Tile t sits in buffer (t - t_begin) & 1.  Tiles [t_full, t_full_end)
  // need no mask (unless there is a bias, or a row of the wave is past Nq
  // or sees no key); the unmasked run starts at an even distance from
  // t_begin, in buffer 0 (a tile moved into a masked run is still computed
  // correctly).
  const std::true_type mask_on;
  const std::false_type mask_off;
  const bool any_full = !BIAS && wave_all_live;
  int tf = any_full ? min(max(t_full, t_begin), t_end) : t_end;
  tf = min(tf + ((tf - t_begin) & 1), t_end);
  const int tfe = any_full ? max(min(t_full_end, t_end), tf) : tf;
  int t = t_begin;
  for (; t < tf; ++t) {
    if ((t - t_begin) & 1)
      tile(mask_on, t, K1, V1, K0, V0);
    else
      tile(mask_on, t, K0, V0, K1, V1);
  }
  for (; t + 1 < tfe; t += 2) {
    tile(mask_off, t, K0, V0, K1, V1);
    tile(mask_off, t + 1, K1, V1, K0, V0);
  }
  if (t < tfe) {
    tile(mask_off, t, K0, V0, K1, V1);
    ++t;
  }
  for (; t < t_end; ++t) {
    if ((t - t_begin) & 1)
      tile(mask_on, t, K1, V1, K0, V0);
    else
      tile(mask_on, t, K0, V0, K1, V1);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!rvalid[qb]) continue;
    uint16_t* out = dq + (bh * Nq + row[qb]) * (size_t)DK;
#pragma unroll
    for (int d = 0; d < DK / 16; ++d) {
      u32x2 w;
      w[0] = cvt_pk_bf16(acc[qb][d][0] * scale, acc[qb][d][1] * scale);
      w[1] = cvt_pk_bf16(acc[qb][d][2] * scale, acc[qb][d][3] * scale);
      *reinterpret_cast<u32x2*>(out + 16 * d + 4 * g) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------

template <int DK, int DV, bool BIAS, bool DROP, int W>
__global__ __launch_bounds__(64 * W, 2) void bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ cvec,
    const float* __restrict__ bias, const int32_t* __restrict__ k_len, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int H, int Nq, int Nk, float scale, KeyRange mr, DropoutSpec dsp,
    float drop_scale) {
  // Q and G (= dO) tiles, double buffered in separate arrays selected at
  // compile time (the loop below is unrolled by two)
  __shared__ __attribute__((aligned(1024))) char qb0[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char qb1[Tile<DK>::BYTES];
  __shared__ __attribute__((aligned(1024))) char gb0[Tile<DV>::BYTES];
  __shared__ __attribute__((aligned(1024))) char gb1[Tile<DV>::BYTES];
  __shared__ __attribute__((aligned(16))) float lbuf[2][kTile];  // L_i log2 e (0 for rows without a key)
  __shared__ __attribute__((aligned(16))) float cbuf[2][kTile];  // c_i
  __shared__ int lobuf[2][kTile];       // per row: first visible key
  __shared__ unsigned spbuf[2][kTile];  // per row: number of visible keys (0 for rows without a key)
  // dropout words of the query tile: row rr, group g', word w at
  // [rr * kZRow + 4 g' + w] (kZRow = 17: odd stride, few bank conflicts)
  constexpr int kZRow = 17;
  __shared__ uint32_t zbuf[DROP ? 2 : 1][DROP ? kTile * kZRow : 1];
  lds_char* const Q0 = (lds_char*)qb0;
  lds_char* const Q1 = (lds_char*)qb1;
  lds_char* const G0 = (lds_char*)gb0;
  lds_char* const G1 = (lds_char*)gb1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  static_assert(W == 4 || (!BIAS && !DROP), "eight waves: plain instance only");
  constexpr int kKeys = 16 * W;  // keys per work-group, 16 per wave
  const TileCoord tc = map_tile(blockIdx.x, gridDim.x, (Nk + kKeys - 1) / kKeys, false);
  const size_t bh = (size_t)tc.bh;
  const int b = (int)(bh / H);
  const int j0 = tc.qt * kKeys;
  const int klen = clamp_klen(k_len, b, Nk);
  const int key = j0 + 16 * wave + r16;  // this lane's key
  const bool kvalid = key < Nk;    // dK, dV rows written (zero past the key length)
  const bool kread = key < klen;   // K, V rows read: none at or past the key length

  TileAddr<DK, W> qa;
  TileAddr<DV, W> ga;
  qa.init(lane, wave);
  ga.init(lane, wave);
  const HeadBuf qh = head_buf(q + bh * Nq * DK, (uint32_t)Nq * DK * 2);
  const HeadBuf gh = head_buf(dout + bh * Nq * DV, (uint32_t)Nq * DV * 2);

  bf16x8 kf[DK / 32], vf[DV / 32];
  load_rows_b<DK>(kf, k + bh * Nk * DK, key, kread, g);
  load_rows_b<DV>(vf, v + bh * Nk * DV, key, kread, g);
  const float c2 = scale * kLog2e;

  f32x4 acc_v[DV / 16], acc_k[DK / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) acc_v[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < DK / 16; ++d) acc_k[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  // query tiles whose rows can see a key of this work-group below klen:
  // key_end(r) > j0 and key_lo(r) <= key_last
  const int key_last = min(j0 + kKeys, klen) - 1;
  const int r_lo = mr.wr >= 0 ? (int)max(0LL, (long long)j0 - mr.off - mr.wr) : 0;
  const int r_hi = j0 >= klen ? 0 : (mr.wl >= 0 ? (int)min((long long)Nq, (long long)key_last - mr.off + mr.wl + 1) : Nq);
  const int t0 = r_lo / kTile;
  const int t_end = r_hi > r_lo ? (r_hi + kTile - 1) / kTile : t0;
  const int n_tiles = max(t_end - t0, 0);

  // Per-row values of query tile qt, staged in LDS by threads 0..63: the
  // loads (fetch_rows) are issued before the tile loads, and the LDS writes
  // (store_rows) come after the products, so that waiting for these few
  // values never waits for the tiles in flight.
  struct Rows {
    float l, c;
  };
  auto fetch_rows = [&](int qt) {
    Rows w{kNegInf, 0.f};
    const int r = qt * kTile + tid;
    if (tid < kTile && r < Nq) {
      w.l = lse[bh * Nq + r];
      w.c = cvec[bh * Nq + r];
    }
    return w;
  };
  auto store_rows = [&](const Rows& w, int qt, int buf) {
    if (tid < kTile) {
      const int r = qt * kTile + tid;
      const bool live = w.l != kNegInf;
      lbuf[buf][tid] = live ? w.l * kLog2e : 0.f;
      cbuf[buf][tid] = w.c;
      const int lo = key_lo(mr, r), end = live ? key_end(mr, r, klen) : 0;
      lobuf[buf][tid] = lo;
      spbuf[buf][tid] = end > lo ? (unsigned)(end - lo) : 0u;
    }
    if (DROP) {
      // one generator call per thread: row tid / 4 of the tile, group tid % 4
      const Philox4 zw = dropout_words(dsp, qt * kTile + (tid >> 2), j0 / kTile, (uint32_t)bh, tid & 3);
      uint32_t* z = &zbuf[buf][(tid >> 2) * kZRow + 4 * (tid & 3)];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = zw.x[e];
    }
  };

  // query tile it (in qt_l, gt_l, row values in buffer par) while tile
  // it + 1 loads into qn, gn
  // no mask when every row of the tile exists and sees every key of the group
  // (with a bias every tile is masked; with dropout an unmasked copy spills
  // registers and a masked copy that selects per element ran 12% slower
  // than testing the mask per tile, so the dropout kernel keeps that)
  constexpr bool kSplit = !BIAS && !DROP;
  const auto tile_masked = [&](int qt) {
    const int q0 = qt * kTile;
    return BIAS || q0 + kTile > Nq || key_last < j0 + kKeys - 1 || key_lo(mr, q0 + kTile - 1) > j0 ||
           key_end(mr, q0, klen) < j0 + kKeys;
  };
  auto tile = [&](auto mask_c, int it, const lds_char* qt_l, const lds_char* gt_l, lds_char* qn, lds_char* gn,
                  int par) {
    // split runs: the mask as the run says; otherwise the test per tile (a
    // uniform branch per element, cheaper here than a select per element)
    const int qt = t0 + it;
    const bool masked = kSplit ? decltype(mask_c)::value : tile_masked(qt);
    wait_loads();
    __syncthreads();  // tile it and its row values visible; tile it-1's buffers free
    const int q0 = qt * kTile;
    const bool more = it + 1 < n_tiles;
    Rows nxt{kNegInf, 0.f};
    if (more) {
      nxt = fetch_rows(qt + 1);
      load_tile<DK, 0, W>(qh, q0 + kTile, qa.ld, qn, wave);
      load_tile<DV, 0, W>(gh, q0 + kTile, ga.ld, gn, wave);
    }
    // S and dP: row block rb, a lane holds rows 16rb + 4g + j of `key`
    f32x4 s[4], dp[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      s[rb] = dp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < DK / 32; ++i) s[rb] = mfma(frag_read(qt_l + qa.frag[i] + 16 * rb * Tile<DK>::ROW), kf[i], s[rb]);
#pragma unroll
      for (int i = 0; i < DV / 32; ++i) dp[rb] = mfma(frag_read(gt_l + ga.frag[i] + 16 * rb * Tile<DV>::ROW), vf[i], dp[rb]);
    }
    f32x4 pv[4], dsv[4];
    const auto p_and_d = [&](auto mask_t) {
      constexpr bool mtest = decltype(mask_t)::value;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      // the four rows 16rb + 4g .. +3 of this lane: one 16-byte read each
      const f32x4 lv = *reinterpret_cast<const f32x4*>(&lbuf[par][16 * rb + 4 * g]);
      const f32x4 cv = *reinterpret_cast<const f32x4*>(&cbuf[par][16 * rb + 4 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * rb + 4 * g + j;  // row within the tile
        float arg = fmaf(s[rb][j], c2, -lv[j]);
        if (BIAS) {
          const int r = min(q0 + rr, Nq - 1);
          arg = fmaf(bias[(bh * Nq + r) * (size_t)Nk + min(key, Nk - 1)], kLog2e, arg);
        }
        float p = fast_exp2(arg);
        if (mtest && (unsigned)(key - lobuf[par][rr]) >= spbuf[par][rr]) p = 0.f;
        float zr = 1.f;
        if (DROP) {
          // byte r16 % 4 of word `wave` of row rr's call for group r16 / 4
          const uint32_t w = zbuf[par][rr * kZRow + 4 * (r16 >> 2) + wave];
          zr = dropout_keep(w, r16 & 3, dsp.keep) ? drop_scale : 0.f;
        }
        pv[rb][j] = zr * p;
        dsv[rb][j] = p * (zr * dp[rb][j] - cv[j]);
      }
    }
    };
    if (masked)
      p_and_d(std::true_type{});
    else
      p_and_d(std::false_type{});
    // dV^T += G^T P and dK^T += Q^T D over the tile's two 32-row steps
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const bf16x8 pop = pack_b(pv[2 * k2], pv[2 * k2 + 1]);
      const bf16x8 dop = pack_b(dsv[2 * k2], dsv[2 * k2 + 1]);
#pragma unroll
      for (int db = 0; db < DV / 16; ++db)
        acc_v[db] = mfma(tr_read(gt_l + ga.tr[db] + 32 * k2 * Tile<DV>::ROW, 16 * Tile<DV>::ROW), pop, acc_v[db]);
#pragma unroll
      for (int db = 0; db < DK / 16; ++db)
        acc_k[db] = mfma(tr_read(qt_l + qa.tr[db] + 32 * k2 * Tile<DK>::ROW, 16 * Tile<DK>::ROW), dop, acc_k[db]);
    }
    if (more) store_rows(nxt, qt + 1, par ^ 1);
  };
  if (n_tiles > 0) {
    load_tile<DK, 0, W>(qh, t0 * kTile, qa.ld, Q0, wave);
    load_tile<DV, 0, W>(gh, t0 * kTile, ga.ld, G0, wave);
    store_rows(fetch_rows(t0), t0, 0);
  }
  // The unmasked query tiles form one run [ia, ib) (each condition above
  // holds on a prefix or a suffix of the tiles): bounds from the mask's
  // closed form, then tightened with the exact test at both ends.  Tile it
  // sits in buffer it & 1; the unmasked run starts at an even it, in buffer
  // 0 (a tile moved into a masked run is still computed correctly).
  int ia = n_tiles, ib = n_tiles;
  if (kSplit && n_tiles > 0 && key_last >= j0 + kKeys - 1) {
    long long lo = t0, hi = min((long long)t0 + n_tiles, (long long)(Nq / kTile));
    if (mr.wr >= 0) lo = max(lo, ((long long)j0 + kKeys - 1 - mr.off - mr.wr + 64LL * kTile) / kTile - 64);
    if (mr.wl >= 0) {
      const long long x = (long long)j0 - (kTile - 1) - mr.off + mr.wl;  // q0 <= x
      hi = min(hi, x < 0 ? lo : x / kTile + 1);
    }
    int a = (int)max(lo, (long long)t0), b = (int)max(min(hi, (long long)t0 + n_tiles), (long long)a);
    while (a < b && tile_masked(a)) ++a;
    while (b > a && tile_masked(b - 1)) --b;
    ia = a - t0;
    ib = b - t0;
    ia = min(ia + (ia & 1), ib);
    if (ia == ib) ia = ib = n_tiles;
  }
  const std::true_type mask_on;
  const std::false_type mask_off;
  int it = 0;
  if (!kSplit) {
    for (; it < n_tiles; it += 2) {
      tile(mask_on, it, Q0, G0, Q1, G1, 0);
      if (it + 1 < n_tiles) tile(mask_on, it + 1, Q1, G1, Q0, G0, 1);
    }
  } else {
    for (; it < ia; ++it) {
      if (it & 1)
        tile(mask_on, it, Q1, G1, Q0, G0, 1);
      else
        tile(mask_on, it, Q0, G0, Q1, G1, 0);
    }
    for (; it + 1 < ib; it += 2) {
      tile(mask_off, it, Q0, G0, Q1, G1, 0);
      tile(mask_off, it + 1, Q1, G1, Q0, G0, 1);
    }
    if (it < ib) {
      tile(mask_off, it, Q0, G0, Q1, G1, 0);
      ++it;
    }
    for (; it < n_tiles; ++it) {
      if (it & 1)
        tile(mask_on, it, Q1, G1, Q0, G0, 1);
      else
        tile(mask_on, it, Q0, G0, Q1, G1, 0);
    }
  }

  if (kvalid) {
    uint16_t* ov = dv + (bh * Nk + key) * (size_t)DV;
    uint16_t* ok = dk + (bh * Nk + key) * (size_t)DK;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      u32x2 w;
      w[0] = cvt_pk_bf16(acc_v[d][0], acc_v[d][1]);
      w[1] = cvt_pk_bf16(acc_v[d][2], acc_v[d][3]);
      *reinterpret_cast<u32x2*>(ov + 16 * d + 4 * g) = w;
    }
#pragma unroll
    for (int d = 0; d < DK / 16; ++d) {
      u32x2 w;
      w[0] = cvt_pk_bf16(acc_k[d][0] * scale, acc_k[d][1] * scale);
      w[1] = cvt_pk_bf16(acc_k[d][2] * scale, acc_k[d][3] * scale);
      *reinterpret_cast<u32x2*>(ok + 16 * d + 4 * g) = w;
    }
  }
}

template <int DK, int DV, bool BIAS, bool DROP>
hipError_t launch_t(const BwdArgs& a, hipStream_t stream) {
  // dK/dV work-groups of 8 waves (128 keys) share each Q/G tile among twice
  // the keys: half the tile loads and LDS writes per product.  Measured
  // against 4 waves on the causal 4x32x4096 d = 128 backward (100 calls x 3,
  // same box): 1.972 against 2.014 ms.  Bias and dropout instances keep 4
  // (their per-row LDS staging assumes 64 keys per work-group).
  constexpr int KV_W = (BIAS || DROP) ? 4 : 8;
  const KeyRange mr{a.off, a.wl, a.wr};
  const DropoutSpec dsp{a.seed_lo, a.seed_hi, a.keep_256};
  const float drop_scale = 256.f / (float)a.keep_256;
  const unsigned bh = (unsigned)(a.B * a.H);
  // dQ first: it stores c for the dK/dV kernel
  // eight waves (256 query rows) per dQ work-group halve the K/V tile loads
  // per product for the plain instance: 1.875 against 1.892 ms per backward
  // call (100 calls x 3, same box)
  constexpr int QW = (BIAS || DROP) ? 4 : 8;
  if ((long long)a.B * a.H * a.Nq > 0)
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<DK, DV, BIAS, DROP, QW>),
                       dim3((unsigned)((a.Nq + 32 * QW - 1) / (32 * QW)) * bh), dim3(64 * QW), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.ws_c, a.bias, a.k_len,
                       (uint16_t*)a.dq_out, a.H, a.Nq, a.Nk, a.scale, mr, dsp, drop_scale);
  if (a.Nk > 0)
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DK, DV, BIAS, DROP, KV_W>),
                       dim3((unsigned)((a.Nk + 16 * KV_W - 1) / (16 * KV_W)) * bh), dim3(64 * KV_W), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.ws_c, a.bias, a.k_len, (uint16_t*)a.dk_out,
                       (uint16_t*)a.dv_out, a.H, a.Nq, a.Nk, a.scale, mr, dsp, drop_scale);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_b(const BwdArgs& a, hipStream_t s) {
  if (a.keep_256 < 256)
    return a.bias ? launch_t<DK, DV, true, true>(a, s) : launch_t<DK, DV, false, true>(a, s);
  return a.bias ? launch_t<DK, DV, true, false>(a, s) : launch_t<DK, DV, false, false>(a, s);
}

}  // namespace

bool bwd_bf16_mfma_eligible(const BwdArgs& a) {
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  // tiles are read with buffer loads: a head's Q, dO, K and V bytes must fit 31 bits
  const int dmax = a.dk > a.dv ? a.dk : a.dv;
  return (a.dk == 64 || a.dk == 128) && (a.dv == 64 || a.dv == 128) && aligned(a.q) && aligned(a.k) &&
         aligned(a.v) && aligned(a.dout) && aligned(a.dq_out) && aligned(a.dk_out) && aligned(a.dv_out) &&
         tiles::head_fits(a.Nq, dmax) && tiles::head_fits(a.Nk, dmax);
}

hipError_t launch_bwd_bf16_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.dk == 64 && a.dv == 64) return launch_b<64, 64>(a, s);
  if (a.dk == 64) return launch_b<64, 128>(a, s);
  if (a.dv == 64) return launch_b<128, 64>(a, s);
  return launch_b<128, 128>(a, s);
}

}  // namespace fa
