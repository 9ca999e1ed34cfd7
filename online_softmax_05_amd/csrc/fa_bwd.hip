// Attention backward by recomputation ([GS] section 7, "Why training need
// not save the full probability matrix"; [VW] Step 8, "Backward pass: the
// recompute trade").
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//
// The forward pass keeps only O and the per-row log-sum-exp L.  With the
// upstream gradient G (row g_i = dLoss/do_i) the gradients are rebuilt tile by
// tile, never storing P:
//
//   p_ij = exp(s_ij - L_i) on the allowed set, 0 elsewhere
//          (s_ij = scale q_i.k_j + b_ij, the forward's logit)
//   c_i  = g_i . o_i                      (softmax Jacobian row reduction)
//   D_ij = p_ij (g_i . v_j - c_i)         (gradient w.r.t. the scaled logit)
//   dV = P^T G,   dQ = scale D K,   dK = scale D^T Q
//
// Rows with lse = -inf (no allowed key) contribute nothing.  The bias is a
// fixed input (no gradient).  The position masks (causal in either
// alignment, sliding windows) are those of the forward (fa_mask.h).  With
// dropout ([GS] section 6: the backward replays the forward's mask and
// scaling) the forward used P~ = z r P (r = 256/keep, fa_dropout.h), so
// dV = P~^T G and D_ij = p_ij (z_ij r (g_i . v_j) - c_i), c_i = g_i . o_i
// with the dropped output.  Three launches, all deterministic (no
// atomics): c per row; dK and dV per key tile looping over query rows; dQ
// per query tile looping over key tiles.
//
// This file holds c and the general kernels: fp32 arithmetic for fp32 and
// bf16 inputs, any head dims 1..128, LDS-staged tiles.  bf16 inputs with head
// dims 64/128 take the matrix-core kernels of fa_bwd_bf16.hip.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_mask.h"
#include "launch.h"

namespace fa {
namespace {

template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ float to_elem<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t to_elem<uint16_t>(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

constexpr int kThreads = 256;
constexpr int kKeys = 32;  // keys per tile
constexpr int kRows = 16;  // query rows per tile

// c_i = g_i . o_i in fp32, one wave per row ([GS] section 7).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dot_kernel(const T* __restrict__ dout, const T* __restrict__ o,
                                                           float* __restrict__ c, long long rows, int dv) {
  const long long row = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // wave-uniform
  float acc = 0.f;
  for (int d = lane; d < dv; d += 64) acc += ldf(dout + row * dv + d) * ldf(o + row * dv + d);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) c[row] = acc;
}

// Shared-memory tiles of the general kernels (fp32, one padding column
// against bank conflicts).
struct GenTiles {
  float* ks;  // [kKeys][dk + 1]
  float* vs;  // [kKeys][dv + 1]
  float* qs;  // [kRows][dk + 1]
  float* gs;  // [kRows][dv + 1]   upstream gradient rows
  float* ps;  // [kRows][kKeys + 1]
  float* ds;  // [kRows][kKeys + 1]
  float* ls;  // [kRows] lse
  float* cs;  // [kRows] c
  __device__ GenTiles(float* sm, int dk, int dv) {
    ks = sm;
    vs = ks + kKeys * (dk + 1);
    qs = vs + kKeys * (dv + 1);
    gs = qs + kRows * (dk + 1);
    ps = gs + kRows * (dv + 1);
    ds = ps + kRows * (kKeys + 1);
    ls = ds + kRows * (kKeys + 1);
    cs = ls + kRows;
  }
  static size_t bytes(int dk, int dv) {
    return sizeof(float) *
           (size_t)(kKeys * (dk + 1) + kKeys * (dv + 1) + kRows * (dk + 1) + kRows * (dv + 1) + 2 * kRows * (kKeys + 1) +
                    2 * kRows);
  }
};

template <typename T>
__device__ __forceinline__ void load_rows(float* dst, int ld, const T* src, int first, int count, int limit, int d) {
  for (int idx = threadIdx.x; idx < count * d; idx += kThreads) {
    const int r = idx / d, e = idx - r * d;
    dst[r * ld + e] = (first + r < limit) ? ldf(src + (size_t)(first + r) * d + e) : 0.f;
  }
}

// P and D for the kRows x kKeys block (rows r0.., keys j0..), by definition
// from the forward's logit and the saved lse.  Each thread takes two
// (row, key) entries.
struct Geom {
  int nq, nk, klen;
  KeyRange mr;  // position masks (fa_mask.h)
  float scale;
  const float* bias_bh;  // [Nq, Nk] of this (b, h) or null
  DropoutSpec dsp;       // dropout (fa_dropout.h); keep == 256: none
  float drop_scale;      // 256 / keep
  uint32_t bh;
};

__device__ __forceinline__ void pd_block(const GenTiles& t, const Geom& g, int r0, int j0, int dk, int dv) {
  const int key = threadIdx.x % kKeys;
  const int j = j0 + key;
  for (int rr = threadIdx.x / kKeys; rr < kRows; rr += kThreads / kKeys) {
    const int row = r0 + rr;
    float s = 0.f, dp = 0.f;
    for (int e = 0; e < dk; ++e) s = fmaf(t.qs[rr * (dk + 1) + e], t.ks[key * (dk + 1) + e], s);
    for (int e = 0; e < dv; ++e) dp = fmaf(t.gs[rr * (dv + 1) + e], t.vs[key * (dv + 1) + e], dp);
    const float l = t.ls[rr];
    const bool ok = row < g.nq && j >= key_lo(g.mr, row) && j < key_end(g.mr, row, g.klen) && l != kNegInf;
    float p = 0.f;
    if (ok) {
      float x = s * g.scale;
      if (g.bias_bh != nullptr) x += g.bias_bh[(size_t)row * g.nk + j];
      p = fast_exp2((x - l) * kLog2e);  // exp(s_ij - L_i)
    }
    // dropout: the forward used z r p in place of p (r = 256/keep), so
    // dV takes z r p and D_ij = p (z r dP_ij - c_i)
    const float zr = (g.dsp.keep < 256 && !dropout_keep_at(g.dsp, row, j, g.bh)) ? 0.f : g.drop_scale;
    t.ps[rr * (kKeys + 1) + key] = zr * p;
    t.ds[rr * (kKeys + 1) + key] = p * (zr * dp - t.cs[rr]);  // D_ij
  }
}

// dK and dV of one kKeys-key tile: loop over the query rows that can see it.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_general_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ c, const float* __restrict__ bias,
    const int32_t* __restrict__ k_len, T* __restrict__ dk, T* __restrict__ dv, int H, int Nq, int Nk, int DK, int DV,
    float scale, KeyRange mr, DropoutSpec dsp, float drop_scale) {
  extern __shared__ float sm[];
  GenTiles t(sm, DK, DV);
  const size_t bh = blockIdx.y;
  const int b = (int)(bh / H);
  const int j0 = blockIdx.x * kKeys;
  Geom g{Nq, Nk, clamp_klen(k_len, b, Nk), mr, scale, bias == nullptr ? nullptr : bias + bh * Nq * (size_t)Nk,
         dsp, drop_scale, (uint32_t)bh};

  load_rows(t.ks, DK + 1, k + bh * Nk * DK, j0, kKeys, g.klen, DK);
  load_rows(t.vs, DV + 1, v + bh * Nk * DV, j0, kKeys, g.klen, DV);

  // this thread's outputs: key kk, dims sub + 8m
  const int kk = threadIdx.x >> 3, sub = threadIdx.x & 7;
  float acc_v[16], acc_k[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc_v[m] = acc_k[m] = 0.f;

  // rows that can see a key of this tile below klen ([GS] section 6: global
  // positions): key_end(r) > j0 and key_lo(r) <= the tile's last such key
  const int jl = min(j0 + kKeys, g.klen) - 1;
  const int r_lo = mr.wr >= 0 ? (int)max(0LL, (long long)j0 - mr.off - mr.wr) : 0;
  const int r_hi = j0 >= g.klen ? 0 : (mr.wl >= 0 ? (int)min((long long)Nq, (long long)jl - mr.off + mr.wl + 1) : Nq);
  for (int r0 = r_lo; r0 < r_hi; r0 += kRows) {
    __syncthreads();  // previous tile's readers are done
    load_rows(t.qs, DK + 1, q + bh * Nq * DK, r0, kRows, Nq, DK);
    load_rows(t.gs, DV + 1, dout + bh * Nq * DV, r0, kRows, Nq, DV);
    if (threadIdx.x < kRows) {
      const int row = r0 + threadIdx.x;
      t.ls[threadIdx.x] = row < Nq ? lse[bh * Nq + row] : kNegInf;
      t.cs[threadIdx.x] = row < Nq ? c[bh * Nq + row] : 0.f;
    }
    __syncthreads();
    pd_block(t, g, r0, j0, DK, DV);
    __syncthreads();
    for (int rr = 0; rr < kRows; ++rr) {
      const float p = t.ps[rr * (kKeys + 1) + kk], d = t.ds[rr * (kKeys + 1) + kk];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int e = sub + 8 * m;
        if (e < DV) acc_v[m] = fmaf(p, t.gs[rr * (DV + 1) + e], acc_v[m]);  // dV += P^T G
        if (e < DK) acc_k[m] = fmaf(d, t.qs[rr * (DK + 1) + e], acc_k[m]);  // dK += D^T Q
      }
    }
  }
  const int j = j0 + kk;
  if (j < Nk) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int e = sub + 8 * m;
      if (e < DV) dv[(bh * Nk + j) * DV + e] = to_elem<T>(acc_v[m]);
      if (e < DK) dk[(bh * Nk + j) * DK + e] = to_elem<T>(acc_k[m] * scale);
    }
  }
}

// dQ of one kRows-row tile: loop over the key tiles its rows can see.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dq_general_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ c, const float* __restrict__ bias,
    const int32_t* __restrict__ k_len, T* __restrict__ dq, int H, int Nq, int Nk, int DK, int DV, float scale,
    KeyRange mr, DropoutSpec dsp, float drop_scale) {
  extern __shared__ float sm[];
  GenTiles t(sm, DK, DV);
  const size_t bh = blockIdx.y;
  const int b = (int)(bh / H);
  const int r0 = blockIdx.x * kRows;
  Geom g{Nq, Nk, clamp_klen(k_len, b, Nk), mr, scale, bias == nullptr ? nullptr : bias + bh * Nq * (size_t)Nk,
         dsp, drop_scale, (uint32_t)bh};

  load_rows(t.qs, DK + 1, q + bh * Nq * DK, r0, kRows, Nq, DK);
  load_rows(t.gs, DV + 1, dout + bh * Nq * DV, r0, kRows, Nq, DV);
  if (threadIdx.x < kRows) {
    const int row = r0 + threadIdx.x;
    t.ls[threadIdx.x] = row < Nq ? lse[bh * Nq + row] : kNegInf;
    t.cs[threadIdx.x] = row < Nq ? c[bh * Nq + row] : 0.f;
  }
  // this thread's outputs: row rr, dims sub + 16m
  const int rr = threadIdx.x >> 4, sub = threadIdx.x & 15;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.f;

  // key tiles that meet the union of the rows' ranges
  const int kbeg = key_lo(mr, r0);
  const int kend = key_end(mr, min(r0 + kRows, Nq) - 1, g.klen);
  for (int j0 = (kbeg / kKeys) * kKeys; j0 < kend; j0 += kKeys) {
    __syncthreads();
    load_rows(t.ks, DK + 1, k + bh * Nk * DK, j0, kKeys, g.klen, DK);
    load_rows(t.vs, DV + 1, v + bh * Nk * DV, j0, kKeys, g.klen, DV);
    __syncthreads();
    pd_block(t, g, r0, j0, DK, DV);
    __syncthreads();
    for (int kk = 0; kk < kKeys; ++kk) {
      const float d = t.ds[rr * (kKeys + 1) + kk];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int e = sub + 16 * m;
        if (e < DK) acc[m] = fmaf(d, t.ks[kk * (DK + 1) + e], acc[m]);  // dQ += D K
      }
    }
  }
  const int row = r0 + rr;
  if (row < Nq) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int e = sub + 16 * m;
      if (e < DK) dq[(bh * Nq + row) * DK + e] = to_elem<T>(acc[m] * scale);
    }
  }
}

template <typename T>
void launch_dot(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  if (rows > 0)
    hipLaunchKernelGGL(bwd_dot_kernel<T>, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, stream,
                       (const T*)a.dout, (const T*)a.o, a.ws_c, rows, a.dv);
}

template <typename T>
hipError_t launch_general(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  const unsigned bh = (unsigned)(a.B * a.H);
  launch_dot<T>(a, stream);
  const size_t smem = GenTiles::bytes(a.dk, a.dv);
  if (a.Nk > 0)  // with no query rows this writes dK = dV = 0
    hipLaunchKernelGGL(bwd_dkdv_general_kernel<T>, dim3((unsigned)((a.Nk + kKeys - 1) / kKeys), bh), dim3(kThreads),
                       smem, stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse, a.ws_c,
                       a.bias, a.k_len, (T*)a.dk_out, (T*)a.dv_out, a.H, a.Nq, a.Nk, a.dk, a.dv, a.scale,
                       KeyRange{a.off, a.wl, a.wr}, DropoutSpec{a.seed_lo, a.seed_hi, a.keep_256},
                       256.f / (float)a.keep_256);
  if (rows > 0)
    hipLaunchKernelGGL(bwd_dq_general_kernel<T>, dim3((unsigned)((a.Nq + kRows - 1) / kRows), bh), dim3(kThreads),
                       smem, stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse, a.ws_c,
                     a.bias, a.k_len, (T*)a.dq_out, a.H, a.Nq, a.Nk, a.dk, a.dv, a.scale, KeyRange{a.off, a.wl, a.wr},
                     DropoutSpec{a.seed_lo, a.seed_hi, a.keep_256}, 256.f / (float)a.keep_256);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t s) { return launch_general<float>(a, s); }

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (!bwd_bf16_mfma_eligible(a)) return launch_general<uint16_t>(a, s);
  return launch_bwd_bf16_mfma(a, s);  // forms c itself
}

}  // namespace fa
