// Split-KV attention for a few query rows per sequence against a KV cache:
// chunked prefill or several speculative tokens at once.
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//
// Nq <= 16 query rows of sequence b are its last Nq positions, so with the
// causal flag row i sees keys j < k_len[b] with j <= i + k_len[b] - Nq (the
// bottom-right alignment of [GS] section 6, taken against the sequence's own
// length).  As in single-token decode the key axis is split into chunks
// ([GS] section 8, split KV loading for short queries): one work-group per
// (chunk, batch, head) forms every row's chunk state (m, l, u), and one merge
// per (batch, head, row) rebases and sums the states in ascending chunk
// order ([GS] section 4; [VW] Step 5) and divides once.  A (chunk, row) pair
// with no allowed key stores the empty state m = -inf, l = 0, u = 0, which
// the merge skips; a row with no allowed key at all gets o = 0, lse = -inf
// ([GS] section 6).
//
// Matrix-core path (bf16, dk = dv = 128): wave w owns keys 16w .. 16w+15 of
// every 64-key tile of the chunk, for all rows, and runs its own pipeline
// with two tiles in flight ahead of the one it consumes.  Its K rows go
// straight into registers in the A-operand layout of S^T = K Q^T
// (v_mfma_f32_16x16x32_bf16; a lane then holds 4 keys of one row); its V rows
// go into its own rows of a three-slot LDS ring, since O^T += V^T P^T
// (v_mfma_f32_16x16x16_bf16, whose B operand layout is exactly the S^T
// accumulator's, so P^T needs no data movement) wants V^T, which
// ds_read_b64_tr_b16 gives.  No wave reads another's rows, so the waves meet
// only at the end of the chunk, where their online states ([GS] section 5)
// are merged.  V is loaded nontemporal (each cache row is read once per
// call); K is not: its loads read 64 of a row's 256 bytes each, and the
// nontemporal form of those measured slower.
//
// General path (fp32 inputs, other head dims): the chunk state of each row
// by its definition -- logits to LDS, chunk maximum, then exponentials and
// the weighted value sum -- one row after another.
#include "fa_common.h"
#include "fa_merge.h"
#include "fa_tiles.h"
#include "launch.h"

namespace fa {
namespace {

using tiles::cvt_pk_bf16;
using tiles::HeadBuf;
using tiles::head_buf;
using tiles::kTile;
using tiles::kWaves;
using tiles::lds_char;
using tiles::load_tile;
using tiles::Tile;
using tiles::TileAddr;
using tiles::wait_loads;

constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 16;
constexpr int kMaxChunk = 2048;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) float lds_float;

// Keys visible to row i of nq against a sequence of klen keys.
__device__ __forceinline__ int row_key_end(int i, int nq, int klen, int causal) {
  if (i >= nq) return 0;
  return causal ? max(0, min(klen, i + klen - nq + 1)) : klen;
}

__device__ __forceinline__ size_t state_index(size_t bh, int c, int i, int max_chunks, int nq) {
  return (bh * max_chunks + c) * nq + i;
}

// ---------------------------------------------------------------------------
// general partial kernel
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__global__ __launch_bounds__(kThreads) void mq_partial_general_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ k_len,
    float* __restrict__ ws_u, float* __restrict__ ws_ml, int H, int BH, int Nq, int Nk, int dk, int dv, int chunk,
    int max_chunks, float scale_log2, int causal) {
  __shared__ float sc[kMaxChunk];
  __shared__ float qs[128];
  __shared__ float red[kThreads];
  const int tid = threadIdx.x;
  const int c = blockIdx.x / BH;
  const size_t bh = blockIdx.x - (size_t)c * BH;
  const int b = (int)(bh / H);
  const int klen = clamp_klen(k_len, b, Nk);
  const int c0 = c * chunk;
  if (c0 >= klen) return;  // the merge reads only chunks below k_len
  const T* kbh = k + bh * Nk * dk;
  const T* vbh = v + bh * Nk * dv;

  for (int i = 0; i < Nq; ++i) {
    const int len = min(c0 + chunk, row_key_end(i, Nq, klen, causal)) - c0;  // keys of this row in the chunk
    const size_t si = state_index(bh, c, i, max_chunks, Nq);
    float* wu = ws_u + si * dv;
    if (len <= 0) {  // empty state
      for (int d = tid; d < dv; d += kThreads) wu[d] = 0.f;
      if (tid == 0) {
        ws_ml[si * 2] = kNegInf;
        ws_ml[si * 2 + 1] = 0.f;
      }
      continue;
    }
    __syncthreads();  // previous row's readers of qs and sc are done
    for (int d = tid; d < dk; d += kThreads) qs[d] = ldf(q + (bh * Nq + i) * dk + d);
    __syncthreads();
    for (int j = tid; j < len; j += kThreads) {
      const T* kr = kbh + (size_t)(c0 + j) * dk;
      float s = 0.f;
      for (int d = 0; d < dk; ++d) s = fmaf(qs[d], ldf(kr + d), s);
      sc[j] = s * scale_log2;
    }
    __syncthreads();
    float mx = kNegInf;
    for (int j = tid; j < len; j += kThreads) mx = fmaxf(mx, sc[j]);
    red[tid] = mx;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
      __syncthreads();
    }
    const float m_c = red[0];
    __syncthreads();
    float ls = 0.f;
    for (int j = tid; j < len; j += kThreads) {
      const float p = fast_exp2(sc[j] - m_c);
      sc[j] = p;
      ls += p;
    }
    red[tid] = ls;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const float l_c = red[0];
    for (int d = tid; d < dv; d += kThreads) {
      float u = 0.f;
      for (int j = 0; j < len; ++j) u = fmaf(sc[j], ldf(vbh + (size_t)(c0 + j) * dv + d), u);
      wu[d] = u;
    }
    if (tid == 0) {
      ws_ml[si * 2] = m_c;
      ws_ml[si * 2 + 1] = l_c;
    }
  }
}

// ---------------------------------------------------------------------------
// matrix-core partial kernel (bf16, dk = dv = 128)
// ---------------------------------------------------------------------------

constexpr int kD = 128;
constexpr int kStages = 3;  // V ring slots: two tiles in flight ahead of the consumed one

// max / sum over the four lanes q, q+16, q+32, q+48 that share a row
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

template <int S>
__global__ __launch_bounds__(kThreads, 3) void mq_partial_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ k_len, float* __restrict__ ws_u, float* __restrict__ ws_ml, int H, int BH, int Nq,
    int Nk, int chunk, int max_chunks, float scale_log2, int causal) {
  constexpr int ROW = Tile<kD>::ROW;
  static_assert(S >= 2 && S <= 4, "the end-of-chunk merge uses two ring buffers; four slots at most");
  // V ring of S tile buffers; wave w only ever writes and reads rows
  // 16w .. 16w+15 of each, so the waves run their pipelines independently.
  // Separate arrays, not one indexed array: the compiler then knows that a
  // read of one slot does not wait for the direct loads into another.
  __shared__ __attribute__((aligned(1024))) char vr0[Tile<kD>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vr1[Tile<kD>::BYTES];
  __shared__ __attribute__((aligned(1024))) char vr2[S > 2 ? Tile<kD>::BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char vr3[S > 3 ? Tile<kD>::BYTES : 1];
  const auto vring = [&](int s) -> lds_char* {
    return (lds_char*)(s == 0 ? vr0 : s == 1 ? vr1 : s == 2 ? vr2 : vr3);
  };
  __shared__ float red_ml[kWaves][kMaxRows][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int c = blockIdx.x / BH;
  const size_t bh = blockIdx.x - (size_t)c * BH;
  const int b = (int)(bh / H);
  const int klen = clamp_klen(k_len, b, Nk);
  const int c0 = c * chunk;
  if (c0 >= klen) return;  // the merge reads only chunks below k_len

  const bool rvalid = r16 < Nq;
  bf16x8 qf[kD / 32];
#pragma unroll
  for (int t = 0; t < kD / 32; ++t)
    qf[t] = rvalid ? *reinterpret_cast<const bf16x8*>(q + (bh * Nq + r16) * kD + 32 * t + 8 * g) : bf16x8{};
  const int row_end = row_key_end(r16, Nq, klen, causal);
  const int c_end = min(c0 + chunk, klen);
  const int n_tiles = (c_end - c0 + kTile - 1) / kTile;

  TileAddr<kD> ta;
  ta.init(lane, wave);
  // the chunk's rows of K and V as buffers ending at c_end: loads past it
  // fail the hardware range check and arrive as zeros without a memory
  // access, so the pipeline below issues its loads unconditionally
  const uint32_t cbytes = (uint32_t)(c_end - c0) * kD * 2;
  const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + (bh * Nk + c0) * kD), (short)0, (int)cbytes,
                                                    0x00020000);
  const HeadBuf vh = head_buf(v + (bh * Nk + c0) * kD, cbytes);
  // K straight into registers in the A-operand layout of the S^T product:
  // lane (r16, g) holds key 16 wave + r16, dims 32i + 8g .. +7 for k-step i
  const uint32_t k_lane = (uint32_t)((16 * wave + r16) * ROW + 16 * g);

  float m = kNegInf, l = 0.f;  // this wave's state for row r16 (l: this lane's share)
  f32x4 o[kD / 16];            // O^T: dims 16db + 4g + j of row r16
#pragma unroll
  for (int d = 0; d < kD / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kr[S][kD / 32];
  auto issue = [&](int t, u32x4 (&kx)[kD / 32], lds_char* vdst) {
#pragma unroll
    for (int i = 0; i < kD / 32; ++i)
      kx[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (uint32_t)(t * kTile * ROW) + k_lane + 64 * i, 0, 0);
    load_tile<kD, tiles::kNonTemporal>(vh, t * kTile, ta.ld, vdst, wave);
  };
  auto compute = [&](int t, const u32x4 (&kx)[kD / 32], const lds_char* vt) {
    // S^T for this wave's 16 keys: a lane holds keys 16 wave + 4g + j of row r16
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kD / 32; ++i)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx[i]), qf[i], sc, 0, 0, 0);
    const int key0 = c0 + t * kTile + 16 * wave + 4 * g;
    float x[4];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = (key0 + j < row_end) ? sc[j] * scale_log2 : kNegInf;
      mx = fmaxf(mx, x[j]);
    }
    const float m_new = fmaxf(m, quad_max(mx));
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);  // 0 from the empty state
    m = m_new;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(x[j] - m_use);
    l = fmaf(alpha, l, (p[0] + p[1]) + (p[2] + p[3]));
    const u32x2 pw = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])};
    const v4i16 pb = __builtin_bit_cast(v4i16, pw);
    // O^T += V^T P^T over these 16 keys: V^T (dims 16db + lane % 16, keys 4g + e)
#pragma unroll
    for (int d = 0; d < kD / 16; ++d) {
      o[d] *= alpha;
      const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vt + ta.tr[d] + 16 * wave * ROW));
      o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[d], 0, 0, 0);
    }
  };

  // S - 1 tiles in flight ahead of the one being consumed; tile t uses ring
  // slot t % S (the loop is unrolled by S so every slot is a compile-time
  // address)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, kr[s], vring(s));
  for (int t0 = 0; t0 < n_tiles; t0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int t = t0 + s;
      if (t >= n_tiles) break;
      issue(t + S - 1, kr[(s + S - 1) % S], vring((s + S - 1) % S));
      compute(t, kr[s], vring(s));
    }
  }

  // merge the four waves' states per row ([GS] section 4) through LDS
  l = quad_sum(l);
  wait_loads();
  __syncthreads();  // ring buffers are free
  // [wave][row][dim]: waves 0 and 1 in ring slot 0, waves 2 and 3 in slot 1
  const auto red_u = [&](int w) { return (lds_float*)(vring(w >> 1) + (w & 1) * kMaxRows * kD * 4); };
  lds_float* const mine = red_u(wave);
#pragma unroll
  for (int d = 0; d < kD / 16; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[r16 * kD + 16 * d + 4 * g + j] = o[d][j];
  if (g == 0) {
    red_ml[wave][r16][0] = m;
    red_ml[wave][r16][1] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < Nq * kD; idx += kThreads) {
    const int i = idx / kD, dd = idx - i * kD;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, red_ml[w][i][0]);
    const float mu = (mm == kNegInf) ? 0.f : mm;
    float u = 0.f, ll = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = fast_exp2(red_ml[w][i][0] - mu);
      u = fmaf(a, red_u(w)[i * kD + dd], u);
      ll = fmaf(a, red_ml[w][i][1], ll);
    }
    const size_t si = state_index(bh, c, i, max_chunks, Nq);
    ws_u[si * kD + dd] = u;
    if (dd == 0) {
      ws_ml[si * 2] = mm;
      ws_ml[si * 2 + 1] = ll;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one wave per (batch, head, row)
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ T store_elem(float x);
template <>
__device__ __forceinline__ float store_elem<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t store_elem<uint16_t>(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

template <typename T>
__global__ __launch_bounds__(64) void mq_merge_kernel(const float* __restrict__ ws_u, const float* __restrict__ ws_ml,
                                                      const int32_t* __restrict__ k_len, T* __restrict__ o,
                                                      float* __restrict__ lse, int H, int Nq, int Nk, int dv,
                                                      int chunk, int max_chunks) {
  const size_t row = blockIdx.x;  // (b, h, i)
  const int i = (int)(row % Nq);
  const size_t bh = row / Nq;
  const int b = (int)(bh / H);
  const int klen = clamp_klen(k_len, b, Nk);
  const int n_c = (klen + chunk - 1) / chunk;
  const size_t s0 = state_index(bh, 0, i, max_chunks, Nq);  // chunk c: s0 + c * Nq
  merge_chunk_states(ws_u + s0 * dv, (size_t)Nq * dv, ws_ml + s0 * 2, (size_t)Nq * 2, n_c, dv, o + row * dv,
                     lse != nullptr ? lse + row : nullptr, [](float x) { return store_elem<T>(x); });
}

template <typename T>
hipError_t launch_mq(const DecodeMqArgs& a, hipStream_t stream, bool mfma) {
  const int BH = a.B * a.H;
  const long long n_part = (long long)BH * a.max_chunks;
  if (n_part > 0) {
    if (mfma)
      hipLaunchKernelGGL(mq_partial_bf16_kernel<kStages>, dim3((unsigned)n_part), dim3(kThreads), 0, stream,
                         (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.k_len, a.ws_u, a.ws_ml,
                         a.H, BH, a.Nq, a.Nk, a.chunk, a.max_chunks, a.scale * kLog2e, a.causal);
    else
      hipLaunchKernelGGL(mq_partial_general_kernel<T>, dim3((unsigned)n_part), dim3(kThreads), 0, stream,
                         (const T*)a.q, (const T*)a.k, (const T*)a.v, a.k_len, a.ws_u, a.ws_ml, a.H, BH, a.Nq, a.Nk,
                         a.dk, a.dv, a.chunk, a.max_chunks, a.scale * kLog2e, a.causal);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mq_merge_kernel<T>, dim3((unsigned)((long long)BH * a.Nq)), dim3(64), 0, stream, a.ws_u,
                     a.ws_ml, a.k_len, (T*)a.o, a.lse, a.H, a.Nq, a.Nk, a.dv, a.chunk, a.max_chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mq_bf16(const DecodeMqArgs& a, hipStream_t s) {
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  // each chunk's K and V rows are read through buffer descriptors of their
  // own (64-bit base at the chunk), so only one chunk must fit their 31-bit
  // byte range, not the whole head
  const bool mfma = a.dk == kD && a.dv == kD && aligned(a.q) && aligned(a.k) && aligned(a.v) &&
                    tiles::head_fits(a.chunk < a.Nk ? a.chunk : a.Nk, kD);
  return launch_mq<uint16_t>(a, s, mfma);
}
hipError_t launch_decode_mq_f32(const DecodeMqArgs& a, hipStream_t s) { return launch_mq<float>(a, s, false); }

}  // namespace fa
