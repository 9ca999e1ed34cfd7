// Single-token decode against a KV cache, split over key chunks.
//
// Sources, cited by title and section:
//   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
//   [VW] "Flash attention and efficient attention: Visual walkthrough"
//
// With one query row there is nothing to reuse: every cached key and value
// is read once, so the pass is bound by HBM bandwidth ([GS] section 8, the
// single-token decode case).  To spread one row's keys over the whole chip
// the key axis is split into chunks ([GS] section 8, split KV loading for
// short queries):
//
//   partial kernel  one work-group per (batch, head, chunk) that holds at
//                   least one allowed key.  It computes the chunk's own state
//                   (m_c, l_c, u_c) by its definition ([VW] Step 4): pass 1
//                   streams K and writes the chunk's logits to LDS, the chunk
//                   maximum is reduced, pass 2 streams V and accumulates
//                   u_c = sum exp(t - m_c) v.  Inside a chunk the maximum is
//                   known before any exponential is taken, so no rescaling is
//                   needed there.
//   merge kernel    one wave per (batch, head): rebases every chunk state to
//                   the common maximum and sums, in ascending chunk order
//                   ([GS] section 4; [VW] Step 5), then divides once.  A
//                   sequence with no key gets o = 0, lse = -inf ([GS]
//                   section 6).
//
// Logits are carried in the base-2 domain (t = s * log2 e), so m_c is a
// base-2 maximum and lse = ln2 * (m + log2 l).
#include "fa_common.h"
#include "fa_merge.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunk = 2048;  // LDS logit buffer (8 KiB)

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {
  static constexpr int VEC = 8;  // elements per 16-byte load
  __device__ static void load(const uint16_t* row, int d0, int d, bool vec, float* out) {
    if (vec) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (d0 < d) w = *reinterpret_cast<const u32x4*>(row + d0);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        out[2 * p] = bf16_lo(w[p]);
        out[2 * p + 1] = bf16_hi(w[p]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = (d0 + e < d) ? bf16_to_f32(row[d0 + e]) : 0.f;
    }
  }
  __device__ static uint16_t store(float x) { return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
};

template <>
struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ static void load(const float* row, int d0, int d, bool vec, float* out) {
    if (vec) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if (d0 < d) w = *reinterpret_cast<const f32x4*>(row + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = w[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (d0 + e < d) ? row[d0 + e] : 0.f;
    }
  }
  __device__ static float store(float x) { return x; }
};

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane
// of a group ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = 1; off < G; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename T, int DKP, int DVP>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ k_len,
    float* __restrict__ ws_u, float* __restrict__ ws_ml, int H, int Nk, int dk, int dv, int chunk, int max_chunks,
    float scale_log2, int vec_k, int vec_v) {
  using E = Elem<T>;
  constexpr int VEC = E::VEC;
  constexpr int LPK = DKP / VEC;  // lanes per K row
  constexpr int RPK = 64 / LPK;   // K rows per wave load
  constexpr int LPV = DVP / VEC;
  constexpr int RPV = 64 / LPV;
  __shared__ float sc[kMaxChunk];
  __shared__ float red[4][DVP];
  __shared__ float stat[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bhi = blockIdx.x / max_chunks;
  const int c = blockIdx.x - bhi * max_chunks;
  const int b = bhi / H;
  const int klen = clamp_klen(k_len, b, Nk);
  const int c0 = c * chunk;
  if (c0 >= klen) return;  // no allowed key in this chunk: no state
  const int len = min(chunk, klen - c0);

  const size_t bh = (size_t)bhi;
  const T* kbh = k + bh * Nk * dk;
  const T* vbh = v + bh * Nk * dv;

  // ---- pass 1: logits of the chunk (base 2) ------------------------------
  float qf[VEC];
  E::load(q + bh * dk, (lane % LPK) * VEC, dk, vec_k != 0, qf);
  const int n_groups_k = (len + RPK - 1) / RPK;
#pragma unroll 4
  for (int g = wave; g < n_groups_k; g += 4) {
    const int r = g * RPK + lane / LPK;  // row within the chunk
    float kf[VEC];
    if (r < len) {
      E::load(kbh + (size_t)(c0 + r) * dk, (lane % LPK) * VEC, dk, vec_k != 0, kf);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) kf[e] = 0.f;
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = fmaf(qf[e], kf[e], dot);
    dot = group_sum<LPK>(dot);
    if ((lane % LPK) == 0 && r < len) sc[r] = dot * scale_log2;
  }
  __syncthreads();

  // ---- chunk maximum and denominator ----------------------------------
  float mx = kNegInf;
  for (int j = tid; j < len; j += kThreads) mx = fmaxf(mx, sc[j]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) stat[wave] = mx;
  __syncthreads();
  const float m_c = fmaxf(fmaxf(stat[0], stat[1]), fmaxf(stat[2], stat[3]));
  float ls = 0.f;
  for (int j = tid; j < len; j += kThreads) ls += fast_exp2(sc[j] - m_c);
  ls = group_sum<64>(ls);
  if (lane == 0) stat[4 + wave] = ls;

  // ---- pass 2: u_c = sum_j exp2(t_j - m_c) v_j ----------------------------
  float u[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) u[e] = 0.f;
  const int n_groups_v = (len + RPV - 1) / RPV;
#pragma unroll 4
  for (int g = wave; g < n_groups_v; g += 4) {
    const int r = g * RPV + lane / LPV;
    if (r < len) {
      float vf[VEC];
      E::load(vbh + (size_t)(c0 + r) * dv, (lane % LPV) * VEC, dv, vec_v != 0, vf);
      const float p = fast_exp2(sc[r] - m_c);
#pragma unroll
      for (int e = 0; e < VEC; ++e) u[e] = fmaf(p, vf[e], u[e]);
    }
  }
  // lanes holding the same dims: reduce across the rows of a wave
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
#pragma unroll
    for (int off = LPV; off < 64; off <<= 1) u[e] += __shfl_xor(u[e], off);
  }
  if (lane < LPV) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[wave][lane * VEC + e] = u[e];
  }
  __syncthreads();
  float* wu = ws_u + (bh * max_chunks + c) * (size_t)dv;
  for (int d = tid; d < dv; d += kThreads) wu[d] = red[0][d] + red[1][d] + red[2][d] + red[3][d];
  if (tid == 0) {
    float* wml = ws_ml + (bh * max_chunks + c) * 2;
    wml[0] = m_c;
    wml[1] = stat[4] + stat[5] + stat[6] + stat[7];
  }
}

template <typename T>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ ws_u,
                                                          const float* __restrict__ ws_ml,
                                                          const int32_t* __restrict__ k_len, T* __restrict__ o,
                                                          float* __restrict__ lse, int H, int Nk, int dv, int chunk,
                                                          int max_chunks) {
  const int bhi = blockIdx.x;
  const int b = bhi / H;
  const int klen = clamp_klen(k_len, b, Nk);
  const int n_c = (klen + chunk - 1) / chunk;
  const size_t base = (size_t)bhi * max_chunks;
  merge_chunk_states(ws_u + base * dv, (size_t)dv, ws_ml + base * 2, 2, n_c, dv, o + (size_t)bhi * dv,
                     lse != nullptr ? lse + bhi : nullptr, [](float x) { return Elem<T>::store(x); });
}

// ---------------------------------------------------------------------------
// Fast partial kernel for bf16 with dk = dv = 128 and 16-byte aligned
// tensors.  One pass streams K and V together: each 256-byte key row is
// spread over 16 lanes (16 bytes each) and four consecutive rows fill a
// wave-wide load, so K and V rows sit in the same lanes and the probability
// of a row is already in the lanes that hold its value row.  Each of the
// four 16-lane row groups of a wave keeps its own online state (m, l, u)
// over the rows it sees (the pages' sequential update, [GS] section 5);
// the states are merged once at the end -- across the row groups, then
// across the waves through LDS -- with the rule of [GS] section 4.
// Work-groups are numbered chunk-major, so the (b, h, chunk) triples past a
// sequence's length -- which exit at once -- cluster at the end of the grid.
constexpr int kFastD = 128;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes of a DPP row: xor 1, xor 2, then mirrors
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Taking the element by value matters: a bit cast applied directly to an
// indexed element of a vector held by reference was lowered as a cast of
// element 0.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2_t, x); }

__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b) {
  float d = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[p]), as_bf16x2(b[p]), d, false);
  return d;
}

struct DecState {
  float m, l, u[8];
};

// merge with the state held by lane ^ off ([GS] section 4); an empty state
// (m = -inf) contributes nothing
__device__ __forceinline__ void merge_lanes(DecState& st, int off) {
  const float m_o = __shfl_xor(st.m, off);
  const float l_o = __shfl_xor(st.l, off);
  const float m_new = fmaxf(st.m, m_o);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float a = fast_exp2(st.m - m_use), bo = fast_exp2(m_o - m_use);
  st.l = a * st.l + bo * l_o;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.u[e] = a * st.u[e] + bo * __shfl_xor(st.u[e], off);
  st.m = m_new;
}

__global__ __launch_bounds__(kThreads) void decode_partial_fast_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ k_len, float* __restrict__ ws_u, float* __restrict__ ws_ml, int H, int BH, int Nk,
    int chunk, int max_chunks, float scale_log2) {
  constexpr int D = kFastD;
  __shared__ float red_u[4][D];
  __shared__ float red_ml[4][2];
  // uniform: the buffer descriptors below stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x / BH;
  const int bhi = blockIdx.x - c * BH;
  const int b = bhi / H;
  const int klen = clamp_klen(k_len, b, Nk);
  const int c0 = c * chunk;
  if (c0 >= klen) return;  // no allowed key in this chunk: no state
  const int len = min(chunk, klen - c0);

  const size_t bh = (size_t)bhi;
  const int col = lane & 15, grp = lane >> 4;  // 16-byte column of a row; row group
  const u32x4 qf = *reinterpret_cast<const u32x4*>(q + bh * D + col * 8);

  // rows of this wave: one quarter of the chunk (a multiple of 16 rows)
  const int quarter = chunk / 4;
  const int r_begin = wave * quarter;
  const int r_end = min(r_begin + quarter, len);
  // This wave's rows of K and V as buffers of r_end - r_begin rows: a load
  // at or past r_end fails the hardware range check and returns zeros, so
  // the loads need no branch (rows of other waves and rows at or past the
  // key length are never read).  Cache policy 2 = nontemporal: every cache
  // row is read once per call.
  const uint32_t bytes = (uint32_t)max(r_end - r_begin, 0) * D * 2;
  const size_t first = (bh * Nk + c0 + r_begin) * D;
  const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + first), (short)0, (int)bytes, 0x00020000);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + first), (short)0, (int)bytes, 0x00020000);
  const uint32_t lane_off = (uint32_t)(grp * D * 2 + col * 16);

  DecState st;
  st.m = kNegInf;
  st.l = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.u[e] = 0.f;

  // kSteps 16-row steps per iteration: their 8 * kSteps loads are issued
  // together, so each wave keeps that many in flight (measured on the
  // decode workload: 4 steps 1.2% faster than 1 step of guarded loads)
  constexpr int kSteps = 4;
  for (int r00 = r_begin; r00 < r_end; r00 += 16 * kSteps) {
    u32x4 kv[kSteps][4], vv[kSteps][4];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)(r00 - r_begin + 16 * s + 4 * i) * (D * 2) + lane_off;
        kv[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 2);
        vv[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 2);
      }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int r0 = r00 + 16 * s;
      float sc[4];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = row16_sum(dot8_bf16(kv[s][i], qf));
        sc[i] = (r0 + 4 * i + grp < r_end) ? d * scale_log2 : kNegInf;
        mx = fmaxf(mx, sc[i]);
      }
      const float m_new = fmaxf(st.m, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(st.m - m_use);
      st.m = m_new;
      float psum = 0.f;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(sc[i] - m_use);
        psum += p[i];
      }
      st.l = fmaf(alpha, st.l, psum);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.u[e] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          st.u[2 * w] = fmaf(p[i], bf16_lo(vv[s][i][w]), st.u[2 * w]);
          st.u[2 * w + 1] = fmaf(p[i], bf16_hi(vv[s][i][w]), st.u[2 * w + 1]);
        }
      }
    }
  }

  // merge the four row groups of the wave, then the four waves
  merge_lanes(st, 16);
  merge_lanes(st, 32);
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_u[wave][col * 8 + e] = st.u[e];
    if (col == 0) {
      red_ml[wave][0] = st.m;
      red_ml[wave][1] = st.l;
    }
  }
  __syncthreads();
  if (tid < D) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, red_ml[w][0]);
    float l = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = fast_exp2(red_ml[w][0] - m);  // m is finite: the chunk holds a key
      l = fmaf(a, red_ml[w][1], l);
      u = fmaf(a, red_u[w][tid], u);
    }
    ws_u[(bh * max_chunks + c) * D + tid] = u;
    if (tid == 0) {
      float* wml = ws_ml + (bh * max_chunks + c) * 2;
      wml[0] = m;
      wml[1] = l;
    }
  }
}

template <typename T, int DKP, int DVP>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int vec = Elem<T>::VEC;
  const uintptr_t m16 = 15;
  const bool vec_k = (a.dk % vec == 0) && (((uintptr_t)a.k & m16) == 0) && (((uintptr_t)a.q & m16) == 0);
  const bool vec_v = (a.dv % vec == 0) && (((uintptr_t)a.v & m16) == 0);
  const long long n_part = (long long)a.B * a.H * a.max_chunks;
  if (n_part > 0) {
    hipLaunchKernelGGL((decode_partial_kernel<T, DKP, DVP>), dim3((unsigned)n_part), dim3(kThreads), 0, stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.k_len, a.ws_u, a.ws_ml, a.H, a.Nk, a.dk, a.dv,
                       a.chunk, a.max_chunks, a.scale * kLog2e, (int)vec_k, (int)vec_v);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<T>), dim3((unsigned)(a.B * a.H)), dim3(64), 0, stream, a.ws_u, a.ws_ml,
                     a.k_len, (T*)a.o, a.lse, a.H, a.Nk, a.dv, a.chunk, a.max_chunks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const bool k64 = a.dk <= 64, v64 = a.dv <= 64;
  if (k64 && v64) return launch_t<T, 64, 64>(a, s);
  if (k64) return launch_t<T, 64, 128>(a, s);
  if (v64) return launch_t<T, 128, 64>(a, s);
  return launch_t<T, 128, 128>(a, s);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const bool fast = a.dk == kFastD && a.dv == kFastD && aligned(a.q) && aligned(a.k) && aligned(a.v) &&
                    a.chunk % 64 == 0;
  if (!fast) return launch_d<uint16_t>(a, s);
  const long long n_part = (long long)a.B * a.H * a.max_chunks;
  if (n_part > 0) {
    hipLaunchKernelGGL(decode_partial_fast_kernel, dim3((unsigned)n_part), dim3(kThreads), 0, s, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, a.k_len, a.ws_u, a.ws_ml, a.H, a.B * a.H, a.Nk,
                       a.chunk, a.max_chunks, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_merge_kernel<uint16_t>), dim3((unsigned)(a.B * a.H)), dim3(64), 0, s, a.ws_u, a.ws_ml,
                     a.k_len, (uint16_t*)a.o, a.lse, a.H, a.Nk, a.dv, a.chunk, a.max_chunks);
  return hipGetLastError();
}
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) { return launch_d<float>(a, s); }

}  // namespace fa
