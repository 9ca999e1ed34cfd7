// Host front end of libfa.so: argument validation and kernel dispatch for
// the C ABI declared in include/fa.h.  Validation never dereferences a
// pointer and never touches the GPU, so the fa_check_* entry points run on
// machines without one.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>

#include "launch.h"

namespace {

constexpr int kMaxHeadDim = 128;
constexpr int kMaxChunk = 2048;
constexpr long long kInt32Max = std::numeric_limits<int32_t>::max();

bool product_fits(std::initializer_list<long long> xs, long long limit) {
  long long p = 1;
  for (long long x : xs) {
    if (x < 0) return false;
    if (x != 0 && p > limit / x) return false;
    p *= x;
  }
  return p <= limit;
}

int check_fwd(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len,
              const void* o, const float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype,
              float scale, int causal, int block_n) {
  (void)bias;
  (void)k_len;
  (void)lse;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (dk < 1 || dv < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (dk > kMaxHeadDim || dv > kMaxHeadDim) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (block_n != 0 && block_n != 32 && block_n != 64 && block_n != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_UNSUPPORTED;
  // element offsets are formed in 64 bits; grid sizes and per-(b,h) row
  // counts must fit the 32-bit launch and index arithmetic
  const long long n_qt = (Nq + 127LL) / 128;
  if (!product_fits({n_qt, H, B}, kInt32Max)) return FA_ERR_SHAPE;
  if (!product_fits({B, H}, kInt32Max)) return FA_ERR_SHAPE;
  if (Nq > kInt32Max - Nk) return FA_ERR_SHAPE;
  if ((long long)B * H * Nq == 0) return FA_OK;  // nothing to compute
  if (q == nullptr || o == nullptr) return FA_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL;
  return FA_OK;
}

int check_masks(int align, int window_left, int window_right, int keep_256) {
  if (align != FA_ALIGN_BOTTOM_RIGHT && align != FA_ALIGN_TOP_LEFT) return FA_ERR_UNSUPPORTED;
  if (window_left < -1 || window_right < -1) return FA_ERR_UNSUPPORTED;
  if (keep_256 < 1 || keep_256 > 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_fwd_ex(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len,
                 const void* o, const float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype,
                 float scale, int causal, int align, int window_left, int window_right, int keep_256,
                 int block_n) {
  const int st = check_masks(align, window_left, window_right, keep_256);
  if (st != FA_OK) return st;
  return check_fwd(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, block_n);
}

// The position masks folded into (off, wl, wr): causal is the right width 0,
// which is also the narrowest right window.
struct Masks {
  int off, wl, wr;
};
Masks fold_masks(int Nq, int Nk, int causal, int align, int window_left, int window_right) {
  return Masks{align == FA_ALIGN_BOTTOM_RIGHT ? Nk - Nq : 0, window_left, causal ? 0 : window_right};
}

fa::FwdArgs make_fwd_args(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len,
                          void* o, float* lse, int B, int H, int Nq, int Nk, int dk, int dv, float scale,
                          int causal, int align, int window_left, int window_right, int keep_256, uint64_t seed,
                          int block_n) {
  const Masks m = fold_masks(Nq, Nk, causal, align, window_left, window_right);
  fa::FwdArgs a{q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, scale, block_n == 0 ? 64 : block_n,
                m.off, m.wl, m.wr, keep_256, (uint32_t)seed, (uint32_t)(seed >> 32)};
  return a;
}

int launch_fwd(const fa::FwdArgs& a, int dtype, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == FA_BF16)
    e = fa::fwd_bf16_fast_eligible(a) ? fa::launch_fwd_bf16_fast(a, s) : fa::launch_fwd_bf16(a, s);
  else
    e = fa::launch_fwd_f32(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               const float* bias, const int32_t* k_len, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
               int d_k, int d_v, int dtype, float scale, int causal, int align, int window_left, int window_right,
               int keep_256, uint64_t seed, void* workspace, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Masks m = fold_masks(Nq, Nk, causal, align, window_left, window_right);
  fa::BwdArgs a{q,     k,     v,    o,    dout,     lse,      bias,          k_len, dq, dk, dv,
                static_cast<float*>(workspace), B, H, Nq, Nk, d_k, d_v, scale, causal,
                m.off, m.wl,  m.wr, keep_256, (uint32_t)seed, (uint32_t)(seed >> 32)};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_bwd_bf16(a, s) : fa::launch_bwd_f32(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int check_decode(const void* q, const void* k, const void* v, const int32_t* k_len, const void* o,
                 const float* lse, int B, int H, int Nk, int dk, int dv, int chunk, int dtype, float scale,
                 const void* workspace, size_t workspace_bytes) {
  (void)lse;
  if (B < 0 || H < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (dk < 1 || dv < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (dk > kMaxHeadDim || dv > kMaxHeadDim) return FA_ERR_UNSUPPORTED;
  if (chunk < 64 || chunk > kMaxChunk || chunk % 64 != 0) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_UNSUPPORTED;
  const long long max_chunks = (Nk + (long long)chunk - 1) / chunk;
  if (!product_fits({B, H, std::max(max_chunks, 1LL)}, kInt32Max)) return FA_ERR_SHAPE;
  if ((long long)B * H == 0) return FA_OK;
  if (q == nullptr || o == nullptr || k_len == nullptr) return FA_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL;
  const size_t need = fa_decode_splitk_workspace_bytes(B, H, Nk, dv, chunk);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return FA_ERR_WORKSPACE;
  }
  return FA_OK;
}

int check_decode_mq(const void* q, const void* k, const void* v, const int32_t* k_len, const void* o,
                    const float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int chunk, int dtype, float scale,
                    int causal, const void* workspace, size_t workspace_bytes) {
  (void)lse;
  if (B < 0 || H < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (Nq < 1 || Nq > 16) return FA_ERR_UNSUPPORTED;
  if (dk < 1 || dv < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (dk > kMaxHeadDim || dv > kMaxHeadDim) return FA_ERR_UNSUPPORTED;
  if (chunk < 64 || chunk > kMaxChunk || chunk % 64 != 0) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_UNSUPPORTED;
  const long long max_chunks = (Nk + (long long)chunk - 1) / chunk;
  if (!product_fits({B, H, std::max(max_chunks, 1LL), Nq}, kInt32Max)) return FA_ERR_SHAPE;
  if ((long long)B * H == 0) return FA_OK;
  if (q == nullptr || o == nullptr || k_len == nullptr) return FA_ERR_NULL;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL;
  const size_t need = fa_decode_splitk_mq_workspace_bytes(B, H, Nq, Nk, dv, chunk);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return FA_ERR_WORKSPACE;
  }
  return FA_OK;
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const float* bias, const int32_t* k_len, const void* dq, const void* dk, const void* dv, int B, int H,
              int Nq, int Nk, int d_k, int d_v, int dtype, float scale, int causal, const void* workspace,
              size_t workspace_bytes) {
  (void)bias;
  (void)k_len;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (d_k < 1 || d_v < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d_k > kMaxHeadDim || d_v > kMaxHeadDim) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_UNSUPPORTED;
  // general kernels: grids (row or key tiles, B*H) with a 16-bit second
  // dimension; matrix-core kernels: one dimension of tiles * B * H
  if (!product_fits({B, H}, 65535)) return FA_ERR_SHAPE;
  if (!product_fits({(std::max(Nq, Nk) + 63LL) / 64, B, H}, kInt32Max)) return FA_ERR_SHAPE;
  if (Nq > kInt32Max - Nk) return FA_ERR_SHAPE;
  const long long bhq = (long long)B * H * Nq, bhk = (long long)B * H * Nk;
  if (bhq == 0 && bhk == 0) return FA_OK;  // nothing to compute
  if (bhk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) return FA_ERR_NULL;
  if (bhq > 0 && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr || dq == nullptr))
    return FA_ERR_NULL;
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return FA_ERR_WORKSPACE;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 105; }

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large shape";
    case FA_ERR_UNSUPPORTED:
      return "unsupported dtype, head dim, block_n, chunk, causal flag, alignment, window, dropout keep or scale";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small (static scratch: the call needs more than FA_STATIC_SCRATCH_BYTES)";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int fa_check_fwd(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len,
                 const void* o, const float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype,
                 float scale, int causal, int block_n) {
  return check_fwd(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, block_n);
}

int fa_fwd(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len, void* o,
           float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype, float scale, int causal,
           int block_n, void* stream) {
  const int st = check_fwd(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, block_n);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0) return FA_OK;
  return launch_fwd(make_fwd_args(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, scale, causal,
                                  FA_ALIGN_BOTTOM_RIGHT, -1, -1, 256, 0, block_n),
                    dtype, stream);
}

int fa_check_fwd_ex(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len,
                    const void* o, const float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype,
                    float scale, int causal, int align, int window_left, int window_right, int keep_256,
                    uint64_t seed, int block_n) {
  (void)seed;
  return check_fwd_ex(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, align, window_left,
                      window_right, keep_256, block_n);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, const float* bias, const int32_t* k_len, void* o,
              float* lse, int B, int H, int Nq, int Nk, int dk, int dv, int dtype, float scale, int causal,
              int align, int window_left, int window_right, int keep_256, uint64_t seed, int block_n,
              void* stream) {
  const int st = check_fwd_ex(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, dtype, scale, causal, align,
                              window_left, window_right, keep_256, block_n);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0) return FA_OK;
  return launch_fwd(make_fwd_args(q, k, v, bias, k_len, o, lse, B, H, Nq, Nk, dk, dv, scale, causal, align,
                                  window_left, window_right, keep_256, seed, block_n),
                    dtype, stream);
}

size_t fa_decode_splitk_workspace_bytes(int B, int H, int Nk_max, int dv, int chunk) {
  if (B < 0 || H < 0 || Nk_max < 0 || dv < 1 || chunk < 64 || chunk % 64 != 0) return 0;
  const size_t max_chunks = ((size_t)Nk_max + chunk - 1) / chunk;
  return (size_t)B * H * max_chunks * ((size_t)dv + 2) * sizeof(float);
}

int fa_check_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* k_len, const void* o,
                    const float* lse, int B, int H, int Nk_max, int dk, int dv, int chunk, int dtype, float scale,
                    const void* workspace, size_t workspace_bytes) {
  return check_decode(q, k_cache, v_cache, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale, workspace,
                      workspace_bytes);
}

int fa_decode_splitk(const void* q, const void* k_cache, const void* v_cache, const int32_t* k_len, void* o,
                     float* lse, int B, int H, int Nk_max, int dk, int dv, int chunk, int dtype, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_decode(q, k_cache, v_cache, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale,
                              workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0) return FA_OK;
  const int max_chunks = (int)(((long long)Nk_max + chunk - 1) / chunk);
  float* ws = static_cast<float*>(workspace);
  fa::DecodeArgs a{q, k_cache, v_cache, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, scale,
                   ws, ws == nullptr ? nullptr : ws + (size_t)B * H * max_chunks * dv, max_chunks};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_decode_bf16(a, static_cast<hipStream_t>(stream))
                                        : fa::launch_decode_f32(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_splitk_static(const void* q, const void* k_cache, const void* v_cache, const int32_t* k_len,
                            void* o, float* lse, int B, int H, int Nk_max, int dk, int dv, int chunk, int dtype,
                            float scale, void* stream) {
  // host checks first (no GPU call): the states must fit the static array,
  // which then stands in for the workspace in the usual argument checks
  const size_t need = fa_decode_splitk_workspace_bytes(B, H, Nk_max, dv, chunk);
  if (need > FA_STATIC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void* const placeholder = reinterpret_cast<void*>(uintptr_t{256});  // aligned, never dereferenced
  int st = check_decode(q, k_cache, v_cache, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale, placeholder,
                        FA_STATIC_SCRATCH_BYTES);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0) return FA_OK;
  void* scratch = nullptr;
  if (fa::static_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  return fa_decode_splitk(q, k_cache, v_cache, k_len, o, lse, B, H, Nk_max, dk, dv, chunk, dtype, scale, scratch,
                          FA_STATIC_SCRATCH_BYTES, stream);
}

size_t fa_decode_splitk_mq_workspace_bytes(int B, int H, int Nq, int Nk_max, int dv, int chunk) {
  if (B < 0 || H < 0 || Nq < 1 || Nq > 16 || Nk_max < 0 || dv < 1 || chunk < 64 || chunk % 64 != 0) return 0;
  const size_t max_chunks = ((size_t)Nk_max + chunk - 1) / chunk;
  return (size_t)B * H * max_chunks * Nq * ((size_t)dv + 2) * sizeof(float);
}

int fa_check_decode_mq(const void* q, const void* k_cache, const void* v_cache, const int32_t* k_len, const void* o,
                       const float* lse, int B, int H, int Nq, int Nk_max, int dk, int dv, int chunk, int dtype,
                       float scale, int causal, const void* workspace, size_t workspace_bytes) {
  return check_decode_mq(q, k_cache, v_cache, k_len, o, lse, B, H, Nq, Nk_max, dk, dv, chunk, dtype, scale, causal,
                         workspace, workspace_bytes);
}

int fa_decode_splitk_mq(const void* q, const void* k_cache, const void* v_cache, const int32_t* k_len, void* o,
                        float* lse, int B, int H, int Nq, int Nk_max, int dk, int dv, int chunk, int dtype, float scale,
                        int causal, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_decode_mq(q, k_cache, v_cache, k_len, o, lse, B, H, Nq, Nk_max, dk, dv, chunk, dtype, scale,
                                 causal, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0) return FA_OK;
  const int max_chunks = (int)(((long long)Nk_max + chunk - 1) / chunk);
  float* ws = static_cast<float*>(workspace);
  fa::DecodeMqArgs a{q,     k_cache, v_cache, k_len, o,      lse,   B,  H,
                     Nq,    Nk_max,  dk,      dv,    chunk,  scale, causal,
                     ws,    ws == nullptr ? nullptr : ws + (size_t)B * H * max_chunks * Nq * dv, max_chunks};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == FA_BF16 ? fa::launch_decode_mq_bf16(a, s) : fa::launch_decode_mq_f32(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq) {
  if (B < 0 || H < 0 || Nq < 0) return 0;
  return (size_t)B * H * Nq * sizeof(float);
}

int fa_check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 const float* bias, const int32_t* k_len, const void* dq, const void* dk, const void* dv, int B, int H,
                 int Nq, int Nk, int d_k, int d_v, int dtype, float scale, int causal, const void* workspace,
                 size_t workspace_bytes) {
  return check_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale, causal,
                   workspace, workspace_bytes);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           const float* bias, const int32_t* k_len, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
           int d_k, int d_v, int dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
           void* stream) {
  const int st = check_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale,
                           causal, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0 && (long long)B * H * Nk == 0) return FA_OK;
  return launch_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale, causal,
                    FA_ALIGN_BOTTOM_RIGHT, -1, -1, 256, 0, workspace, stream);
}

int fa_check_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const float* bias, const int32_t* k_len, const void* dq, const void* dk, const void* dv, int B,
                    int H, int Nq, int Nk, int d_k, int d_v, int dtype, float scale, int causal, int align,
                    int window_left, int window_right, int keep_256, uint64_t seed, const void* workspace,
                    size_t workspace_bytes) {
  (void)seed;
  const int st = check_masks(align, window_left, window_right, keep_256);
  if (st != FA_OK) return st;
  return check_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale, causal,
                   workspace, workspace_bytes);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const float* bias, const int32_t* k_len, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
              int d_k, int d_v, int dtype, float scale, int causal, int align, int window_left, int window_right,
              int keep_256, uint64_t seed, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = fa_check_bwd_ex(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype,
                                 scale, causal, align, window_left, window_right, keep_256, seed, workspace,
                                 workspace_bytes);
  if (st != FA_OK) return st;
  if ((long long)B * H * Nq == 0 && (long long)B * H * Nk == 0) return FA_OK;
  return launch_bwd(q, k, v, o, dout, lse, bias, k_len, dq, dk, dv, B, H, Nq, Nk, d_k, d_v, dtype, scale, causal,
                    align, window_left, window_right, keep_256, seed, workspace, stream);
}

}  // extern "C"
