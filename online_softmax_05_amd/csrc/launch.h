// Internal launcher interface between the C-ABI front end (fa_api.cpp) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;
  const int32_t* k_len;
  void* o;
  float* lse;
  int B, H, Nq, Nk, dk, dv;
  float scale;
  int block_n;  // 32, 64 or 128 (already resolved from "auto")
  // position masks, see fa_mask.h: row i sits at key position i + off and
  // sees keys [pos - wl, pos + wr] (a negative width is unbounded; causal is
  // folded into wr = 0)
  int off;
  int wl;
  int wr;
  // dropout of P (fa_dropout.h): keep_256 == 256 means none
  int keep_256;
  uint32_t seed_lo, seed_hi;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* k_len;
  void* o;
  float* lse;
  int B, H, Nk, dk, dv, chunk;
  float scale;
  float* ws_u;   // [B*H*max_chunks, dv]
  float* ws_ml;  // [B*H*max_chunks, 2]  (m in the base-2 domain, l)
  int max_chunks;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;  // upstream gradient dLoss/dO
  const float* lse;
  const float* bias;
  const int32_t* k_len;
  void* dq_out;
  void* dk_out;
  void* dv_out;
  float* ws_c;  // [B*H*Nq]: c_i = dO_i . O_i
  int B, H, Nq, Nk, dk, dv;
  float scale;
  int causal;  // unused by the kernels: the position masks below include it
  // position masks as for the forward (fa_mask.h) and dropout (fa_dropout.h)
  int off;
  int wl;
  int wr;
  int keep_256;
  uint32_t seed_lo, seed_hi;
};

struct DecodeMqArgs {
  const void* q;  // [B, H, Nq, dk]
  const void* k;
  const void* v;
  const int32_t* k_len;
  void* o;     // [B, H, Nq, dv]
  float* lse;  // [B, H, Nq] or null
  int B, H, Nq, Nk, dk, dv, chunk;
  float scale;
  int causal;
  float* ws_u;   // [B*H*max_chunks*Nq, dv]
  float* ws_ml;  // [B*H*max_chunks*Nq, 2]
  int max_chunks;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// fast bf16 path: head dims 64/128, 16-byte aligned tensors, 64-key tiles
bool fwd_bf16_fast_eligible(const FwdArgs& a);
hipError_t launch_fwd_bf16_fast(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);
// Device address of the library's static scratch array on the current
// device (looked up once per device; fa_scratch.hip).
hipError_t static_scratch(void** out);
hipError_t launch_decode_mq_bf16(const DecodeMqArgs& a, hipStream_t stream);
hipError_t launch_decode_mq_f32(const DecodeMqArgs& a, hipStream_t stream);
// backward: c = dO.O, then dK/dV and dQ (bf16 with head dims 64/128 and
// 16-byte aligned tensors on the matrix cores, everything else general)
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
bool bwd_bf16_mfma_eligible(const BwdArgs& a);
hipError_t launch_bwd_bf16_mfma(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
