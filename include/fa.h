/*
 * fa.h -- C ABI of the exact attention forward library (libfa.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, for every batch entry b, head h and query row i,
 *
 *     s_ij  = scale * (q_i . k_j) + bias_ij          for keys j in J_i
 *     o_i   = sum_j softmax_j(s_i.) v_j,  lse_i = ln sum_{j in J_i} exp(s_ij)
 *
 * tile by tile with the per-row running state (max m, denominator l,
 * unnormalised weighted value sum u); l and u are both rescaled by
 * exp(m_old - m_new) when the maximum rises and each row is divided once at
 * the end.  S and P never reach device memory.  Sources, cited by title and
 * section:
 *   [GS] "How Does FlashAttention Preserve Global Softmax Across Tiles?"
 *   [VW] "Flash attention and efficient attention: Visual walkthrough"
 *   [OA] "Reducing Memory Traffic with Output Accumulation in FlashAttention"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major, contiguous, last dimension fastest:
 *   [B, H, N, d] for Q/K/V/O, [B, H, Nq] for lse, [B, H, Nq, Nk] for bias.
 * - Every pointer argument is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or synchronises; it only enqueues kernels on
 *   `stream` (a hipStream_t; NULL means the default stream) and returns.
 *   Kernel faults surface at the caller's next synchronisation.
 * - Validation happens on the host before any launch; on failure nothing is
 *   launched and nothing is written, and the return value is a nonzero
 *   fa_status.  Values inside device arrays (k_len) are not validated: the
 *   kernels clamp them to [0, Nk].
 * - The allowed key set J_i ([GS] sections 1 and 6) is the intersection of
 *   the key-length mask j < clamp(k_len[b], 0, Nk) and, if causal, the
 *   bottom-right causal mask j <= i + Nk - Nq (zero-based, the ends of the two
 *   sequences aligned).  A row whose J_i is empty gets o_i = 0 and
 *   lse_i = -inf exactly ([GS] section 6); no NaN is produced.
 * - Inputs are assumed finite ([GS] section 1).  Accumulation is fp32 for
 *   both dtypes; bf16 inputs use bf16 MFMA products (P is rounded to bf16
 *   before P.V), fp32 inputs use fp32 MFMA.
 * - The library is stateless and reentrant.
 * - fa_fwd_ex / fa_bwd_ex add the mask variants of [GS] section 6 (top-left
 *   alignment, sliding windows) and dropout with a counter-based mask.
 */
#ifndef ONLINE_SOFTMAX_FA_H
#define ONLINE_SOFTMAX_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O.  bias and lse are always fp32. */
typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  FA_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be,
                             or too large for 32-bit grid/index arithmetic   */
  FA_ERR_UNSUPPORTED = 3, /* dtype, head dim (> 128), block_n, chunk, causal
                             flag, alignment, window width or scale outside
                             what the kernels support                        */
  FA_ERR_WORKSPACE = 4,   /* workspace missing, misaligned or too small     */
  FA_ERR_HIP = 5          /* the HIP runtime reported an error at launch    */
} fa_status;

/*
 * fa_fwd -- prefill / general forward pass ([GS] sections 1, 5-7; [OA]
 * "Completing the Output by Traversing Tiles").
 *
 *   q     [B, H, Nq, dk]  dtype        read only
 *   k     [B, H, Nk, dk]  dtype        read only (may be NULL if Nk == 0)
 *   v     [B, H, Nk, dv]  dtype        read only (may be NULL if Nk == 0)
 *   bias  [B, H, Nq, Nk]  fp32 or NULL; added after scaling, before masking;
 *                                      must be finite at allowed positions
 *   k_len [B] int32 or NULL (NULL: every sequence has Nk keys); rows
 *                                      j >= k_len[b] of k and v are never
 *                                      read (their contents do not matter)
 *   o     [B, H, Nq, dv]  dtype        written in full
 *   lse   [B, H, Nq] fp32 or NULL      natural-log log-sum-exp per row
 *   1 <= dk, dv <= 128; B, H, Nq, Nk >= 0.  B*H*Nq == 0 is a no-op (FA_OK,
 *   pointers may then be NULL).  Nk == 0 yields o = 0, lse = -inf.
 *   scale : finite; the usual value is 1/sqrt(dk) (computed by the caller).
 *   causal: 0 or 1 (bottom-right alignment).
 *   block_n: key-tile width; 0 = automatic, or 32, 64, 128.  The result does
 *   not depend on it beyond rounding ([GS] section 9).
 */
int fa_fwd(const void* q, const void* k, const void* v, const float* bias,
           const int32_t* k_len, void* o, float* lse, int B, int H, int Nq,
           int Nk, int dk, int dv, int dtype, float scale, int causal,
           int block_n, void* stream);

/* Host-only validation of fa_fwd's arguments (no pointer is dereferenced and
 * no GPU is touched).  Returns the status fa_fwd would return before
 * launching. */
int fa_check_fwd(const void* q, const void* k, const void* v,
                 const float* bias, const int32_t* k_len, const void* o,
                 const float* lse, int B, int H, int Nq, int Nk, int dk,
                 int dv, int dtype, float scale, int causal, int block_n);

/* Where query row i sits on the key axis ([GS] section 6): with the ENDS of
 * the two sequences aligned (bottom-right, the convention since
 * FlashAttention 2.1) at position i + Nk - Nq; with their STARTS aligned
 * (top-left, the earlier convention) at position i. */
typedef enum { FA_ALIGN_BOTTOM_RIGHT = 0, FA_ALIGN_TOP_LEFT = 1 } fa_align;

/*
 * fa_fwd_ex -- fa_fwd with the mask variants of [GS] section 6: a causal
 * alignment choice and a sliding window measured from the same aligned
 * position.  Arguments as for fa_fwd, plus
 *
 *   align        FA_ALIGN_BOTTOM_RIGHT or FA_ALIGN_TOP_LEFT; the row's key
 *                position is pos_i = i + Nk - Nq or pos_i = i.  It applies
 *                to the causal mask and to both window edges.
 *   window_left  -1 (no left edge) or w >= 0: keys j >= pos_i - w only
 *   window_right -1 (no right edge) or w >= 0: keys j <= pos_i + w only
 *
 * J_i = { j : j < clamp(k_len[b], 0, Nk), j <= pos_i if causal,
 *             j >= pos_i - window_left if window_left >= 0,
 *             j <= pos_i + window_right if window_right >= 0 }.
 * The usual sliding window of width W is causal = 1, window_left = W - 1.
 * Rows whose J_i is empty (a window entirely past k_len, or before key 0)
 * get o_i = 0, lse_i = -inf.  Every kernel (both dtypes, the bf16 head-dim
 * 64/128 fast path included) visits only the key tiles that meet the union
 * of a row block's ranges and masks only the edge tiles.
 *
 *   keep_256     dropout of the attention probabilities ([GS] section 6:
 *                a training backward must replay the mask and scaling):
 *                256 = no dropout; T in 1..255 keeps an element iff its
 *                random byte is < T (keep probability T/256) and multiplies
 *                kept probabilities by 256/T:
 *                  o_i = (256/T) sum_j z_ij p_ij v_j,  lse_i undropped.
 *   seed         64-bit seed of the dropout mask (ignored without dropout).
 *
 * Dropout mask layout: the random byte of element (b, h, i, j) comes from
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 * Easy as 1, 2, 3", SC 2011) with key (seed mod 2^32, seed div 2^32) and
 * counter (i, j div 64, b*H + h, (j div 4) mod 4); it is byte (j mod 4)
 * (bits 8(j mod 4) .. +7) of output word (j div 16) mod 4.  fa_bwd_ex with
 * the same seed and keep_256 replays the same mask.
 *
 * With align = BOTTOM_RIGHT, both widths -1 and keep_256 = 256 the result
 * equals fa_fwd's bit for bit.  Returns FA_ERR_UNSUPPORTED for another align
 * value, a width below -1 or keep_256 outside 1..256.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, const float* bias,
              const int32_t* k_len, void* o, float* lse, int B, int H,
              int Nq, int Nk, int dk, int dv, int dtype, float scale,
              int causal, int align, int window_left, int window_right,
              int keep_256, uint64_t seed, int block_n, void* stream);

/* Host-only validation of fa_fwd_ex's arguments. */
int fa_check_fwd_ex(const void* q, const void* k, const void* v,
                    const float* bias, const int32_t* k_len, const void* o,
                    const float* lse, int B, int H, int Nq, int Nk, int dk,
                    int dv, int dtype, float scale, int causal, int align,
                    int window_left, int window_right, int keep_256,
                    uint64_t seed, int block_n);

/*
 * Bytes of fp32 workspace fa_decode_splitk needs:
 *   B * H * ceil(Nk_max / chunk) * (dv + 2) * 4.
 * Returns 0 for invalid arguments (negative sizes, chunk not a positive
 * multiple of 64).
 */
size_t fa_decode_splitk_workspace_bytes(int B, int H, int Nk_max, int dv,
                                        int chunk);

/*
 * fa_decode_splitk -- single-token decode against a KV cache, split over
 * key chunks ([GS] section 8, split KV loading for short queries; the
 * per-chunk states are merged with the rule of [GS] section 4 / [VW] Step 5).
 *
 *   q       [B, H, dk]         dtype   (one query token per sequence)
 *   k_cache [B, H, Nk_max, dk] dtype   only keys j < k_len[b] are read
 *   v_cache [B, H, Nk_max, dv] dtype
 *   k_len   [B] int32, required; clamped to [0, Nk_max]
 *   o       [B, H, dv] dtype; lse [B, H] fp32 or NULL
 *   chunk   keys per partial state: a positive multiple of 64 (512 usual)
 *   workspace: device buffer of at least
 *              fa_decode_splitk_workspace_bytes(B, H, Nk_max, dv, chunk)
 *              bytes, 16-byte aligned; its contents on entry are ignored.
 * Two kernels are enqueued on `stream`: one partial state (m_c, l_c, u_c)
 * per (b, h, chunk) with chunk < ceil(k_len[b] / chunk), then one merge per
 * (b, h) in ascending chunk order.  A sequence with k_len = 0 gets o = 0,
 * lse = -inf.
 */
int fa_decode_splitk(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* k_len, void* o, float* lse, int B, int H,
                     int Nk_max, int dk, int dv, int chunk, int dtype,
                     float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * fa_decode_splitk_static -- fa_decode_splitk for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * fa_decode_splitk (the same kernels run), without the workspace: the
 * partial states live in a static device array of the library,
 * FA_STATIC_SCRATCH_BYTES per GPU, loaded with the library's code object and
 * held until the process ends.  The call allocates and frees nothing.
 *
 *   Returns FA_ERR_WORKSPACE when the partial states of the call,
 *   fa_decode_splitk_workspace_bytes(B, H, Nk_max, dv, chunk), exceed
 *   FA_STATIC_SCRATCH_BYTES (e.g. B * H = 2048 sequence-heads of 8192 keys
 *   in 512-key chunks with dv = 128 need 17 MB); other errors as
 *   fa_decode_splitk.  The array's device address is looked up once per
 *   device, on the first call made while that device is current.
 *   All calls on one GPU share the array: calls ordered on one stream are
 *   safe, calls that overlap in time on one GPU (two streams, two host
 *   threads) race on it and give undefined results.  Nothing in the array
 *   needs clearing between calls (every state the merge reads is written
 *   by the same call).
 */
#define FA_STATIC_SCRATCH_BYTES (32u * 1024u * 1024u)
int fa_decode_splitk_static(const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* k_len,
                            void* o, float* lse, int B, int H, int Nk_max,
                            int dk, int dv, int chunk, int dtype, float scale,
                            void* stream);

/*
 * Bytes of fp32 workspace fa_decode_splitk_mq needs:
 *   B * H * ceil(Nk_max / chunk) * Nq * (dv + 2) * 4.
 * Returns 0 for invalid arguments (negative sizes, Nq outside 1..16, chunk
 * not a positive multiple of 64).
 */
size_t fa_decode_splitk_mq_workspace_bytes(int B, int H, int Nq, int Nk_max,
                                           int dv, int chunk);

/*
 * fa_decode_splitk_mq -- split-KV attention for a few query rows per
 * sequence against a KV cache (chunked prefill, several speculative tokens):
 * the key axis split into chunks ([GS] section 8, split KV loading for short
 * queries), chunk states merged per row with the rule of [GS] section 4 /
 * [VW] Step 5.
 *
 *   q       [B, H, Nq, dk]     dtype, 1 <= Nq <= 16: the LAST Nq positions
 *                              of each sequence
 *   k_cache [B, H, Nk_max, dk] dtype   only keys j < k_len[b] are read
 *   v_cache [B, H, Nk_max, dv] dtype
 *   k_len   [B] int32, required; clamped to [0, Nk_max]
 *   o       [B, H, Nq, dv] dtype; lse [B, H, Nq] fp32 or NULL
 *   causal  0: every row sees the k_len[b] keys; 1: row i sees keys
 *           j <= i + k_len[b] - Nq (bottom-right alignment against the
 *           sequence's own length, [GS] section 6); rows left with no key
 *           get o = 0, lse = -inf
 *   chunk   a positive multiple of 64, at most 2048 (512 usual)
 *   workspace: at least fa_decode_splitk_mq_workspace_bytes(...) bytes,
 *              16-byte aligned; contents on entry are ignored.
 * Two kernels on `stream`: the chunk states (one work-group per chunk, batch
 * and head, chunks below k_len[b] only), then one merge per (b, h, row) in
 * ascending chunk order.
 */
int fa_decode_splitk_mq(const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* k_len, void* o,
                        float* lse, int B, int H, int Nq, int Nk_max, int dk,
                        int dv, int chunk, int dtype, float scale, int causal,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Host-only validation of fa_decode_splitk_mq's arguments. */
int fa_check_decode_mq(const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* k_len,
                       const void* o, const float* lse, int B, int H, int Nq,
                       int Nk_max, int dk, int dv, int chunk, int dtype,
                       float scale, int causal, const void* workspace,
                       size_t workspace_bytes);

/* Host-only validation of fa_decode_splitk's arguments. */
int fa_check_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* k_len, const void* o, const float* lse,
                    int B, int H, int Nk_max, int dk, int dv, int chunk,
                    int dtype, float scale, const void* workspace,
                    size_t workspace_bytes);

/*
 * Bytes of fp32 workspace fa_bwd needs: B * H * Nq * 4 (one scalar per query
 * row).  Returns 0 for negative sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq);

/*
 * fa_bwd -- gradients of fa_fwd by recomputation ([GS] section 7, "Why
 * training need not save the full probability matrix"; [VW] Step 8).  The
 * forward's O and lse are consumed; the probabilities are rebuilt tile by
 * tile from Q, K, the same masks and the same bias, and never stored:
 *
 *   p_ij = exp(s_ij - lse_i) on the allowed set (0 elsewhere)
 *   c_i  = dO_i . O_i,   D_ij = p_ij (dO_i . v_j - c_i)
 *   dV = P^T dO,   dQ = scale * D K,   dK = scale * D^T Q
 *
 *   q, k, v    as for fa_fwd                           read only
 *   o          [B, H, Nq, dv] dtype: fa_fwd's output    read only
 *   dout       [B, H, Nq, dv] dtype: dLoss/dO           read only
 *   lse        [B, H, Nq] fp32: fa_fwd's lse, required  read only
 *   bias, k_len, scale, causal: exactly as passed to fa_fwd (the bias is a
 *              fixed input: no bias gradient is formed); as in fa_fwd,
 *              rows j >= k_len[b] of k and v are never read
 *   dq [B, H, Nq, dk], dk [B, H, Nk, dk], dv [B, H, Nk, dv]  dtype,
 *              written in full (keys no row can see get zero)
 *   workspace: device buffer of at least fa_bwd_workspace_bytes(B, H, Nq)
 *              bytes, 16-byte aligned; contents on entry are ignored.
 *   1 <= dk, dv <= 128; B * H <= 65535 and ceil(max(Nq, Nk) / 64) * B * H
 *   < 2^31 (FA_ERR_SHAPE otherwise).  Rows whose lse is -inf (no allowed
 *   key) contribute nothing.  Launches (all on `stream`, no atomics, results
 *   bitwise reproducible): bf16 with head dims 64/128 -- dQ per query tile
 *   (it also forms c = dO.O per row into the workspace), then dK/dV per key
 *   tile; otherwise c per row, then dK/dV, then dQ.  Inputs must be finite;
 *   lse must be the forward's (a different lse rescales the rebuilt
 *   probabilities).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, const float* bias,
           const int32_t* k_len, void* dq, void* dk, void* dv, int B, int H,
           int Nq, int Nk, int d_k, int d_v, int dtype, float scale,
           int causal, void* workspace, size_t workspace_bytes, void* stream);

/* Host-only validation of fa_bwd's arguments. */
int fa_check_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, const float* bias,
                 const int32_t* k_len, const void* dq, const void* dk,
                 const void* dv, int B, int H, int Nq, int Nk, int d_k,
                 int d_v, int dtype, float scale, int causal,
                 const void* workspace, size_t workspace_bytes);

/*
 * fa_bwd_ex -- fa_bwd for the forwards of fa_fwd_ex: the same position
 * masks (causal, align, window_left, window_right) and the same dropout
 * (keep_256, seed), replayed exactly ([GS] section 6: the backward must
 * reproduce the forward's random mask and scaling).  With dropout, for
 * r = 256/keep_256 and z the kept elements:
 *
 *   dV = (z r P)^T dO,   D_ij = p_ij (z_ij r (dO_i . v_j) - c_i),
 *   c_i = dO_i . O_i (the dropped forward output),
 *   dQ = scale D K,   dK = scale D^T Q.
 *
 * o and lse must be those fa_fwd_ex returned for the same arguments.  Other
 * arguments, workspace and errors as for fa_bwd; FA_ERR_UNSUPPORTED also for
 * an invalid align, a width below -1 or keep_256 outside 1..256.  With the
 * defaults (BOTTOM_RIGHT, -1, -1, 256) it equals fa_bwd bit for bit.
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, const float* bias,
              const int32_t* k_len, void* dq, void* dk, void* dv, int B,
              int H, int Nq, int Nk, int d_k, int d_v, int dtype, float scale,
              int causal, int align, int window_left, int window_right,
              int keep_256, uint64_t seed, void* workspace,
              size_t workspace_bytes, void* stream);

/* Host-only validation of fa_bwd_ex's arguments. */
int fa_check_bwd_ex(const void* q, const void* k, const void* v,
                    const void* o, const void* dout, const float* lse,
                    const float* bias, const int32_t* k_len, const void* dq,
                    const void* dk, const void* dv, int B, int H, int Nq,
                    int Nk, int d_k, int d_v, int dtype, float scale,
                    int causal, int align, int window_left, int window_right,
                    int keep_256, uint64_t seed, const void* workspace,
                    size_t workspace_bytes);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_str(int status);

/* Version of this ABI (major * 100 + minor). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ONLINE_SOFTMAX_FA_H */
