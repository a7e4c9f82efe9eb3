/*
 * attn.h -- C ABI of the exact tiled attention library for MI355X (gfx950).
 *
 * The operation is exact softmax attention,
 *
 *     O = softmax(scale * Q K^T + mask) V      (dropout on the probabilities),
 *
 * computed as one fused, tiled kernel: a block of Q rows stays on chip while
 * blocks of K and V stream through, a running row maximum m and denominator l
 * are updated per block (the online softmax), O is rescaled and accumulated,
 * and only O and the per-row log-sum-exp are written. No N x N matrix reaches
 * device memory. The backward pass recomputes the scores and probabilities
 * from Q, K and the saved log-sum-exp.
 *
 * Sources (web pages on the method):
 *   - "Why FlashAttention Is a Kernel Story" (praveentn.live), sections
 *     "The real bottleneck" (the unfused chain and its memory traffic),
 *     "Tiling: fitting the work inside SRAM" (the online-softmax update, the
 *     final O / l, and the O(Nd) traffic), "Why this only works as a fused
 *     kernel", and "When it falls down" (backward recomputation from the
 *     output and log-sum-exp).
 *   - anthology-of-the-sota practice SOTA-114 (dmarx.github.io), "The general
 *     form of the practice above it" (the fused chain matmul, scale, mask,
 *     softmax, dropout, matmul) and "Cost" (each mask/dropout/head-dim/dtype
 *     combination is its own code path; a silent fallback is a hazard).
 *   - anthology-of-the-sota practice SOTA-085, "What 'when hardware supports
 *     it' is carrying" (the result is exact; O(N) extra memory).
 *
 * Conventions shared by every entry point
 *   Layout.  Q, O, dO, dQ are dense row-major (B, H, N, d) arrays: element
 *            (b, h, i, c) sits at ((b*H + h)*N + i)*d + c. K, V, dK, dV are
 *            (B, H, Nk, d) in the same layout (Nk = N for self-attention,
 *            Nk != N for cross-attention on a non-square grid). lse is
 *            (B, H, N) float32 (the backward's D lives in its workspace,
 *            see attn_bwd_workspace_bytes).
 *   Masks.   Query i lines up with key c_i = i + Nk - N (the last query with
 *            the last key; c_i = i when Nk = N). Every set mask must keep a
 *            key for it to be visible:
 *            causal: j <= c_i.
 *            sliding window: c_i - window_left <= j <= c_i + window_right,
 *            each side unbounded when its value is -1 (Mistral-style: causal
 *            with window_left = w - 1; Longformer-style: both sides w).
 *            key padding: kv_len is a device array of B int32; key j is
 *            visible iff j < kv_len[b] (values are clamped to [0, Nk]; query
 *            rows are all computed).
 *            A query row with no visible key yields O = 0, lse = -inf and
 *            zero gradients.
 *            ("Why FlashAttention Is a Kernel Story", section "When it falls
 *            down": sliding-window attention and cross-attention with
 *            non-square K, V grids are the variants that change the tiling;
 *            the alignment and the window bounds are this library's reading.)
 *   Dropout. p in [0, 1). Each probability is kept iff the 32-bit draw
 *            u = Philox4x32-10(counter = (j >> 2, i, h, b), key = seed)[j & 3]
 *            satisfies u >= floor(p_f32 * 2^32); kept values are scaled by
 *            1 / (1 - p). The log-sum-exp is over the undropped scores.
 *            (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3".)
 *   Memory.  All tensor pointers are device pointers owned by the caller and
 *            must be 16-byte aligned; the pointer of a tensor with no elements
 *            may be NULL (it is never read or written). Outputs must not alias
 *            inputs. The library never allocates, frees or synchronises; it
 *            keeps no global state, so calls from several host threads are
 *            safe.
 *   Streams. `stream` is a hipStream_t (NULL = the default stream). Work is
 *            enqueued asynchronously; faults inside a kernel surface at the
 *            caller's next synchronisation.
 *   Errors.  Every argument is validated on the host before anything is
 *            enqueued. An unsupported combination (head dimension, dtype)
 *            returns ATTN_ERR_UNSUPPORTED: there is never a fallback path.
 *            ATTN_ERR_LAUNCH reports a launch failure from the HIP runtime.
 */
#ifndef EXACT_TILED_ATTN_H
#define EXACT_TILED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F16 = 0,   /* IEEE binary16 */
  ATTN_BF16 = 1,  /* bfloat16 */
  ATTN_F32 = 2,   /* IEEE binary32 (outputs only) */
  ATTN_E4M3 = 3   /* OCP FP8 E4M3 ("e4m3fn": bias 7, no infinities, max 448),
                     one byte per element; inputs of attn_fwd only, d = 128,
                     out_dtype BF16 or F32 (see attn_fwd) */
} attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,  /* NULL/misaligned pointer, bad size, bad p ... */
  ATTN_ERR_UNSUPPORTED = 2,  /* valid request with no kernel (e.g. d = 96)  */
  ATTN_ERR_WORKSPACE = 3,    /* backward workspace missing or too small     */
  ATTN_ERR_LAUNCH = 4,       /* the HIP runtime rejected a kernel launch    */
  ATTN_ERR_TOO_LARGE = 5     /* beyond attn_bwd_noalloc's fixed scratch     */
} attn_status;

typedef struct {
  int32_t B, H, N, d;      /* batch, heads, sequence length, head dim.
                              B, H, N >= 0 (see "Empty problems");
                              d in {64, 128, 256};
                              N*d and Nk*d must be below 2^31 (per-head
                              index math) and the element counts of every
                              tensor below about 2^62.                     */
  int32_t dtype;           /* attn_dtype of Q, K, V, dO: ATTN_F16 or BF16
                              (ATTN_E4M3 for the forward, see attn_fwd)    */
  int32_t out_dtype;       /* attn_dtype of O, dQ, dK, dV: == dtype or F32
                              (BF16 or F32 when dtype is ATTN_E4M3)        */
  float scale;             /* multiplies Q K^T; finite and > 0             */
  int32_t causal;          /* 0 or 1                                       */
  const int32_t* kv_len;   /* device int32[B] of valid key counts, or NULL */
  float dropout_p;         /* 0 <= p < 1; 0 disables dropout               */
  uint64_t seed;           /* Philox key for dropout                       */
  int32_t Nk;              /* rows of K, V, dK, dV (>= 0); Nk = N for
                              self-attention. Always explicit: Nk = 0 means
                              no keys (every row sees none).               */
  int32_t window_left;     /* sliding window, keys before c_i; -1 = none   */
  int32_t window_right;    /* sliding window, keys after c_i;  -1 = none   */
} attn_params;

/* Forward: O (out_dtype, (B,H,N,d)) and lse (float32, (B,H,N)), where
 * lse_i = log sum_j exp(scale * Q_i . K_j) over the visible keys. K and V are
 * (B,H,Nk,d). Reads Q, K, V once per query block; writes only O and lse.
 * ("Why FlashAttention Is a Kernel Story", section "Tiling: fitting the work
 * inside SRAM": per-block running max and denominator, rescaled O, final
 * O / l; the single log-sum-exp replaces the page's separate l and m.
 * SOTA-114, "The general form of the practice above it": scale, mask,
 * softmax and dropout fused between the two products.)
 *
 * fp8: with dtype ATTN_E4M3 (d = 128, out_dtype BF16 or F32) both products
 * run on fp8 operands with fp32 accumulation. The scores are exact (products
 * of e4m3 values are exact in fp32); the probabilities are rounded to e4m3
 * relative to the running reference maximum before the product with V, and O
 * is normalised by the fp32 sum of the unrounded probabilities, so each term
 * of O carries a relative error of at most 2^-4 (absolute 2^-10 / L_i below
 * 2^-6). ("Why FlashAttention Is a Kernel Story", section "When it falls
 * down": FP8 score tiles need care with precision.) */
attn_status attn_fwd(const attn_params* p, const void* q, const void* k,
                     const void* v, void* o, float* lse, void* stream);

/* Size in bytes of the workspace attn_bwd needs for these parameters:
 * two float32 (B,H,Np) arrays (D_i = dO_i . O_i and lse_i * log2(e); Np = N
 * rounded up to a multiple of 4), each rounded up to 256 bytes; 0 if the
 * parameters are invalid or N = 0. Callers size the workspace with this
 * function, not with a formula of their own (the layout changed in 0.5.0).
 * (The backward's row statistics: "Why FlashAttention Is a Kernel Story",
 * section "When it falls down", recomputation from the stored output and
 * log-sum-exp.) */
size_t attn_bwd_workspace_bytes(const attn_params* p);

/* Backward: given Q, K, V, the forward's O (out_dtype) and lse, and dO
 * (dtype), writes dQ (B,H,N,d), dK and dV (B,H,Nk,d), all in out_dtype.
 * Scores and probabilities are recomputed from lse; nothing N x Nk is stored.
 * `workspace` is a device buffer of at least attn_bwd_workspace_bytes(p)
 * bytes, owned by the caller, 256-byte aligned (NULL when that size is 0);
 * its contents on entry do not matter. With N = 0 it writes dK = dV = 0;
 * with Nk = 0 it writes dQ = 0.
 * ("Why FlashAttention Is a Kernel Story", section "When it falls down",
 * backward pass: S and P are rebuilt from Q, K and the saved log-sum-exp
 * rather than read back from memory.) */
attn_status attn_bwd(const attn_params* p, const void* q, const void* k,
                     const void* v, const void* o, const float* lse,
                     const void* d_o, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The three steps attn_bwd enqueues, callable one at a time (same arguments
 * and validation as attn_bwd; each ignores the outputs it does not write).
 * Calling them in this order on one stream equals attn_bwd:
 *   ATTN_BWD_STAGE_PREPROCESS  D_i = dO_i . O_i and lse_i * log2(e) into the
 *                              workspace
 *   ATTN_BWD_STAGE_DKDV        dK, dV (reads the workspace)
 *   ATTN_BWD_STAGE_DQ          dQ     (reads the workspace)
 * Useful for timing each kernel with events, or for overlapping dQ with
 * other work on a second stream once the preprocess step has run. */
typedef enum {
  ATTN_BWD_STAGE_PREPROCESS = 0,
  ATTN_BWD_STAGE_DKDV = 1,
  ATTN_BWD_STAGE_DQ = 2
} attn_bwd_stage_id;

attn_status attn_bwd_stage(const attn_params* p, int32_t stage, const void* q,
                           const void* k, const void* v, const void* o,
                           const float* lse, const void* d_o, void* dq, void* dk,
                           void* dv, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Test aid: writes the dropout keep-mask keep[b][h][i][j] (uint8 0/1, device,
 * (B,H,N,Nk)) that attn_fwd and attn_bwd use for these parameters. Masking by
 * causal/window/kv_len is not applied here: it is the raw Philox keep
 * decision. (SOTA-114, "The general form of the practice above it": dropout
 * is one of the fused steps; the generator is Philox4x32-10 from Salmon et
 * al., SC'11, keyed as described under "Dropout" above.) */
attn_status attn_dropout_mask(const attn_params* p, uint8_t* keep, void* stream);

/* Static, human-readable text for a status code. (SOTA-114, "Cost": an
 * unsupported combination is reported, never served by a slower path.) */
const char* attn_status_string(attn_status s);

/* Empty problems.  When B, H or N is 0 (and the other fields are valid),
 * attn_fwd returns ATTN_OK without reading any pointer or enqueueing work;
 * so does attn_dropout_mask when B*H*N*Nk is 0, and attn_bwd_workspace_bytes
 * returns 0. attn_bwd and attn_bwd_stage do nothing when B or H is 0 or when
 * N = Nk = 0; with N = 0 and Nk > 0 they write dK = dV = 0, and with Nk = 0
 * and N > 0 they write dQ = 0 (each row sees no key: O = 0, lse = -inf). */

/* The backward of attn_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). It takes the same arguments as
 * attn_bwd minus the workspace and gives bit-identical results: the
 * workspace lives in a fixed, file-scope device array of
 * attn_bwd_noalloc_max_workspace_bytes() bytes (16 MiB) per GPU, held by each
 * GPU the library runs on until the process ends. Nothing is allocated.
 * Limit: attn_bwd_workspace_bytes(p) must not exceed that size (about 2^21
 * query rows B*H*N in all); larger problems return ATTN_ERR_TOO_LARGE before
 * anything is enqueued. Parameter errors are reported as attn_bwd reports
 * them. The array belongs to the GPU of `stream` (the current device for the
 * NULL stream); its address is looked up once per GPU. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (from two
 * host threads, or on two streams with no ordering between them) race on it.
 * Calls ordered on one stream are safe, and nothing in the array needs to
 * start at zero. */
attn_status attn_bwd_noalloc(const attn_params* p, const void* q, const void* k,
                             const void* v, const void* o, const float* lse,
                             const void* d_o, void* dq, void* dk, void* dv, void* stream);

/* Size in bytes of attn_bwd_noalloc's per-GPU scratch array (its limit on
 * attn_bwd_workspace_bytes). */
size_t attn_bwd_noalloc_max_workspace_bytes(void);

/* Library version as major*10000 + minor*100 + patch (0.3.0: Nk explicit;
 * 0.4.0: fp8 forward; 0.5.0: backward workspace rows padded to a multiple of 4). */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTN_H */
