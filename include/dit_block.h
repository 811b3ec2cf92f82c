/*
 * dit_block.h - C ABI of the token-chunked, activation-bounded forward pass of
 * one DiT transformer block on MI355X (gfx950).
 *
 * The method is the one of "LayerStream: H3 Chunking"
 * (comfy.icu/node/LayerStreamH3Chunking), sections "How the slicing works" and
 * "The two numbers you set", and of "Proposal: Generic memory-aware streaming
 * execution for transformer models" (github.com/Comfy-Org/ComfyUI/discussions/
 * 15920), sections "MLP planning" and "Attention requires a stronger
 * contract":
 *   - norms, modulation, projections and the MLP are token-wise and run on
 *     token slices that add into the residual stream in place;
 *   - attention runs in two passes: pass 1 keeps only K and V for all tokens;
 *     pass 2 recomputes Q per slice, attends the slice against the full K/V,
 *     out-projects and adds into the residual;
 *   - the gated MLP can additionally be split along its FFN features, each
 *     slice projected, activated, down-projected and accumulated.
 *
 * The block computed (fp64 meaning; the oracle is this definition):
 *   n1 = LN(x) * (1 + scale1) + shift1          LN: no affine, biased var, eps
 *   q, k, v = n1 Wq^T, n1 Wk^T, n1 Wv^T          Wq|Wk|Wv = rows of w_qkv
 *   o  = softmax(q k^T / sqrt(dh)) v             per head, bidirectional, no mask
 *   x1 = x + gate1 * (o Wo^T)
 *   n2 = LN(x1) * (1 + scale2) + shift2
 *   y  = x1 + gate2 * ((silu(n2 Wg^T) * (n2 Wu^T)) Wd^T)   Wg|Wu = rows of w_gu
 *
 * All functions are thread-safe for distinct handles. A handle may be used by
 * one stream at a time. No function allocates device memory; dit_block_forward
 * only enqueues kernels on the given stream and never synchronises.
 */
#ifndef DIT_BLOCK_H
#define DIT_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Every argument error is reported before any kernel is
 * enqueued; nothing falls back to another path (the streaming proposal's
 * "Patch compatibility" section: fail closed rather than degrade). */
#define DIT_OK 0
#define DIT_EINVAL (-1)  /* bad argument: null pointer, shape, chunk value, alignment */
#define DIT_ENOSPC (-2)  /* workspace_bytes below dit_block_peak_workspace() */
#define DIT_EHIP (-3)    /* the HIP runtime reported a launch error */
#define DIT_ETOOBIG (-4) /* dit_block_forward_noalloc: the sizes need more than
                            DIT_STATIC_WORKSPACE_BYTES of workspace */

/* Storage types. F32: activations and weights fp32, fp32 arithmetic.
 * BF16: activations and weights bf16, fp32 accumulation and softmax.
 * W8_BF16: bf16 activations, int8 weights with one fp32 scale per output row
 * (W[n][k] = s[n] * q[n][k]; the per-row weight_scale of the Ascend port's
 * TensorWiseINT8 layout, m.qwbw.cn/news/87515, section 2.2). */
#define DIT_F32 0
#define DIT_BF16 1
#define DIT_W8_BF16 2

typedef struct dit_block dit_block;

typedef struct dit_block_desc {
  int64_t d;         /* hidden size; must equal n_heads * head_dim */
  int64_t n_heads;
  int64_t head_dim;  /* 64 or 128 */
  int64_t ffn;       /* SwiGLU width F; multiple of 64 */
  int32_t dtype;     /* DIT_F32, DIT_BF16 or DIT_W8_BF16 */
  float eps;         /* LayerNorm epsilon (1e-6 for the DiT blocks here) */
} dit_block_desc;

/* Device pointers, row-major [out][in], borrowed: the caller keeps them alive
 * and unchanged until dit_block_destroy. Element type: fp32 (F32), bf16
 * (BF16) or int8 (W8_BF16). 16-byte aligned. */
typedef struct dit_block_weights {
  const void* w_qkv;   /* [3d][d]: rows [0,d) = Wq, [d,2d) = Wk, [2d,3d) = Wv;
                          head h owns rows h*dh .. h*dh+dh-1 of each */
  const void* w_o;     /* [d][d] */
  const void* w_gu;    /* [2F][d]: rows [0,F) = gate, [F,2F) = up; feature f
                          pairs gate row f with up row F+f */
  const void* w_down;  /* [d][F] */
  const float* s_qkv;  /* W8_BF16 only: fp32 scale per output row, [3d] */
  const float* s_o;    /* [d] */
  const float* s_gu;   /* [2F] */
  const float* s_down; /* [d] */
  /* Optional QK RMSNorm weights, fp32 [head_dim], shared by all heads (NULL =
   * no normalization): per token and head, t <- t / sqrt(mean(t^2) + eps) * w,
   * applied to Q and K after their projection ("Proposal: Generic
   * memory-aware streaming execution ...", "Attention requires a stronger
   * contract": the model's Q normalization inside the streamed-Q plan). */
  const float* q_norm;
  const float* k_norm;
} dit_block_weights;

/* Validate the descriptor and weight pointers and create a handle that holds
 * only host metadata (no device calls). *out is set on success.
 * Errors: DIT_EINVAL for a null pointer, d != n_heads*head_dim, head_dim not
 * in {64,128}, ffn < 64 or not a multiple of 64, an unknown dtype, eps <= 0,
 * a weight pointer not 16-byte aligned, or a missing W8 scale; also when
 * (ffn + 256) * d or 256 * ffn weight or activation elements reach 2^32 bytes
 * (the projections address one tile's rows with 32-bit byte offsets). */
int dit_block_create(const dit_block_desc* desc, const dit_block_weights* w, dit_block** out);

/* Exact workspace bytes that dit_block_forward needs for these arguments
 * (host arithmetic only). With e = activation bytes (4 for F32, else 2),
 * Ca = attn_chunk_tokens (0 -> N), Cm = mlp_chunk_tokens, fc =
 * ffn_chunk_features (0 -> F), each clamped to N (fc to F), S = max(Ca, Cm)
 * and Np = N rounded up to 64, each region rounded up to 256 bytes:
 *     N*d*e           global K            (kept for the whole sequence)
 *   + d*Np*e          global V, stored transposed [d][Np]
 *   + S*d*4           fp32 residual staging for one super-slice
 *   + max(2*Ca*d*e, Cm*d*e + Cm*fc*e)    slabs: norm/O + Q, or norm2 + h
 *   + (S > 1 only) S*Ca*d*4 + S*Ca*H*2*4 the key ranges' partial O, m and l
 *     (S = min(attention splits, ceil(N/64)), H = n_heads; see
 *     dit_block_set_attention_splits)
 * Only the K/V terms grow with N ("Where people get burned": K and V for the
 * whole sequence stay resident and set the memory floor). Same argument
 * rules and errors as dit_block_forward. */
int dit_block_peak_workspace(const dit_block* h, int64_t n_tokens, int64_t attn_chunk_tokens,
                             int64_t mlp_chunk_tokens, int64_t ffn_chunk_features,
                             size_t* bytes_out);

/* Automatic chunk sizing: the largest chunks whose workspace fits
 * `budget_bytes` ("Proposal: Generic memory-aware streaming execution ...",
 * section "Automatic chunk sizing": pick the largest chunks that fit a memory
 * envelope; "LayerStream: H3 Chunking", "The two numbers you set": use the
 * largest chunk that fits).
 * Candidates use one token chunk C for both attention and MLP slices: all N
 * tokens, or a multiple of 256 (the node's step) below N. The FFN width fc is
 * F, F/2, F/4, ... while it stays a multiple of 64. The choice maximises C,
 * and among equal C prefers the largest fc (no feature slicing when possible).
 * Outputs: *attn_chunk_tokens (0 when C covers all N tokens),
 * *mlp_chunk_tokens = C, *ffn_chunk_features (0 when fc = F); then
 * dit_block_peak_workspace(h, n_tokens, ...) <= budget_bytes.
 * Errors: DIT_EINVAL for a null pointer or n_tokens < 1; DIT_ENOSPC when not
 * even C = 256 fits (global K/V alone is N*d*e + d*Np*e bytes: the floor
 * that chunking cannot go below, "Where people get burned"). */
int dit_block_plan_chunks(const dit_block* h, int64_t n_tokens, size_t budget_bytes,
                          int64_t* attn_chunk_tokens, int64_t* mlp_chunk_tokens,
                          int64_t* ffn_chunk_features);

/* One block forward, in place.
 *   x          [N][d] activations (fp32 for F32, else bf16), read and
 *              overwritten with the block output y. 16-byte aligned.
 *   mod        [6][d] fp32: shift1, scale1, gate1, shift2, scale2, gate2.
 *   n_tokens   N >= 1, and head_dim * Np * e < 2^32 (Np = N rounded up to
 *              64, e = activation bytes): the attention kernel addresses a
 *              head's rows of the transposed V with 32-bit offsets (N below
 *              16.7 M tokens for bf16 at head_dim 128); larger N is DIT_EINVAL.
 *   attn_chunk_tokens   query tokens per attention slice (>= 0; 0 = one slice
 *              of all N tokens, the pages' "stock attention" setting).
 *   mlp_chunk_tokens    tokens per MLP slice (>= 1).
 *   ffn_chunk_features  FFN features per MLP slice (0 = all F; otherwise a
 *              multiple of 64; the last slice may be shorter).
 *   Chunk values above N (F) are clamped. Output bytes are identical for every
 *   (attn_chunk_tokens, mlp_chunk_tokens) at a fixed ffn_chunk_features.
 *   workspace  device scratch of at least dit_block_peak_workspace() bytes,
 *              16-byte aligned, owned by the caller; contents undefined after.
 *   stream     a hipStream_t (NULL = the null stream).
 * Enqueues and returns; no allocation, no host synchronisation.
 * Errors: DIT_EINVAL (null pointer, N < 1, negative chunk, mlp_chunk_tokens <
 * 1, ffn_chunk_features not a multiple of 64, misaligned pointer),
 * DIT_ENOSPC, DIT_EHIP. On an error return nothing has been enqueued, except
 * for DIT_EHIP, which reports a failed launch. */
int dit_block_forward(dit_block* h, void* x, const float* mod, int64_t n_tokens,
                      int64_t attn_chunk_tokens, int64_t mlp_chunk_tokens,
                      int64_t ffn_chunk_features, void* workspace, size_t workspace_bytes,
                      void* stream);

/* dit_block_forward with a rotary positional transform of Q and K: for token
 * i and head pair j, (t[2j], t[2j+1]) <- (a cos - b sin, a sin + b cos) with
 * cos = rope_cos[i][j], sin = rope_sin[i][j] (device, fp32 [N][head_dim/2],
 * 16-byte aligned, read-only), applied after the QK normalization if any (the
 * "positional encoding/RoPE step" of the same plan). Tables may be NULL
 * together (then this equals dit_block_forward); one NULL alone is
 * DIT_EINVAL. Other arguments, errors and guarantees as dit_block_forward. */
int dit_block_forward_rope(dit_block* h, void* x, const float* mod, const float* rope_cos,
                           const float* rope_sin, int64_t n_tokens, int64_t attn_chunk_tokens,
                           int64_t mlp_chunk_tokens, int64_t ffn_chunk_features, void* workspace,
                           size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as dit_block_forward_rope, with the workspace taken from a buffer
 * the library owns instead of a caller argument.
 *   The buffer is a static device array of DIT_STATIC_WORKSPACE_BYTES (64 MiB)
 *   per GPU, loaded with the library's code and held until the process ends.
 *   The first call on a device looks up that device's copy of the array
 *   (hipGetSymbolAddress, host side, with that device current); no call
 *   allocates device memory or calls hipMalloc / hipFree.
 *   The current device's copy is used: `stream` must belong to the current
 *   device.
 *   Sizes whose dit_block_peak_workspace() exceeds DIT_STATIC_WORKSPACE_BYTES
 *   are refused with DIT_ETOOBIG before anything is enqueued (for example a
 *   bf16 block with d = 1024 and F = 4096 needs 44 MiB for 4096 tokens at
 *   chunks of 2048, and 72 MiB at chunks of 4096, which is refused).
 *   Every call on one GPU shares that GPU's buffer, and the buffer keeps the
 *   last call's contents: the forward needs no part of it cleared (every
 *   region is written before it is read), but calls that overlap in time on
 *   one GPU (different streams, or different host threads) race on it and
 *   must be serialised by the caller.
 * Arguments, results and other errors as dit_block_forward_rope (rope tables
 * may be NULL together). */
#define DIT_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int dit_block_forward_noalloc(dit_block* h, void* x, const float* mod, const float* rope_cos,
                              const float* rope_sin, int64_t n_tokens, int64_t attn_chunk_tokens,
                              int64_t mlp_chunk_tokens, int64_t ffn_chunk_features, void* stream);

/* Key ranges per query in the attention of this handle's forwards (default
 * 1). With splits > 1 every query's keys are cut into S = min(splits,
 * ceil(N/64)) contiguous ranges of 64-key tiles, attended by separate
 * workgroups and merged in a fixed order (dit_attention_split), so a short
 * attention slice (small attn_chunk_tokens) still fills the GPU: an
 * attention launch has ceil(Ca/256) * n_heads * S workgroups. The cut
 * depends only on N and splits, so the output bytes are still identical for
 * every (attn_chunk_tokens, mlp_chunk_tokens) at a fixed splits; across
 * different splits they agree within rounding. The workspace grows by the
 * partials' S*Ca*d*4 + S*Ca*H*8 bytes (dit_block_peak_workspace).
 * Host metadata only. Errors: DIT_EINVAL for a null handle or splits
 * outside 1..64. */
int dit_block_set_attention_splits(dit_block* h, int64_t splits);

/* One activation-space adapter ("ComfyUI-StaticPipeline", section
 * "Activation-space LoRA (bypass mode)"): a projection y = W a of the block
 * becomes y = W a + alpha * B (A a), applied to activations so that W stays
 * as stored (int8 weights stay packed int8).
 *   a      device [rank][in], row-major, activation type (fp32 for DIT_F32,
 *          bf16 for DIT_BF16 and DIT_W8_BF16), 16-byte aligned
 *   b      device [out][rank], row-major, same type, 16-byte aligned
 *   rank   0 = no adapter on this projection; else a multiple of 16, <= 256
 *   alpha  the adapter's scale (finite)
 * (in, out) are (d, d) for q, k, v and o, (d, F) for gate and up, (F, d) for
 * down. On the GPU, t = alpha * (A a) is formed in fp32 (bf16 blocks: by a
 * kernel whose workgroups own 32 token rows and split the contraction into a
 * fixed number of contiguous parts, added in a fixed order). The projection's MFMA contraction adds B t to W a in the
 * same fp32 accumulator (int8 weights: after their per-row scale); for bf16,
 * t enters it as its bf16 rounding plus the bf16 rounding of the residual, so
 * the adapter adds no rounding point of its own, and the projection's output
 * is rounded once, as without an adapter. */
typedef struct dit_lora {
  const void* a;
  const void* b;
  int64_t rank;
  float alpha;
} dit_lora;

typedef struct dit_block_lora {
  dit_lora q, k, v, o, gate, up, down;
} dit_block_lora;

/* Attach adapters to the handle (pointers borrowed like the weights; the
 * struct itself is copied). NULL, or every rank 0, detaches them. Host
 * metadata only. With adapters attached, dit_block_peak_workspace grows by
 *   round_up(4 * max(Ca * max(rk + rv, rq, ro), Cm * (rgate + rup + rdown)), 256)
 * bytes (fp32 t of the adapters of one launch group), placed after the other
 * regions. Errors: DIT_EINVAL for a null handle, a rank that is negative, not
 * a multiple of 16 or above 256, a null or misaligned a/b of a present
 * adapter, or a non-finite alpha; the attached set is then unchanged. */
int dit_block_set_lora(dit_block* h, const dit_block_lora* lora);

/* Release the handle (host memory only; the weights stay the caller's). */
void dit_block_destroy(dit_block* h);

/* Static message for a return code. */
const char* dit_block_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DIT_BLOCK_H */
