/*
 * dit_block_steps.h - step-level entry points of the DiT block library.
 *
 * Each call enqueues exactly one kernel of the block forward, so each step of
 * the method can be checked and timed on its own. Same conventions as
 * dit_block.h: device pointers, row-major, 16-byte aligned; return codes
 * DIT_OK / DIT_EINVAL / DIT_EHIP; validation before any launch; nothing
 * allocated; `stream` is a hipStream_t (NULL = null stream).
 * Type codes: DIT_F32 (fp32), DIT_BF16 (bf16), DIT_W8_BF16 (bf16 activations,
 * int8 weights with fp32 per-row scales).
 */
#ifndef DIT_BLOCK_STEPS_H
#define DIT_BLOCK_STEPS_H

#include <stddef.h>
#include <stdint.h>

#include "dit_block.h"

#ifdef __cplusplus
extern "C" {
#endif

/* adaLN-modulated LayerNorm of `rows` token rows ("LayerStream: H3 Chunking",
 * "How the slicing works": the normalisation and modulation are token-wise):
 *   out[r][c] = (x[r][c] - mean_r) / sqrt(var_r + eps) * (1 + scale[c]) + shift[c]
 * mean and biased variance over the d values of row r, in fp32.
 * x: [rows][ldx] of in_dtype (DIT_F32 or DIT_BF16); out: [rows][ldo] of
 * out_dtype; shift, scale: [d] fp32. d % 8 == 0, 8 <= d <= 8192,
 * ldx, ldo >= d and multiples of 8. rows == 0 enqueues nothing. */
int dit_modnorm(int32_t in_dtype, int32_t out_dtype, const void* x, int64_t ldx,
                const float* shift, const float* scale, void* out, int64_t ldo, int64_t rows,
                int64_t d, float eps, void* stream);

/* Softmax attention of a query slice against global K/V (pass 2 of "How the
 * slicing works"; "Attention requires a stronger contract" of the streaming
 * proposal: bounded Q, global K and V, output in Q-sized slabs):
 *   o[i][h] = sum_j softmax_j(q[i][h] . k[j][h] / sqrt(head_dim)) v[j][h]
 * over all n_kv keys j, bidirectional, no mask; [h] = columns h*head_dim ..
 * h*head_dim + head_dim - 1.
 * q: [n_q][ldq], k: [n_kv][ldk], o: [n_q][ldo]; vt: V transposed,
 * [n_heads*head_dim][ldvt] (row c holds column c of V for all keys).
 * dtype DIT_F32 or DIT_BF16 (fp32 softmax, bf16 P and O for DIT_BF16).
 * head_dim 64 or 128; ldq, ldk, ldo >= n_heads*head_dim; ldvt >= n_kv and
 * head_dim * ldvt * (element bytes) < 2^32 (32-bit offsets within a head's V^T rows);
 * all leading dimensions multiples of 8. The bf16 kernel may read V^T
 * columns n_kv .. (n_kv rounded up to 8) - 1 (inside each row, since ldvt is
 * a multiple of 8) and never lets their values reach o, whatever they hold.
 * n_q == 0 enqueues nothing. */
int dit_attention(int32_t dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                  const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv,
                  int64_t n_heads, int64_t head_dim, void* stream);

/* dit_attention with each query's keys cut into contiguous ranges that
 * separate workgroups attend, merged afterwards: more workgroups for short
 * query slices. Range p of S = min(splits, ceil(n_kv/64)) is key tiles
 * [p*T/S, (p+1)*T/S) of the T = ceil(n_kv/64) 64-key tiles (the cut depends
 * only on n_kv and splits, never on the query rows). Each range's
 * unnormalised fp32 O, running max m and row sum l go to the workspace; a
 * second kernel forms O = (sum_p w_p O_p) / (sum_p w_p l_p) with
 * w_p = exp2((m_p - max_p m_p) * log2(e) / sqrt(head_dim)), p in order.
 * The result is within rounding of dit_attention (splits = 1 is
 * dit_attention exactly), and a query's bits do not depend on the other
 * query rows of the call.
 * workspace: at least dit_attention_split_workspace() bytes, 16-byte aligned,
 * device memory owned by the caller (unused when S = 1).
 * Other arguments and errors as dit_attention; splits outside 1..64 is
 * DIT_EINVAL, a smaller workspace DIT_ENOSPC. */
int dit_attention_split(int32_t dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                        const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv,
                        int64_t n_heads, int64_t head_dim, int64_t splits, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes of dit_attention_split (host arithmetic): with S as there
 * and d = n_heads*head_dim, 0 when S = 1, else
 *   round_up(S*n_q*d*4, 256) + round_up(S*n_q*n_heads*2*4, 256). */
int dit_attention_split_workspace(int64_t n_q, int64_t n_kv, int64_t n_heads, int64_t head_dim, int64_t splits,
                                  size_t* bytes_out);

/* QK RMSNorm and/or RoPE in place on `rows` token rows (the Q normalization /
 * positional transform of the streamed-Q plan, "Attention requires a stronger
 * contract" of the streaming proposal):
 *   norm_w != NULL: per head, t <- t / sqrt(mean(t^2) + eps) * norm_w  ([head_dim] fp32)
 *   rope_cos/sin != NULL: per head pair j of row i, (a, b) <- (a c - b s, a s + b c),
 *     c = rope_cos[i*ld_rope + j], s = rope_sin[i*ld_rope + j]
 * x: [rows][ldx] of dtype DIT_F32 or DIT_BF16, d = n_heads*head_dim;
 * head_dim 64 or 128; d <= 8192; ldx >= d, multiple of 8; ld_rope >=
 * head_dim/2, multiple of 4; rope tables both or neither. */
int dit_qk_transform(int32_t dtype, void* x, int64_t ldx, int64_t rows, int64_t n_heads, int64_t head_dim,
                     const float* norm_w, const float* rope_cos, const float* rope_sin, int64_t ld_rope,
                     float eps, void* stream);

/* Epilogues of dit_linear (acc = sum_k a[m][k] * w[n][k] * s[n]). */
#define DIT_EPI_STORE 0    /* out[m][n] = acc (activation type) */
#define DIT_EPI_STORE_T 1  /* out[n][m] = acc (transposed store, used for V) */
#define DIT_EPI_RESID 2    /* out[m][n] (fp32) = aux[m][n] + gate[n] * acc: the gated
                              residual of the out-projection ("How the slicing works":
                              project and add into the residual) */
#define DIT_EPI_GATEUP 3   /* out[m][f] = silu(acc over w row f) * (acc over w row
                              f + up_offset): SwiGLU ("MLP planning" of the streaming
                              proposal); n counts features f */
#define DIT_EPI_ACCUM 4    /* out[m][n] (fp32) += gate[n] * acc: one FFN feature slice's
                              partial ("MLP planning": accumulate into the output) */
#define DIT_EPI_FINAL 5    /* out[m][n] = aux[m][n] (fp32) + gate[n] * acc, rounded once
                              to the activation type */

/* One projection over token rows with a fused epilogue.
 *   a: [m][lda] activations (fp32 for DIT_F32, else bf16); k columns used.
 *   w: [n][ldw] weight rows (fp32 / bf16 / int8 by dtype); k columns used.
 *   w_scale: per weight row fp32 scale (DIT_W8_BF16 only, else NULL).
 *   up_offset: DIT_EPI_GATEUP only, rows from a gate row to its up row.
 *   out: [m][ldo] (or [n][ldo] for DIT_EPI_STORE_T); aux: [m][ldaux];
 *   gate: [n] fp32 (RESID, ACCUM, FINAL).
 * k % 64 == 0 (k % 32 for DIT_F32); n % 64 == 0; leading dims multiples of 8
 * (of 16 for int8 weights). The kernel reaches the rows of one 256-row tile
 * through 32-bit byte offsets, so 256 * lda * (activation bytes) and
 * R * ldw * (weight bytes) must stay below 2^32, with R = up_offset + 256 for
 * DIT_EPI_GATEUP and 256 otherwise; else DIT_EINVAL. m == 0 enqueues nothing. */
int dit_linear(int32_t dtype, int32_t epilogue, const void* a, int64_t lda, const void* w,
               int64_t ldw, const float* w_scale, int64_t up_offset, int64_t m, int64_t n,
               int64_t k, void* out, int64_t ldo, const void* aux, int64_t ldaux,
               const float* gate, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_BLOCK_STEPS_H */
