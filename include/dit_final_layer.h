/*
 * dit_final_layer.h - the output head that follows the last DiT block, with
 * bounded activation memory.
 *
 * "LayerStream: H3 Chunking", section "How the slicing works": the output head
 * runs in fp32, and it is the one place where the pack slices by tokens only
 * when memory runs out. "Proposal: Generic memory-aware streaming execution
 * for transformer models", section "Summary": the final projection and
 * modulation are bounded like the block's token-wise steps.
 *
 * Computed (fp32 arithmetic throughout):
 *   out[t][j] = sum_c (LN(x[t])[c] * (1 + scale[c]) + shift[c]) * w_out[j][c]
 * LN as in the block: no affine, mean and biased variance over the d values of
 * row t, eps inside the square root. No bias term.
 *
 * Memory: the head is token-wise and this library fuses it into one kernel
 * whose token slab is 64 rows per workgroup, so the normalised and modulated
 * rows never exist in device memory: the only device memory touched besides
 * the inputs is `out`. No workspace, no allocation. Since rows are
 * independent, a caller may also call it on any range of rows (x + r0*ldx,
 * out + r0*ldo); each row's output bits are the same whichever range it was
 * computed in.
 *
 * Conventions as dit_block.h: device pointers, row-major; return codes DIT_OK /
 * DIT_EINVAL / DIT_EHIP; validation before any launch; `stream` is a
 * hipStream_t (NULL = the null stream); nothing synchronises.
 */
#ifndef DIT_FINAL_LAYER_H
#define DIT_FINAL_LAYER_H

#include <stddef.h>
#include <stdint.h>

#include "dit_block.h"

#ifdef __cplusplus
extern "C" {
#endif

/* x: [n_tokens][ldx] activations, x_dtype DIT_F32 or DIT_BF16, 16-byte aligned,
 *    ldx >= d and a multiple of 8. Read only.
 * shift, scale: [d] fp32, 16-byte aligned (the head's modulation vectors).
 * w_out: [out_dim][d] fp32 row-major, 16-byte aligned (the projection; output
 *    column j uses row j).
 * out: [n_tokens][ldo] fp32, 4-byte aligned, ldo >= out_dim; written.
 * d % 64 == 0, 64 <= d <= 8192; 1 <= out_dim <= 128; eps > 0.
 * n_tokens == 0 enqueues nothing (x and out may then be NULL).
 * Errors: DIT_EINVAL for any violation above or a null pointer; DIT_EHIP if
 * the launch fails. */
int dit_final_layer(int32_t x_dtype, const void* x, int64_t ldx, int64_t n_tokens, int64_t d, const float* shift,
                    const float* scale, const float* w_out, int64_t out_dim, float* out, int64_t ldo, float eps,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_FINAL_LAYER_H */
