/*
 * dit_block_profile.h - optional per-kernel timing of dit_block_forward.
 *
 * While enabled, dit_block_forward (and dit_final_layer) records a pair of HIP events on its stream
 * around every kernel it enqueues, tagged with the step of the block that the
 * kernel computes. Reading waits for those events and returns the summed
 * elapsed time and the launch count per step. Off by default; when off the
 * forward records nothing. Enabling is process-wide and not meant for
 * concurrent forwards on several streams. HIP events are created on first
 * use while enabled (host-side handles only; no device memory is allocated)
 * and reused afterwards.
 */
#ifndef DIT_BLOCK_PROFILE_H
#define DIT_BLOCK_PROFILE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Steps of the block, as tagged by the profiler. */
#define DIT_K_MODNORM 0    /* norm1 (modulated LayerNorm of x) */
#define DIT_K_KV_PROJ 1    /* pass 1: K and V projections of a token slab */
#define DIT_K_Q_PROJ 2     /* pass 2: Q projection of a slice */
#define DIT_K_ATTENTION 3  /* pass 2: attention of a slice against global K/V */
#define DIT_K_OUT_PROJ 4   /* out-projection + gated residual into fp32 staging */
#define DIT_K_GATE_UP 5    /* SwiGLU gate/up projection of an MLP slab */
#define DIT_K_DOWN 6       /* down projection + gated residual, in place */
#define DIT_K_QK 7         /* optional QK RMSNorm / RoPE of a Q or K slab */
#define DIT_K_FINAL 8      /* dit_final_layer: the output head */
#define DIT_K_LORA 9       /* adapter inputs t = alpha * (A a) of one launch group */
#define DIT_K_NORM2 10     /* norm2 (modulated LayerNorm of the fp32 staged residual) */
#define DIT_K_COUNT 11

/* on != 0: clear all records and start recording; on == 0: stop recording
 * (records are kept for dit_profile_read). Returns DIT_OK. */
int dit_profile_enable(int on);

/* Summed elapsed milliseconds and launch count of one step over the records
 * since the last enable. Synchronises on the recorded events.
 * DIT_EINVAL for a bad kind or null pointer, DIT_EHIP on a HIP error. */
int dit_profile_read(int kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DIT_BLOCK_PROFILE_H */
