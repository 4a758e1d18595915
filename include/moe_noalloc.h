/*
 * moe_noalloc.h -- the routed MoE layer's forward pass for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same conventions as
 * moe.h, whose types it uses.
 */
#ifndef MOE_MI355X_NOALLOC_H
#define MOE_MI355X_NOALLOC_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the library's own forward scratch on each GPU: 64 MiB. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward with its workspace taken from a device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library keeps on each GPU it runs on
 * (loaded with the library, held until the process ends); the caller still
 * passes the plan, x, the weights and y, and everything else follows
 * moe_forward. It allocates no device memory and calls no allocating
 * routine: MOE_OPT_PHASE_EVENTS is ignored (recording would create events)
 * and every launch stays on `stream`, as with MOE_OPT_ONE_STREAM (the
 * second stream of moe_forward is created on its first use).
 * A call whose moe_forward_workspace_bytes exceeds the scratch returns
 * MOE_EWORKSPACE before any launch (decode-shaped calls and short prompts
 * fit: the 128-token prompt over 128 experts of d_model 2048 / d_ff 768
 * needs about 46 MiB). The scratch keeps the last call's contents; nothing
 * in it needs to start at zero. Every call on one GPU uses that GPU's one
 * array: calls that overlap on a GPU (other streams, other host threads)
 * race and give wrong results, so serialise them. */
moe_status moe_forward_noalloc(const moe_plan *plan, const void *x,
                               int32_t x_dtype, moe_weight w_gate,
                               moe_weight w_up, moe_weight w_down, int32_t D,
                               int32_t F, void *y, int32_t y_dtype,
                               const moe_options *opt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_NOALLOC_H */
