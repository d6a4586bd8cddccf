/*
 * moe_prof.h -- kernel timing for measurement tools (benchmarks, profilers).
 *
 * While enabled on a layer, every launch of a selected kernel family is
 * bracketed by two HIP events recorded on the stream of the call that
 * launched it, so the elapsed time between them is that kernel's duration on
 * its own stream.  Not needed for computing anything; the layer behaves the
 * same with timing on or off apart from the two event records per launch.
 * Sources: the LazyLoRA README ("Cost, measured" / LAZYLORA_PROFILE) and the
 * Two Desks write-up (Act IV: a measurement step that cannot measure is an error, not a pass) time
 * the engine's own kernels; this is the same facility for the GPU layer.
 */
#ifndef MOE_PROF_H
#define MOE_PROF_H

#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* kernel families */
typedef enum {
    MOE_PROF_ROUTER_LOGITS = 0,  /* fp32 router logits and error bounds */
    MOE_PROF_ROUTER_TOPK = 1,    /* top-k selection, fp64 re-ranking, softmax */
    MOE_PROF_GROUP = 2,          /* histogram / scan / stable permute */
    MOE_PROF_GATEUP = 3,         /* dequant + gate/up + SwiGLU */
    MOE_PROF_DOWN = 4,           /* dequant + down + routing weight */
    MOE_PROF_COMBINE = 5,        /* fixed-order combine */
    MOE_PROF_BWD_DOWN = 6,       /* transposed down product + SwiGLU backward */
    MOE_PROF_BWD_GATEUP = 7,     /* transposed gate/up products */
    MOE_PROF_BWD_FINAL = 8,      /* slot reduction + router term */
    MOE_PROF_XTERMS = 9,         /* x as two E4M3 terms for the block-scaled gate/up */
    MOE_PROF_NKERNELS = 10
} moe_prof_kernel;

/* Enable timing of the families whose bit (1u << family) is set in mask, for
 * at most max_launches launches per family (events are created here, on the
 * host, before any timed work); mask = 0 disables timing and releases the
 * events.  Clears previous records.  Returns MOE_ERR_INVALID_ARG for a NULL
 * layer or max_launches outside 1..65536, MOE_ERR_DEVICE if events cannot be
 * created. */
moe_status moe_prof_enable(moe_layer *L, uint32_t mask, int32_t max_launches);

/* Total milliseconds and number of recorded launches of one family since the
 * last enable.  Waits for the recorded events (a host synchronization). */
moe_status moe_prof_read(moe_layer *L, int32_t family, double *total_ms, int32_t *launches);

/* Reference stream: reads `bytes` of the device buffer buf once with a plain coalesced
 * kernel (16 bytes per lane, 2048 blocks of 256 threads), enqueued on stream, and
 * returns that kernel's own duration in *ms (waits for it: a host synchronization).  It
 * gives the practical HBM read rate for a transfer of that size (launch ramp and tail
 * included), beside the 8 TB/s peak, for judging the expert stream kernels.  buf must
 * be 16-byte aligned and bytes a nonzero multiple of 16 (else MOE_ERR_INVALID_ARG);
 * nothing is written.  MOE_ERR_DEVICE if the launch or the events fail. */
moe_status moe_prof_hbm_read(const void *buf, size_t bytes, void *stream, double *ms);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROF_H */
