// Bench-only diagnostic, outside the MoE path and outside the library's ABI
// (include/moe.h): a dense register-only MFMA loop for stating a measured
// MFMA peak beside the published one.  Built into libmoe_probe.so.
#pragma once
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif
/* Enqueues one kernel of `blocks` workgroups of 4 waves; every wave runs
 * iters x 16 MFMA 32x32x16 bf16 instructions from registers only (no memory
 * traffic, no LDS), then each thread writes one float to out[blocks * 256]
 * (device memory, caller-owned).  Work: blocks * iters * 4 * 16 * 32768
 * flops; time it with events on the stream.  Returns 0, -1 for blocks or
 * iters < 1 or out NULL, else the HIP error code of the launch. */
int moe_probe_mfma_rate(int32_t blocks, int32_t iters, float* out, void* stream);
#ifdef __cplusplus
}
#endif
