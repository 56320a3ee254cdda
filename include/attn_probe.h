/* attn_probe.h -- design probes of the attention library (libattn_probe.so).
 *
 * Not part of the attention path: each entry point times an alternative
 * design against which the library's own choice was measured.  Same
 * conventions as attn.h (bf16 tensors in device memory, a HIP stream or NULL
 * for the null stream; work is only queued).
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Large-head-dim alternative that splits the output columns across the waves
 * of a workgroup (one kernel, no materialised scores): O = softmax(scale Q K^T) V
 * for B x H independent heads, q, k, v, out contiguous bf16 [B, H, L, 1024].
 * It is the streaming softmax of the FastVideo / cuDNN pages (running row
 * maximum and sum, exp2 with the scale folded in) with each 1024-long dot
 * product split into eight 128-channel shares summed through LDS.  Returns 0,
 * 1 for a NULL pointer, 2 for d != 1024 or sizes out of range, 8 for a failed
 * launch.  No mask. */
int attn_probe_split_columns(const void* q, const void* k, const void* v, void* out, int64_t B,
                             int64_t H, int64_t L, int64_t d, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
