/*
 * Device side of the seeded synthetic-input generator (not part of the decode path).
 *
 * Element i of tensor (seed, tensor_id) is produced from the i-th output of a
 * SplitMix64 stream (Steele, Lea and Flood, OOPSLA 2014; Vigna's splitmix64.c):
 *   x0  = mix((seed ^ (tensor_id << 32)) + GAMMA)          (first output of that seed)
 *   r_i = mix(x0 + (i + 1) * GAMMA),   GAMMA = 0x9e3779b97f4a7c15, arithmetic mod 2^64
 *   z_i = (u0 + u1 + u2 + u3 - 131070) * (sqrt(3) / 65536)    u_j = 16-bit fields of r_i
 * mode 0 (normal): value = fp32(z_i * std)
 * mode 1 (gain):   value = fp32(1 + z_i * std)
 * mode 2 (const):  value = fp32(std)
 * every step an IEEE double operation rounded to nearest even (no fused multiply-add);
 * bf16 tensors round the fp32 value to bf16 (nearest even).  The host generator in the
 * `synth` Python module implements the same definition, so values are bit-identical.
 * Lets 15 GB of weights be made on the GPU instead of crossing PCIe.
 */
#ifndef DLLM_SYNTH_H
#define DLLM_SYNTH_H
#include <stdint.h>
#include "dllm.h"
#ifdef __cplusplus
extern "C" {
#endif

/* dst: device buffer of n elements of dtype (dllm_dtype).  Enqueued on stream.      */
dllm_status dllm_synth_fill(void* dst, int64_t n, int32_t dtype, uint64_t seed,
                            uint32_t tensor_id, double std, int32_t mode,
                            dllm_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
