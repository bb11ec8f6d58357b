/*
 * fa355 measurement aid (not part of the attention library): a dense
 * matrix-core throughput probe, so that kernel efficiencies can be quoted
 * against the peak the chip actually delivers at the clock it actually runs,
 * next to the published one.  Built as libfa355_probe.so.
 */
#ifndef FA355_PROBE_H
#define FA355_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launch `blocks` workgroups of 256 threads on `stream`; every wave runs
 * `iters` rounds of 8 independent MFMA accumulations:
 *   kind 0: v_mfma_f32_32x32x16_bf16       (32768 FLOP per instruction)
 *   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands
 *           (131072 FLOP per instruction)
 * FLOPs of the launch = blocks * 4 * iters * 8 * (FLOP per instruction).
 * clocks: DEVICE uint64 [4], written by the first wave: shader-clock counter
 * (s_memtime) and 100 MHz reference counter (s_memrealtime) at its start and
 * end, so the shader clock = 100 MHz * d(memtime) / d(memrealtime).
 * sink: DEVICE float [blocks] (keeps the results live; contents meaningless).
 * Returns 0, or the HIP error code of the launch; 1 for a bad argument.
 */
int fa355_mfma_probe(int kind, int iters, int blocks, uint64_t* clocks,
                     float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
