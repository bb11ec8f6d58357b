/*
 * fa355 measurement aids (not part of the attention library): a dense
 * matrix-core throughput probe, so that kernel efficiencies can be quoted
 * against the peak the chip actually delivers at the clock it actually runs,
 * next to the published one, and a co-issue probe of the execution units
 * one CU shares.  Built as libfa355_probe.so.
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

/*
 * Co-issue probe: how the matrix core, the vector ALUs, the transcendental
 * unit and LDS reads share one CU.  Launch `blocks` workgroups of 8 waves
 * (at most one per CU; waves w and w + 4 share a SIMD) on `stream`.  Each
 * wave runs `iters` iterations of the role its mode gives it:
 *   MFMA     8 independent v_mfma_f32_32x32x16_bf16 chains (8 per iteration)
 *   FMA      16 independent v_fma_f32 chains, 64 instructions per iteration
 *   EXP      16 independent v_exp_f32 chains, 16 instructions per iteration
 *   LDS      8 ds_read_b128 per iteration (1 KiB per wave-wide read)
 *   LDS-TR   8 ds_read_b64_tr_b16 per iteration (512 bytes per read)
 *   MFMA+EXP the MFMA role with 4 v_exp_f32 after every MFMA (one wave)
 *   MFMA+FMA the MFMA role with 16 v_fma_f32 after every MFMA (one wave)
 *   BURST    the 8 MFMAs of an iteration back to back, then 128 v_fma_f32
 *   MIXk     k v_fma_f32 after every MFMA (k = 2, 4, 6, 8); MIX5E1: five
 *            v_fma_f32 and one v_exp_f32 after every MFMA
 *   idle     nothing
 * mode: roles of (waves 0-3, waves 4-7):
 *    0 (MFMA, MFMA)     1 (MFMA, idle)     2 (MFMA, FMA)    3 (MFMA, EXP)
 *    4 (idle, FMA)      5 (idle, EXP)      6 (FMA, FMA)     7 (LDS, LDS)
 *    8 (LDS-TR, LDS-TR) 9 (MFMA+EXP, idle) 10 (MFMA+FMA, idle)
 *   11 (MFMA, LDS)     12 (MFMA, LDS-TR)  13 (EXP, EXP)    14 (LDS, idle)
 *   15 (MFMA+FMA, MFMA+FMA)                16 (MFMA+EXP, MFMA+EXP)
 *   17 (BURST, BURST)  18 (MIX2, MIX2)    19 (MIX4, MIX4)  20 (MIX6, MIX6)
 *   21 (MIX8, MIX8)    22 (MIX5E1, MIX5E1)
 * cycles: DEVICE uint64 [16 * blocks]: entry 16 b + w is the shader-clock
 * span (s_memtime) of wave w of block b around its role, entry 16 b + 8 + w
 * the span of the 100 MHz reference counter (s_memrealtime).
 * sink: DEVICE float [512 * blocks] (keeps results live; meaningless).
 * Returns 0, or the HIP error code of the launch; 1 for a bad argument
 * (mode outside 0..22, iters or blocks < 1, null pointer).
 */
int fa355_coexec_probe(int mode, int iters, int blocks, uint64_t* cycles,
                       float* sink, void* stream);

/*
 * Atomic-accumulation probe: the HBM traffic of forming dQ inside the
 * key-outer dK/dV kernel ("FlashAttention: making attention IO-aware", "The
 * backward pass: recompute, don't store": dQ_i accumulates scale dS_ij K_j
 * over every key block j).  Launch BH * ceil(N / 128) workgroups of 512
 * threads on `stream`, in the head-grouped order of the dK/dV kernel; each
 * adds one 64 x d fp32 tile per 64-row query tile that its 128 keys see
 * (all tiles, or under a causal mask those from its first key on) into
 * dq with global fp32 atomic adds (2^-10 per element per visit).
 * dq: DEVICE float [BH, N, d], caller-owned; incremented in place.
 * Returns 0, or the HIP error code of the launch; 1 for a bad argument
 * (BH or N < 1, d not 64 or 128, null dq).
 */
int fa355_atomic_probe(int BH, int N, int d, int causal, float* dq,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif
