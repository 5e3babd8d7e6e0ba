/*
 * moe_probe.h -- machine-rate probes of libmoe for the measurement harness.
 * They are not part of the layer: they measure, on the GPU at hand, the two
 * ceilings the expert GEMMs run against, so that achieved rates can be given
 * as fractions of measured peaks as well as of the published ones.
 *
 * Both calls launch one kernel on `stream` (a hipStream_t; NULL = the null
 * stream) and return at once; the caller times them with events on the same
 * stream.  Return value: MOE_OK (0), MOE_ERR_ARG (1) for a bad argument (then
 * nothing is launched and moe_last_error() says why), or MOE_ERR_HIP (4) if
 * the launch failed.  Pointers are device pointers owned by the caller.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HBM read rate through global -> LDS direct copies, the way the expert GEMMs
 * stream their weights.  `blocks` workgroups of 512 threads (one per CU at a
 * time: each holds 128 KB of LDS) each read a contiguous bytes/blocks share of
 * buf in 64 KB steps through two LDS stages, and fold one word per step into
 * sink[block * 512 + thread] (u32) so the reads cannot be dropped.
 *  buf    [bytes]        read only; 16-byte aligned
 *  bytes  a positive multiple of blocks * 65536, below 2^40
 *  blocks 1 .. 65536
 *  sink   [blocks * 512] u32, written
 */
int moe_probe_hbm_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream);

/* MFMA rate of a register-resident loop of the expert GEMMs' instruction:
 * `blocks` workgroups of 8 waves (2 per SIMD, as in the GEMMs), each wave
 * running `iters` rounds of 10 independent accumulations.
 *  dtype MOE_BF16:      v_mfma_f32_32x32x16_bf16, 32768 flop each
 *  dtype MOE_FP8_E4M3:  v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales),
 *                       131072 flop each
 * so flop = blocks * 8 * iters * 10 * (flop each).
 *  iters  1 .. 2^24;  blocks 1 .. 65536
 *  sink   [blocks * 512] fp32, written (the accumulator sums)
 */
int moe_probe_mfma(int32_t dtype, int32_t iters, int blocks, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
