/*
 * libvit_probe.so: measurement support, not part of the attention path and
 * not part of libvit.so.  No page defines this operation; bench.py uses it to
 * state what a bf16 MFMA kernel can sustain on data like its inputs.
 */
#ifndef VIT_PROBE_H
#define VIT_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The sustained bf16 MFMA rate on given operand data.  MI355X lowers its
 * clock when MFMA operands toggle many bits, so the rate depends on the data;
 * timing this probe with operands drawn like the inputs brackets what any
 * bf16 MFMA kernel can reach on them.  Runs `blocks` workgroups of 4 waves;
 * each wave issues 32 * iters v_mfma_f32_32x32x16_bf16 (4 * 32 * iters *
 * 32768 FLOP per workgroup) on operands read once.
 *  operands      device, 16-byte aligned, at least 4 MiB (64 slices of 256
 *                threads x 256 bytes, read as bf16); operand_bytes its size.
 *  sink          device float [blocks * 256], written (keeps the work live).
 *  blocks        1 .. 65536; iters 1 .. 2^20.
 * Returns 0, 1 (invalid argument, checked before the launch) or 3 (HIP
 * launch error); the message of a failed call is in vit_probe_last_error().
 */
int vit_probe_mfma(const void* operands, int64_t operand_bytes, int blocks, int iters, float* sink,
                   hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* vit_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif  // VIT_PROBE_H
