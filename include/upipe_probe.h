/*
 * upipe_probe.h - a measurement probe of the MI355X (gfx950) matrix cores
 * under sustained load.  The benchmark reports with it the bf16 MFMA rate
 * the chip attains on given operand data beside the published peak: under
 * MFMA load the chip is power-limited and its clock depends on the data.
 * Not part of the attention layer.
 *
 * upipe_probe_mfma enqueues on `stream` one kernel of `workgroups`
 * workgroups of 256 threads (4 waves), each holding 64 KB of LDS so that a
 * CU runs at most two of them: 2 * CUs workgroups give two waves per SIMD.  Each wave loads eight A and eight B operand fragments of
 * v_mfma_f32_32x32x16_bf16 from `operands` once and then runs `iters`
 * rounds of 32 such MFMAs (four independent accumulator chains cycling
 * through the fragments), i.e. 32 * 32768 FLOP per round and wave.  It then
 * writes
 *   sink[t]             a sum of thread t's accumulators (keeps the work);
 *   clocks[2 w]         shader-clock ticks (s_memtime) over wave w's loop;
 *   clocks[2 w + 1]     constant 100 MHz ticks (s_memrealtime) over it;
 * so the caller derives the FLOP rate from its own timing of the launch
 * and the clock the waves ran at from the tick ratio.
 *   operands   device, operand_bytes >= 16 MiB of bf16 values (uint16 bits,
 *              16-byte aligned): the operand data to probe, e.g. N(0, 1)
 *              draws or a constant
 *   sink       device, workgroups * 256 floats
 *   clocks     device, workgroups * 4 * 2 uint64 (8-byte aligned)
 * Returns UPIPE_OK, UPIPE_EINVAL (a NULL or misaligned pointer,
 * operand_bytes < 16 MiB, iters < 1, workgroups < 1 or above 2^22) or
 * UPIPE_EHIP.  Never allocates, never synchronizes.
 */
#ifndef UPIPE_PROBE_H
#define UPIPE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "upipe_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

int upipe_probe_mfma(const uint16_t* operands, size_t operand_bytes, int32_t iters,
                     int32_t workgroups, float* sink, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_PROBE_H */
