/*
 * Achievable-peak probes (gfx950), built as libcwprobes.so beside the weight-gradient
 * library and used only to measure the chip (not part of its C ABI).
 *
 * The weight-gradient kernels are priced against the chip's nominal HBM
 * bandwidth (8 TB/s) and dense MFMA rates (f32 157.3 TFLOP/s, bf16 / fp16
 * 2516.6 TFLOP/s).  These two entry points measure what the chip sustains on
 * the same two resources with the simplest kernels that use them, so that a
 * kernel's fraction of the nominal peak can be read beside the fraction a
 * plain kernel reaches.  They compute nothing of the gradient.
 *
 * Both enqueue one kernel on `stream` (a hipStream_t; NULL = the null stream)
 * and return without synchronising.  begin / end, when not NULL, are
 * hipEvent_t created by the caller; the launch records them at the kernel's
 * own start and end (hipExtLaunchKernel), so hipEventElapsedTime(begin, end)
 * is the kernel's duration.  Status codes are those of conv_wgrad.h.
 */
#ifndef CWPROBES_H_
#define CWPROBES_H_

#include <stdint.h>

#include "../../include/conv_wgrad.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read: `blocks` workgroups of 256 lanes read the nbytes of src
 * once with 16-byte loads in a grid-stride order (consecutive lanes read
 * consecutive 16-byte words; four loads in flight per lane), and fold them
 * into a per-lane value that decides a store to sink, so no load can be
 * dropped.  Bytes moved per call: nbytes.
 *   src    : device pointer, 16-byte aligned (MISALIGNED otherwise), read only
 *   nbytes : > 0 and a multiple of 16 (BAD_SHAPE otherwise)
 *   blocks : 1 .. 65536 (BAD_SHAPE otherwise)
 *   sink   : device pointer to `blocks` uint32 words; its content is
 *            meaningless (stored to only for one specific folded value)
 * NULL src or sink is NULL_ARG; a launch failure is ERR_HIP.
 */
conv_wgrad_status_t cwprobe_read(const void* src, int64_t nbytes, int32_t blocks,
                                         uint32_t* sink, void* stream, void* begin, void* end);

/*
 * MFMA loop: `blocks` workgroups of four waves; every wave issues iters
 * rounds of independent accumulation chains of one MFMA instruction on
 * register operands (no memory traffic in the loop), then each lane stores the
 * sum of its accumulators to sink.  One round per wave:
 *   dtype  : CONV_WGRAD_F32 -> 8 x v_mfma_f32_16x16x4_f32 (2048 FLOP each,
 *            16384 per round),
 *            CONV_WGRAD_BF16 -> 4 x v_mfma_f32_32x32x16_bf16,
 *            CONV_WGRAD_F16 -> 4 x v_mfma_f32_32x32x16_f16 (32768 FLOP each,
 *            131072 per round);
 *            anything else is BAD_DTYPE
 *   iters  : 1 .. 2^31 - 1 (BAD_SHAPE otherwise)
 *   blocks : 1 .. 65536 (BAD_SHAPE otherwise)
 *   sink   : device pointer to blocks * 256 floats, overwritten
 * FLOPs per call: blocks * 4 * iters * (16384 for f32, 131072 for bf16 / f16).
 * NULL sink is NULL_ARG; a launch failure is ERR_HIP.
 */
conv_wgrad_status_t cwprobe_mfma(int32_t dtype, int64_t iters, int32_t blocks, float* sink,
                                         void* stream, void* begin, void* end);

/* cwprobe_mfma16: as cwprobe_mfma for bf16, with 8 independent chains of
 * v_mfma_f32_16x16x32_bf16 (16384 FLOP each, 131072 per round and wave), the
 * form the 16-bit weight-gradient kernels issue.  FLOPs per call:
 * blocks * 4 * iters * 131072.  Same argument checks and errors. */
conv_wgrad_status_t cwprobe_mfma16(int64_t iters, int32_t blocks, float* sink, void* stream, void* begin,
                                   void* end);

/* cwprobe_lds: LDS read rate.  `blocks` workgroups of 256 lanes, each with a
 * 32 KB LDS array, run `iters` rounds of 8 reads per lane at the addressing
 * of the 16-bit kernels' operand reads (16 pixel rows of 64 channels at a
 * 160-byte pitch per wave), every read folded into registers:
 *   mode 0: ds_read_b64_tr_b16 (8 bytes per lane), 1: ds_read_b64 (8 bytes),
 *   2: ds_read_b128 (16 bytes); anything else is BAD_SHAPE
 *   iters  : 1 .. 2^31 - 1, blocks: 1 .. 65536 (BAD_SHAPE otherwise)
 *   sink   : device pointer to blocks uint32 (written only if the folded
 *            value hits a fixed constant)
 * LDS bytes read per call: blocks * 256 * iters * 8 * (8, 8 or 16).  NULL
 * sink is NULL_ARG; a launch failure is ERR_HIP. */
conv_wgrad_status_t cwprobe_lds(int32_t mode, int64_t iters, int32_t blocks, uint32_t* sink, void* stream,
                                void* begin, void* end);

#ifdef __cplusplus
}
#endif

#endif /* CWPROBES_H_ */
