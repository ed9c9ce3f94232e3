/* Matrix-core microbenchmarks on gfx950 (libsfa_probe.so): the ceilings the
 * attention kernel's roofline report compares against.
 *
 * The attention of "HeyGen x Google Cloud: Bringing Avatar IV to TPUs" (sections
 * "Deleting the mask" and "Unchaining softmax") is a chain of bf16 matrix products
 * with an exp2 softmax between them. These kernels run the same instruction mix with
 * no HBM traffic, so their rates bound what the real kernel can reach:
 *
 *   SFA_PROBE_MFMA_CHAIN  independent chains of v_mfma_f32_32x32x16_bf16 on every SIMD,
 *                         no memory at all: the measured matrix-core peak;
 *   SFA_PROBE_TILE_LOOP   per 32-key tile of each wave's 32 query rows: 8 QK^T MFMAs with
 *                         the key operand read from LDS, the fixed-maximum softmax
 *                         (exp2, bf16 pack, row sum), 8 PV MFMAs with the V^T operand
 *                         read from LDS; no barriers, no DMA;
 *   SFA_PROBE_TILE_LOOP64 the same with 64 query rows per wave (every LDS operand feeds
 *                         two MFMAs);
 *   SFA_PROBE_TILE_NOEXP  the 32-row tile loop without the softmax (MFMA + LDS reads).
 *
 * Every call launches one workgroup per compute unit on the current device, on the
 * given hipStream_t (NULL: the null stream), and waits for it. Results:
 *   ms          kernel time from HIP events,
 *   tflops      32768 flops per MFMA issued / ms,
 *   clock_ghz   shader clock over the run: s_memtime cycles / s_memrealtime ticks,
 *               averaged over the workgroups,
 *   mfma_busy   MFMA cycles issued per SIMD / (ms * clock) (32 cycles per MFMA).
 * scratch: caller-owned device memory of at least sfa_probe_scratch_bytes() bytes
 * (per-thread sinks that keep the results live, and per-workgroup clock readings).
 * Returns 0, -1 for bad arguments (unknown kind, waves not 4 or 8, iters < 1, scratch
 * too small, null result), -3 on a HIP error. */
#ifndef SFA_PROBE_H
#define SFA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFA_PROBE_MFMA_CHAIN 0
#define SFA_PROBE_TILE_LOOP 1
#define SFA_PROBE_TILE_LOOP64 2
#define SFA_PROBE_TILE_NOEXP 3

typedef struct {
  double ms;
  double tflops;
  double clock_ghz;
  double mfma_busy;
} sfa_probe_result;

size_t sfa_probe_scratch_bytes(void);

int sfa_probe_run(int32_t kind, int32_t waves, int32_t iters, void* scratch,
                  size_t scratch_bytes, void* stream, sfa_probe_result* result);

#ifdef __cplusplus
}
#endif

#endif
