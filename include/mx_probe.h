/* mx_probe.h — measurement aid for the matrix-core roofline (libmx_probe.so). Not part of the
 * quantize/GEMM interface in mx.h.
 *
 * The GEMMs are priced against the dense MXFP4 peak of the matrix cores. That peak assumes the
 * top clock; with random operand bits the cores draw more power and the clock falls, so the
 * attainable rate is lower. This probe measures it: each 256-thread workgroup (one wave per
 * SIMD) issues `iters` rounds of 16 independent 32x32x64 block-scaled FP4 matrix instructions
 * per wave (the 4x4 accumulator tiles a GEMM wave owns), on random FP4 operands with E8M0 scales
 * of 1/2 or 1, with no memory traffic. The work is
 * workgroups * 4 waves * iters * 16 * 2 * 32 * 32 * 64 flops; time it with events on `stream`.
 *
 * sink: device buffer of workgroups * 256 floats (caller-owned), written once per lane so the
 * work is not dead code; its values carry no meaning.
 * Returns 0 on success, otherwise a HIP error code (invalid value for workgroups <= 0,
 * iters <= 0 or a NULL sink, checked before any launch). Asynchronous on `stream`
 * (hipStream_t passed as void*). */
#ifndef MX_PROBE_H
#define MX_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t mx_probe_mfma_fp4(int32_t workgroups, int32_t iters, uint32_t seed, float* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_PROBE_H */
