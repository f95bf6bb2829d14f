/* Machine-ceiling probes of the OAL library (liboal.so) for gfx950.
 *
 * These two calls are not part of the attention method.  They measure the
 * two limits against which the attention kernels are judged on the machine
 * at hand: the HBM bandwidth of a kernel that reads and writes every byte
 * once, and the throughput of the bf16 MFMA instruction that the prefill
 * kernels issue.  Both are asynchronous launches on `stream` (a hipStream_t,
 * or NULL for the null stream); the caller times them.
 */
#ifndef OAL_CEILINGS_H
#define OAL_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In-place streaming update buf[i] <- 0.999 buf[i] + 0.001 over n_floats
 * fp32 values in DEVICE memory: n_floats * 4 bytes read and as many
 * written.  buf must be 16-byte aligned and n_floats a positive multiple of
 * 4 (OAL_ERR_INVALID_ARG otherwise).  The contents are overwritten. */
int oal_ceiling_stream_rw(float* buf, size_t n_floats, void* stream);

/* n_workgroups workgroups of four waves each run `iters` rounds of eight
 * independent v_mfma_f32_16x16x32_bf16 on register operands, then each
 * thread writes one float to out (DEVICE, n_workgroups * 256 floats).
 * Returns OAL_OK, OAL_ERR_INVALID_ARG (null out, n_workgroups not positive,
 * iters not a positive multiple of 16) or OAL_ERR_HIP. */
int oal_ceiling_mfma(float* out, int n_workgroups, int iters, void* stream);

/* Floating-point operations of one oal_ceiling_mfma launch (2 m n k per
 * MFMA). */
double oal_ceiling_mfma_flops(int n_workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* OAL_CEILINGS_H */
