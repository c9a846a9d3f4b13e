/*
 * kvstore_calib.h -- C ABI of libkvstore_calib.so, a device calibration used
 * by the benchmark beside the attention library (it is not part of the
 * attention path and libkvstore.so does not export it).
 *
 * The benchmark reports each attention kernel's MFMA rate as a fraction of
 * the published bf16 peak and also of the rate this GPU actually sustains;
 * the second needs a loop of bf16 MFMAs with no memory traffic, timed by the
 * caller with events ("Transformer 추론 커널: GEMM·Attention·FlashAttention·
 * Fusion (3/10)", §25-§26: fix the manifest and the measurement method before
 * comparing against a roofline).
 */
#ifndef KVSTORE_CALIB_H
#define KVSTORE_CALIB_H

#include "kvstore.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * kvs_mfma_peak_launch -- the MFMA rate this GPU sustains, for the benchmark's
 * roofline fractions ("Transformer 추론 커널 (3/10)", §25-§26).  Enqueues
 * `workgroups` workgroups of 4 waves, each
 * wave running 4 independent chains of `iters` 32x32x16 bf16 MFMAs (32768 FLOP
 * each) with no memory traffic in the loop (FLOP = workgroups * 4 * 4 * iters
 * * 32768).  `src`: 512 readable bytes, 16-byte aligned, device memory
 * (operand data); `dst`: workgroups * 256 floats written, device memory.
 * KVS_ERR_INVALID on a bad argument (nothing enqueued), KVS_ERR_HIP if the
 * launch fails.  Asynchronous on `stream`; allocates nothing.
 */
kvs_status kvs_mfma_peak_launch(const void* src, void* dst, int workgroups, int iters, kvs_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSTORE_CALIB_H */
