/*
 * gqa_measure.h -- measurement aid exported by libgqa.so beside the attention calls of gqa.h.
 *
 * Decode is bound by reading the KV cache from memory [GQA paper digest page (51969.com),
 * section "QA"; "Hands-on: implementing GQA in PyTorch", section 2.1, bytes per decode step],
 * so its kernels are compared with the rate at which the device streams plain reads. This
 * call is that plain read; the benchmark also uses it to evict the 256 MB Infinity Cache
 * before a timed run.
 */
#ifndef GQA_MEASURE_H
#define GQA_MEASURE_H

#include <stddef.h>

#include "gqa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of device memory at `buf` once, in 16-byte loads spread over every
 * compute unit, and write nothing but (practically never) one int of `sink`.
 *
 *   buf    device pointer, 16-byte aligned, caller-owned, only read
 *   bytes  a positive multiple of 16
 *   sink   device int[1024], caller-owned; its contents are unspecified afterwards
 *
 * Enqueues one kernel on `stream` and returns. GQA_ERR_INVALID_ARG for a null pointer, a
 * misaligned buffer or a size that is zero or not a multiple of 16 (checked before any HIP
 * call); GQA_ERR_HIP when the launch fails.
 */
gqa_status gqa_hbm_stream_read(const void *buf, size_t bytes, int *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_MEASURE_H */
