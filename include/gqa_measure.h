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

/*
 * Per-workgroup timeline of the decode kernels (diagnostic build only). The library built with
 * GQA_TIMELINE (libgqa_timeline.so, from build.py --timeline) has thread 0 of every decode
 * workgroup w < 4096 record the device's constant 100 MHz clock at fixed points into slots
 * [w][0..31] of a device array (unsigned 64-bit): 0 entry; 1 sequence length(s) and work layout
 * known; for the workgroup's piece p < 3 (a key range of one sequence and KV head), slots
 * 2 + 6 p + 0 start, + 1 first block done, + 2 block loop done, + 3 waves merged and partials
 * issued, + 4 arrival counted (split ranges merged in the kernel), + 5 end; 20 exit; 21 the
 * number of pieces (a count); for the workgroup's last piece, 22 all four waves' block loops done
 * (the first barrier of the merge of the waves) and 23 the waves' partial sums written to LDS
 * (its second barrier); 31 where the workgroup ran (a value: the HW_ID register, which holds the
 * CU, shader-array and shader-engine numbers, in the low 32 bits, XCC_ID above). Slots a
 * workgroup never reaches keep their value.
 *
 * gqa_timeline_clear zeroes the array; gqa_timeline_read copies its first `bytes` bytes (at
 * most 4096 * 32 * 8) to host memory `dst`. Both are synchronous (they wait for the device's
 * prior work) and belong between decode calls, never during one. The library proper returns
 * GQA_ERR_UNSUPPORTED from both (and GQA_ERR_INVALID_ARG for a null dst); GQA_ERR_HIP when a
 * copy fails.
 */
gqa_status gqa_timeline_read(void *dst, size_t bytes);
gqa_status gqa_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_MEASURE_H */
