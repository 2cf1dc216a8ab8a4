// Plain streaming read of a device buffer: the measured "achievable" HBM read rate that the
// decode kernels are compared with (decode is bound by reading the KV cache from memory [GQA
// paper digest page (51969.com), section "QA"]), and the pass that evicts the 256 MB Infinity
// Cache before a timed run reads cold data.
//
// One workgroup per compute unit; every thread keeps eight 16-byte nontemporal loads in flight
// (grid-stride: a wave reads 1 KB runs, every cache line once). Measured on gfx950 over 2 GiB:
// this form 7.1 TB/s; ordinary loads 5.0-6.3 TB/s whatever the workgroup count, loads in
// flight or order (grid-stride or a contiguous chunk per workgroup). The XOR of everything read
// decides a single store that practically never happens, so the loads cannot be dropped and
// nothing else touches memory.
#include "gqa_internal.h"
#include "gqa_measure.h"
#include "mfma_util.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const i32x4_t *__restrict__ p, long n16, int *sink) {
    const long stride = (long)gridDim.x * kThreads;
    long i = (long)blockIdx.x * kThreads + threadIdx.x;
    int acc = 0;
    for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
        i32x4_t x[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) x[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) acc ^= x[j][0] ^ x[j][1] ^ x[j][2] ^ x[j][3];
    }
    for (; i < n16; i += stride) {
        const i32x4_t x = __builtin_nontemporal_load(p + i);
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    if (acc == 0x5EEDF00D) sink[blockIdx.x & 1023] = acc;
}

}  // namespace
}  // namespace gqa

extern "C" gqa_status gqa_hbm_stream_read(const void *buf, size_t bytes, int *sink, hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0) return GQA_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return GQA_ERR_HIP;
    const long n16 = (long)(bytes / 16);
    long blocks = cus > 0 ? cus : 256;  // one workgroup per compute unit
    const long need = (n16 + gqa::kThreads - 1) / gqa::kThreads;
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(gqa::stream_read_kernel, dim3((unsigned)blocks), dim3(gqa::kThreads), 0, stream,
                       static_cast<const gqa::i32x4_t *>(buf), n16, sink);
    return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}
