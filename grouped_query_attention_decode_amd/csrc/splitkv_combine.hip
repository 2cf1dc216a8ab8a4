// Split-KV log-sum-exp combine.
//
// A long cache is cut into S key ranges that separate workgroups process at once, and
// their partial results are then reduced ["GQA revolution: how xformers speeds up LLM
// inference", section on split-KV block computation; the page names the split and the
// reduction but gives no formula]. Each range s left, per query head, the running
// maximum m_s of its base-2 scores, the running sum l_s = sum_j 2^(s_j - m_s) and the
// unnormalised accumulator acc_s = sum_j 2^(s_j - m_s) v_j. With M = max_s m_s and
// w_s = 2^(m_s - M):
//     out = (sum_s w_s acc_s) / (sum_s w_s l_s),
// which is exactly the softmax-weighted sum over all keys. A range with no keys has
// m_s = -inf, l_s = 0, acc_s = 0 and gets weight 0; a row with no keys at all is 0.
#include "dtypes.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplits = 1024;

template <typename QT>
__global__ __launch_bounds__(kThreads) void splitkv_combine_kernel(const float *__restrict__ part_acc,
                                                                   const float *__restrict__ part_ml,
                                                                   QT *__restrict__ out, int S, int D) {
    __shared__ float w_s[kMaxSplits];
    __shared__ float red[kThreads / 64];
    __shared__ float M_s, den_s;
    const int tid = threadIdx.x;
    const long bh = blockIdx.x;
    const float *ml = part_ml + bh * S * 2;

    // M = max_s m_s (block reduction).
    float mx = -INFINITY;
    for (int s = tid; s < S; s += kThreads) mx = fmaxf(mx, ml[2 * s]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        float m = red[0];
        for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, red[i]);
        M_s = m;
    }
    __syncthreads();
    const float M = M_s;

    float den = 0.f;
    for (int s = tid; s < S; s += kThreads) {
        const float m = ml[2 * s];
        const float w = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
        w_s[s] = w;
        den += w * ml[2 * s + 1];
    }
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = den;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
        for (int i = 0; i < kThreads / 64; ++i) t += red[i];
        den_s = t;
    }
    __syncthreads();
    const float dsum = den_s;

    const float *acc = part_acc + bh * S * D;
    for (int d = tid; d < D; d += kThreads) {
        float num = 0.f;
        for (int s = 0; s < S; ++s) {
            const float w = w_s[s];
            if (w != 0.f) num += w * acc[(long)s * D + d];
        }
        store_f32(out, bh * D + d, dsum > 0.f ? num / dsum : 0.f);
    }
}

}  // namespace

hipError_t launch_combine(const AttnArgs &a, hipStream_t stream) {
    if (a.num_splits > kMaxSplits) return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.B * a.H));
    dim3 block(kThreads);
    if (a.q_dtype == DT_F32)
        hipLaunchKernelGGL(splitkv_combine_kernel<float>, grid, block, 0, stream, a.part_acc, a.part_ml,
                           static_cast<float *>(a.out), a.num_splits, a.D);
    else
        hipLaunchKernelGGL(splitkv_combine_kernel<uint16_t>, grid, block, 0, stream, a.part_acc, a.part_ml,
                           static_cast<uint16_t *>(a.out), a.num_splits, a.D);
    return hipGetLastError();
}

}  // namespace gqa
