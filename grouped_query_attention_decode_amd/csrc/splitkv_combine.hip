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
// which is exactly the softmax-weighted sum over all keys. Only the ranges that hold
// keys of this sequence (the first ceil(L_b / split_len)) are read; a row with no keys at
// all is 0.
#include "dtypes.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplits = 1024;

template <typename QT>
__global__ __launch_bounds__(kThreads) void splitkv_combine_kernel(const float *__restrict__ part_acc,
                                                                   const float *__restrict__ part_ml,
                                                                   const int32_t *__restrict__ seq_lens,
                                                                   QT *__restrict__ out, int H, int S, int D,
                                                                   int split_len, int Tk) {
    __shared__ float w_s[kMaxSplits];
    __shared__ float half_s[kThreads];
    __shared__ float M_s, den_s;
    const int tid = threadIdx.x;
    const long bh = blockIdx.x;
    const int b = (int)(bh / H);
    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > Tk ? Tk : L);
    int SA = (L + split_len - 1) / split_len;  // ranges that hold keys
    SA = SA < S ? SA : S;
    const float *ml = part_ml + bh * S * 2;

    if (tid < 64) {
        float mx = -INFINITY;
        for (int s = tid; s < SA; s += 64) mx = fmaxf(mx, ml[2 * s]);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float den = 0.f;
        for (int s = tid; s < SA; s += 64) {
            const float m = ml[2 * s];
            const float w = (mx == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - mx);
            w_s[s] = w;
            den += w * ml[2 * s + 1];
        }
        for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
        if (tid == 0) {
            M_s = mx;
            den_s = den;
        }
    }
    __syncthreads();
    const float dsum = den_s;

    // Two threads per head dim, each over every other range; independent loads, no branch.
    const float *acc = part_acc + bh * S * D;
    const int d = tid % (kThreads / 2);
    const int s0 = tid / (kThreads / 2);
    for (int dd = d; dd < D; dd += kThreads / 2) {
        float num = 0.f;
#pragma unroll 8
        for (int s = s0; s < SA; s += 2) {
            const float w = w_s[s];
            const float x = acc[(long)s * D + dd];
            num += w != 0.f ? w * x : 0.f;
        }
        half_s[tid] = num;
        __syncthreads();
        if (s0 == 0) {
            const float tot = num + half_s[tid + kThreads / 2];
            store_f32(out, bh * D + dd, dsum > 0.f ? tot / dsum : 0.f);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_combine(const AttnArgs &a, hipStream_t stream) {
    if (a.num_splits > kMaxSplits) return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.B * a.H));
    dim3 block(kThreads);
    if (a.q_dtype == DT_F32)
        hipLaunchKernelGGL(splitkv_combine_kernel<float>, grid, block, 0, stream, a.part_acc, a.part_ml, a.seq_lens,
                           static_cast<float *>(a.out), a.H, a.num_splits, a.D, a.split_len, a.Tk);
    else
        hipLaunchKernelGGL(splitkv_combine_kernel<uint16_t>, grid, block, 0, stream, a.part_acc, a.part_ml,
                           a.seq_lens, static_cast<uint16_t *>(a.out), a.H, a.num_splits, a.D, a.split_len, a.Tk);
    return hipGetLastError();
}

}  // namespace gqa
