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
// which is exactly the softmax-weighted sum over all keys. Every range writes its
// partials, an empty one (m, l) = (-inf, 0), so the combine needs no sequence length: all
// its loads (the per-head (m, l) pairs are uniform across the workgroup and go through
// the scalar cache) leave in one round trip. A row with no keys at all is 0.
#include "dtypes.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kChunk = 32;  // ranges whose loads are in flight together

// One workgroup per (sequence, query head); thread d owns head dim d.
template <typename QT>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(const float *__restrict__ part_acc,
                                                              const float *__restrict__ part_ml,
                                                              QT *__restrict__ out, int S, int D) {
    const long bh = blockIdx.x;
    const int d = threadIdx.x < D ? threadIdx.x : D - 1;  // spare lanes load a valid dim
    const float *ml = part_ml + bh * S * 2;
    const float *acc = part_acc + bh * S * D + d;
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int s0 = 0; s0 < S; s0 += kChunk) {
        float m[kChunk], l[kChunk], x[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int s = s0 + j < S ? s0 + j : S - 1;
            m[j] = ml[2 * s];
            l[j] = ml[2 * s + 1];
            x[j] = acc[(long)s * D];
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) Mc = fmaxf(Mc, m[j]);  // the clamped repeats change nothing
        if (Mc == -INFINITY) continue;                          // no keys in any range so far
        const float alpha = M == -INFINITY ? 0.f : exp2f(M - Mc);
        num *= alpha;
        den *= alpha;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const float w = (s0 + j < S && m[j] != -INFINITY) ? exp2f(m[j] - Mc) : 0.f;
            num += w != 0.f ? w * x[j] : 0.f;  // never 0 * (unwritten value)
            den += w * l[j];
        }
        M = Mc;
    }
    if (threadIdx.x < D) store_f32(out, bh * D + d, den > 0.f ? num / den : 0.f);
}

}  // namespace

hipError_t launch_combine(const AttnArgs &a, hipStream_t stream) {
    if (a.D > 256) return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.B * a.H));
    dim3 block((unsigned)((a.D + 63) / 64 * 64));
    if (a.q_dtype == DT_F32)
        hipLaunchKernelGGL(splitkv_combine_kernel<float>, grid, block, 0, stream, a.part_acc, a.part_ml,
                           static_cast<float *>(a.out), a.num_splits, a.D);
    else
        hipLaunchKernelGGL(splitkv_combine_kernel<uint16_t>, grid, block, 0, stream, a.part_acc, a.part_ml,
                           static_cast<uint16_t *>(a.out), a.num_splits, a.D);
    return hipGetLastError();
}

}  // namespace gqa
