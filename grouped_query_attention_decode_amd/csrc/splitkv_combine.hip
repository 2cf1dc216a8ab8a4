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
#include "splitkv.h"

namespace gqa {

namespace {

constexpr int kChunk = 32;  // ranges whose loads are in flight together

// Flat layout (splitkv.h): the number of pieces of this row's (sequence, KV head) segment,
// from the sequence lengths, by the whole workgroup.
__device__ int flat_row_pieces(const AttnArgs &a, int b, int g) {
    __shared__ int red_s[2][4];
    int tot = 0, pre = 0;
    for (int bb = threadIdx.x; bb < a.B; bb += blockDim.x) {
        const int t = flat_span(clamp_len(a.seq_lens[bb], a.Tk), a.flat_pad);
        tot += t;
        if (bb < b) pre += t;
    }
    tot = wave_sum(tot);
    pre = wave_sum(pre);
    const int wave = threadIdx.x >> 6, nwave = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) {
        red_s[0][wave] = tot;
        red_s[1][wave] = pre;
    }
    __syncthreads();
    int Ng = 0, Pb = 0;
    for (int w = 0; w < nwave; ++w) {
        Ng += red_s[0][w];
        Pb += red_s[1][w];
    }
    Ng = __builtin_amdgcn_readfirstlane(Ng);
    Pb = __builtin_amdgcn_readfirstlane(Pb);
    const int C = flat_chunk(a.G * Ng, a.flat_nw, a.flat_cmin);
    return flat_pieces(Ng, C, Pb, clamp_len(a.seq_lens[b], a.Tk), g, a.flat_pad);
}

// One workgroup per (sequence, query head); thread d owns head dim d. Uniform layout: all
// S slots (an empty range left m = -inf); flat layout: the row's pieces, and nothing to do
// for a row that one piece covered (the decode kernel wrote it).
template <typename QT, bool FLAT>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(AttnArgs a) {
    const float *__restrict__ part_acc = a.part_acc;
    const float *__restrict__ part_ml = a.part_ml;
    QT *__restrict__ out = static_cast<QT *>(a.out);
    const int S = a.num_splits, D = a.D;
    const long bh = blockIdx.x;
    int n = S;
    if constexpr (FLAT) {
        const int b = (int)(bh / a.H), g = (int)(bh % a.H) / (a.H / a.G);
        n = flat_row_pieces(a, b, g);
        if (n == 1) return;
    }
    const int d = threadIdx.x < D ? threadIdx.x : D - 1;  // spare lanes load a valid dim
    const float *ml = part_ml + bh * S * 2;
    const float *acc = part_acc + bh * S * D + d;
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int s0 = 0; s0 < n; s0 += kChunk) {
        float m[kChunk], l[kChunk], x[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int s = s0 + j < n ? s0 + j : n - 1;
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
            const float w = (s0 + j < n && m[j] != -INFINITY) ? exp2f(m[j] - Mc) : 0.f;
            num += w != 0.f ? w * x[j] : 0.f;  // never 0 * (unwritten value)
            den += w * l[j];
        }
        M = Mc;
    }
    if (threadIdx.x < D) store_f32(out, bh * D + d, den > 0.f ? num / den : 0.f);
}

// Head dims a multiple of 4: D threads per (sequence, query head). The four lanes of a quad
// share head dims 4 (t / 4) .. +3 and take ranges s = t mod 4, +4, ..., eight per chunk of 32
// ranges, with one 16-byte accumulator load and one 8-byte (m, l) load per range -- all of a
// chunk's loads in flight at once; the quad then adds its sums with lane shuffles. Every quad
// sees the same ranges, so the running maximum is the same in every lane. The first chunk is
// requested before the flat layout's piece count is known (slots below S are allocated);
// ranges at or past the count get weight 0 and their values are never used.
template <typename QT, bool FLAT>
__global__ __launch_bounds__(256) void splitkv_combine4_kernel(AttnArgs a) {
    const int S = a.num_splits, D = a.D;
    const long bh = blockIdx.x;
    const int t = threadIdx.x, p = t & 3, d = 4 * (t >> 2);
    const float *ml = a.part_ml + bh * S * 2;
    const float *acc = a.part_acc + bh * S * D + d;
    f32x4_t x[8];
    f32x2_t mlv[8];
    auto load_chunk = [&](int s0, int lim) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = min(s0 + 4 * j + p, lim - 1);
            x[j] = *(const f32x4_t *)(acc + (long)s * D);
            mlv[j] = *(const f32x2_t *)(ml + 2 * s);
        }
    };
    load_chunk(0, S);
    int n = S;
    if constexpr (FLAT) {
        const int b = (int)(bh / a.H), g = (int)(bh % a.H) / (a.H / a.G);
        n = flat_row_pieces(a, b, g);
        if (n == 1) return;
    }
    float M = -INFINITY, den = 0.f;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n; s0 += 32) {
        if (s0 > 0) load_chunk(s0, n);
        float Mc = M;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + 4 * j + p < n) Mc = fmaxf(Mc, mlv[j][0]);
        Mc = fmaxf(Mc, __shfl_xor(Mc, 1));
        Mc = fmaxf(Mc, __shfl_xor(Mc, 2));
        if (Mc == -INFINITY) continue;  // no keys in any range so far
        const float alpha = M == -INFINITY ? 0.f : exp2f(M - Mc);
        den *= alpha;
#pragma unroll
        for (int c = 0; c < 4; ++c) num[c] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float m = mlv[j][0];
            const float w = (s0 + 4 * j + p < n && m != -INFINITY) ? exp2f(m - Mc) : 0.f;
            if (w != 0.f) {  // never 0 * (unwritten value)
                den += w * mlv[j][1];
#pragma unroll
                for (int c = 0; c < 4; ++c) num[c] += w * x[j][c];
            }
        }
        M = Mc;
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
        den += __shfl_xor(den, o);
#pragma unroll
        for (int c = 0; c < 4; ++c) num[c] += __shfl_xor(num[c], o);
    }
    if (p == 0) {
        const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) store_f32(static_cast<QT *>(a.out), bh * D + d + c, den > 0.f ? num[c] * inv : 0.f);
    }
}

// Zero-fill of n ints (the split arrival counters of fresh workspace memory). A kernel rather
// than hipMemsetAsync, so that the stream carries only kernel work.
__global__ __launch_bounds__(256) void zero_ints_kernel(int *p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_ints(int *p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs &a, hipStream_t stream) {
    if (a.D > 256) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.B * a.H));
    const bool f32 = a.q_dtype == DT_F32;
    if (a.D % 4 == 0) {
        const dim3 block((unsigned)a.D);
        if (f32) {
            if (a.flat) hipLaunchKernelGGL((splitkv_combine4_kernel<float, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((splitkv_combine4_kernel<float, false>), grid, block, 0, stream, a);
        } else {
            if (a.flat) hipLaunchKernelGGL((splitkv_combine4_kernel<uint16_t, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((splitkv_combine4_kernel<uint16_t, false>), grid, block, 0, stream, a);
        }
        return hipGetLastError();
    }
    const dim3 block((unsigned)((a.D + 63) / 64 * 64));
    if (f32) {
        if (a.flat) hipLaunchKernelGGL((splitkv_combine_kernel<float, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((splitkv_combine_kernel<float, false>), grid, block, 0, stream, a);
    } else {
        if (a.flat) hipLaunchKernelGGL((splitkv_combine_kernel<uint16_t, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((splitkv_combine_kernel<uint16_t, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gqa
