// Split-KV partial results and their in-kernel log-sum-exp merge (decode kernels).
//
// A long cache is cut into key ranges that separate workgroups process at once; their
// partial results are then reduced ["GQA revolution: how xformers speeds up LLM
// inference", section on split-KV block computation; the page gives no formula]. Range s
// leaves, per query head, the running maximum m_s of its base-2 scores, l_s = sum_j
// 2^(s_j - m_s) and acc_s = sum_j 2^(s_j - m_s) v_j. With M = max_s m_s and
// w_s = 2^(m_s - M), out = (sum_s w_s acc_s) / (sum_s w_s l_s).
//
// When the partials of one (sequence, KV head) are small, the workgroup that finishes that
// group's last range merges them itself instead of a second kernel. gfx950 gives every XCD
// its own L2, and a device-scope release/acquire fence writes back and invalidates that whole
// cache, which costs more than the merge saves. So the partials bypass the fences instead:
// they are written and read with device-scope atomic stores and loads, which the hardware
// keeps coherent across the L2s. Only the order of the operations remains to be enforced:
// every thread waits until its own partial stores have completed, the workgroup synchronises,
// and one thread increments the group's arrival counter; the one that sees count = ranges - 1
// merges in a fixed order (deterministic) and resets the counter to 0 for the next call. Its
// loads issue only after the counter's value has returned. The counters live in the caller's
// workspace, which must be zero when first used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dtypes.h"
#include "gqa_internal.h"
#include "mfma_util.h"

namespace gqa {

// Number of key ranges of sequence b that hold at least one key.
__device__ __forceinline__ int active_splits(int L, int split_len, int S) {
    const int n = (L + split_len - 1) / split_len;
    return n < S ? n : S;
}

// Store one partial value: device-coherent when another workgroup of the same launch will
// merge it, a plain store when the combine kernel reads it after this launch.
__device__ __forceinline__ void splitkv_store(float *p, float v, int coherent) {
    if (coherent)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

__device__ __forceinline__ void splitkv_store4(float *p, f32x4_t v, int coherent) {
    if (coherent) {
#pragma unroll
        for (int i = 0; i < 4; ++i) __hip_atomic_store(p + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        *(f32x4_t *)p = v;
    }
}

__device__ __forceinline__ float splitkv_load(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All threads call this after writing their partials with splitkv_store(.., 1). Returns, in
// every thread of the workgroup, whether this workgroup arrived last for its group.
__device__ __forceinline__ bool splitkv_arrive(int *counter, int n_active) {
    __shared__ int last_s;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == n_active - 1;
        // Every other range has arrived: reset for the next call.
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = last;
    }
    __syncthreads();
    return last_s != 0;
}

// Largest R * n_active a fused merge handles; the host fuses only when
// S * R * (D + 2) * 4 bytes <= 64 KiB, so R * S <= 126 for D = 128.
constexpr int kMergeMaxPairs = 128;

// Merge the n_active partials of query heads head0 .. head0+R-1 into out (bf16), using the
// whole workgroup. part layout: acc [B*H][S][D], ml [B*H][S][2]. Every load of another
// workgroup's partials is a device-coherent load and each costs a trip to memory, so they
// are issued in batches: all (m, l) pairs at once, then eight ranges per output element.
__device__ __forceinline__ void splitkv_merge_bf16(const AttnArgs &a, long head0, int R, int n_active,
                                                   uint16_t *out) {
    __shared__ float m_s[kMergeMaxPairs], w_s[kMergeMaxPairs];
    const int S = a.num_splits, D = a.D, n = n_active;
    for (int t = threadIdx.x; t < R * n; t += blockDim.x) {
        const int h = t / n, s = t - h * n;
        const float *ml = a.part_ml + ((head0 + h) * S + s) * 2;
        m_s[t] = splitkv_load(ml);
        w_s[t] = splitkv_load(ml + 1);
    }
    __syncthreads();
    // Per head: M = max_s m_s, den = sum_s 2^(m_s - M) l_s; w_s becomes 2^(m_s - M) / den.
    for (int h = threadIdx.x; h < R; h += blockDim.x) {
        float M = -INFINITY;
        for (int s = 0; s < n; ++s) M = fmaxf(M, m_s[h * n + s]);
        float den = 0.f;
        for (int s = 0; s < n; ++s) {
            const float m = m_s[h * n + s];
            const float w = m == -INFINITY ? 0.f : exp2f(m - M);
            den += w * w_s[h * n + s];
            m_s[h * n + s] = w;
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        for (int s = 0; s < n; ++s) w_s[h * n + s] = m_s[h * n + s] * inv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
        const int h = e / D, d = e - (e / D) * D;
        const float *acc = a.part_acc + (head0 + h) * S * D + d;
        float num = 0.f;
        for (int s0 = 0; s0 < n; s0 += 8) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = s0 + j < n ? s0 + j : n - 1;  // past the end: a valid, unused range
                x[j] = splitkv_load(acc + (long)s * D);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float w = s0 + j < n ? w_s[h * n + s0 + j] : 0.f;
                num += w != 0.f ? w * x[j] : 0.f;
            }
        }
        out[(head0 + h) * D + d] = f32_to_bf16(num);
    }
}

}  // namespace gqa
