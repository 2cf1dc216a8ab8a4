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
    return __builtin_amdgcn_readfirstlane(last_s) != 0;
}

// Largest R * n_active a fused merge handles (the host checks R * S against it).
constexpr int kMergeMaxPairs = 128;
// Ranges whose accumulator loads one thread keeps in flight together.
constexpr int kMergeBatch = 32;

// out[h][d] = sum_s w[h][s] * acc_s[h][d] for the R heads of one group; each thread keeps
// NB ranges' loads in flight at once.
template <int NB>
__device__ __forceinline__ void splitkv_merge_rows(const AttnArgs &a, long head0, int R, int n, const float *w_s,
                                                   uint16_t *out) {
    const int S = a.num_splits, D = a.D;
    for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
        const int h = e / D, d = e - (e / D) * D;
        const float *acc = a.part_acc + (head0 + h) * S * D + d;
        float num = 0.f;
        for (int s0 = 0; s0 < n; s0 += NB) {
            float x[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int s = s0 + j < n ? s0 + j : n - 1;  // past the end: a valid, unused range
                x[j] = splitkv_load(acc + (long)s * D);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float w = s0 + j < n ? w_s[h * n + s0 + j] : 0.f;
                num += w != 0.f ? w * x[j] : 0.f;
            }
        }
        out[(head0 + h) * D + d] = f32_to_bf16(num);
    }
}

// Merge the n_active partials of query heads head0 .. head0+R-1 into out (bf16), using the
// whole workgroup. part layout: acc [B*H][S][D], ml [B*H][S][2]. Every load of another
// workgroup's partials is a device-coherent load and each costs a trip to memory, so they
// are issued in batches: all (m, l) pairs at once, then up to 32 ranges per output element.
__device__ __forceinline__ void splitkv_merge_bf16(const AttnArgs &a, long head0, int R, int n_active,
                                                   uint16_t *out) {
    __shared__ float m_s[kMergeMaxPairs], w_s[kMergeMaxPairs];
    const int S = a.num_splits, n = n_active;
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
    if (n <= 2)
        splitkv_merge_rows<2>(a, head0, R, n, w_s, out);
    else if (n <= 8)
        splitkv_merge_rows<8>(a, head0, R, n, w_s, out);
    else if (n <= 16)
        splitkv_merge_rows<16>(a, head0, R, n, w_s, out);
    else
        splitkv_merge_rows<kMergeBatch>(a, head0, R, n, w_s, out);
}

// ---- Flat layout of a ragged batch ----
// The valid rows of every (sequence b, KV head g) segment are laid end to end, KV head
// outermost: segment (b, g) starts at g * Ng + P_b, with T_b the clamped length of sequence
// b, Ng = sum_b T_b and P_b = sum_{b' < b} T_b'. Workgroup w takes rows [w C, (w + 1) C) of
// this sequence, so every workgroup streams the same number of rows whatever the lengths.
// The part of a segment that one workgroup covers is a "piece"; the pieces of segment (b, g)
// belong to workgroups first .. last = (start) / C .. (start + T_b - 1) / C and leave their
// partials in slots 0 .. last - first. The host uses this layout only when B * G * T_cap
// < 2^31, so every row index fits in 32 bits.

__device__ __forceinline__ int clamp_len(int L, int Tk) { return L < 0 ? 0 : (L > Tk ? Tk : L); }

// Rows per workgroup: the N rows spread over nw workgroups, at least cmin, a multiple of 32.
__device__ __forceinline__ int flat_chunk(int N, int nw, int cmin) {
    int c = (int)(((unsigned)N + nw - 1) / (unsigned)nw);
    if (c < cmin) c = cmin;
    return (c + 31) & ~31;
}

// Wave-wide sum of one value per lane.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Wave-wide inclusive prefix sum of one value per lane.
__device__ __forceinline__ int wave_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// Whole wave: Ng = sum_b T_b.
__device__ __forceinline__ int flat_total(const int32_t *seq_lens, int B, int Tk, int lane) {
    int tot = 0;
    for (int k0 = 0; k0 < B; k0 += 64) {
        const int b = k0 + lane;
        tot += wave_sum(b < B ? clamp_len(seq_lens[b], Tk) : 0);
    }
    return tot;
}

// Whole wave: the sequence b holding row `local` (0 <= local < Ng) of a KV head's run of
// segments, and its start P_b.
__device__ __forceinline__ void flat_find(const int32_t *seq_lens, int B, int Tk, int local, int lane, int &b_out,
                                          int &p_out) {
    int run = 0;
    b_out = B - 1;
    p_out = 0;
    for (int k0 = 0; k0 < B; k0 += 64) {
        const int b = k0 + lane;
        const int t = b < B ? clamp_len(seq_lens[b], Tk) : 0;
        const int incl = wave_scan(t, lane) + run;
        const int excl = incl - t;
        const unsigned long long hit = __ballot(b < B && excl <= local && local < incl);
        if (hit) {
            const int j = __ffsll((long long)hit) - 1;
            b_out = k0 + j;
            p_out = __shfl(excl, j);
            return;
        }
        run = __shfl(incl, 63);
    }
}

// Number of pieces (partial slots) of segment (b, g): 0 for an empty sequence.
__device__ __forceinline__ int flat_pieces(int Ng, int C, int Pb, int Tb, int g) {
    if (Tb <= 0) return 0;
    const unsigned s0 = (unsigned)(g * Ng + Pb);
    return (int)((s0 + Tb - 1) / (unsigned)C - s0 / (unsigned)C + 1);
}

}  // namespace gqa
