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
// they are written and read with the cache policy of device-scope atomic stores and loads
// (sc1; 16-byte buffer accesses for the accumulators), which the hardware keeps coherent
// across the L2s. Only the order of the operations remains to be enforced:
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

__device__ __forceinline__ float splitkv_load(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (m, l) of one range and query head as one 8-byte device-coherent store / load.
__device__ __forceinline__ void splitkv_store_ml(float *p, float m, float l, int coherent) {
    const unsigned long long bits = (unsigned long long)__float_as_uint(m) | ((unsigned long long)__float_as_uint(l) << 32);
    if (coherent)
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *reinterpret_cast<unsigned long long *>(p) = bits;
}

__device__ __forceinline__ f32x2_t splitkv_load_ml(const float *p) {
    const unsigned long long bits =
        __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2_t{__uint_as_float((uint32_t)bits), __uint_as_float((uint32_t)(bits >> 32))};
}

// Buffer resource over the partial accumulators [R][S][D] of query heads head0 .. head0+R-1
// (workgroup-uniform), for 16-byte device-coherent accesses: buffer loads and stores with the
// cache-policy bit (sc1) that agent-scope atomic loads and stores carry. Offsets past the
// resource's size read zero and write nothing instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t splitkv_acc_rsrc(const AttnArgs &a, long head0, int R) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(a.part_acc + head0 * a.num_splits * a.D), (short)0,
                                             R * a.num_splits * a.D * 4, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void splitkv_store4c(__amdgpu_buffer_rsrc_t r, unsigned byte_off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, /*sc1*/ 16);
}

__device__ __forceinline__ f32x4_t splitkv_load4(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, /*sc1*/ 16));
}

// All threads call this after writing their partials with splitkv_store(.., 1). Returns, in
// every thread of the workgroup, whether this workgroup arrived last for its group. `then` runs
// in every thread once the partial stores have completed, after the counter increment has been
// issued and before its result is awaited: loads it issues (the next piece's first block) are
// in flight during that round trip instead of after it.
template <typename Then>
__device__ __forceinline__ bool splitkv_arrive(int *counter, int n_active, Then then) {
    __shared__ int last_s;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    int old = 0;
    if (threadIdx.x == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    then();
    if (threadIdx.x == 0) {
        const int last = old == n_active - 1;
        // Every other range has arrived: reset for the next call.
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = last;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(last_s) != 0;
}

__device__ __forceinline__ bool splitkv_arrive(int *counter, int n_active) {
    return splitkv_arrive(counter, n_active, [] {});
}

// Largest R * n_active a fused merge handles (the host checks R * S against it).
constexpr int kMergeMaxPairs = 128;

// Merge the n partials of query heads head0 .. head0+R-1 into out (bf16), using the whole
// workgroup of NT threads. part layout: acc [B*H][S][D], ml [B*H][S][2]. Every load
// of another workgroup's partials travels to memory, and one compute unit completes only so
// many of them at a time, so the accumulators are read 16 bytes per load and all loads are
// issued before any is used: each (m, l) pair and up to NB ranges per thread at once, the
// weights formed while the accumulators are in flight. A work item is 4 head dims of one
// head; P = 1, 2 or 4 consecutive lanes share an item and take its ranges in turn, then add
// their sums with lane shuffles. Ranges past n are not loaded into the sums (weight 0).
template <int NT, int D, int NB>
__device__ __forceinline__ void splitkv_merge_t(const AttnArgs &a, long head0, int R, int n, uint16_t *out) {
    static_assert(D % 4 == 0, "16-byte accumulator loads");
    __shared__ float m_s[kMergeMaxPairs], l_s[kMergeMaxPairs], w_s[kMergeMaxPairs];
    constexpr int nt = NT;
    const int S = a.num_splits, t = threadIdx.x;
    const int I = R * (D / 4);                                 // work items
    const int P = 4 * I <= nt ? 4 : (2 * I <= nt ? 2 : 1);     // lanes per item
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)(a.part_acc + head0 * S * D), (short)0,
                                                                          R * S * D * 4, 0x00020000);
    f32x2_t ml0 = {0.f, 0.f};
    if (t < R * n) {
        const int h = t / n, s = t - h * n;
        ml0 = splitkv_load_ml(a.part_ml + ((head0 + h) * S + s) * 2);
    }
    const int p = t % P;
    for (int i0 = 0; i0 < I; i0 += nt / P) {
        const int item = min(i0 + t / P, I - 1);
        const int h = item / (D / 4), d = 4 * (item - h * (D / 4));
        f32x4_t num = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < n; s0 += NB * P) {
            f32x4_t x[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int sr = min(s0 + j * P + p, n - 1);
                x[j] = splitkv_load4(rsrc, (unsigned)(((h * S + sr) * D + d) * 4));
            }
            if (i0 == 0 && s0 == 0) {
                // Weight of pair t = (head h, range s): with M = max_s m_s and
                // den = sum_s 2^(m_s - M) l_s of its head, w = 2^(m - M) / den. One thread per
                // pair; every thread of a head forms M and den in the same order.
                if (t < R * n) {
                    m_s[t] = ml0[0];
                    l_s[t] = ml0[1];
                }
                __syncthreads();
                if (t < R * n) {
                    // Unrolled so that the LDS reads go out eight at a time rather than one
                    // round trip per range.
                    const int hb = (t / n) * n;
                    float M = -INFINITY;
#pragma unroll 8
                    for (int s = 0; s < n; ++s) M = fmaxf(M, m_s[hb + s]);
                    float den = 0.f;
#pragma unroll 8
                    for (int s = 0; s < n; ++s) {
                        const float m = m_s[hb + s], e = exp2f(m - M) * l_s[hb + s];
                        den += m == -INFINITY ? 0.f : e;
                    }
                    w_s[t] = ml0[0] == -INFINITY || !(den > 0.f) ? 0.f : exp2f(ml0[0] - M) / den;
                }
                __syncthreads();
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int sr = s0 + j * P + p;
                const float w = sr < n ? w_s[h * n + sr] : 0.f;
                if (w != 0.f) {
                    num[0] += w * x[j][0];
                    num[1] += w * x[j][1];
                    num[2] += w * x[j][2];
                    num[3] += w * x[j][3];
                }
            }
        }
        for (int o = 1; o < P; o <<= 1)
#pragma unroll
            for (int c = 0; c < 4; ++c) num[c] += __shfl_xor(num[c], o);
        if (p == 0 && i0 + t / P < I) {
            uint16_t *dst = out + (head0 + h) * D + d;
            *(i32x2_t *)dst = i32x2_t{(int)((uint32_t)f32_to_bf16(num[0]) | ((uint32_t)f32_to_bf16(num[1]) << 16)),
                                      (int)((uint32_t)f32_to_bf16(num[2]) | ((uint32_t)f32_to_bf16(num[3]) << 16))};
        }
    }
}

// Merge for a workgroup of NT threads and head dim D (compile-time: no division by D and no
// read of the launch's block size on the critical path).
template <int NT, int D>
__device__ __forceinline__ void splitkv_merge_bf16(const AttnArgs &a, long head0, int R, int n_active,
                                                   uint16_t *out) {
    splitkv_merge_t<NT, D, 8>(a, head0, R, n_active, out);
}

// ---- Flat layout of a ragged batch ----
// The valid rows of every (sequence b, KV head g) segment are laid end to end, KV head
// outermost, each non-empty segment preceded by `pad` rows of no work: segment (b, g) spans
// X_b = T_b + pad rows (0 when T_b = 0) from g * Ng + P_b, its valid rows from g * Ng + P_b +
// pad, with T_b the clamped length of sequence b, Ng = sum_b X_b and P_b = sum_{b' < b} X_b'.
// Workgroup w takes rows [w C, (w + 1) C) of this sequence. The part of a segment's valid rows
// that one workgroup covers is a "piece"; each piece has a fixed cost (its first round trip,
// the merge of its waves, its partials and arrival), which the pad rows stand for: a
// workgroup whose run is cut into several pieces gets correspondingly fewer valid rows, so
// every workgroup has about the same work whatever the lengths. The pieces of segment (b, g)
// belong to workgroups first .. last = r0 / C .. (r0 + T_b - 1) / C, r0 being its first valid
// row, and leave their partials in slots 0 .. last - first. The host uses this layout only when
// B * G * (T_cap + pad) < 2^31, so every row index fits in 32 bits.

__device__ __forceinline__ int clamp_len(int L, int Tk) { return L < 0 ? 0 : (L > Tk ? Tk : L); }

// Rows that a sequence of T valid rows occupies in each KV head's run.
__device__ __forceinline__ int flat_span(int T, int pad) { return T > 0 ? T + pad : 0; }

// Rows per workgroup: the N rows spread over nw workgroups, at least cmin, a multiple of 32.
__device__ __forceinline__ int flat_chunk(int N, int nw, int cmin) {
    int c = (int)(((unsigned)N + nw - 1) / (unsigned)nw);
    if (c < cmin) c = cmin;
    return (c + 31) & ~31;
}

// Wave-wide sum of one value per lane: rows of 16 by two rotations and two quad permutes,
// then the four rows by two lane swaps.
__device__ __forceinline__ int wave_sum(int x) {
    x += dpp_move<0x128>(x);
    x += dpp_move<0x124>(x);
    x += dpp_move<0x4E>(x);
    x += dpp_move<0xB1>(x);
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(p[0] + p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)(q[0] + q[1]);
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

// Whole wave: the sequence b holding row `local` (0 <= local < Ng) of a KV head's run of
// segments, and its start P_b. len(b) gives the clamped length of sequence b.
template <typename Len>
__device__ __forceinline__ void flat_find(Len len, int B, int pad, int local, int lane, int &b_out, int &p_out) {
    int run = 0;
    b_out = B - 1;
    p_out = 0;
    for (int k0 = 0; k0 < B; k0 += 64) {
        const int b = k0 + lane;
        const int t = b < B ? flat_span(len(b), pad) : 0;
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
__device__ __forceinline__ int flat_pieces(int Ng, int C, int Pb, int Tb, int g, int pad) {
    if (Tb <= 0) return 0;
    const unsigned r0 = (unsigned)(g * Ng + Pb + pad);  // its first valid row
    return (int)((r0 + Tb - 1) / (unsigned)C - r0 / (unsigned)C + 1);
}

}  // namespace gqa
