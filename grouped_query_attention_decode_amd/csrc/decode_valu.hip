// Narrow-group GQA decode on the vector ALUs (bf16 KV cache, D = 128, R = H/G <= 8).
//
// With few query heads per KV head (R = 4 for a GQA-8 model with 32 query heads) decode
// does only 4*R flops per cached bf16 element, which the vector ALUs sustain at HBM rate;
// matrix cores would mostly multiply padding. Each KV row is still read once per
// (sequence, KV head) and used for all R heads of the group [GQA paper digest page
// (51969.com), section "Grouped-query attention (GQA)"; group of head h is h / (H/G), "LLM
// principles -- code implementation of multi-head attention (MQA and GQA)", section 5].
//
// Work: one workgroup (4 waves) per (sequence b, KV head g, key range). A wave streams
// 32-row tiles of K and V with 16-byte loads: lane l reads 8 head dims (chunk l%16) of row
// 4*i + l/16 for i = 0..7, so one wave instruction covers four whole 256-byte rows. Each
// lane forms the partial dot products of its 8 dims with the R query rows; a butterfly
// over the 16 lanes of the row completes them. The online softmax state (running max,
// running sum, 8-dim accumulators per head) is kept per lane and updated once per tile
// (one rescale per 8 rows); the 16 lane groups x 4 waves states are merged at the end in a
// fixed order.
#include "dtypes.h"
#include "gqa_internal.h"
#include "mfma_util.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;  // rows per wave tile (8 per lane)
constexpr int kD = 128;

__device__ __forceinline__ void bf16x8_to_f32(const i32x4_t &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = (uint32_t)w[i];
        x[2 * i] = __uint_as_float(u << 16);
        x[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
}

template <int RP>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(AttnArgs a) {
    constexpr int NST = kWaves * 4;  // softmax states per workgroup (4 row groups per wave)
    __shared__ float st_m[NST][RP], st_l[NST][RP];
    __shared__ float M_s[RP], l_s[RP];
    __shared__ __attribute__((aligned(16))) float O_s[RP][kD];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;    // row group inside the wave
    const int chunk = lane & 15;  // 8 head dims: 8*chunk .. 8*chunk+7
    // Split-major block order (see decode_mfma.hip).
    const int S = a.num_splits;
    const int split = blockIdx.x / (a.B * a.G);
    const int bg = blockIdx.x % (a.B * a.G);
    const int G = a.G, H = a.H, R = H / G;
    const int b = bg / G, g = bg % G;
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.Tk ? a.Tk : L);
    const int kb = split * a.split_len;
    const int ke = kb + a.split_len < L ? kb + a.split_len : L;
    const long head0 = (long)b * H + (long)g * R;

    if (kb >= ke) {
        if (S == 1) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            for (int e = threadIdx.x; e < R * kD; e += kThreads) out[head0 * kD + e] = 0;
        } else {
            for (int h = threadIdx.x; h < R; h += kThreads) {
                a.part_ml[((head0 + h) * S + split) * 2] = -INFINITY;
                a.part_ml[((head0 + h) * S + split) * 2 + 1] = 0.f;
            }
        }
        return;
    }

    // This lane's 8 dims of every query row of the group, pre-scaled into the base-2 domain.
    float q[RP][8];
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + head0 * kD;
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        if (h < R) {
            const i32x4_t w = *(const i32x4_t *)(qp + (long)h * kD + 8 * chunk);
            bf16x8_to_f32(w, q[h]);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[h][e] *= a.scale_log2;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[h][e] = 0.f;
        }
    }

    const char *kbase = static_cast<const char *>(a.k) + (long)bg * a.Tk * (kD * 2);
    const char *vbase = static_cast<const char *>(a.v) + (long)bg * a.Tk * (kD * 2);

    float m[RP], lsum[RP], acc[RP][8];
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    i32x4_t kn[8], vn[8];
    auto load = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int row = t0 + 4 * i + grp;
            row = row < ke ? row : ke - 1;
            kn[i] = *(const i32x4_t *)(kbase + (long)row * (kD * 2) + 16 * chunk);
            vn[i] = *(const i32x4_t *)(vbase + (long)row * (kD * 2) + 16 * chunk);
        }
    };

    int t0 = kb + wave * kRows;
    if (t0 < ke) load(t0);
    for (; t0 < ke; t0 += kWaves * kRows) {
        i32x4_t kc[8], vc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kc[i] = kn[i];
            vc[i] = vn[i];
        }
        // Unconditional, branch-free prefetch of the next tile (past the end it re-reads this
        // tile from cache), pinned ahead of this tile's work.
        load(t0 + kWaves * kRows < ke ? t0 + kWaves * kRows : t0);
        __builtin_amdgcn_sched_barrier(0);

        float s[8][RP], mx[RP];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float k[8];
            bf16x8_to_f32(kc[i], k);
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(q[h][e], k[e], d);
                s[i][h] = d;
            }
        }
        // Complete the dot products across the 16 lanes of each row.
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                float d = s[i][h];
                d += __shfl_xor(d, 8);
                d += __shfl_xor(d, 4);
                d += __shfl_xor(d, 2);
                d += __shfl_xor(d, 1);
                const int t = t0 + 4 * i + grp;
                s[i][h] = t < ke ? d : -INFINITY;
            }
#pragma unroll
        for (int h = 0; h < RP; ++h) {
            float bm = s[0][h];
#pragma unroll
            for (int i = 1; i < 8; ++i) bm = fmaxf(bm, s[i][h]);
            // A tail tile can leave this row group with no valid row yet (mn = -inf): use 0
            // as the exponent reference then, so every exp2 sees -inf and yields 0.
            const float mn = fmaxf(m[h], bm);
            const float mref = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[h] - mref);
            m[h] = mn;
            mx[h] = mref;
            lsum[h] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v[8];
            bf16x8_to_f32(vc[i], v);
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                const float p = fast_exp2(s[i][h] - mx[h]);
                lsum[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
            }
        }
    }

    // ---- merge the 16 states (4 row groups x 4 waves) in a fixed order ----
    const int sid = wave * 4 + grp;
    if (chunk == 0) {
#pragma unroll
        for (int h = 0; h < RP; ++h) {
            st_m[sid][h] = m[h];
            st_l[sid][h] = lsum[h];
        }
    }
    __syncthreads();
    if (threadIdx.x < RP) {
        const int h = threadIdx.x;
        float M = st_m[0][h];
        for (int i = 1; i < NST; ++i) M = fmaxf(M, st_m[i][h]);
        float l = 0.f;
        for (int i = 0; i < NST; ++i) l += st_m[i][h] == -INFINITY ? 0.f : fast_exp2(st_m[i][h] - M) * st_l[i][h];
        M_s[h] = M;
        l_s[h] = l;
    }
    __syncthreads();
    float f[RP];
#pragma unroll
    for (int h = 0; h < RP; ++h) f[h] = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - M_s[h]);
    for (int s = 0; s < NST; ++s) {
        if (sid == s) {
#pragma unroll
            for (int h = 0; h < RP; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float *dst = &O_s[h][8 * chunk + e];
                    *dst = (s == 0 ? 0.f : *dst) + acc[h][e] * f[h];
                }
        }
        __syncthreads();
    }

    if (S == 1) {
        uint16_t *out = static_cast<uint16_t *>(a.out);
        for (int e = threadIdx.x; e < R * kD; e += kThreads) {
            const int h = e / kD;
            out[head0 * kD + e] = f32_to_bf16(O_s[h][e % kD] / l_s[h]);
        }
    } else {
        for (int e = threadIdx.x; e < R * kD; e += kThreads) {
            const int h = e / kD, d = e % kD;
            a.part_acc[((head0 + h) * S + split) * kD + d] = O_s[h][d];
        }
        for (int h = threadIdx.x; h < R; h += kThreads) {
            a.part_ml[((head0 + h) * S + split) * 2] = M_s[h];
            a.part_ml[((head0 + h) * S + split) * 2 + 1] = l_s[h];
        }
    }
}

template <int RP>
hipError_t launch_rp(const AttnArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_valu_kernel<RP>), dim3((unsigned)(a.B * a.G * a.num_splits)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

bool decode_valu_supports(const AttnArgs &a) {
    return a.decode && a.D == kD && a.q_dtype == DT_BF16 && a.kv_dtype == DT_BF16 && a.H / a.G <= 8;
}

hipError_t launch_decode_valu(const AttnArgs &a, hipStream_t stream) {
    if (!decode_valu_supports(a)) return hipErrorInvalidValue;
    const int R = a.H / a.G;
    if (R <= 1) return launch_rp<1>(a, stream);
    if (R <= 2) return launch_rp<2>(a, stream);
    if (R <= 4) return launch_rp<4>(a, stream);
    return launch_rp<8>(a, stream);
}

}  // namespace gqa
