// Narrow-group GQA decode on the vector ALUs (bf16 KV cache, D = 128, R = H/G <= 8).
//
// With few query heads per KV head (R = 4 for a GQA-8 model with 32 query heads) decode
// does only 4*R flops per cached bf16 element, which the vector ALUs sustain at HBM rate.
// The library's default is still the matrix-core kernel, whose per-block instruction count
// is lower; this kernel is an independent second implementation, selected explicitly
// (GQA_PATH_VALU) and checked against the same inputs. Each KV row is read once per (sequence,
// KV head) and used for all R heads of the group [GQA paper digest page (51969.com),
// section "Grouped-query attention (GQA)"; group of head h is h / (H/G), "LLM principles --
// code implementation of multi-head attention (MQA and GQA)", section 5].
//
// Work: one workgroup of 4 independent waves per (sequence b, KV head g, key range); wave w
// streams 32-row tiles w, w+4, ... of the range with 16-byte loads: lane l reads 8 head dims
// (chunk l%16) of row 4*i + l/16, i = 0..7, so one instruction covers four whole 256-byte
// rows. Each lane forms the partial dot products of its 8 dims with the R query rows and a
// DPP reduction over the 16 lanes of the row completes them (no LDS traffic). Each lane
// group keeps its own online-softmax state (running max, running sum, 8-dim accumulators
// per head), updated once per tile; the 16 states of the workgroup are merged in one LDS
// step at the end. Each wave's first tile is requested before the sequence length is
// known, so its latency overlaps the seq_lens read; rows past the end are masked by index.
// Split ranges either leave partials for the combine kernel or, when small, are merged by
// the workgroup that finishes last (splitkv.h).
#include "dtypes.h"
#include "gqa_internal.h"
#include "mfma_util.h"
#include "splitkv.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32;  // rows per tile (8 per lane)
constexpr int kStates = 4 * kWaves;  // softmax states per workgroup (4 row groups per wave)
constexpr int kPassHeads = 4;        // heads merged per LDS pass
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;

__device__ __forceinline__ void bf16x8_to_f32(const i32x4_t &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = (uint32_t)w[i];
        x[2 * i] = __uint_as_float(u << 16);
        x[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
}

// DPP lane moves inside a row of 16 lanes. quad_perm [1,0,3,2] and [2,3,0,1] swap within
// quads; row_half_mirror and row_mirror reverse within 8 and 16 lanes. After the two quad
// steps every lane of a quad holds the quad sum, so the mirrors complete a full 16-lane sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

template <int RP>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(AttnArgs a) {
    constexpr int PH = RP < kPassHeads ? RP : kPassHeads;
    __shared__ float st_m[kStates][RP], st_l[kStates][RP];
    __shared__ float M_s[RP], l_s[RP];
    __shared__ __attribute__((aligned(16))) float st_acc[kStates][PH][kD];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar
    const int grp = lane >> 4;    // row group: rows 4*i + grp of each tile
    const int chunk = lane & 15;  // head dims 8*chunk .. 8*chunk+7
    // Split-major block order (see decode_mfma.hip).
    const int S = a.num_splits;
    const int nbg = a.B * a.G;
    const int split = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int G = a.G, H = a.H, R = H / G;
    const int b = bg / G, g = bg % G;
    const int kb = split * a.split_len;
    const long head0 = (long)b * H + (long)g * R;

    const char *kbase = static_cast<const char *>(a.k) + (long)bg * a.Tk * kRowBytes;
    const char *vbase = static_cast<const char *>(a.v) + (long)bg * a.Tk * kRowBytes;

    i32x4_t kn[8], vn[8];
    auto load = [&](int t0, int last) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int row = t0 + 4 * i + grp;
            row = row < last ? row : last;
            kn[i] = *(const i32x4_t *)(kbase + (long)row * kRowBytes + 16 * chunk);
            vn[i] = *(const i32x4_t *)(vbase + (long)row * kRowBytes + 16 * chunk);
        }
    };

    // The query rows and the first tile do not depend on the length (the tile's rows are
    // clamped to the allocation), so all three requests share one memory round trip.
    i32x4_t qraw[RP];
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + head0 * kD;
#pragma unroll
    for (int h = 0; h < RP; ++h) qraw[h] = *(const i32x4_t *)(qp + (long)(h < R ? h : R - 1) * kD + 8 * chunk);
    if (kb + wave * kRows < a.Tk) load(kb + wave * kRows, a.Tk - 1);

    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.Tk ? a.Tk : L);
    const int ke = kb + a.split_len < L ? kb + a.split_len : L;

    if (kb >= ke) {
        // Nothing to attend to in this range. Fused merges count only non-empty ranges, so
        // an empty one only has to produce the zero row of an empty sequence.
        if (S == 1 || (a.fuse_combine && L == 0 && split == 0)) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            for (int e = threadIdx.x; e < R * kD; e += kThreads) out[head0 * kD + e] = 0;
        } else if (!a.fuse_combine) {
            for (int h = threadIdx.x; h < R; h += kThreads) {
                a.part_ml[((head0 + h) * S + split) * 2] = -INFINITY;
                a.part_ml[((head0 + h) * S + split) * 2 + 1] = 0.f;
            }
        }
        return;
    }

    // This lane's 8 dims of every query row of the group, pre-scaled into the base-2 domain.
    float q[RP][8];
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        if (h < R) {
            bf16x8_to_f32(qraw[h], q[h]);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[h][e] *= a.scale_log2;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[h][e] = 0.f;
        }
    }

    float m[RP], lsum[RP], acc[RP][8];
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int t0 = kb + wave * kRows; t0 < ke; t0 += kWaves * kRows) {
        i32x4_t kc[8], vc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kc[i] = kn[i];
            vc[i] = vn[i];
        }
        // Unconditional, branch-free prefetch of the next tile (past the end it re-reads this
        // tile from cache), pinned ahead of this tile's work.
        load(t0 + kWaves * kRows < ke ? t0 + kWaves * kRows : t0, ke - 1);
        __builtin_amdgcn_sched_barrier(0);

        // Rows at or past the end (the last tile, or a first tile loaded before the length
        // was known) may hold anything, NaN included: zero their values, mask their scores.
        const bool tail = t0 + kRows > ke;
        if (tail) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (t0 + 4 * i + grp >= ke) {
                    kc[i] = i32x4_t{0, 0, 0, 0};
                    vc[i] = i32x4_t{0, 0, 0, 0};
                }
        }

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
                d = row16_sum(d);
                s[i][h] = (!tail || t0 + 4 * i + grp < ke) ? d : -INFINITY;
            }
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

    // ---- merge the 16 states of the workgroup (fixed order: deterministic) ----
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
        for (int i = 1; i < kStates; ++i) M = fmaxf(M, st_m[i][h]);
        float l = 0.f;
        for (int i = 0; i < kStates; ++i) l += st_m[i][h] == -INFINITY ? 0.f : fast_exp2(st_m[i][h] - M) * st_l[i][h];
        M_s[h] = M;
        l_s[h] = l;
    }
    __syncthreads();
    uint16_t *out = static_cast<uint16_t *>(a.out);
#pragma unroll
    for (int h0 = 0; h0 < RP; h0 += PH) {
#pragma unroll
        for (int hh = 0; hh < PH; ++hh) {
            const float f = m[h0 + hh] == -INFINITY ? 0.f : fast_exp2(m[h0 + hh] - M_s[h0 + hh]);
            *(f32x4_t *)&st_acc[sid][hh][8 * chunk] =
                f32x4_t{acc[h0 + hh][0] * f, acc[h0 + hh][1] * f, acc[h0 + hh][2] * f, acc[h0 + hh][3] * f};
            *(f32x4_t *)&st_acc[sid][hh][8 * chunk + 4] =
                f32x4_t{acc[h0 + hh][4] * f, acc[h0 + hh][5] * f, acc[h0 + hh][6] * f, acc[h0 + hh][7] * f};
        }
        __syncthreads();
        for (int e = threadIdx.x; e < PH * kD; e += kThreads) {
            const int hh = e / kD, d = e % kD, h = h0 + hh;
            if (h < R) {
                float x = 0.f;
#pragma unroll
                for (int i = 0; i < kStates; ++i) x += st_acc[i][hh][d];
                if (S == 1)
                    out[(head0 + h) * kD + d] = f32_to_bf16(x / l_s[h]);
                else
                    splitkv_store(&a.part_acc[((head0 + h) * S + split) * kD + d], x, a.fuse_combine);
            }
        }
        __syncthreads();
    }
    if (S == 1) return;
    for (int h = threadIdx.x; h < R; h += kThreads) {
        splitkv_store(&a.part_ml[((head0 + h) * S + split) * 2], M_s[h], a.fuse_combine);
        splitkv_store(&a.part_ml[((head0 + h) * S + split) * 2 + 1], l_s[h], a.fuse_combine);
    }
    if (a.fuse_combine) {
        const int n_active = active_splits(L, a.split_len, S);
        if (splitkv_arrive(a.counters + bg, n_active)) splitkv_merge_bf16<kThreads, kD>(a, head0, R, n_active, out);
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
