// Narrow-group GQA decode on the vector ALUs (bf16 KV cache, D = 128, R = H/G <= 8).
//
// With few query heads per KV head (R = 4 for a GQA-8 model with 32 query heads) decode
// does only 4*R flops per cached bf16 element, which the vector ALUs sustain at HBM rate;
// matrix cores would mostly multiply padding. Each KV row is read once per (sequence,
// KV head) and used for all R heads of the group [GQA paper digest page (51969.com),
// section "Grouped-query attention (GQA)"; group of head h is h / (H/G), "LLM principles --
// code implementation of multi-head attention (MQA and GQA)", section 5].
//
// Work: one single-wave workgroup per (sequence b, KV head g, key range), so there is no
// barrier anywhere. The wave streams 32-row tiles of K and V with 16-byte loads: lane l
// reads 8 head dims (chunk l%16) of row 4*i + l/16, i = 0..7, so one instruction covers
// four whole 256-byte rows. Each lane forms the partial dot products of its 8 dims with the
// R query rows and a DPP reduction over the 16 lanes of the row completes them (no LDS
// traffic). The four row groups keep separate online-softmax states (running max, running
// sum, 8-dim accumulators per head), updated once per tile, and merge at the end with four
// cross-row exchanges. The first tile is requested before the sequence length is known, so
// its latency overlaps the seq_lens read; rows past the end are masked by index.
#include "dtypes.h"
#include "gqa_internal.h"
#include "mfma_util.h"

namespace gqa {

namespace {

constexpr int kRows = 32;  // rows per tile (8 per lane)
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
__global__ __launch_bounds__(64) void decode_valu_kernel(AttnArgs a) {
    const int lane = threadIdx.x;
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

    // First tile first: its rows are known before the length (clamped to the allocation).
    if (kb < a.Tk) load(kb, a.Tk - 1);

    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.Tk ? a.Tk : L);
    const int ke = kb + a.split_len < L ? kb + a.split_len : L;

    if (kb >= ke) {
        if (S == 1) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            for (int e = lane; e < R * kD; e += 64) out[head0 * kD + e] = 0;
        } else {
            for (int h = lane; h < R; h += 64) {
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

    float m[RP], lsum[RP], acc[RP][8];
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int t0 = kb; t0 < ke; t0 += kRows) {
        i32x4_t kc[8], vc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kc[i] = kn[i];
            vc[i] = vn[i];
        }
        // Unconditional, branch-free prefetch of the next tile (past the end it re-reads this
        // tile from cache), pinned ahead of this tile's work.
        load(t0 + kRows < ke ? t0 + kRows : t0, ke - 1);
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

    // ---- merge the four row-group states (lanes chunk, chunk+16, +32, +48), fixed order ----
#pragma unroll
    for (int h = 0; h < RP; ++h) {
        float M = fmaxf(m[h], __shfl_xor(m[h], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float f = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - M);
        float l = lsum[h] * f;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[h][e] * f;
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[h][e] = x;
        }
        m[h] = M;
        lsum[h] = l;
    }

    if (grp == 0) {
        if (S == 1) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                if (h < R) {
                    const float inv = 1.f / lsum[h];
                    i32x4_t w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = pack_bf16_rne(acc[h][2 * e] * inv, acc[h][2 * e + 1] * inv);
                    *(i32x4_t *)(out + (head0 + h) * kD + 8 * chunk) = w;
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < RP; ++h) {
                if (h < R) {
                    float *pa = a.part_acc + ((head0 + h) * S + split) * kD + 8 * chunk;
                    *(f32x4_t *)pa = f32x4_t{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
                    *(f32x4_t *)(pa + 4) = f32x4_t{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
                    if (chunk == 0) {
                        a.part_ml[((head0 + h) * S + split) * 2] = m[h];
                        a.part_ml[((head0 + h) * S + split) * 2 + 1] = lsum[h];
                    }
                }
            }
        }
    }
}

template <int RP>
hipError_t launch_rp(const AttnArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_valu_kernel<RP>), dim3((unsigned)(a.B * a.G * a.num_splits)), dim3(64), 0, stream,
                       a);
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
