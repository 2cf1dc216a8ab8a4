// Generic GQA attention kernel: any head dim 1..256, fp32 / bf16 / fp8-E4M3FN / INT4 KV.
//
// Serves the shapes the vectorised kernels do not (tiny or odd head dims such as the
// 12-dim, 4-head toy with D = 3) and is the family every fast kernel is cross-checked
// against. One workgroup owns one (sequence, KV head g) and a block of query rows made
// of `hpw` heads of group g times `tm` query positions, so each K/V row it stages in
// LDS is read from memory once and used by all of those heads -- query head h reads KV
// head h / (H/G) [GQA paper digest page (51969.com), section "Grouped-query attention
// (GQA)"; "LLM principles -- code implementation of multi-head attention (MQA and
// GQA)", section 5]. Scores use the online (running max / running sum) form of the
// softmax, in base 2 with log2(e) folded into the scale; that equals the page's
// softmax(QK^T / sqrt(d)) V (same page, section 3) in exact arithmetic. Modes: decode (one
// query row at the sequence's last position), prefill, and prefill of a chunk of Tq queries
// against a cache of seq_lens[b] rows (the chunk's rows at the end, causal from there).
#include "dtypes.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 16;                       // keys per LDS tile
constexpr int kSlots = 16;                       // accumulator elements per thread
constexpr int kRowElems = kThreads * kSlots;     // rows * D must fit (4096)
constexpr int kRowsMax = 64;
constexpr int kDMax = 256;

template <typename QT, int KVT>
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(AttnArgs a, int hpw, int tm) {
    using KT = typename KvElem<KVT>::T;
    __shared__ float q_s[kRowElems];
    __shared__ float k_s[kTileN * kDMax];
    __shared__ float v_s[kTileN * kDMax];
    __shared__ float p_s[kRowsMax * kTileN];
    __shared__ float m_s[kRowsMax], l_s[kRowsMax], alpha_s[kRowsMax];
    __shared__ int head_s[kRowsMax], pos_s[kRowsMax];

    const int tid = threadIdx.x;
    const int D = a.D, H = a.H, G = a.G;
    const int R = H / G;
    // blockIdx.x enumerates (head chunk, query tile, sequence * KV head), fastest first.
    const int nhc = (R + hpw - 1) / hpw;
    const int nqt = a.decode ? 1 : (a.Tq + tm - 1) / tm;
    const int hc = blockIdx.x % nhc;
    const int qt = (blockIdx.x / nhc) % nqt;
    const int bg = blockIdx.x / (nhc * nqt);
    const int b = bg / G, g = bg % G;
    const int split = blockIdx.y;
    const int rows = hpw * tm;

    // Key range of this workgroup. A chunk against a cache (a.cached) holds the last Tq of
    // L positions: query row i sits at position off + i, off = L - Tq (0 for a plain prefill).
    int kb, ke, dec_pos = 0, off = 0;
    if (a.decode) {
        int L = a.seq_lens[b];
        L = L < 0 ? 0 : (L > a.Tk ? a.Tk : L);
        dec_pos = L - 1;
        kb = split * a.split_len;
        ke = kb + a.split_len < L ? kb + a.split_len : L;
    } else {
        int L = a.Tk;
        if (a.cached) {
            L = a.seq_lens[b];
            L = L < 0 ? 0 : (L > a.Tk ? a.Tk : L);
            off = L - a.Tq;
        }
        kb = 0;
        const int last = off + qt * tm + tm - 1;
        ke = a.causal ? (last + 1 < L ? last + 1 : L) : L;
        ke = ke < 0 ? 0 : ke;
    }

    for (int r = tid; r < rows; r += kThreads) {
        const int rh = hc * hpw + r / tm;
        const int pos = a.decode ? dec_pos : qt * tm + r % tm;
        const bool ok = rh < R && (a.decode || pos < a.Tq);
        head_s[r] = ok ? g * R + rh : -1;
        pos_s[r] = pos;
        m_s[r] = -INFINITY;
        l_s[r] = 0.f;
    }
    __syncthreads();

    const QT *q = static_cast<const QT *>(a.q);
    for (int e = tid; e < rows * D; e += kThreads) {
        const int r = e / D, d = e - (e / D) * D;
        const int h = head_s[r];
        float x = 0.f;
        if (h >= 0) {
            const long row = a.decode ? (long)b * H + h : ((long)b * H + h) * a.Tq + pos_s[r];
            x = load_f32(q, row * D + d) * a.scale_log2;
        }
        q_s[e] = x;
    }

    float acc[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) acc[s] = 0.f;

    // Element index of this slab's first value (packed INT4 holds two values per byte, so the
    // offset is kept in elements and added to every index).
    const long slab = ((long)b * G + g) * (long)a.Tk * D;
    const KT *kp = static_cast<const KT *>(a.k);
    const KT *vp = static_cast<const KT *>(a.v);
    const float ksc = KVT == DT_FP8 || KVT == DT_INT4 ? a.k_scale[bg] : 1.f;
    const float vsc = KVT == DT_FP8 || KVT == DT_INT4 ? a.v_scale[bg] : 1.f;

    for (int t0 = kb; t0 < ke; t0 += kTileN) {
        const int n = ke - t0 < kTileN ? ke - t0 : kTileN;
        __syncthreads();  // previous tile fully consumed
        for (int e = tid; e < n * D; e += kThreads) {
            k_s[e] = load_f32(kp, slab + (long)t0 * D + e) * ksc;
            v_s[e] = load_f32(vp, slab + (long)t0 * D + e) * vsc;
        }
        __syncthreads();
        // Scores in the base-2 domain; masked or absent keys are -inf.
        for (int pidx = tid; pidx < rows * kTileN; pidx += kThreads) {
            const int r = pidx / kTileN, j = pidx % kTileN;
            float s = -INFINITY;
            const bool live = j < n && head_s[r] >= 0 && (a.decode || !a.causal || t0 + j <= off + pos_s[r]);
            if (live) {
                float dot = 0.f;
                for (int d = 0; d < D; ++d) dot += q_s[r * D + d] * k_s[j * D + d];
                s = dot;
            }
            p_s[pidx] = s;
        }
        __syncthreads();
        // Online softmax update, one thread per row.
        for (int r = tid; r < rows; r += kThreads) {
            float mx = -INFINITY;
            for (int j = 0; j < n; ++j) mx = fmaxf(mx, p_s[r * kTileN + j]);
            const float m_old = m_s[r];
            const float m_new = fmaxf(m_old, mx);
            float alpha = 1.f, sum = 0.f;
            if (m_new != -INFINITY) {
                alpha = exp2f(m_old - m_new);  // 0 when m_old is -inf
                for (int j = 0; j < n; ++j) {
                    const float p = exp2f(p_s[r * kTileN + j] - m_new);
                    p_s[r * kTileN + j] = p;
                    sum += p;
                }
            } else {
                for (int j = 0; j < n; ++j) p_s[r * kTileN + j] = 0.f;
            }
            l_s[r] = l_s[r] * alpha + sum;
            m_s[r] = m_new;
            alpha_s[r] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const int e = tid + s * kThreads;
            if (e < rows * D) {
                const int r = e / D, d = e - (e / D) * D;
                float o = acc[s] * alpha_s[r];
                for (int j = 0; j < n; ++j) o += p_s[r * kTileN + j] * v_s[j * D + d];
                acc[s] = o;
            }
        }
    }
    __syncthreads();

    if (a.num_splits <= 1) {
        QT *out = static_cast<QT *>(a.out);
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const int e = tid + s * kThreads;
            if (e < rows * D) {
                const int r = e / D, d = e - (e / D) * D;
                const int h = head_s[r];
                if (h >= 0) {
                    const long row = a.decode ? (long)b * H + h : ((long)b * H + h) * a.Tq + pos_s[r];
                    const float l = l_s[r];
                    store_f32(out, row * D + d, l > 0.f ? acc[s] / l : 0.f);
                }
            }
        }
    } else {
        const int S = a.num_splits;
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const int e = tid + s * kThreads;
            if (e < rows * D) {
                const int r = e / D, d = e - (e / D) * D;
                const int h = head_s[r];
                if (h >= 0) a.part_acc[(((long)b * H + h) * S + split) * D + d] = acc[s];
            }
        }
        for (int r = tid; r < rows; r += kThreads) {
            const int h = head_s[r];
            if (h >= 0) {
                const long i = (((long)b * H + h) * S + split) * 2;
                a.part_ml[i] = m_s[r];
                a.part_ml[i + 1] = l_s[r];
            }
        }
    }
}

}  // namespace

hipError_t launch_generic(const AttnArgs &a, hipStream_t stream) {
    const int R = a.H / a.G;
    int rows_cap = kRowElems / a.D;
    if (rows_cap > kRowsMax) rows_cap = kRowsMax;
    const int hpw = R < rows_cap ? R : rows_cap;
    int tm = a.decode ? 1 : rows_cap / hpw;
    if (tm < 1) tm = 1;
    if (!a.decode && tm > a.Tq) tm = a.Tq;
    const int nhc = (R + hpw - 1) / hpw;
    const int nqt = a.decode ? 1 : (a.Tq + tm - 1) / tm;
    dim3 grid((unsigned)(nhc * nqt * a.B * a.G), (unsigned)(a.decode ? a.num_splits : 1));
    dim3 block(kThreads);
    if (a.q_dtype == DT_F32 && a.kv_dtype == DT_F32)
        hipLaunchKernelGGL((attn_generic_kernel<float, DT_F32>), grid, block, 0, stream, a, hpw, tm);
    else if (a.q_dtype == DT_BF16 && a.kv_dtype == DT_BF16)
        hipLaunchKernelGGL((attn_generic_kernel<uint16_t, DT_BF16>), grid, block, 0, stream, a, hpw, tm);
    else if (a.q_dtype == DT_BF16 && a.kv_dtype == DT_FP8)
        hipLaunchKernelGGL((attn_generic_kernel<uint16_t, DT_FP8>), grid, block, 0, stream, a, hpw, tm);
    else if (a.q_dtype == DT_BF16 && a.kv_dtype == DT_INT4)
        hipLaunchKernelGGL((attn_generic_kernel<uint16_t, DT_INT4>), grid, block, 0, stream, a, hpw, tm);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gqa
