// Cache append as its own kernel, for the decode families that do not fuse it (generic and
// vector-ALU) and for new rows that are not 16-byte aligned: the current token's key and
// value, [B*G][D] in q's dtype, are stored at (logical) row
// L_b - 1 of every (b, g) with 1 <= L_b <= T_cap ("LLM principles -- code implementation of
// multi-head attention (MQA and GQA)", sections 3 and 5: the new K/V are appended to the
// cache before the scores). fp32 and bf16 caches take the values unchanged; fp8 caches take
// E4M3FN codes of x / scale with the slab's fixed scale, saturated at 448, and INT4 caches the
// nearest integer field clamped to -8 .. 7 ("GQA revolution: how xformers speeds up LLM
// inference", section on mixed-precision KV storage).
#include "dtypes.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

// One workgroup per (b, g); thread d handles head dim d.
template <typename QT, typename KT, bool FP8>
__global__ __launch_bounds__(256) void kv_append_kernel(AttnArgs a) {
    const int bg = blockIdx.x;
    const int b = bg / a.G, g = bg - b * a.G;
    const int L = a.seq_lens[b];
    const int d = threadIdx.x;
    if (L < 1 || L > a.Tk || d >= a.D) return;
    long i;  // element index of row L-1, head dim d
    if (a.block_table) {
        // Paged cache [num_pages][G][page_size][D]; page ids outside the pool are clamped.
        const int r = L - 1, ps = 1 << a.ps_log2;
        int page = a.block_table[(long)b * a.pages_per_seq + (r >> a.ps_log2)];
        page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
        i = (((long)page * a.G + g) * ps + (r & (ps - 1))) * a.D + d;
    } else {
        i = ((long)bg * a.Tk + (L - 1)) * a.D + d;
    }
    const float k = load_f32(static_cast<const QT *>(a.k_new), (long)bg * a.D + d);
    const float v = load_f32(static_cast<const QT *>(a.v_new), (long)bg * a.D + d);
    if constexpr (FP8) {
        static_cast<uint8_t *>(const_cast<void *>(a.k))[i] = (uint8_t)quant_e4m3fn_x4(k, 0.f, 0.f, 0.f, a.k_scale[bg]);
        static_cast<uint8_t *>(const_cast<void *>(a.v))[i] = (uint8_t)quant_e4m3fn_x4(v, 0.f, 0.f, 0.f, a.v_scale[bg]);
    } else {
        store_f32(static_cast<KT *>(const_cast<void *>(a.k)), i, k);  // exact: same type
        store_f32(static_cast<KT *>(const_cast<void *>(a.v)), i, v);
    }
}

// INT4 caches: thread j quantises head dims 2j and 2j+1 into byte j of the row.
__global__ __launch_bounds__(128) void kv_append_i4_kernel(AttnArgs a) {
    const int bg = blockIdx.x;
    const int b = bg / a.G, g = bg - b * a.G;
    const int L = a.seq_lens[b];
    const int j = threadIdx.x, nb = a.D / 2;
    if (L < 1 || L > a.Tk || j >= nb) return;
    long row;  // row index of L-1 in [.. rows ..][D/2] bytes
    if (a.block_table) {
        const int r = L - 1, ps = 1 << a.ps_log2;
        int page = a.block_table[(long)b * a.pages_per_seq + (r >> a.ps_log2)];
        page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
        row = ((long)page * a.G + g) * ps + (r & (ps - 1));
    } else {
        row = (long)bg * a.Tk + (L - 1);
    }
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) + (long)bg * a.D + 2 * j;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) + (long)bg * a.D + 2 * j;
    const float ks = a.k_scale[bg], vs = a.v_scale[bg];
    static_cast<uint8_t *>(const_cast<void *>(a.k))[row * nb + j] =
        (uint8_t)(quant_int4(bf16_to_f32(kn[0]), ks) | (quant_int4(bf16_to_f32(kn[1]), ks) << 4));
    static_cast<uint8_t *>(const_cast<void *>(a.v))[row * nb + j] =
        (uint8_t)(quant_int4(bf16_to_f32(vn[0]), vs) | (quant_int4(bf16_to_f32(vn[1]), vs) << 4));
}

}  // namespace

hipError_t launch_kv_append(const AttnArgs &a, hipStream_t stream) {
    if (a.kv_dtype == DT_INT4) {
        if (a.D > 256 || a.D % 2 != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kv_append_i4_kernel, dim3((unsigned)(a.B * a.G)), dim3(128), 0, stream, a);
        return hipGetLastError();
    }
    if (a.D > 256) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.B * a.G)), block(256);
    if (a.kv_dtype == DT_F32)
        hipLaunchKernelGGL((kv_append_kernel<float, float, false>), grid, block, 0, stream, a);
    else if (a.kv_dtype == DT_BF16)
        hipLaunchKernelGGL((kv_append_kernel<uint16_t, uint16_t, false>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((kv_append_kernel<uint16_t, uint8_t, true>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace gqa
