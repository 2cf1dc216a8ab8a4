// Host layer of libgqa.so: the C ABI declared in include/gqa.h.
//
// Every check runs before the first HIP call, so a rejected call leaves the device and
// the stream untouched. The launch sequence is: (optional) stream-ordered workspace,
// the cache append when it is not fused, the attention kernel, the split-KV combine when
// the cache was split, and the release of the workspace -- all on the caller's stream,
// with no host synchronisation.
#include <math.h>
#include <stddef.h>
#include <string.h>

#include <mutex>

#include "gqa.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kMaxDim = 256;
constexpr int kMaxSplitsAbi = 1024;
constexpr int kNumDevicesMax = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Bytes per KV row of D values (INT4 packs two values per byte).
long row_bytes(int dt, long D) { return dt == DT_F32 ? 4 * D : dt == DT_BF16 ? 2 * D : dt == DT_FP8 ? D : (D + 1) / 2; }

bool valid_dtype(int dt) { return dt == DT_F32 || dt == DT_BF16 || dt == DT_FP8 || dt == DT_INT4; }

// Copy the caller's options over defaults, honouring struct_size (older, shorter
// layouts keep the defaults for the fields they do not have).
bool read_opts(const gqa_opts *in, gqa_opts *o) {
    gqa_opts_init(o);
    if (!in) return true;
    if (in->struct_size < offsetof(gqa_opts, kv_dtype) + sizeof(int32_t)) return false;
    const size_t n = in->struct_size < sizeof(gqa_opts) ? in->struct_size : sizeof(gqa_opts);
    memcpy(o, in, n);
    o->struct_size = sizeof(gqa_opts);
    return true;
}

// Key-range splits for decode. A split is the unit of work of one workgroup. Aim at
// about two workgroups per compute unit on the 256-CU part, but keep each split long
// enough that its partial results (R heads x (D + 2) floats, written and read once) stay
// under 1/8 of the K/V bytes it streams, and at least one 64-key tile long. The partials
// rule yields to filling every CU once: with small rows (INT4) and many heads per KV head
// it would leave CUs idle, which costs more than the extra partials (INT4 MQA decode,
// B8 H32 G1 L32768: 16 ranges 34.2 us, 32 ranges 23.9 us).
int auto_splits(long B, long H, long G, long D, long T_cap, int kv_dtype) {
    const long R = H / G;
    const long units = B * G;
    const long target = 512;
    long min_len = (8L * R * (D + 2) * 4 * 2) / (2L * row_bytes(kv_dtype, D));
    if (min_len < 64) min_len = 64;
    long by_len = (T_cap + min_len - 1) / min_len;
    const long fill = (256 + units - 1) / units, fill_cap = (T_cap + 63) / 64;
    if (by_len < fill) by_len = fill < fill_cap ? fill : fill_cap;
    long by_units = (target + units - 1) / units;
    long s = by_len < by_units ? by_len : by_units;
    if (s < 1) s = 1;
    if (s > kMaxSplitsAbi) s = kMaxSplitsAbi;
    return (int)s;
}

bool decode_sizes_ok(int B, int H, int G, int D, int T_cap) {
    if (B < 1 || H < 1 || G < 1 || D < 1 || T_cap < 1) return false;
    if (H % G != 0 || D > kMaxDim) return false;
    // Element counts must stay well inside int64 and grid sizes inside 2^31.
    const double kv = (double)B * G * (double)T_cap * D;
    if (kv > 9.0e15) return false;
    if ((double)B * H > 2.0e9 || (double)B * G * H > 2.0e9) return false;
    return true;
}

int resolve_splits(int B, int H, int G, int D, int T_cap, int kv_dtype, int requested) {
    int s = requested > 0 ? requested : auto_splits(B, H, G, D, T_cap, kv_dtype);
    if (s > T_cap) s = requested > 0 ? s : T_cap;
    return s;
}

// Partial results of one key range merged inside the decode kernel up to this size.
constexpr size_t kFuseMaxBytes = 64 * 1024;
bool fuse_combine_for(long H, long G, long D, long S) {
    // The in-kernel merge keeps one weight per (head, range) in a 128-entry LDS table.
    return S > 1 && S * (H / G) <= 128 && (size_t)S * (H / G) * (D + 2) * sizeof(float) <= kFuseMaxBytes;
}

// Decode work layout. The flat layout (equal rows per workgroup whatever the lengths) serves
// the matrix-core family when asked for, or by default for batches of at least
// kFlatMinBatch sequences, where lengths usually differ; its fixed cost (every workgroup
// first reads all lengths) does not pay off for a few sequences. Otherwise uniform key ranges.
struct DecodePlan {
    int flat = 0;
    int S = 1;          // key ranges (uniform) or partial slots per head (flat)
    int split_len = 0;  // uniform
    int nw = 0;         // flat: workgroups
    int cmin = 0;       // flat: fewest rows per workgroup
    int pad = 0;        // flat: rows of no work in front of each non-empty segment
    int fuse = 0;       // merge inside the decode kernel
};

constexpr int kNominalCUs = 256;
constexpr int kFlatMinBatch = 16;

// The fixed cost of one piece of the flat layout (its first round trip, the merge of its waves,
// its partials and arrival: a few microseconds at the ~27 GB/s one CU streams) as the K/V bytes
// a workgroup would stream meanwhile, and as rows of a cache type. Measured on the ragged
// Llama-70B batch (pads of 0 / 40 / 80 / 120 / 160 / 240 KiB): bf16 35.4 / 34.9 / 34.6 / 33.7 /
// 33.8 / 34.0 us; a ragged fp8 MQA batch (B16 H32 G1, 2k-16k keys) 26.0 / 23.9 / 22.2 / 21.5 /
// 21.5 / 21.3 us. Again with the next piece requested before the wave merge: bf16 at 80 / 100 /
// 120 / 140 / 170 KiB 34.2 / 34.1 / 33.0 / 33.4 / 33.7 us; the INT4 cache (two workgroups per
// CU) at 50 / 65 / 80 / 95 / 115 KiB 17.9 / 17.6 / 18.2 / 18.4 / 18.4 us.
int flat_pad_rows(long D, int kv_dtype) {
    const long cost = kv_dtype == DT_INT4 ? 64 * 1024 : 120 * 1024;
    return (int)(cost / (2 * row_bytes(kv_dtype, D)));
}

bool flat_possible(int B, int G, int T_cap, int D, int kv_dtype, int path, int requested) {
    return path == GQA_PATH_MFMA && requested == 0 && (long)B * G * (T_cap + flat_pad_rows(D, kv_dtype)) < (1L << 31);
}

// `path` is the resolved kernel family (not AUTO); `layout` a gqa_layout the caller checked.
DecodePlan plan_decode(int B, int H, int G, int D, int T_cap, int kv_dtype, int requested, int path, int layout) {
    DecodePlan p;
    const long R = H / G;
    const bool mfma_path = path == GQA_PATH_MFMA;
    const bool flat = flat_possible(B, G, T_cap, D, kv_dtype, path, requested) &&
                      (layout == GQA_LAYOUT_FLAT || (layout == GQA_LAYOUT_AUTO && B >= kFlatMinBatch));
    if (flat) {
        p.flat = 1;
        p.pad = flat_pad_rows(D, kv_dtype);
        // One workgroup per CU: each streams a long run of rows, so the per-piece fixed costs
        // (lengths, first block, merge) stay small against it. INT4 caches take two per CU: their
        // blocks are bound by the widening arithmetic of one wave per SIMD, which a second
        // workgroup overlaps (ragged Llama-70B batch, 256 / 512 / 768 workgroups: INT4 19.8 /
        // 18.0 / 18.7 us, in 16-row pages 21.8 / 20.1 / 20.9 us; bf16 33.4 / 34.6 / 39.9 us).
        p.nw = kv_dtype == DT_INT4 ? 2 * kNominalCUs : kNominalCUs;
        const long per_slot = R * (D + 2) * (long)sizeof(float);
        const long fuse_slots = (long)kFuseMaxBytes / per_slot;
        const long full_chunk = ((long)B * G * T_cap + p.nw - 1) / p.nw;  // rows per workgroup, full caches
        long cmin = 256;
        if (fuse_slots >= 3 && fuse_slots * R <= 128) {
            // Fuse when a chunk long enough to bound the slots by fuse_slots still spreads a full
            // batch over every workgroup.
            const long need = ((T_cap + fuse_slots - 2) / (fuse_slots - 1) + 31) / 32 * 32;
            if (need <= full_chunk) {
                cmin = need > 128 ? need : 128;
                p.fuse = 1;
            }
        }
        p.cmin = (int)cmin;
        // A segment of T rows meets at most ceil((T - 1) / C) + 1 chunks of C >= cmin rows.
        p.S = (int)((T_cap - 1 + cmin - 1) / cmin + 1);
        if (p.fuse && !fuse_combine_for(H, G, D, p.S)) p.fuse = 0;
        return p;
    }
    p.S = resolve_splits(B, H, G, D, T_cap, kv_dtype, requested);
    if (requested == 0 && mfma_path && !fuse_combine_for(H, G, D, p.S)) {
        // Prefer a split count whose partials merge inside the kernel (no second kernel), if
        // halving reaches one while at least 128 workgroups remain.
        int s = p.S;
        while (s > 1 && !fuse_combine_for(H, G, D, s) && (long)B * G * (s / 2) >= 128) s /= 2;
        if (s > 1 && fuse_combine_for(H, G, D, s)) p.S = s;
    }
    p.split_len = (T_cap + p.S - 1) / p.S;
    p.fuse = path != GQA_PATH_GENERIC && fuse_combine_for(H, G, D, p.S);
    return p;
}

// AUTO resolves to the matrix-core family wherever it applies: head dim 128 with a bf16 or fp8
// cache (the cache type fixes q's: bf16), at most 64 query heads per KV head.
int auto_path(int H, int G, int D, int kv_dtype) {
    if (D == 128 && (kv_dtype == DT_BF16 || kv_dtype == DT_FP8 || kv_dtype == DT_INT4) && H / G <= 64)
        return GQA_PATH_MFMA;
    return GQA_PATH_GENERIC;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return ((x + kAlign - 1) / kAlign) * kAlign; }

// Workspace layout: [B*G] int arrival counters | [B*H][S][D] fp32 partial accumulators |
// [B*H][S][2] fp32 (running max, running sum); each part 256-byte aligned.
size_t counter_bytes(long B, long G) { return round_up((size_t)B * G * sizeof(int)); }
size_t acc_bytes(long B, long H, long D, long S) { return round_up((size_t)B * H * S * D * sizeof(float)); }

size_t workspace_bytes_for(long B, long H, long G, long D, long S) {
    if (S <= 1) return 0;
    return counter_bytes(B, G) + acc_bytes(B, H, D, S) + (size_t)B * H * S * 2 * sizeof(float);
}


// gfx950 check, once per device.
std::mutex g_arch_mu;
signed char g_arch_ok[kNumDevicesMax];  // 0 unknown, 1 ok, -1 not gfx950

gqa_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
    if (dev < 0 || dev >= kNumDevicesMax) return GQA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_arch_mu);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GQA_ERR_HIP;
        g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_arch_ok[dev] == 1 ? GQA_OK : GQA_ERR_UNSUPPORTED;
}

// ---- Device scratch of gqa_decode_noalloc ----
// One array per GPU, in the library's own code object, held until the process ends: a fixed
// region of split arrival counters (only ever used as counters, so the invariant that a
// completed call leaves them at zero holds across calls of any size), then the split partials.
// In host code `scratch` names a host-side stand-in, not device memory: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
constexpr int kScratchCounters = 65536;                     // B * G at most
constexpr size_t kScratchCounterBytes = kScratchCounters * sizeof(int);
constexpr size_t kScratchPartialBytes = size_t(32) << 20;   // 32 MiB of split partials at most
static __device__ __align__(256) char scratch[kScratchCounterBytes + kScratchPartialBytes];

std::mutex g_scratch_mu;
char *g_scratch[kNumDevicesMax];  // device address of `scratch`, per device; null until set up

// The current device's scratch: on its first use on a device, look up the array's address there
// and zero its counters on `stream` (ordered before the call's kernels on that stream).
gqa_status device_scratch(hipStream_t stream, char **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
    if (dev < 0 || dev >= kNumDevicesMax) return GQA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GQA_ERR_HIP;
        if (launch_zero_ints(static_cast<int *>(p), kScratchCounters, stream) != hipSuccess) return GQA_ERR_HIP;
        g_scratch[dev] = static_cast<char *>(p);
    }
    *out = g_scratch[dev];
    return GQA_OK;
}

}  // namespace

}  // namespace gqa

using namespace gqa;

extern "C" {

void gqa_opts_init(gqa_opts *o) {
    if (!o) return;
    memset(o, 0, sizeof(*o));
    o->struct_size = sizeof(gqa_opts);
    o->q_dtype = GQA_DTYPE_BF16;
    o->kv_dtype = GQA_DTYPE_BF16;
    o->path = GQA_PATH_AUTO;
}

const char *gqa_status_string(gqa_status s) {
    switch (s) {
        case GQA_OK: return "GQA_OK";
        case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG";
        case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
        case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
        case GQA_ERR_HIP: return "GQA_ERR_HIP";
    }
    return "GQA_ERR_UNKNOWN";
}

int gqa_decode_num_splits(int B, int H, int G, int D, int kv_capacity, int kv_dtype, int num_splits) {
    if (!decode_sizes_ok(B, H, G, D, kv_capacity) || !valid_dtype(kv_dtype)) return 0;
    if (num_splits < 0 || num_splits > kMaxSplitsAbi) return 0;
    return plan_decode(B, H, G, D, kv_capacity, kv_dtype, num_splits, auto_path(H, G, D, kv_dtype), GQA_LAYOUT_AUTO)
        .S;
}

size_t gqa_decode_workspace_size(int B, int H, int G, int D, int kv_capacity, int kv_dtype, int num_splits) {
    int S = gqa_decode_num_splits(B, H, G, D, kv_capacity, kv_dtype, num_splits);
    if (S == 0) return SIZE_MAX;
    // Enough for every kernel family and layout a caller may force as well.
    const int path = auto_path(H, G, D, kv_dtype);
    for (int layout : {GQA_LAYOUT_UNIFORM, GQA_LAYOUT_FLAT}) {
        const int s = plan_decode(B, H, G, D, kv_capacity, kv_dtype, num_splits, path, layout).S;
        if (s > S) S = s;
    }
    const int s_generic = plan_decode(B, H, G, D, kv_capacity, kv_dtype, num_splits, GQA_PATH_GENERIC,
                                      GQA_LAYOUT_UNIFORM).S;
    if (s_generic > S) S = s_generic;
    return workspace_bytes_for(B, H, G, D, S);
}

}  // extern "C"

namespace gqa {
namespace {

// Paged cache geometry (null for the contiguous cache).
struct PagedDesc {
    const int32_t *block_table;
    int page_size, pages_per_seq, num_pages;
};

// use_scratch: the allocation-free variant (split partials in the library's static device
// scratch; opts->workspace must be NULL).
gqa_status decode_impl(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, void *out,
                       int B, int H, int G, int D, float scale, hipStream_t stream, const gqa_opts *opts_in,
                       const PagedDesc *pg, bool use_scratch = false) {
    // ---- host-side validation (no HIP calls) ----
    if (!q || !k_cache || !v_cache || !seq_lens || !out || !opts_in) return GQA_ERR_INVALID_ARG;
    gqa_opts o;
    if (!read_opts(opts_in, &o)) return GQA_ERR_INVALID_ARG;
    int ps_log2 = 0;
    if (pg) {
        // Rows per page: a power of two from 16 (a 32-row block then spans at most three
        // pages) to 2^20; the capacity replaces opts->kv_capacity.
        if (!pg->block_table || pg->pages_per_seq < 1 || pg->num_pages < 1) return GQA_ERR_INVALID_ARG;
        if (pg->page_size < 16 || pg->page_size > (1 << 20) || (pg->page_size & (pg->page_size - 1)) != 0)
            return GQA_ERR_INVALID_ARG;
        while ((1 << ps_log2) < pg->page_size) ++ps_log2;
        if ((long)pg->pages_per_seq * pg->page_size > 0x7fffffffL) return GQA_ERR_INVALID_ARG;
        o.kv_capacity = pg->pages_per_seq * pg->page_size;
    }
    if (o.layout < GQA_LAYOUT_AUTO || o.layout > GQA_LAYOUT_FLAT) return GQA_ERR_INVALID_ARG;
    if (o.layout == GQA_LAYOUT_FLAT && o.num_splits > 0) return GQA_ERR_INVALID_ARG;
    if (!decode_sizes_ok(B, H, G, D, o.kv_capacity)) return GQA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
    if (o.num_splits < 0 || o.num_splits > kMaxSplitsAbi) return GQA_ERR_INVALID_ARG;
    if (o.path < GQA_PATH_AUTO || o.path > GQA_PATH_MFMA) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(o.q_dtype) || !valid_dtype(o.kv_dtype)) return GQA_ERR_INVALID_ARG;
    const bool pair_ok = (o.q_dtype == DT_F32 && o.kv_dtype == DT_F32) ||
                         (o.q_dtype == DT_BF16 && o.kv_dtype == DT_BF16) ||
                         (o.q_dtype == DT_BF16 && o.kv_dtype == DT_FP8) ||
                         (o.q_dtype == DT_BF16 && o.kv_dtype == DT_INT4);
    if (!pair_ok) return GQA_ERR_UNSUPPORTED;
    const bool scaled = o.kv_dtype == DT_FP8 || o.kv_dtype == DT_INT4;
    if (scaled && (!o.k_scale || !o.v_scale)) return GQA_ERR_INVALID_ARG;
    if (o.kv_dtype == DT_INT4 && D % 2 != 0) return GQA_ERR_UNSUPPORTED;  // whole bytes per row
    if ((o.k_new == nullptr) != (o.v_new == nullptr)) return GQA_ERR_INVALID_ARG;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k_cache; a.v = v_cache; a.out = out; a.seq_lens = seq_lens;
    a.k_scale = scaled ? o.k_scale : nullptr;
    a.v_scale = scaled ? o.v_scale : nullptr;
    a.B = B; a.H = H; a.G = G; a.D = D;
    a.Tq = 1; a.Tk = o.kv_capacity;
    a.causal = 0; a.decode = 1;
    a.scale_log2 = scale * kLog2e;
    a.q_dtype = o.q_dtype; a.kv_dtype = o.kv_dtype;
    if (pg) {
        a.block_table = pg->block_table;
        a.ps_log2 = ps_log2;
        a.pages_per_seq = pg->pages_per_seq;
        a.num_pages = pg->num_pages;
    }
    int path = o.path;
    if (path == GQA_PATH_AUTO) path = decode_mfma_supports(a) ? GQA_PATH_MFMA : GQA_PATH_GENERIC;
    if (pg && path != GQA_PATH_MFMA) return GQA_ERR_UNSUPPORTED;  // paged: matrix-core family only
    if (path == GQA_PATH_VALU && !decode_valu_supports(a)) return GQA_ERR_UNSUPPORTED;
    if (path == GQA_PATH_MFMA && !decode_mfma_supports(a)) return GQA_ERR_UNSUPPORTED;

    if (o.layout == GQA_LAYOUT_FLAT && !flat_possible(B, G, o.kv_capacity, D, o.kv_dtype, path, o.num_splits))
        return GQA_ERR_UNSUPPORTED;
    const DecodePlan plan = plan_decode(B, H, G, D, o.kv_capacity, o.kv_dtype, o.num_splits, path, o.layout);
    a.num_splits = plan.S;
    a.split_len = plan.split_len;
    a.flat = plan.flat;
    a.flat_nw = plan.nw;
    a.flat_cmin = plan.cmin;
    a.flat_pad = plan.pad;

    const size_t need = workspace_bytes_for(B, H, G, D, a.num_splits);
    if (need > 0 && o.workspace && o.workspace_bytes < need) return GQA_ERR_WORKSPACE;
    if (need > 0 && o.workspace && ((uintptr_t)o.workspace % 16) != 0) return GQA_ERR_INVALID_ARG;
    if (use_scratch) {
        if (o.workspace) return GQA_ERR_INVALID_ARG;
        const size_t part = need > 0 ? need - counter_bytes(B, G) : 0;
        if (need > 0 && ((long)B * G > kScratchCounters || part > kScratchPartialBytes)) return GQA_ERR_WORKSPACE;
    }

    // ---- device work ----
    gqa_status st = check_device();
    if (st != GQA_OK) return st;

    void *ws = o.workspace;
    bool owned = false;
    if (need > 0 && use_scratch) {
        char *base = nullptr;
        st = device_scratch(stream, &base);
        if (st != GQA_OK) return st;
        a.counters = reinterpret_cast<int *>(base);
        a.part_acc = reinterpret_cast<float *>(base + kScratchCounterBytes);
        a.part_ml = reinterpret_cast<float *>(base + kScratchCounterBytes + acc_bytes(B, H, D, a.num_splits));
        a.fuse_combine = plan.fuse;
    } else if (need > 0 && !ws) {
        // Stream-ordered memory of this call's own. Not while the stream is being captured into
        // a graph: the allocation and its release would become graph nodes.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return GQA_ERR_HIP;
        if (cap != hipStreamCaptureStatusNone) return GQA_ERR_WORKSPACE;
        if (hipMallocAsync(&ws, need, stream) != hipSuccess) return GQA_ERR_HIP;
        owned = true;
        // Fresh memory: the arrival counters must start at zero.
        if (launch_zero_ints(static_cast<int *>(ws), B * G, stream) != hipSuccess) {
            (void)hipFreeAsync(ws, stream);
            return GQA_ERR_HIP;
        }
    }
    if (need > 0 && !use_scratch) {
        char *base = static_cast<char *>(ws);
        a.counters = reinterpret_cast<int *>(base);
        a.part_acc = reinterpret_cast<float *>(base + counter_bytes(B, G));
        a.part_ml = reinterpret_cast<float *>(base + counter_bytes(B, G) + acc_bytes(B, H, D, a.num_splits));
        a.fuse_combine = plan.fuse;
    }

    hipError_t e = hipSuccess;
    if (o.k_new) {
        // The matrix-core kernel stores the new row itself, from the registers it attends with
        // (its 16-byte loads need 16-byte aligned rows); every other case copies it first.
        const bool fused = path == GQA_PATH_MFMA && o.kv_dtype != DT_INT4 && ((uintptr_t)o.k_new % 16) == 0 &&
                           ((uintptr_t)o.v_new % 16) == 0;
        a.k_new = o.k_new;
        a.v_new = o.v_new;
        if (!fused) {
            e = launch_kv_append(a, stream);
            a.k_new = a.v_new = nullptr;
        }
    }
    if (e == hipSuccess) {
        if (path == GQA_PATH_MFMA) e = launch_decode_mfma(a, stream);
        else if (path == GQA_PATH_VALU) e = launch_decode_valu(a, stream);
        else e = launch_generic(a, stream);
    }
    if (e == hipSuccess && a.num_splits > 1 && !a.fuse_combine) e = launch_combine(a, stream);
    if (owned) {
        const hipError_t f = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // namespace
// Chunk against a cache, contiguous (pg null) or paged.
gqa_status prefill_cached_impl(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                               void *out, int B, int Tq, int H, int G, int D, float scale, int causal,
                               hipStream_t stream, const gqa_opts *opts_in, const PagedDesc *pg) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out || !opts_in) return GQA_ERR_INVALID_ARG;
    gqa_opts o;
    if (!read_opts(opts_in, &o)) return GQA_ERR_INVALID_ARG;
    int ps_log2 = 0;
    if (pg) {
        // As for the paged decode; the capacity replaces opts->kv_capacity.
        if (!pg->block_table || pg->pages_per_seq < 1 || pg->num_pages < 1) return GQA_ERR_INVALID_ARG;
        if (pg->page_size < 16 || pg->page_size > (1 << 20) || (pg->page_size & (pg->page_size - 1)) != 0)
            return GQA_ERR_INVALID_ARG;
        while ((1 << ps_log2) < pg->page_size) ++ps_log2;
        if ((long)pg->pages_per_seq * pg->page_size > 0x7fffffffL) return GQA_ERR_INVALID_ARG;
        o.kv_capacity = pg->pages_per_seq * pg->page_size;
    }
    if (o.layout < GQA_LAYOUT_AUTO || o.layout > GQA_LAYOUT_FLAT) return GQA_ERR_INVALID_ARG;
    if (Tq < 1 || !decode_sizes_ok(B, H, G, D, o.kv_capacity)) return GQA_ERR_INVALID_ARG;
    if ((double)B * H * (double)Tq * D > 9.0e15 || (double)B * G * H * (double)Tq > 2.0e9) return GQA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
    if (o.path < GQA_PATH_AUTO || o.path > GQA_PATH_MFMA) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(o.q_dtype) || !valid_dtype(o.kv_dtype)) return GQA_ERR_INVALID_ARG;
    const bool pair_ok = (o.q_dtype == DT_F32 && o.kv_dtype == DT_F32) ||
                         (o.q_dtype == DT_BF16 && o.kv_dtype == DT_BF16) ||
                         (o.q_dtype == DT_BF16 && o.kv_dtype == DT_FP8);
    if (!pair_ok) return GQA_ERR_UNSUPPORTED;
    if (o.kv_dtype == DT_FP8 && (!o.k_scale || !o.v_scale)) return GQA_ERR_INVALID_ARG;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k_cache; a.v = v_cache; a.out = out; a.seq_lens = seq_lens;
    a.k_scale = o.kv_dtype == DT_FP8 ? o.k_scale : nullptr;
    a.v_scale = o.kv_dtype == DT_FP8 ? o.v_scale : nullptr;
    a.B = B; a.H = H; a.G = G; a.D = D;
    a.Tq = Tq; a.Tk = o.kv_capacity;
    a.causal = causal; a.decode = 0; a.cached = 1;
    a.num_splits = 1; a.split_len = o.kv_capacity;
    a.scale_log2 = scale * kLog2e;
    a.q_dtype = o.q_dtype; a.kv_dtype = o.kv_dtype;
    if (pg) {
        a.block_table = pg->block_table;
        a.ps_log2 = ps_log2;
        a.pages_per_seq = pg->pages_per_seq;
        a.num_pages = pg->num_pages;
    }

    int path = o.path;
    if (path == GQA_PATH_AUTO) path = prefill_mfma_supports(a) ? GQA_PATH_MFMA : GQA_PATH_GENERIC;
    if (path == GQA_PATH_VALU) return GQA_ERR_UNSUPPORTED;
    if (pg && path != GQA_PATH_MFMA) return GQA_ERR_UNSUPPORTED;  // paged: matrix-core family only
    if (path == GQA_PATH_MFMA && !prefill_mfma_supports(a)) return GQA_ERR_UNSUPPORTED;

    gqa_status st = check_device();
    if (st != GQA_OK) return st;
    const hipError_t e = path == GQA_PATH_MFMA ? launch_prefill_mfma(a, stream) : launch_generic(a, stream);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // namespace gqa

extern "C" {

gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                      void *out, int B, int H, int G, int D, float scale, hipStream_t stream,
                      const gqa_opts *opts) {
    return gqa::decode_impl(q, k_cache, v_cache, seq_lens, out, B, H, G, D, scale, stream, opts, nullptr);
}

gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                              void *out, int B, int H, int G, int D, float scale, hipStream_t stream,
                              const gqa_opts *opts) {
    return gqa::decode_impl(q, k_cache, v_cache, seq_lens, out, B, H, G, D, scale, stream, opts, nullptr, true);
}

gqa_status gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                            const int32_t *seq_lens, void *out, int B, int H, int G, int D, float scale,
                            int page_size, int pages_per_seq, int num_pages, hipStream_t stream,
                            const gqa_opts *opts) {
    const gqa::PagedDesc pg = {block_table, page_size, pages_per_seq, num_pages};
    return gqa::decode_impl(q, k_pages, v_pages, seq_lens, out, B, H, G, D, scale, stream, opts, &pg);
}

gqa_status gqa_prefill(const void *q, const void *k, const void *v, void *out, int B, int T, int H, int G,
                       int D, float scale, int causal, hipStream_t stream, const gqa_opts *opts_in) {
    if (!q || !k || !v || !out) return GQA_ERR_INVALID_ARG;
    gqa_opts o;
    if (!read_opts(opts_in, &o)) return GQA_ERR_INVALID_ARG;
    if (o.layout < GQA_LAYOUT_AUTO || o.layout > GQA_LAYOUT_FLAT) return GQA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || H < 1 || G < 1 || D < 1 || H % G != 0 || D > kMaxDim) return GQA_ERR_INVALID_ARG;
    if ((double)B * H * (double)T * D > 9.0e15 || (double)B * G * H * (double)T > 2.0e9)
        return GQA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return GQA_ERR_INVALID_ARG;
    if (o.path < GQA_PATH_AUTO || o.path > GQA_PATH_MFMA) return GQA_ERR_INVALID_ARG;
    if (!valid_dtype(o.q_dtype) || !valid_dtype(o.kv_dtype)) return GQA_ERR_INVALID_ARG;
    if (o.q_dtype != o.kv_dtype || o.q_dtype == DT_FP8 || o.q_dtype == DT_INT4) return GQA_ERR_UNSUPPORTED;

    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.B = B; a.H = H; a.G = G; a.D = D;
    a.Tq = T; a.Tk = T;
    a.causal = causal; a.decode = 0;
    a.num_splits = 1; a.split_len = T;
    a.scale_log2 = scale * kLog2e;
    a.q_dtype = o.q_dtype; a.kv_dtype = o.kv_dtype;

    int path = o.path;
    if (path == GQA_PATH_AUTO) path = prefill_mfma_supports(a) ? GQA_PATH_MFMA : GQA_PATH_GENERIC;
    if (path == GQA_PATH_VALU) return GQA_ERR_UNSUPPORTED;
    if (path == GQA_PATH_MFMA && !prefill_mfma_supports(a)) return GQA_ERR_UNSUPPORTED;

    gqa_status st = check_device();
    if (st != GQA_OK) return st;
    const hipError_t e = path == GQA_PATH_MFMA ? launch_prefill_mfma(a, stream) : launch_generic(a, stream);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status gqa_prefill_cached(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                              void *out, int B, int Tq, int H, int G, int D, float scale, int causal,
                              hipStream_t stream, const gqa_opts *opts_in) {
    return gqa::prefill_cached_impl(q, k_cache, v_cache, seq_lens, out, B, Tq, H, G, D, scale, causal, stream,
                                    opts_in, nullptr);
}

gqa_status gqa_prefill_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, void *out, int B, int Tq, int H, int G, int D, float scale,
                             int causal, int page_size, int pages_per_seq, int num_pages, hipStream_t stream,
                             const gqa_opts *opts) {
    const gqa::PagedDesc pg = {block_table, page_size, pages_per_seq, num_pages};
    return gqa::prefill_cached_impl(q, k_pages, v_pages, seq_lens, out, B, Tq, H, G, D, scale, causal, stream, opts,
                                    &pg);
}

}  // extern "C"
