// GQA decode on the matrix cores (bf16, fp8-E4M3FN or INT4 KV cache, D = 128, any R = H/G <= 64).
//
// Both contractions run as bf16 MFMA, even for narrow groups (R = 4), where most MFMA rows
// are padding: a decode step is latency-bound per wave, and the matrix cores finish a block
// in about a third of the instructions the vector ALUs need. Each KV row is read from HBM
// exactly once per (sequence, KV head) and multiplied against all R query heads of its group
// inside one MFMA -- the group sharing that defines GQA [GQA paper digest page (51969.com),
// section "Grouped-query attention (GQA)"; the KV head of query head h is h / (H/G), "LLM
// principles -- code implementation of multi-head attention (MQA and GQA)", section 5].
//
// Work: a workgroup (4 waves) attends to one key range of one (sequence b, KV head g). Each
// wave streams its own 32-token blocks of the range (blocks wave, wave+4, ...), keeping an
// independent online-softmax state; the four states are merged at the end, and a split
// range leaves (acc, max, sum) partials for the log-sum-exp merge (splitkv.h). Key ranges
// come from one of two layouts: uniform (grid = range x sequence x KV head) or flat (equal
// runs of the concatenated valid keys of all segments, splitkv.h).
//
// Per 32-token block, per wave:
//   S^T (32 tokens x 16 heads per head block) = K . Q^T          -- 16x16x32 bf16 MFMA
//        K rows are loaded whole (four bf16 or eight fp8 rows per wave instruction), written
//        to a wave-private LDS tile and read back in the MFMA A-operand layout (an INT4 row
//        is 64 bytes, one operand row: loaded straight into registers); rows are assigned to
//        MFMA rows so that afterwards each lane holds 8 consecutive tokens of one head,
//        which is exactly the B-operand layout of the next product.
//   online softmax in base 2 (scale * log2(e) * k_scale applied to the fp32 scores)
//   O^T (128 d x 16 heads) += V^T . P^T                          -- 16x16x32 bf16 MFMA
//        V rows are loaded coalesced (4 rows of 256 bytes per wave instruction), written to
//        a wave-private LDS tile, and read back transposed with ds_read_b64_tr_b16
//        (ds_read_b64_tr_b8 + exact fp8->bf16 widening for fp8; INT4 rows are widened to
//        bf16 on their way into the tile, and K fields straight into the operands).
// Tokens at or beyond the valid length are masked by index and their values zeroed: a wave's
// first block is requested before the length is known (rows clamped to the allocation), the
// later ones clamp their rows to the last row of the range.
// v_scale multiplies the output once, in the epilogue.
// With a cache append, the wave whose block holds the last valid row swaps the caller's new
// key/value (quantised for fp8) into its registers and stores that row: no separate pass.
#include "dtypes.h"
#include "gqa_internal.h"
#include "gqa_measure.h"
#include "mfma_util.h"
#include "splitkv.h"

namespace gqa {

// ---- Per-workgroup timeline (diagnostic build only) ----
// Built with GQA_TIMELINE (libgqa_timeline.so: build.py --timeline), thread 0 of every
// workgroup records the device's constant 100 MHz clock (s_memrealtime) at fixed points of
// the decode kernels into g_timeline[workgroup][slot]; in the library proper every stamp is
// empty. Slots: 0 entry; 1 length(s) and work layout known; for piece p < 3 of the workgroup,
// 2 + 6 p + {0 start, 1 first block done, 2 block loop done (both wave 0), 3 waves merged and
// partials issued, 4 arrival counted, 5 end}; 20 exit; 21 number of pieces (a count).
#ifdef GQA_TIMELINE
constexpr int kTlWorkgroups = 4096, kTlSlots = 32;
__device__ unsigned long long g_timeline[kTlWorkgroups * kTlSlots];
__device__ __forceinline__ void tl_put(int slot, unsigned long long v) {
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kTlWorkgroups && slot >= 0 && slot < kTlSlots)
        g_timeline[blockIdx.x * kTlSlots + slot] = v;
}
__device__ __forceinline__ void tl_stamp(int slot) { tl_put(slot, __builtin_amdgcn_s_memrealtime()); }
// Where the workgroup runs: the HW_ID register (CU, shader array and engine fields) in the low
// 32 bits, XCC_ID above.
__device__ __forceinline__ void tl_where() {
    tl_put(31, (unsigned long long)__builtin_amdgcn_s_getreg(0xF804) |
                   ((unsigned long long)__builtin_amdgcn_s_getreg(0xF814) << 32));
}
#else
__device__ __forceinline__ void tl_put(int, unsigned long long) {}
__device__ __forceinline__ void tl_stamp(int) {}
__device__ __forceinline__ void tl_where() {}
#endif

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockT = 32;  // tokens per wave iteration
constexpr int kD = 128;
constexpr int kDP = kD + 4;      // row stride of the wave-merge tile: rows of 16 heads on distinct LDS banks
constexpr int kLenCache = 256;  // flat layout: sequence lengths kept in LDS for batches up to this

// MFMA row m of token sub-block `blk` (0/1) holds token tau(blk, m) of the 32-token block,
// so that C row 4*(l/16)+i of both sub-blocks lands in lane l as tokens 8*(l/16) + 4*blk + i.
__device__ __forceinline__ int tau(int blk, int m) { return ((m >> 2) << 3) + (blk << 2) + (m & 3); }

// XOR swizzles of the 16-byte chunk position inside a V-tile row (bank-conflict avoidance
// for the transposed reads); bf16 rows have 16 chunks, fp8 rows 8.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 1) | (r & 8) | ((r >> 4) & 1); }
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
// K tiles: the matrix-operand reads take the 16 rows tau(blk, 0..15) of a sub-block at one
// chunk position; these XORs send them to 16 distinct 16-byte bank groups (bf16: 256-byte rows,
// rows bits 1:0 and 4:3; fp8: 128-byte rows, two per 256 bytes, row bits 1 and 4:3).
__device__ __forceinline__ int swzk16(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
__device__ __forceinline__ int swzk8(int r) { return ((r >> 1) & 1) | (((r >> 3) & 3) << 1); }

// KV cache formats of this kernel. INT4 rows are widened to bf16 on the fly (see i4x8_to_bf16x8).
enum : int { KV_BF16 = 0, KV_FP8 = 1, KV_I4 = 2 };

// Bytes of one cache row in HBM, and of one V-tile row in LDS (INT4 V is widened to bf16).
template <int KV> constexpr int kRowBytes = KV == KV_FP8 ? 128 : (KV == KV_I4 ? 64 : 256);
template <int KV> constexpr int kLdsRowBytes = KV == KV_FP8 ? 128 : 256;
// Bytes of one K-tile row in LDS (INT4 K goes from registers straight into the operands).
template <int KV> constexpr int kKRowBytes = KV == KV_I4 ? 0 : kRowBytes<KV>;
// LDS of a workgroup: the V and K tiles of its four waves, later reused by the wave merge.
template <int KV, int NHB> constexpr int kLdsBytes =
    kWaves * kBlockT * (kLdsRowBytes<KV> + kKRowBytes<KV>) > kWaves * 16 * NHB * kDP * 4
        ? kWaves * kBlockT * (kLdsRowBytes<KV> + kKRowBytes<KV>)
        : kWaves * 16 * NHB * kDP * 4;

// INT4 field u in a bf16 operand: bf16 bits 0x4300 | u are exactly 128 + u = 136 + code (bf16
// has unit spacing in [128, 256)). The constant 136 is taken out of the products afterwards:
// 136 * sum(q) from each score, 136 * sum(p) from each output.
constexpr float kI4Offset = 136.f;
constexpr float kRescaleSlack = 8.f;  // base-2 headroom of the lazy softmax reference

// Eight INT4 fields (byte i: field 2i low, 2i+1 high) -> eight bf16 values 136 + code, in
// nine instructions: the fields are masked out one per byte (even and odd fields), gathered
// into byte order by two byte permutes, and each output dword is one permute that puts the
// bf16 high byte 0x43 above two of them. (perm(s0, s1, sel): result byte k is byte sel_k of
// s0:s1, s1 being bytes 0-3.)
__device__ __forceinline__ i32x4_t i4x8_to_bf16x8(int w) {
    const uint32_t x = (uint32_t)w;
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;  // fields 2i, 2i+1
    const uint32_t f03 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // fields 0..3
    const uint32_t f47 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // fields 4..7
    const uint32_t c = 0x43434343u;
    i32x4_t r;
    r[0] = (int)__builtin_amdgcn_perm(c, f03, 0x04010400u);
    r[1] = (int)__builtin_amdgcn_perm(c, f03, 0x04030402u);
    r[2] = (int)__builtin_amdgcn_perm(c, f47, 0x04010400u);
    r[3] = (int)__builtin_amdgcn_perm(c, f47, 0x04030402u);
    return r;
}

template <int KV> struct Frag;
template <> struct Frag<KV_BF16> { i32x4_t k[8]; i32x4_t v[8]; };
template <> struct Frag<KV_FP8> { i32x4_t k[4]; i32x4_t v[4]; };
template <> struct Frag<KV_I4> { i32x4_t k[2]; i32x4_t v[2]; };

typedef const __attribute__((address_space(4))) int32_t cint32_t;

// Where the key/value rows of one (sequence, KV head) live. Contiguous: k, v point at row 0
// of the slab. Paged: k, v point at the page pools advanced to KV head g (a page holds the
// 2^ps_log2 rows of all G heads, page_bytes long) and bt at the sequence's block-table row,
// read through the scalar cache (the table is not written during a launch).
struct KvSrc {
    const char *k, *v;
    long page_bytes;
    cint32_t *bt;
    int ps_log2, n_bt, num_pages;
};

// Pool offsets of the (at most three) pages that rows t0 .. t0+31 fall in; pages have at
// least 16 rows. Table positions past the row and page ids outside the pool are clamped, so
// every address stays inside the allocations whatever the table holds.
struct PageOffs {
    long o0, o1, o2;  // separate fields: an array here was indexed through scratch memory
};

template <bool PAGED>
__device__ __forceinline__ PageOffs fetch_pages(const KvSrc &s, int t0) {
    PageOffs p = {};
    if constexpr (PAGED) {
        const int p0 = t0 >> s.ps_log2;
        auto off = [&](int k) { return (long)min(max(s.bt[min(p0 + k, s.n_bt - 1)], 0), s.num_pages - 1) * s.page_bytes; };
        p.o0 = off(0);
        p.o1 = off(1);
        p.o2 = off(2);
    }
    return p;
}

// Byte offset of row r (t0 <= r < t0 + 32) from k / v.
template <bool PAGED, int RB>
__device__ __forceinline__ long row_off(const KvSrc &s, PageOffs p, int t0, int r) {
    if constexpr (PAGED) {
        const int rel = (r >> s.ps_log2) - (t0 >> s.ps_log2);
        const long base = rel == 0 ? p.o0 : (rel == 1 ? p.o1 : p.o2);
        return base + (long)(r & ((1 << s.ps_log2) - 1)) * RB;
    } else {
        return (long)r * RB;
    }
}

// A call reads every KV row once and never again: nontemporal loads. (A plain streaming read
// of 2 GiB on gfx950 measured 5.0-6.3 TB/s with ordinary 16-byte loads, 7.0-7.1 TB/s with
// nontemporal ones.)
__device__ __forceinline__ i32x4_t ld_kv(const char *p) { return __builtin_nontemporal_load((const i32x4_t *)p); }

template <int KV, bool PAGED>
__device__ __forceinline__ void load_block(Frag<KV> &f, const KvSrc &src, PageOffs pg, int t0, int ke,
                                           int lane) {
    constexpr int RB = kRowBytes<KV>;
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
    if constexpr (I4) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            int row = t0 + tau(blk, lane & 15);
            row = row < ke ? row : ke - 1;
            // 32 INT4 fields per lane: head dims 32*(l/16) .. +31, eight per k-step (a 64-byte
            // row is one operand row: whole rows per instruction already).
            f.k[blk] = ld_kv(src.k + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane >> 4));
        }
    }
    // bf16 and fp8 K: whole rows per instruction, as V below (the matrix-operand layout would
    // read half of every 128-byte line per instruction, which streams measurably slower); the
    // block goes through an LDS tile and is read back in that layout.
    if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = t0 + 8 * i + (lane >> 3);
            row = row < ke ? row : ke - 1;
            f.k[i] = ld_kv(src.k + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane & 7));
        }
    } else if constexpr (!I4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int row = t0 + 4 * i + (lane >> 4);
            row = row < ke ? row : ke - 1;
            f.k[i] = ld_kv(src.k + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane & 15));
        }
    }
    if constexpr (I4) {
        // 16 rows of 64 bytes per wave instruction: lane l reads head dims 32*(l%4) .. +31.
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row = t0 + 16 * i + (lane >> 2);
            row = row < ke ? row : ke - 1;
            f.v[i] = ld_kv(src.v + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane & 3));
        }
    } else if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = t0 + 8 * i + (lane >> 3);
            row = row < ke ? row : ke - 1;
            f.v[i] = ld_kv(src.v + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane & 7));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int row = t0 + 4 * i + (lane >> 4);
            row = row < ke ? row : ke - 1;
            f.v[i] = ld_kv(src.v + row_off<PAGED, RB>(src, pg, t0, row) + 16 * (lane & 15));
        }
    }
}

// Q^T as the B operand: lane l holds Q[head 16*hb + l%16][dk .. dk+7] for k-step kk. Padded
// heads (index >= R) load head R-1 so that the loads stay unconditional; attend() zeroes them.
template <int NHB, int KV>
__device__ __forceinline__ void load_q(i32x4_t (&qT)[NHB][4], const uint16_t *qp, int R, int lane) {
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        const int h = hb * 16 + (lane & 15);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // k-step kk covers head dims dk(kk) .. +7 of this lane; fp8 pairs the steps so
            // that one 16-byte K load serves two of them, INT4 lets one serve all four (the
            // same order on both operands).
            const int dk = I4    ? 32 * (lane >> 4) + 8 * kk
                           : FP8 ? 64 * (kk >> 1) + 16 * (lane >> 4) + 8 * (kk & 1)
                                 : 32 * kk + 8 * (lane >> 4);
            qT[hb][kk] = *(const i32x4_t *)(qp + (long)(h < R ? h : R - 1) * kD + dk);
        }
    }
}

// Cache append inside the attention: the block starting at t0 holds row r, the last valid
// row, which the caller's current key and value (bf16, [B*G][128]) replace. The lanes whose
// registers hold a 16-byte chunk of row r -- every chunk sits in exactly one lane, in the K
// operand layout and in the V row layout alike -- put the new chunk (quantised for an fp8
// cache) in its place and store it to the cache, so the row is written once and attended to
// with exactly the bytes stored.
// The current token's key and value as append_row needs them, requested when the piece starts
// so that their round trip overlaps the block loop instead of delaying the last block: bf16,
// the lane's 16-byte chunk of each; fp8, the four values the lane quantises and their scale.
template <int KV> struct AppendIn;
template <> struct AppendIn<KV_BF16> { i32x4_t k, v; };
template <> struct AppendIn<KV_FP8> { i32x2_t w; float sc; };
template <> struct AppendIn<KV_I4> {};

template <int KV>
__device__ __forceinline__ void load_append(AppendIn<KV> &in, const AttnArgs &a, int bg, int lane) {
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new) + (long)bg * kD;
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new) + (long)bg * kD;
    if constexpr (KV == KV_FP8) {
        in.w = *(const i32x2_t *)((lane < 32 ? kn : vn) + 4 * (lane & 31));
        in.sc = lane < 32 ? a.k_scale[bg] : a.v_scale[bg];
    } else if constexpr (KV == KV_BF16) {
        const int d0 = 8 * (lane & 15);
        in.k = *(const i32x4_t *)(kn + d0);
        in.v = *(const i32x4_t *)(vn + d0);
    }
}

template <int KV, bool PAGED>
__device__ __forceinline__ void append_row(Frag<KV> &f, const AppendIn<KV> &in, const KvSrc &src, int t0, int r,
                                           int lane) {
    constexpr int RB = kRowBytes<KV>;
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
    const long ro = row_off<PAGED, RB>(src, fetch_pages<PAGED>(src, t0), t0, r);
    char *kr = const_cast<char *>(src.k) + ro;
    char *vr = const_cast<char *>(src.v) + ro;
    const int rb = r - t0;  // row in the block, 0..31
    // Registers are chosen by per-lane predicates over compile-time indices, so that the
    // fragment stays in registers.
    if constexpr (I4) {
        // INT4 caches are appended by the copy kernel before the attention, never here.
        (void)f; (void)in; (void)kr; (void)vr; (void)rb; (void)lane;
    } else if constexpr (FP8) {
        // The wave quantises the 256 new values once, four per lane (K dims 4l .. 4l+3 in lanes
        // 0-31, V dims in lanes 32-63), and each lane gathers the four words of its chunks.
        const i32x2_t w = in.w;
        const float sc = in.sc;
        const int word = (int)quant_e4m3fn_x4(__uint_as_float((uint32_t)w[0] << 16), __uint_as_float((uint32_t)w[0] & 0xffff0000u),
                                              __uint_as_float((uint32_t)w[1] << 16), __uint_as_float((uint32_t)w[1] & 0xffff0000u), sc);
        auto gather = [&](int l0) { return i32x4_t{__shfl(word, l0), __shfl(word, l0 + 1), __shfl(word, l0 + 2), __shfl(word, l0 + 3)}; };
        const i32x4_t kc = gather(4 * (lane & 7));       // K dims 16 (l%8) .. +15
        const i32x4_t vc = gather(32 + 4 * (lane & 7));  // V dims likewise
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (8 * i + (lane >> 3) == rb) {
                f.k[i] = kc;
                f.v[i] = vc;
                *(i32x4_t *)(kr + 16 * (lane & 7)) = kc;
                *(i32x4_t *)(vr + 16 * (lane & 7)) = vc;
            }
    } else {
        const int d0 = 8 * (lane & 15);
        const i32x4_t xk = in.k;
        const i32x4_t xv = in.v;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (4 * i + (lane >> 4) == rb) {
                f.k[i] = xk;
                f.v[i] = xv;
                *(i32x4_t *)(kr + 2 * d0) = xk;
                *(i32x4_t *)(vr + 2 * d0) = xv;
            }
    }
}

// Where one call of attend() leaves its result.
struct PieceOut {
    int slot;     // partial slot of this key range
    int n_slots;  // key ranges of this (sequence, KV head) that hold keys
    bool direct;  // the range covers the whole sequence: write the output itself
    bool append;  // the range ends at the sequence's last row, which the new token fills
    int seq = 0;  // its place among the workgroup's pieces (timeline build)
};

// The piece a workgroup of the flat layout takes up after the current one. Its query and this
// wave's first block of it are requested into the registers the current piece no longer needs
// (qT, nxt) as soon as the current piece's last block is in registers, before the merge of the
// waves.
struct NextPiece {
    KvSrc src;
    const uint16_t *q;  // its R query heads
    int kb, ke;         // its key rows
    bool valid;         // workgroup-uniform
};

// Attention of query heads head0 .. head0+R-1 over key rows kb .. ke-1 of one (sequence, KV
// head), by the whole workgroup: each wave streams blocks kb + 32 (wave + 4 i), then the four
// waves merge. The caller has requested q (qT) and this wave's first block (nxt) already.
// With np.valid, qT and nxt are refilled with the next piece's query and first block.
template <int NHB, int KV, bool PAGED>
__device__ __forceinline__ void attend(const AttnArgs &a, char *lds, float (*m_w)[16 * NHB], float (*l_w)[16 * NHB],
                                       int lane, int wave, long head0, int R, int bg, int kb, int ke, PieceOut po,
                                       i32x4_t (&qT)[NHB][4], Frag<KV> &nxt, const KvSrc &src, float c,
                                       float vscale, const NextPiece &np) {
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
    const int tls = 2 + 6 * (po.seq < 3 ? po.seq : 2);  // timeline slots of this piece
    tl_stamp(tls);
    constexpr int RBL = kLdsRowBytes<KV>;  // V-tile row bytes in LDS
    constexpr int VT = kBlockT * RBL;      // V tile bytes per wave
    constexpr int HP = 16 * NHB;           // heads padded to MFMA blocks
    const int S = a.num_splits;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
        if (hb * 16 + (lane & 15) >= R)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qT[hb][kk] = i32x4_t{0, 0, 0, 0};
    char *vt = lds + wave * VT;
    char *ktile = lds + kWaves * VT + wave * (kBlockT * kKRowBytes<KV>);
    // INT4: 136 * sum_d q[h][d] for the lane's head, to take out of every score.
    float qoff[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        qoff[hb] = 0.f;
        if constexpr (I4) {
            float sum = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = (uint32_t)qT[hb][kk][e];
                    sum += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
                }
            sum = sum_xor32(sum_xor16(sum));
            qoff[hb] = kI4Offset * sum;
        }
    }

    f32x4_t o[NHB][8];
    float m[NHB], lsum[NHB];
    float lb[NHB];  // INT4: running sum of the bf16-rounded probabilities the P.V product used
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        m[hb] = -INFINITY;
        lsum[hb] = 0.f;
        lb[hb] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[hb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    constexpr int kStep = kWaves * kBlockT;
    // Paged: pool offsets of the pages of the block to prefetch next (the wave's second block);
    // page ids are requested one block before the rows they locate.
    PageOffs pgn = fetch_pages<PAGED>(src, kb + wave * kBlockT + kStep);

    // One 32-token block: `slot` holds its K/V rows (requested earlier) and is refilled with
    // the block `dist` rows ahead (dist = 0: the wave's last block, nothing to refill).
    // tail: std::true_type for the wave's last block, the only one that can reach past the end
    // of the range; only there are rows masked by index.
    auto step = [&](Frag<KV> &slot, int t0, int dist, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        Frag<KV> cur = slot;
        // Rows at or past the end may hold anything, NaN included (a first block requested
        // before the length was known reads up to the allocation). Their scores are masked by
        // index below; zero their values so that the zero probabilities stay exact. (Every
        // INT4 field is finite: nothing to clear.)
        if (!I4 && TAIL && t0 + kBlockT > ke) {
            if constexpr (FP8) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t0 + 8 * i + (lane >> 3) >= ke) cur.v[i] = i32x4_t{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (t0 + 4 * i + (lane >> 4) >= ke) cur.v[i] = i32x4_t{0, 0, 0, 0};
            }
        }
        // V tile -> LDS (row-major, swizzled 16-byte chunks) first, so the V registers are
        // free again before the next block's loads are issued. INT4 rows are widened to the
        // bf16 tile layout on the way (four 8-dim chunks per lane).
        if constexpr (I4) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 16 * i + (lane >> 2);
#pragma unroll
                for (int mq = 0; mq < 4; ++mq)
                    *(i32x4_t *)(vt + r * RBL + 16 * ((4 * (lane & 3) + mq) ^ swz16(r))) = i4x8_to_bf16x8(cur.v[i][mq]);
            }
        } else if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 8 * i + (lane >> 3);
                *(i32x4_t *)(vt + r * RBL + 16 * ((lane & 7) ^ swz8(r))) = cur.v[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + (lane >> 4);
                *(i32x4_t *)(vt + r * RBL + 16 * ((lane & 15) ^ swz16(r))) = cur.v[i];
            }
        }
        // K tile -> LDS likewise (bf16, fp8), for the operand-layout reads below.
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 8 * i + (lane >> 3);
                *(i32x4_t *)(ktile + r * 128 + 16 * ((lane & 7) ^ swzk8(r))) = cur.k[i];
            }
        } else if constexpr (!I4) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + (lane >> 4);
                *(i32x4_t *)(ktile + r * 256 + 16 * ((lane & 15) ^ swzk16(r))) = cur.k[i];
            }
        }
        // Prefetch this slot's next block (dist rows ahead, always inside the range) before this
        // block's work; the barrier keeps the scheduler from sinking it next to its use --
        // otherwise every block waits out a full memory latency.
        if (dist > 0) {
            load_block<KV, PAGED>(slot, src, pgn, t0 + dist, ke, lane);
            if constexpr (PAGED) pgn = fetch_pages<PAGED>(src, t0 + 2 * dist);  // for the next prefetch
        }
        __builtin_amdgcn_sched_barrier(0);

        // S^T = K . Q^T for both 16-token sub-blocks and every head block.
        f32x4_t s[NHB][2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            // Lane l: row tau(blk, l%16) of the block, head dims of k-step kk as in load_q.
            i32x4_t ka[4];
            const int kr = tau(blk, lane & 15);
            if constexpr (I4) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) ka[kk] = i4x8_to_bf16x8(cur.k[blk][kk]);
            } else if constexpr (FP8) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const i32x4_t w = *(const i32x4_t *)(ktile + kr * 128 + 16 * ((4 * p + (lane >> 4)) ^ swzk8(kr)));
                    ka[2 * p] = e4m3x8_to_bf16x8(i32x2_t{w[0], w[1]});
                    ka[2 * p + 1] = e4m3x8_to_bf16x8(i32x2_t{w[2], w[3]});
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    ka[kk] = *(const i32x4_t *)(ktile + kr * 256 + 16 * ((4 * kk + (lane >> 4)) ^ swzk16(kr)));
            }
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma16x16x32(ka[kk], qT[hb][kk], acc);
                s[hb][blk] = acc;
            }
        }

        // Online softmax; lane l holds head l%16 of each head block and tokens
        // t0 + 8*(l/16) + 4*blk + i.
        const int tl = t0 + 8 * (lane >> 4);
        i32x4_t pb[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float x[8];
            float bm = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = tl + 4 * blk + i;
                    const float v = !TAIL || t < ke ? (s[hb][blk][i] - qoff[hb]) * c : -INFINITY;
                    x[blk * 4 + i] = v;
                    bm = fmaxf(bm, v);
                }
            bm = max_xor32(max_xor16(bm));
            // Running max, rescaled every block, on the wave's last block (a wave with a single
            // block pays no test); lazily before it: the reference m moves only when a head's
            // max outgrows it by more than kRescaleSlack, so p <= 2^kRescaleSlack and most
            // blocks skip the O rescale (the merge only needs m, l and O to agree).
            float alpha = 1.f;
            bool resc = TAIL;
            if constexpr (TAIL) {
                const float mn = fmaxf(m[hb], bm);
                alpha = fast_exp2(m[hb] - mn);
                m[hb] = mn;
            } else if (__any(bm > m[hb] + kRescaleSlack)) {
                const float mn = fmaxf(m[hb], bm);
                alpha = fast_exp2(m[hb] - mn);
                m[hb] = mn;
                resc = true;
            }
            const float mr = m[hb];
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = fast_exp2(x[e] - mr);
                ps += x[e];
            }
            lsum[hb] = lsum[hb] * alpha + ps;
            if (resc) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    o[hb][nb][0] *= alpha;
                    o[hb][nb][1] *= alpha;
                    o[hb][nb][2] *= alpha;
                    o[hb][nb][3] *= alpha;
                }
            }
            pb[hb][0] = pack_bf16_rne(x[0], x[1]);
            pb[hb][1] = pack_bf16_rne(x[2], x[3]);
            pb[hb][2] = pack_bf16_rne(x[4], x[5]);
            pb[hb][3] = pack_bf16_rne(x[6], x[7]);
            if constexpr (I4) {
                float sb = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    sb += __uint_as_float((uint32_t)pb[hb][w] << 16) + __uint_as_float((uint32_t)pb[hb][w] & 0xffff0000u);
                lb[hb] = lb[hb] * alpha + sb;
            }
        }

        // O^T += V^T . P^T, 16 head dims per MFMA.
        const int j = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            i32x4_t va;
            if constexpr (FP8) {
                const int r = 8 * grp + (j >> 1);
                const i32x2_t codes = lds_read_tr8(vt + r * RBL + 16 * (nb ^ swz8(r)) + 8 * (j & 1));
                va = e4m3x8_to_bf16x8(codes);
            } else {
                const int r0 = 8 * grp + (j >> 2);
                const int r1 = r0 + 4;
                const int cc = 2 * nb + ((j & 3) >> 1);
                const i32x2_t lo = lds_read_tr16(vt + r0 * RBL + 16 * (cc ^ swz16(r0)) + 8 * (j & 1));
                const i32x2_t hi = lds_read_tr16(vt + r1 * RBL + 16 * (cc ^ swz16(r1)) + 8 * (j & 1));
                va = i32x4_t{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) o[hb][nb] = mfma16x16x32(va, pb[hb], o[hb][nb]);
        }
        };
    AppendIn<KV> ain = {};
    if constexpr (KV != KV_I4 && NHB <= 2)  // (above 32 heads the registers are needed by the loop)
        if (po.append) load_append<KV>(ain, a, bg, lane);
    int t0 = kb + wave * kBlockT;
    if (t0 < ke) {
        // The wave's last block is peeled off the loop: it is the one that may hold the row
        // of a cache append, and code for that kept out of the loop costs it no registers.
        const int tlast = t0 + (ke - 1 - t0) / kStep * kStep;
        for (; t0 < tlast; t0 += kStep) {
            step(nxt, t0, kStep, std::false_type{});
            if (t0 == kb) tl_stamp(tls + 1);
        }
        if (po.append && tlast + kBlockT >= ke) {
            if constexpr (KV != KV_I4 && NHB > 2) load_append<KV>(ain, a, bg, lane);
            append_row<KV, PAGED>(nxt, ain, src, tlast, ke - 1, lane);
        }
        step(nxt, tlast, 0, std::true_type{});
        if (tlast == kb) tl_stamp(tls + 1);
    }
    if constexpr (I4) {
        // Take 136 * sum(p) out of every output: o held sum_t p_t (136 + code_t) v_scale-free.
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            lb[hb] = sum_xor32(sum_xor16(lb[hb]));
            const float corr = kI4Offset * lb[hb];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                o[hb][nb][0] -= corr;
                o[hb][nb][1] -= corr;
                o[hb][nb][2] -= corr;
                o[hb][nb][3] -= corr;
            }
        }
    }

    tl_stamp(tls + 2);
    // The next piece's query and first block are requested as soon as this piece's last block
    // is in registers, so that their round trip overlaps the merge of the waves, the partial
    // stores and the arrival. (Above 32 heads per KV head the caller loads them after the
    // return: the accumulators and the next block together would spill.)
    if constexpr (NHB <= 2) {
        if (np.valid) {
            load_q<NHB, KV>(qT, np.q, R, lane);
            const int t0n = np.kb + wave * kBlockT;
            if (t0n < np.ke) load_block<KV, PAGED>(nxt, np.src, fetch_pages<PAGED>(np.src, t0n), t0n, np.ke, lane);
        }
    }

    // ---- merge the four waves in one LDS round (fixed order: deterministic) ----
    // Each wave writes its accumulators, reference maximum and sum to its own slice as they
    // are; every thread then takes 4 consecutive head dims of one head and sums the four
    // slices, each rescaled to the workgroup maximum (one barrier fewer than rescaling before
    // the write).
    float *o_w = reinterpret_cast<float *>(lds);  // [kWaves][HP][kDP]
    __syncthreads();  // every wave is done with its V tile
    tl_stamp(22);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        lsum[hb] = sum_xor32(sum_xor16(lsum[hb]));
        const int h = hb * 16 + (lane & 15);
        if (h < R) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
                *(f32x4_t *)&o_w[(wave * HP + h) * kDP + 16 * nb + 4 * (lane >> 4)] = o[hb][nb];
            if (lane < 16) {
                m_w[wave][h] = m[hb];
                l_w[wave][h] = lsum[hb];
            }
        }
    }
    __syncthreads();
    tl_stamp(23);
    for (int cidx = threadIdx.x; cidx < R * (kD / 4); cidx += kThreads) {
        const int h = cidx / (kD / 4), d = 4 * (cidx % (kD / 4));
        // All twelve LDS reads of the item go out before any is used: one LDS round trip per
        // item (left to itself, the scheduler spaces them one round trip apart).
        float mw[kWaves], lw[kWaves];
        f32x4_t x[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = m_w[w][h];
            lw[w] = l_w[w][h];
            x[w] = *(const f32x4_t *)&o_w[(w * HP + h) * kDP + d];
        }
        __builtin_amdgcn_sched_barrier(0);
        float M = mw[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
        // A wave without rows of this piece holds m = -inf and zeros: weight 0.
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
            acc[0] += f * x[w][0];
            acc[1] += f * x[w][1];
            acc[2] += f * x[w][2];
            acc[3] += f * x[w][3];
            l += f * lw[w];
        }
        if (po.direct) {
            const float inv = vscale / l;
            uint16_t *out = static_cast<uint16_t *>(a.out) + (head0 + h) * kD + d;
            *(i32x2_t *)out = i32x2_t{pack_bf16_rne(acc[0] * inv, acc[1] * inv), pack_bf16_rne(acc[2] * inv, acc[3] * inv)};
        } else {
            const f32x4_t v = {acc[0] * vscale, acc[1] * vscale, acc[2] * vscale, acc[3] * vscale};
            if (a.fuse_combine)  // whole 16-byte chunks: every wave store writes full lines
                splitkv_store4c(splitkv_acc_rsrc(a, head0, R), (unsigned)(((h * S + po.slot) * kD + d) * 4), v);
            else  // read once, by the combine kernel: streamed past the caches (fp8 MQA decode -0.8 us)
                __builtin_nontemporal_store(v, (f32x4_t *)&a.part_acc[((head0 + h) * S + po.slot) * kD + d]);
            if (d == 0) splitkv_store_ml(&a.part_ml[((head0 + h) * S + po.slot) * 2], M, l, a.fuse_combine);
        }
    }
    tl_stamp(tls + 3);
    if (!po.direct && a.fuse_combine) {
        const bool last = splitkv_arrive(a.counters + bg, po.n_slots);
        tl_stamp(tls + 4);
        if (last) splitkv_merge_bf16<kThreads, kD>(a, head0, R, po.n_slots, static_cast<uint16_t *>(a.out));
    }
    tl_stamp(tls + 5);
}

// The rows of (sequence b, KV head g): a slab of the contiguous cache, or the page pools and
// the sequence's block-table row.
template <bool PAGED, int RB>
__device__ __forceinline__ KvSrc kv_src(const AttnArgs &a, int b, int g, int bg) {
    KvSrc s = {};
    if constexpr (PAGED) {
        const long ps_bytes = (long)RB << a.ps_log2;
        s.k = static_cast<const char *>(a.k) + g * ps_bytes;
        s.v = static_cast<const char *>(a.v) + g * ps_bytes;
        s.page_bytes = a.G * ps_bytes;
        s.bt = (cint32_t *)(a.block_table + (long)b * a.pages_per_seq);
        s.ps_log2 = a.ps_log2;
        s.n_bt = a.pages_per_seq;
        s.num_pages = a.num_pages;
    } else {
        s.k = static_cast<const char *>(a.k) + (long)bg * a.Tk * RB;
        s.v = static_cast<const char *>(a.v) + (long)bg * a.Tk * RB;
    }
    return s;
}

// Uniform layout: workgroup = (key range `split`, sequence b, KV head g), ranges of split_len
// keys. Split-major order: the blocks resident on one CU at once are far apart in the grid.
template <int NHB, int KV, bool PAGED>
// Two workgroups per CU for up to 32 heads per KV head (the register budget then keeps the
// accumulators in VGPRs without spilling): a wave's block is latency-bound, and a second
// workgroup hides it (measured: fp8 MQA decode, R = 32, -9 %; Llama-7B decode -2 %).
__global__ __launch_bounds__(kThreads, NHB <= 2 ? 2 : 1) void decode_mfma_kernel(AttnArgs a) {
    constexpr int RB = kRowBytes<KV>;
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
    constexpr int HP = 16 * NHB;
    constexpr int LDS_BYTES = kLdsBytes<KV, NHB>;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ float m_w[kWaves][HP], l_w[kWaves][HP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar
    const int S = a.num_splits;
    const int nbg = a.B * a.G;
    const int split = blockIdx.x / nbg;
    const int bg = blockIdx.x % nbg;
    const int G = a.G, H = a.H, R = H / G;
    const int b = bg / G, g = bg % G;
    const int kb = split * a.split_len;
    const long head0 = (long)b * H + (long)g * R;  // first query head row of this group
    tl_stamp(0);
    tl_where();

    // The query, the scales and this wave's first block do not depend on the length (the
    // block's rows are clamped to the allocation), so they are requested before it and share
    // its round trip.
    i32x4_t qT[NHB][4];
    load_q<NHB, KV>(qT, static_cast<const uint16_t *>(a.q) + head0 * kD, R, lane);
    const float kscale = FP8 || I4 ? a.k_scale[bg] : 1.f;
    const float vscale = FP8 || I4 ? a.v_scale[bg] : 1.f;
    const KvSrc src = kv_src<PAGED, RB>(a, b, g, bg);
    Frag<KV> nxt;
    if (kb + wave * kBlockT < a.Tk)
        load_block<KV, PAGED>(nxt, src, fetch_pages<PAGED>(src, kb + wave * kBlockT), kb + wave * kBlockT, a.Tk, lane);

    const int Lraw = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    const int L = clamp_len(Lraw, a.Tk);
    const int ke = kb + a.split_len < L ? kb + a.split_len : L;
    tl_stamp(1);

    if (kb >= ke) {  // nothing to attend to in this range
        // Fused merges count only non-empty ranges, so an empty one only has to produce the
        // zero row of an empty sequence.
        if (S == 1 || (a.fuse_combine && L == 0 && split == 0)) {
            uint16_t *out = static_cast<uint16_t *>(a.out);
            for (int e = threadIdx.x; e < R * kD; e += kThreads) out[head0 * kD + e] = 0;
        } else if (!a.fuse_combine) {
            for (int h = threadIdx.x; h < R; h += kThreads) {
                a.part_ml[((head0 + h) * S + split) * 2] = -INFINITY;
                a.part_ml[((head0 + h) * S + split) * 2 + 1] = 0.f;
            }
        }
        tl_stamp(20);
        tl_put(21, 0);
        return;
    }
    PieceOut po;
    po.slot = split;
    po.n_slots = active_splits(L, a.split_len, S);
    // With the in-kernel merge, a sequence whose keys all fall in this range needs no merge.
    po.direct = S == 1 || (a.fuse_combine && po.n_slots == 1);
    po.append = a.k_new && ke == L && Lraw == L;  // Lraw in 1..T_cap: the row exists
    const NextPiece none = {};
    attend<NHB, KV, PAGED>(a, lds, m_w, l_w, lane, wave, head0, R, bg, kb, ke, po, qT, nxt, src,
                            a.scale_log2 * kscale, vscale, none);
    tl_stamp(20);
    tl_put(21, 1);
}

// Flat layout (splitkv.h): workgroup w streams rows [w C, (w + 1) C) of the concatenated
// segments, piece by piece. Every workgroup gets the same number of rows, whatever the mix of
// sequence lengths.
template <int NHB, int KV, bool PAGED>
// Two workgroups per CU where the registers allow it without spills (R <= 16; R <= 32 for
// the 8- and 4-bit caches): ragged fp8 MQA batch (R = 32) -3 %.
__global__ __launch_bounds__(kThreads, NHB == 1 || (NHB == 2 && KV != KV_BF16) ? 2 : 1) void decode_mfma_flat_kernel(
    AttnArgs a) {
    constexpr int RB = kRowBytes<KV>;
    constexpr bool FP8 = KV == KV_FP8, I4 = KV == KV_I4;
    constexpr int HP = 16 * NHB;
    constexpr int LDS_BYTES = kLdsBytes<KV, NHB>;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ float m_w[kWaves][HP], l_w[kWaves][HP];
    __shared__ int lay_s[4];
    // Sequence lengths as stored (clamped where used), read once by the layout step (batches of
    // up to kLenCache sequences; larger ones read them from memory as they go).
    __shared__ int len_s[kLenCache];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar
    const int G = a.G, H = a.H, R = H / G, B = a.B;
    tl_stamp(0);
    tl_where();

    // Layout, once per workgroup: Ng, the chunk C, and the segment holding the first row. The
    // lengths are read from memory once (into LDS, for batches up to kLenCache; the search for
    // the first segment then runs on them there), which is the only round trip before this
    // workgroup's first K/V requests.
    if (wave == 0) {
        const bool cached = B <= kLenCache;
        int Ng = 0;
        for (int k0 = 0; k0 < B; k0 += 64) {
            const int bb = k0 + lane;
            const int raw = bb < B ? a.seq_lens[bb] : 0;
            const int t = clamp_len(raw, a.Tk);
            if (cached && bb < B) len_s[bb] = raw;
            Ng += wave_sum(flat_span(t, a.flat_pad));
        }
        const int C = flat_chunk(G * Ng, gridDim.x, a.flat_cmin);
        const int x0 = (int)blockIdx.x * C;
        int b0 = 0, p0 = 0, g0 = 0;
        if (x0 < G * Ng) {
            g0 = x0 / Ng;
            if (cached)
                flat_find([&](int bb) { return clamp_len(len_s[bb], a.Tk); }, B, a.flat_pad, x0 - g0 * Ng, lane, b0, p0);
            else
                flat_find([&](int bb) { return clamp_len(a.seq_lens[bb], a.Tk); }, B, a.flat_pad, x0 - g0 * Ng, lane,
                          b0, p0);
        }
        if (lane == 0) {
            lay_s[0] = Ng;
            lay_s[1] = C;
            lay_s[2] = g0 * B + b0;
            lay_s[3] = p0;
        }
    }
    __syncthreads();
    // Workgroup-uniform from here on: scalar registers, scalar branches.
    const int Ng = __builtin_amdgcn_readfirstlane(lay_s[0]);
    const int C = __builtin_amdgcn_readfirstlane(lay_s[1]);
    const int gb0 = __builtin_amdgcn_readfirstlane(lay_s[2]);
    int Pb = __builtin_amdgcn_readfirstlane(lay_s[3]);
    const int N = G * Ng;
    tl_stamp(1);

    if (blockIdx.x == 0 && a.fuse_combine) {
        // Sequences without keys belong to no piece: their output rows are zero. (From the
        // lengths in LDS where they are cached: no round trip before this workgroup's loads.)
        uint16_t *out = static_cast<uint16_t *>(a.out);
        for (int k0 = 0; k0 < B; k0 += 64) {
            const int bb = k0 + lane;
            const int t = bb < B ? clamp_len(B <= kLenCache ? len_s[bb] : a.seq_lens[bb], a.Tk) : 1;
            unsigned long long empty = __ballot(t == 0);
            while (empty) {
                const int be = k0 + __ffsll((long long)empty) - 1;
                empty &= empty - 1;
                for (int e = threadIdx.x; e < H * kD; e += kThreads) out[(long)be * H * kD + e] = 0;
            }
        }
    }
    const int xe = (int)blockIdx.x * C + C < N ? (int)blockIdx.x * C + C : N;
    int g = gb0 / B, b = gb0 % B;

    // The piece that holds row x (x < xe) of this workgroup's run: the walk over the segments
    // moves (b, g, Pb) forward past finished and empty segments. r0 is the segment's first valid
    // row; the piece covers its valid rows kb .. ke-1, none when the run ends in the segment's
    // pad rows (ke <= kb).
    struct Piece {
        int b, g, kb, ke, Tb, r0, Pb;
    };
    const int pad = a.flat_pad;
    auto piece_at = [&](int x) {
        for (;;) {
            const int Tb = clamp_len(__builtin_amdgcn_readfirstlane(B <= kLenCache ? len_s[b] : a.seq_lens[b]), a.Tk);
            const int s0 = g * Ng + Pb;  // first row of segment (b, g), pad rows included
            const int X = flat_span(Tb, pad);
            if (x < s0 + X) {
                const int r0 = s0 + pad;
                return Piece{b, g, x > r0 ? x - r0 : 0, (xe < s0 + X ? xe : s0 + X) - r0, Tb, r0, Pb};
            }
            Pb += X;  // segment done (or empty): next one
            if (++b == B) {
                b = 0;
                Pb = 0;
                ++g;
            }
        }
    };

    if ((int)blockIdx.x * C >= xe) {
        tl_stamp(20);
        tl_put(21, 0);
        return;
    }
    Piece cur = piece_at((int)blockIdx.x * C);
    if (cur.ke <= cur.kb) {  // the run holds pad rows only
        tl_stamp(20);
        tl_put(21, 0);
        return;
    }
    int npieces = 0;
    i32x4_t qT[NHB][4];
    Frag<KV> nxt;
    {
        load_q<NHB, KV>(qT, static_cast<const uint16_t *>(a.q) + ((long)cur.b * H + (long)cur.g * R) * kD, R, lane);
        const KvSrc src = kv_src<PAGED, RB>(a, cur.b, cur.g, cur.b * G + cur.g);
        const int t0 = cur.kb + wave * kBlockT;
        if (t0 < cur.ke) load_block<KV, PAGED>(nxt, src, fetch_pages<PAGED>(src, t0), t0, cur.ke, lane);
    }
    for (;;) {
        const int bg = cur.b * G + cur.g;
        const long head0 = (long)cur.b * H + (long)cur.g * R;
        PieceOut po;
        po.n_slots = flat_pieces(Ng, C, cur.Pb, cur.Tb, cur.g, pad);
        po.slot = (int)blockIdx.x - (int)((unsigned)cur.r0 / (unsigned)C);
        po.direct = po.n_slots == 1;
        // The length as stored (not clamped) decides whether row L-1 exists for an append.
        po.append = a.k_new && cur.ke == cur.Tb &&
                    __builtin_amdgcn_readfirstlane(B <= kLenCache ? len_s[cur.b] : a.seq_lens[cur.b]) == cur.Tb;
        po.seq = npieces++;
        const float kscale = FP8 || I4 ? a.k_scale[bg] : 1.f;
        const float vscale = FP8 || I4 ? a.v_scale[bg] : 1.f;
        const KvSrc src = kv_src<PAGED, RB>(a, cur.b, cur.g, bg);
        // The piece after this one, if the run goes on.
        NextPiece np = {};
        Piece following = cur;
        np.valid = cur.r0 + cur.ke < xe;
        if (np.valid) {
            following = piece_at(cur.r0 + cur.ke);
            np.valid = following.ke > following.kb;
        }
        if (np.valid) {
            np.src = kv_src<PAGED, RB>(a, following.b, following.g, following.b * G + following.g);
            np.q = static_cast<const uint16_t *>(a.q) + ((long)following.b * H + (long)following.g * R) * kD;
            np.kb = following.kb;
            np.ke = following.ke;
        }
        attend<NHB, KV, PAGED>(a, lds, m_w, l_w, lane, wave, head0, R, bg, cur.kb, cur.ke, po, qT, nxt, src,
                               a.scale_log2 * kscale, vscale, np);
        if (!np.valid) {
            tl_stamp(20);
            tl_put(21, (unsigned long long)npieces);
            break;
        }
        if constexpr (NHB > 2) {
            load_q<NHB, KV>(qT, np.q, R, lane);
            const int t0 = np.kb + wave * kBlockT;
            if (t0 < np.ke) load_block<KV, PAGED>(nxt, np.src, fetch_pages<PAGED>(np.src, t0), t0, np.ke, lane);
        }
        __syncthreads();  // the next piece reuses the LDS tiles
        cur = following;
    }
}

template <int NHB, int KV, bool PAGED>
hipError_t launch_nhb(const AttnArgs &a, hipStream_t stream) {
    if (a.flat) {
        hipLaunchKernelGGL((decode_mfma_flat_kernel<NHB, KV, PAGED>), dim3((unsigned)a.flat_nw), dim3(kThreads), 0,
                           stream, a);
    } else {
        dim3 grid((unsigned)(a.B * a.G * a.num_splits));
        hipLaunchKernelGGL((decode_mfma_kernel<NHB, KV, PAGED>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <int KV, bool PAGED>
hipError_t launch_kv(const AttnArgs &a, hipStream_t stream) {
    const int R = a.H / a.G;
    if (R <= 16) return launch_nhb<1, KV, PAGED>(a, stream);
    if (R <= 32) return launch_nhb<2, KV, PAGED>(a, stream);
    return launch_nhb<4, KV, PAGED>(a, stream);
}

}  // namespace

bool decode_mfma_supports(const AttnArgs &a) {
    return a.decode && a.D == kD && a.q_dtype == DT_BF16 &&
           (a.kv_dtype == DT_BF16 || a.kv_dtype == DT_FP8 || a.kv_dtype == DT_INT4) &&
           a.H / a.G <= 64;
}

hipError_t launch_decode_mfma(const AttnArgs &a, hipStream_t stream) {
    if (!decode_mfma_supports(a)) return hipErrorInvalidValue;
    if (a.block_table) {
        if (a.kv_dtype == DT_FP8) return launch_kv<KV_FP8, true>(a, stream);
        if (a.kv_dtype == DT_INT4) return launch_kv<KV_I4, true>(a, stream);
        return launch_kv<KV_BF16, true>(a, stream);
    }
    if (a.kv_dtype == DT_FP8) return launch_kv<KV_FP8, false>(a, stream);
    if (a.kv_dtype == DT_INT4) return launch_kv<KV_I4, false>(a, stream);
    return launch_kv<KV_BF16, false>(a, stream);
}

}  // namespace gqa

// Timeline access (gqa_measure.h): the library proper has no timeline and says so.
extern "C" gqa_status gqa_timeline_read(void *dst, size_t bytes) {
    if (!dst) return GQA_ERR_INVALID_ARG;
#ifdef GQA_TIMELINE
    const size_t all = sizeof(unsigned long long) * gqa::kTlWorkgroups * gqa::kTlSlots;
    return hipMemcpyFromSymbol(dst, HIP_SYMBOL(gqa::g_timeline), bytes < all ? bytes : all) == hipSuccess
               ? GQA_OK
               : GQA_ERR_HIP;
#else
    (void)bytes;
    return GQA_ERR_UNSUPPORTED;
#endif
}

extern "C" gqa_status gqa_timeline_clear(void) {
#ifdef GQA_TIMELINE
    static const unsigned long long zeros[gqa::kTlWorkgroups * gqa::kTlSlots] = {};
    return hipMemcpyToSymbol(HIP_SYMBOL(gqa::g_timeline), zeros, sizeof(zeros)) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
#else
    return GQA_ERR_UNSUPPORTED;
#endif
}
