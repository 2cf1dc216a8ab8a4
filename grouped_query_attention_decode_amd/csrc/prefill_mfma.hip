// GQA prefill on the matrix cores (bf16, D = 128, causal or not).
//
// Prefill is compute-bound [GQA paper digest page (51969.com), introduction and section
// "QA": the pre-fill stage is bound by compute, decode by loading the KV cache]. Grouping
// does not change the flops (every query head still scores every visible key) but lets one
// K/V tile serve all R = H/G query heads of its group [same page, section "Grouped-query
// attention (GQA)"; the KV head of query head h is h / R, "LLM principles -- code
// implementation of multi-head attention (MQA and GQA)", section 5]. Softmax of the scaled
// scores with the causal mask (key j visible to row i iff j <= i) follows the same page,
// section 3; it is evaluated online, tile by tile, in base 2.
//
// Work: one workgroup (4 waves, 128 query rows) per (sequence b, KV head g, position
// tile); two workgroups share a CU, so one's softmax overlaps the other's MFMAs. The 128
// rows are the R heads of group g times P = 128 / R consecutive positions, so each 64-key
// K/V tile staged in LDS is used by every head of the group. Each wave owns 32 rows (lane l
// and lane l+32 hold row l%32) and, per key tile:
//   S^T (64 keys x 32 rows) = K . Q^T          16 MFMA 32x32x16 bf16 (K rows read from LDS
//                                              in the A-operand layout; Q^T stays in registers)
//   online softmax, one row per lane: the row max is an in-lane max plus one shuffle
//   O^T (128 d x 32 rows) += V^T . P^T          16 MFMA 32x32x16 (V^T via ds_read_b64_tr_b16;
//                                              P^T comes straight from the S^T registers)
// The softmax keeps a per-row reference max and rescales O only when a row's running max
// exceeds it by more than 8 (base 2), so every probability stays below 2^8 and most tiles
// skip the rescale; the result is the same softmax, since the reference cancels in O / l.
// K/V tiles are loaded with direct global->LDS 16-byte loads into two ping-pong buffers, so
// the next tile streams in while the current one is multiplied. Causal tiles entirely above
// the diagonal are skipped; position tiles are issued heaviest first, and all blocks of one
// (b, g) land on one XCD (block i runs on XCD i mod 8), so its K/V stays in that L2.
// Chunk against a cache (CACHED): the T queries are the last T of the sequence's L_b
// positions, so query i sits at position L_b - T + i; keys come from the cache [B,G,T_cap,D]
// and stop at L_b; the causal diagonal moves by L_b - T ("LLM principles -- code ...",
// sections 3 and 5: keys concatenated to the cache, later keys masked).
#include "dtypes.h"
#include "gqa_internal.h"
#include "mfma_util.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;             // keys per tile
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB
constexpr float kRescaleSlack = 8.f;         // base-2 headroom before O is rescaled

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ f32x16_t mfma32x32x16(const i32x4_t &a, const i32x4_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// S^T row m of a 32-key half holds key tau(m): C row 8i + 4h + j (lane half h) then covers
// keys 16(i/2) + 8h + 4(i%2) + j, i.e. lane half h holds 8 consecutive keys per 16-key step,
// the B-operand layout of the P.V product.
__device__ __forceinline__ int tau(int m) {
    const int i = m >> 3, h = (m >> 2) & 1, j = m & 3;
    return ((i >> 1) << 4) + (h << 3) + ((i & 1) << 2) + j;
}

// XOR swizzle of the 16-byte chunk position inside a 256-byte K/V tile row. Measured on
// gfx950 (SQ_LDS_BANK_CONFLICT) to be conflict-free for both read patterns below: the
// ds_read_b128 K-operand reads and the ds_read_b64_tr_b16 V-operand reads.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Direct buffer -> LDS load of one 64-key tile of K or V (16 KB); each of the 4 waves moves
// 4 KB (four 1 KB instructions). Lane l of instruction n fills LDS slot 64n + l: tile row
// r = 4n + l/16, position p = l%16, which holds chunk p ^ swz(r) of key row k0 + r. The
// buffer resource (built with scalar instructions) starts at row k0 and covers only the rows
// below L, so rows past the end read as zeros: their scores are masked and their zero values
// add nothing. The per-lane byte offsets are the same for every tile (TileOffs), so a tile
// load costs no vector arithmetic.
struct TileOffs {
    int o0, o1, o2, o3;
};
__device__ __forceinline__ TileOffs tile_offsets(int wave, int lane) {
    int o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 4 * (wave * 4 + q) + (lane >> 4);
        o[q] = r * kRowBytes + 16 * ((lane & 15) ^ swz(r));
    }
    return TileOffs{o[0], o[1], o[2], o[3]};
}
__device__ __forceinline__ void load_tile(char *lds_tile, const char *src, int k0, int L, int wave, TileOffs t) {
    const int rows = L - k0;
    const int bytes = rows <= 0 ? 0 : (rows < kBN ? rows : kBN) * kRowBytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(src + (long)k0 * kRowBytes), 0, bytes, 0x00020000);
    char *const dst = lds_tile + wave * 4 * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQA_LDS(void, dst), 16, t.o0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQA_LDS(void, dst + 1024), 16, t.o1, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQA_LDS(void, dst + 2048), 16, t.o2, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GQA_LDS(void, dst + 3072), 16, t.o3, 0, 0, 0);
}

// fp8 (E4M3FN) cache rows: 128 bytes. A wave fetches 16 of a tile's 64 rows into registers --
// lane l, i = 0, 1: row 16 w + 8 i + l/8, 16-byte chunk l % 8 (dims 16 (l % 8) .. +15) --
// through a buffer resource that covers only the rows below L (rows past it read as zeros),
// and later widens them (exactly) into the bf16 tile layout above, so the products are the
// same as for a bf16 cache and the conversion happens once per tile, not once per wave.
constexpr int kRowBytesF8 = kD;
__device__ __forceinline__ void fetch_tile_f8(i32x4_t (&f)[2], const char *src, int k0, int L, int wave, int lane) {
    const int rows = L - k0;
    const int bytes = rows <= 0 ? 0 : (rows < kBN ? rows : kBN) * kRowBytesF8;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(src + (long)k0 * kRowBytesF8), 0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * wave + 8 * i + (lane >> 3);
        f[i] = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, r * kRowBytesF8 + 16 * (lane & 7), 0, 0));
    }
}
// Paged cache (pools [num_pages, G, page_size, D], one block-table row per sequence, read
// through the scalar cache): a wave's 16 rows of a tile start at a multiple of 16 and pages
// hold >= 16 rows, so they lie in one page -- one table read per wave and tile serves its K
// and V loads; each load instruction (4 bf16 or 8 fp8 rows) gets a buffer resource covering
// its valid rows. Table entries and page ids are clamped into range (memory-safe).
typedef const __attribute__((address_space(4))) int32_t cint32_t;
struct PageGeo {
    const char *k, *v;  // pools advanced to KV head g
    long page_bytes;    // one page of all G heads
    cint32_t *bt;       // block-table row of the sequence
    int ps_log2, n_bt, num_pages;
};
// Byte offset, inside the pools, of key row `row` (the page of `row` looked up once).
__device__ __forceinline__ long page_row_base(const PageGeo &pg, int row, int rb) {
    int pi = row >> pg.ps_log2;
    pi = pi < 0 ? 0 : (pi >= pg.n_bt ? pg.n_bt - 1 : pi);
    int page = __builtin_amdgcn_readfirstlane(pg.bt[pi]);
    page = page < 0 ? 0 : (page >= pg.num_pages ? pg.num_pages - 1 : page);
    return page * pg.page_bytes + (long)(row & ((1 << pg.ps_log2) - 1)) * rb;
}
template <int RB, int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char *base, int row0, int L) {
    const int rows = L - row0;
    const int bytes = rows <= 0 ? 0 : (rows < ROWS ? rows : ROWS) * RB;
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, 0x00020000);
}
__device__ __forceinline__ void load_tile_paged(char *lds_tile, const char *pool, long wbase, int k0, int L, int wave,
                                                TileOffs t) {
    char *const dst = lds_tile + wave * 4 * 1024;
    const int r0 = k0 + 16 * wave;        // the wave's first key row; wbase: its offset in the pool
    const char *src = pool + wbase;
    const int n0 = wave * 16 * kRowBytes;  // tile offsets -> offsets from each instruction's first row
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc<kRowBytes, 4>(src, r0, L), GQA_LDS(void, dst), 16, t.o0 - n0,
                                             0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc<kRowBytes, 4>(src + 4 * kRowBytes, r0 + 4, L),
                                             GQA_LDS(void, dst + 1024), 16, t.o1 - n0 - 4 * kRowBytes, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc<kRowBytes, 4>(src + 8 * kRowBytes, r0 + 8, L),
                                             GQA_LDS(void, dst + 2048), 16, t.o2 - n0 - 8 * kRowBytes, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc<kRowBytes, 4>(src + 12 * kRowBytes, r0 + 12, L),
                                             GQA_LDS(void, dst + 3072), 16, t.o3 - n0 - 12 * kRowBytes, 0, 0, 0);
}
__device__ __forceinline__ void fetch_tile_f8_paged(i32x4_t (&f)[2], const char *pool, long wbase, int k0, int L,
                                                    int wave, int lane) {
    const int r0 = k0 + 16 * wave;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const __amdgpu_buffer_rsrc_t rs = rows_rsrc<kRowBytesF8, 8>(pool + wbase + 8 * i * kRowBytesF8, r0 + 8 * i, L);
        f[i] = __builtin_bit_cast(i32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(rs, (lane >> 3) * kRowBytesF8 + 16 * (lane & 7), 0, 0));
    }
}

__device__ __forceinline__ void stage_tile_f8(char *lds_tile, const i32x4_t (&f)[2], int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * wave + 8 * i + (lane >> 3), c = lane & 7;
        char *row = lds_tile + r * kRowBytes;
        *(i32x4_t *)(row + 16 * ((2 * c) ^ swz(r))) = e4m3x8_to_bf16x8(i32x2_t{f[i][0], f[i][1]});
        *(i32x4_t *)(row + 16 * ((2 * c + 1) ^ swz(r))) = e4m3x8_to_bf16x8(i32x2_t{f[i][2], f[i][3]});
    }
}

// R: query heads per KV head, a power of two; 0 = any R <= 64, read at run time (the
// workgroup then holds floor(128 / R) positions of each head and its last 128 mod R rows idle).
// F8: the cache holds E4M3FN codes with one k and one v scale per (sequence, KV head) (chunk
// against a cache only): k_scale joins the score scale, v_scale the final division.
// PG: the cache lives in pages (chunk against a cache only).
template <int R, bool CAUSAL, bool CACHED, bool F8 = false, bool PG = false>
__global__ __launch_bounds__(kThreads, 2) void prefill_mfma_kernel(AttnArgs a) {
    const int Rr = R > 0 ? R : a.H / a.G;
    const int P = kRows / Rr;  // positions per workgroup
    __shared__ __attribute__((aligned(16))) char k_lds0[kTileBytes];
    __shared__ __attribute__((aligned(16))) char v_lds0[kTileBytes];
    __shared__ __attribute__((aligned(16))) char k_lds1[kTileBytes];
    __shared__ __attribute__((aligned(16))) char v_lds1[kTileBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int T = a.Tq;
    const int G = a.G, H = a.H;
    const int nbg = a.B * G;
    const int npt = (T + P - 1) / P;
    const int bg = blockIdx.x % nbg;
    const int pt = CAUSAL ? npt - 1 - (int)(blockIdx.x / nbg) : (int)(blockIdx.x / nbg);
    const int b = bg / G, g = bg % G;
    const int p0 = pt * P;
    // Keys of this sequence, and the position of query row 0: a chunk against a cache holds
    // the last T of Lb positions; a plain prefill is Lb = T, offset 0.
    const int Tk = CACHED ? a.Tk : T;
    int Lb = T;
    if constexpr (CACHED) {
        const int l = a.seq_lens[b];
        Lb = __builtin_amdgcn_readfirstlane(l < 0 ? 0 : (l > Tk ? Tk : l));
    }
    const int off = Lb - T;

    // This lane's query row.
    const int wr = 32 * wave + (lane & 31);  // row inside the workgroup
    const int hq = wr / P;  // head of the group (Rr: an idle row, loads clamped into the group)
    const int head = g * Rr + (hq < Rr ? hq : Rr - 1);
    const int pos = p0 + wr % P;
    const bool row_ok = hq < Rr && pos < T;
    const long qrow = ((long)b * H + head) * T + (row_ok ? pos : T - 1);

    // Base-2 score scale; a negative scale is folded into Q so that c > 0 and the row max
    // can be taken on the raw scores.
    float c = a.scale_log2;
    float vscale = 1.f;
    if constexpr (F8) {
        c *= a.k_scale[bg];
        vscale = a.v_scale[bg];
    }
    const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
    c = fmaxf(fabsf(c), 1e-30f);  // a zero scale stays (numerically) uniform, without 0 * -inf

    // Q^T as the B operand: lane l holds Q[row][16*ks + 8*(l/32) .. +7], ks = 0..7.
    i32x4_t qT[8];
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + qrow * kD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        qT[ks] = *(const i32x4_t *)(qp + 16 * ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) qT[ks][e] ^= qsign;
    }

    constexpr int kRowBytesG = F8 ? kRowBytesF8 : kRowBytes;  // cache row bytes in memory
    const char *kbase = static_cast<const char *>(a.k) + (long)bg * Tk * kRowBytesG;
    const char *vbase = static_cast<const char *>(a.v) + (long)bg * Tk * kRowBytesG;
    PageGeo pgeo = {};
    if constexpr (PG) {
        const long ps_bytes = (long)kRowBytesG << a.ps_log2;
        pgeo.k = static_cast<const char *>(a.k) + g * ps_bytes;
        pgeo.v = static_cast<const char *>(a.v) + g * ps_bytes;
        pgeo.page_bytes = G * ps_bytes;
        pgeo.bt = (cint32_t *)(a.block_table + (long)b * a.pages_per_seq);
        pgeo.ps_log2 = a.ps_log2;
        pgeo.n_bt = a.pages_per_seq;
        pgeo.num_pages = a.num_pages;
    }
    // Fetch / load the K and V tile starting at key k0 (contiguous or paged).
    auto fetch_f8 = [&](i32x4_t (&kf)[2], i32x4_t (&vf)[2], int k0) __attribute__((always_inline)) {
        if constexpr (PG) {
            const long wb = page_row_base(pgeo, k0 + 16 * wave, kRowBytesF8);
            fetch_tile_f8_paged(kf, pgeo.k, wb, k0, Lb, wave, lane);
            fetch_tile_f8_paged(vf, pgeo.v, wb, k0, Lb, wave, lane);
        } else {
            fetch_tile_f8(kf, kbase, k0, Lb, wave, lane);
            fetch_tile_f8(vf, vbase, k0, Lb, wave, lane);
        }
    };

    // Keys this workgroup needs (absolute positions), and the smallest position of this wave.
    const int wg_last = off + (p0 + P - 1 < T - 1 ? p0 + P - 1 : T - 1);
    const int nkt = CAUSAL ? (wg_last < 0 ? 0 : wg_last / kBN + 1) : (Lb + kBN - 1) / kBN;
    // The wave's 32 rows start at position (32 w) mod P and wrap to 0 if they cross a head.
    const int wm0 = (32 * wave) % P;
    const int wave_min_pos = off + p0 + (wm0 + 31 < P ? wm0 : 0);
    const TileOffs toffs = tile_offsets(wave, lane);

    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    float mref = -INFINITY, lsum = 0.f;

    // Per-lane constant parts of the LDS addresses. K operand, key half kh: row r and chunk
    // (2 ks + hl) ^ swz(r); since 2 ks + hl = 2 ks ^ hl, the byte offset is
    // kofs[kh] ^ 32 ks with kofs[kh] = 256 r + 16 (hl ^ swz(r)).
    const int hl = lane >> 5;
    int kofs[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        const int r = 32 * kh + tau(lane & 31);
        kofs[kh] = r * kRowBytes + 16 * (hl ^ swz(r));
    }
    // V operand: rows 16 kk + vrow0 (+4 for the upper half) have the swizzle of vrow0 (+4), so
    // the offset is 4096 kk (an immediate) plus one of eight per-lane constants.
    const int gq = lane >> 4, jj = lane & 15;
    const int vrow0 = 8 * (gq >> 1) + (jj >> 2);
    const int vcol = 16 * (gq & 1) + 4 * (jj & 3);                  // + 32 db
    const int voff = (vcol & 7) * 2;
    int vofs[2][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int chn = (32 * db + vcol) >> 3;
        vofs[0][db] = vrow0 * kRowBytes + voff + 16 * (chn ^ swz(vrow0));
        vofs[1][db] = (vrow0 + 4) * kRowBytes + voff + 16 * (chn ^ swz(vrow0 + 4));
    }

    // stage(): work issued inside the P.V block (the fp8 cache's widening of the next tile).
    auto compute_tile = [&](const char *kt, const char *vt, int k0, bool need_mask, auto stage) {
        // ---- S^T = K . Q^T; the two 32-key halves accumulate independently, so
        // consecutive MFMAs never wait on each other ----
        f32x16_t s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[kh][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const i32x4_t ka = *(const i32x4_t *)(kt + (kofs[kh] ^ (32 * ks)));
                s[kh] = mfma32x32x16(ka, qT[ks], s[kh]);
            }
        // K-operand reads lead their MFMAs by two k-steps, so their LDS latency overlaps
        // MFMAs instead of stalling each pair (measured +2-3 % on the causal 2048 prefill).
        __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);  // LDS reads
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
        // ---- mask (diagonal / tail tiles only) and tile max on the raw scores ----
        if (need_mask) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = e >> 2, j = e & 3;
                    const int key = k0 + 32 * kh + 16 * (i >> 1) + 8 * hl + 4 * (i & 1) + j;
                    const bool vis = key < Lb && (!CAUSAL || key <= off + pos);
                    s[kh][e] = vis ? s[kh][e] : -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[kh][e]);
        tmax = max_xor32(tmax) * c;
        // ---- lazy rescale: move the reference only when the max outgrows it by > 2^8 ----
        if (__any(tmax > mref + kRescaleSlack)) {
            const float mn = fmaxf(mref, tmax);
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(mref - mn);
            mref = mn;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        }
        const float nref = mref == -INFINITY ? 0.f : -mref;
        float ps = 0.f;
        i32x4_t pb[4];  // P^T operands for the four 16-key steps
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = fast_exp2(fmaf(s[kh][8 * half + e], c, nref));
                    ps += p[e];
                }
                pb[2 * kh + half] = i32x4_t{pack_bf16_rne(p[0], p[1]), pack_bf16_rne(p[2], p[3]),
                                            pack_bf16_rne(p[4], p[5]), pack_bf16_rne(p[6], p[7])};
            }
        lsum += ps;
        // ---- O^T += V^T . P^T ----
        // Raised wave priority for this block: while one wave of a SIMD issues its P.V
        // products, the other wave's softmax fills the issue slots around them instead of
        // delaying them (measured +2.5-3 % on non-causal and chunked prefill, neutral causal).
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        stage();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const char *vk = vt + 16 * kk * kRowBytes;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const i32x2_t lo = lds_read_tr16(vk + vofs[0][db]);
                const i32x2_t hi = lds_read_tr16(vk + vofs[1][db]);
                o[db] = mfma32x32x16(i32x4_t{lo[0], lo[1], hi[0], hi[1]}, pb[kk], o[db]);
            }
        }
        // V-operand reads lead their MFMAs by four products (eight transposed reads first, then
        // one product per two reads), so their LDS latency overlaps products as for K
        // (measured: fp8-cache chunked prefill 134.2 -> 130.0 us, bf16 chunk and causal -0.5 %).
        __builtin_amdgcn_sched_group_barrier(0x0100, 8, 0);  // LDS reads
#pragma unroll
        for (int r = 0; r < 12; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
            if constexpr (F8) {
                __builtin_amdgcn_sched_group_barrier(0x0002, 3, 0);  // VALU (the staging)
                __builtin_amdgcn_sched_group_barrier(0x0200, 1, 0);  // LDS writes
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };

    auto load_kv = [&](char *kl, char *vl, int k0) __attribute__((always_inline)) {
        if constexpr (PG) {
            const long wb = page_row_base(pgeo, k0 + 16 * wave, kRowBytes);
            load_tile_paged(kl, pgeo.k, wb, k0, Lb, wave, toffs);
            load_tile_paged(vl, pgeo.v, wb, k0, Lb, wave, toffs);
        } else {
            load_tile(kl, kbase, k0, Lb, wave, toffs);
            load_tile(vl, vbase, k0, Lb, wave, toffs);
        }
    };

    auto tile_needs_mask = [&](int k0) {
        return (CAUSAL && k0 + kBN - 1 > wave_min_pos) || (k0 + kBN > Lb);
    };

    if constexpr (F8) {
        // Tile t+1 is fetched into registers before tile t is multiplied, then widened into
        // the other buffer (free: every wave passed the barrier after the tile that used it).
        i32x4_t kf[2], vf[2];
        fetch_f8(kf, vf, 0);
        wait_vmem_all();
        stage_tile_f8(k_lds0, kf, wave, lane);
        stage_tile_f8(v_lds0, vf, wave, lane);
        __syncthreads();
        // The widening of the next tile runs inside the current tile's P.V block, between its
        // products, so its vector work fills their shadow (132.6 -> 125.7 us on the fp8-cache
        // chunked prefill). With no next tile it re-widens the last fetch into the buffer that
        // no wave reads again.
        for (int kt = 0; kt < nkt; kt += 2) {
            if (kt + 1 < nkt) {
                fetch_f8(kf, vf, (kt + 1) * kBN);
            }
            compute_tile(k_lds0, v_lds0, kt * kBN, tile_needs_mask(kt * kBN), [&] {
                stage_tile_f8(k_lds1, kf, wave, lane);
                stage_tile_f8(v_lds1, vf, wave, lane);
            });
            if (kt + 1 >= nkt) break;
            __syncthreads();
            if (kt + 2 < nkt) {
                fetch_f8(kf, vf, (kt + 2) * kBN);
            }
            compute_tile(k_lds1, v_lds1, (kt + 1) * kBN, tile_needs_mask((kt + 1) * kBN), [&] {
                stage_tile_f8(k_lds0, kf, wave, lane);
                stage_tile_f8(v_lds0, vf, wave, lane);
            });
            if (kt + 2 >= nkt) break;
            __syncthreads();
        }
    } else {
    load_kv(k_lds0, v_lds0, 0);
    wait_vmem_all();
    __syncthreads();
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) {
            load_kv(k_lds1, v_lds1, (kt + 1) * kBN);
        }
        compute_tile(k_lds0, v_lds0, kt * kBN, tile_needs_mask(kt * kBN), [] {});
        wait_vmem_all();
        __syncthreads();
        if (kt + 1 >= nkt) break;
        if (kt + 2 < nkt) {
            load_kv(k_lds0, v_lds0, (kt + 2) * kBN);
        }
        compute_tile(k_lds1, v_lds1, (kt + 1) * kBN, tile_needs_mask((kt + 1) * kBN), [] {});
        wait_vmem_all();
        __syncthreads();
    }
    }

    // ---- epilogue: out[row][d] = O^T[d][row] / l ----
    lsum = sum_xor32(lsum);
    if (row_ok) {
        const float inv = lsum > 0.f ? vscale / lsum : 0.f;
        uint16_t *op = static_cast<uint16_t *>(a.out) + qrow * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 32 * db + 8 * i + 4 * hl;
                i32x2_t w;
                w[0] = pack_bf16_rne(o[db][4 * i] * inv, o[db][4 * i + 1] * inv);
                w[1] = pack_bf16_rne(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv);
                *(i32x2_t *)(op + d) = w;
            }
    }
}

template <int R>
hipError_t launch_r(const AttnArgs &a, hipStream_t stream) {
    const int P = kRows / (R > 0 ? R : a.H / a.G);
    const int npt = (a.Tq + P - 1) / P;
    dim3 grid((unsigned)(a.B * a.G * npt));
#define GQA_PREFILL(C, K, F, PG) hipLaunchKernelGGL((prefill_mfma_kernel<R, C, K, F, PG>), grid, dim3(kThreads), 0, stream, a)
    const bool f8 = a.kv_dtype == DT_FP8, pg = a.block_table != nullptr;
    if (a.cached && pg) {
        if (f8) {
            if (a.causal) GQA_PREFILL(true, true, true, true);
            else GQA_PREFILL(false, true, true, true);
        } else {
            if (a.causal) GQA_PREFILL(true, true, false, true);
            else GQA_PREFILL(false, true, false, true);
        }
    } else if (a.cached) {
        if (f8) {
            if (a.causal) GQA_PREFILL(true, true, true, false);
            else GQA_PREFILL(false, true, true, false);
        } else {
            if (a.causal) GQA_PREFILL(true, true, false, false);
            else GQA_PREFILL(false, true, false, false);
        }
    } else {
        if (a.causal) GQA_PREFILL(true, false, false, false);
        else GQA_PREFILL(false, false, false, false);
    }
#undef GQA_PREFILL
    return hipGetLastError();
}

}  // namespace

bool prefill_mfma_supports(const AttnArgs &a) {
    if (a.decode || a.D != kD || a.q_dtype != DT_BF16) return false;
    if (a.kv_dtype != DT_BF16 && !(a.cached && a.kv_dtype == DT_FP8)) return false;
    const int R = a.H / a.G;
    return R >= 1 && R <= 64;
}

hipError_t launch_prefill_mfma(const AttnArgs &a, hipStream_t stream) {
    if (!prefill_mfma_supports(a)) return hipErrorInvalidValue;
    switch (a.H / a.G) {
        case 1: return launch_r<1>(a, stream);
        case 2: return launch_r<2>(a, stream);
        case 4: return launch_r<4>(a, stream);
        case 8: return launch_r<8>(a, stream);
        case 16: return launch_r<16>(a, stream);
        case 32: return launch_r<32>(a, stream);
        case 64: return launch_r<64>(a, stream);
        default: return launch_r<0>(a, stream);
    }
}

}  // namespace gqa
