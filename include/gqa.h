/*
 * gqa.h -- C ABI of libgqa.so: grouped-query attention (GQA) decode and prefill on
 * AMD Instinct MI355X (gfx950).
 *
 * Grouped-query attention splits H query heads into G groups of R = H / G
 * consecutive heads; all heads of group g read the single key/value head g, so
 * G = H is multi-head attention and G = 1 is multi-query attention [GQA paper
 * digest page (51969.com), section "Grouped-query attention (GQA)", Figure 2;
 * "LLM principles -- code implementation of multi-head attention (MQA and GQA)",
 * section 5, where a head's group is its index divided by the heads per group].
 * Query head h therefore reads KV head h / R. The library never copies a KV head
 * out to its R query heads: every key/value row is read from memory once per
 * (sequence, KV head) and used by all R heads of the group.
 *
 * For one query row q and key/value rows 0..n-1 the library computes
 *     out = sum_j softmax_j(scale * q . k_j) * v_j
 * ["LLM principles -- code ...", sections 3 and 5: Q times K transposed, divided by
 * the square root of the head size, softmax over the keys, times V]. Callers
 * normally pass scale = 1/sqrt(D).
 *
 * Memory: every pointer argument is caller-owned memory. Tensor pointers and
 * seq_lens, k_scale, v_scale and workspace are DEVICE pointers; the options struct
 * is a HOST pointer read during the call only. The library frees nothing it did
 * not allocate, keeps no per-call state, and may be called from several host
 * threads at once. Outputs must not alias inputs.
 *
 * Execution: both compute calls only enqueue work on `stream` and return without
 * waiting; `out` is valid once the stream has drained. Results are deterministic
 * for fixed arguments: partial results are merged in a fixed order (the only atomics are
 * integer arrival counters).
 *
 * Errors: every call returns a gqa_status by value and never aborts or prints.
 * All argument checks run on the host before any HIP call, so a rejected call has
 * touched neither the device nor the stream. GQA_ERR_HIP reports a failure of the
 * HIP runtime (for example a launch error) after work may have been enqueued.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, H % G != 0, non-finite scale, ... */
    GQA_ERR_UNSUPPORTED = 2,   /* dtype pair, head dim, forced path or device not supported */
    GQA_ERR_WORKSPACE = 3,     /* caller workspace smaller than gqa_decode_workspace_size() */
    GQA_ERR_HIP = 4            /* the HIP runtime reported an error */
} gqa_status;

/* Element types. q and out always share one type. */
typedef enum gqa_dtype {
    GQA_DTYPE_F32 = 0,
    GQA_DTYPE_BF16 = 1,
    /* OCP 8-bit float E4M3FN (bias 7, no infinities, max 448). KV cache only; each
     * stored value stands for code * scale with one fp32 scale per (sequence, KV
     * head) ["GQA revolution: how xformers speeds up LLM inference", section on
     * mixed-precision KV storage]. */
    GQA_DTYPE_FP8_E4M3FN = 2,
    /* 4-bit integer KV cache only: rows of D/2 bytes, byte i holding head dims 2i (low four
     * bits) and 2i+1 (high four bits); a field u in 0..15 stands for (u - 8) * scale with one
     * fp32 scale per (sequence, KV head), as for fp8. ["GQA revolution ...", section on
     * mixed-precision KV storage, names 4-bit KV storage and no layout; this is the library's
     * reading.] D must be even. */
    GQA_DTYPE_INT4 = 3
} gqa_dtype;

/* Kernel family for decode. AUTO takes MFMA wherever it applies and GENERIC otherwise;
 * the others force a family so tests can check each against the same inputs. */
typedef enum gqa_path {
    GQA_PATH_AUTO = 0,
    GQA_PATH_GENERIC = 1,  /* any head dim 1..256, any supported dtype pair */
    GQA_PATH_VALU = 2,     /* vector-ALU dot products; bf16 KV, D = 128 */
    GQA_PATH_MFMA = 3      /* matrix cores; bf16, fp8 or INT4 KV, bf16 q, D = 128 */
} gqa_path;

/* Decode work layout. UNIFORM cuts every (sequence, KV head) into the same number of key
 * ranges (num_splits); FLAT lays the valid keys of all sequences end to end and gives every
 * workgroup the same number of them, so a batch of very unequal lengths still keeps every
 * compute unit busy (matrix-core family only, batches with B * G * (kv_capacity + 1024) < 2^31).
 * AUTO takes FLAT for batches of 16 or more sequences on the matrix-core family and UNIFORM
 * otherwise. The split-KV scheme these build on is the one of ["GQA revolution ...", section
 * on split-KV block computation]; the flat layout is this library's own. */
typedef enum gqa_layout {
    GQA_LAYOUT_AUTO = 0,
    GQA_LAYOUT_UNIFORM = 1,
    GQA_LAYOUT_FLAT = 2
} gqa_layout;

typedef struct gqa_opts {
    size_t struct_size;     /* sizeof(gqa_opts); fields past it are taken as defaults */
    int32_t q_dtype;        /* gqa_dtype of q and out (default BF16) */
    int32_t kv_dtype;       /* gqa_dtype of k/v or of the cache (default BF16) */
    int32_t kv_capacity;    /* decode: T_cap, rows allocated per (sequence, KV head); required */
    int32_t num_splits;     /* decode: KV splits per (sequence, KV head); 0 = choose */
    int32_t path;           /* gqa_path (default AUTO) */
    int32_t layout;         /* decode: gqa_layout (default AUTO); FLAT excludes num_splits > 0 */
    const float *k_scale;   /* fp8 / INT4 KV: device fp32 [B*G], index b*G + g; else NULL */
    const float *v_scale;   /* fp8 / INT4 KV: device fp32 [B*G]; else NULL */
    void *workspace;        /* device scratch for split partials, or NULL */
    size_t workspace_bytes; /* size of `workspace` */
    const void *k_new;      /* decode: the current token's key [B, G, D] (q's dtype) to append, or NULL */
    const void *v_new;      /* decode: its value [B, G, D]; set both or neither */
} gqa_opts;

/* Fill `opts` with defaults: struct_size set, BF16/BF16, kv_capacity 0 (must be set
 * for decode), num_splits 0, path AUTO, layout AUTO, no scales, no workspace. */
void gqa_opts_init(gqa_opts *opts);

/*
 * Single-token decode over a KV cache (the memory-bound step: the step reads the
 * whole cache once [GQA paper digest page, section "QA": decoding is bound by
 * loading the KV cache]).
 *
 *   q        [B, H, D]            q_dtype, the current token's query heads
 *   k_cache  [B, G, T_cap, D]     kv_dtype, head dim innermost, T_cap = opts->kv_capacity
 *                                 (INT4: [B, G, T_cap, D/2] bytes)
 *   v_cache  [B, G, T_cap, D]     kv_dtype
 *   seq_lens [B] int32 (device)   valid rows of sequence b, current token included
 *   out      [B, H, D]            q_dtype
 *
 * The caller has already written the current token's k and v at row seq_lens[b]-1
 * ("LLM principles -- code ...", sections 3 and 5 concatenate the new K/V to the
 * cache before forming scores), so query head h of sequence b attends to rows
 * 0 .. seq_lens[b]-1 of KV head h / (H/G), itself included. Rows at or beyond
 * seq_lens[b] (up to T_cap - 1) may be read but never affect the result, whatever they
 * hold, NaN included; nothing past T_cap is read. seq_lens lives on the device and is not
 * checked on the host: a value above T_cap is treated as T_cap, a value <= 0 yields a
 * zero output row.
 *
 * Long caches are split into num_splits key ranges whose partial results are merged
 * by a log-sum-exp combine ["GQA revolution ...", section on split-KV block
 * computation]; that needs device scratch: opts->workspace of at least
 * gqa_decode_workspace_size() bytes, or NULL to let the call take stream-ordered
 * memory with hipMallocAsync/hipFreeAsync on `stream` (zero-filled by a kernel on the same
 * stream). A NULL workspace is refused with GQA_ERR_WORKSPACE while `stream` is being
 * captured into a graph: pass a workspace there. A caller workspace must be
 * zero-filled before its first use (it holds per-(sequence, KV head) arrival counters);
 * every completed call leaves it ready for the next one. Calls that run concurrently must
 * not share a workspace.
 *
 * Cache append (optional): with opts->k_new and opts->v_new set, the call first stores the
 * current token's key and value at row seq_lens[b]-1 of every (b, g) whose length lies in
 * 1..T_cap, then attends over rows 0..seq_lens[b]-1 as above, the stored row included; the
 * caller then need not write the row itself ("LLM principles -- code ...", sections 3 and 5
 * append the new K/V to the cache before the scores). fp32 and bf16 caches receive the values
 * unchanged; an fp8 cache receives the E4M3FN code nearest (ties to even) to the fp32 quotient
 * k_new / k_scale[b*G+g] (v likewise), with the slab's scale kept fixed: magnitudes beyond 448
 * saturate ["GQA revolution ...", section on mixed-precision KV storage, stores code * scale;
 * what happens past the range is this library's reading]. k_cache and v_cache are then written,
 * so they must be writable memory although the signature declares them const. The matrix-core
 * family writes the row inside the attention kernel; the other families run a small copy
 * kernel first.
 *
 * Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN), (BF16, INT4).
 * opts is required (it carries kv_capacity). D in 1..256 (even for INT4). An INT4 append
 * stores the nearest integer to k_new / k_scale (ties to even) clamped to -8 .. 7, by a copy
 * kernel before the attention.
 */
gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *seq_lens, void *out, int B, int H, int G, int D,
                      float scale, hipStream_t stream, const gqa_opts *opts);

/*
 * gqa_decode for callers that cannot allocate device memory during the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same arguments,
 * kernels and results as gqa_decode, except that the split partials and arrival counters live
 * in a static device array inside libgqa.so instead of a workspace. opts->workspace must be
 * NULL (else GQA_ERR_INVALID_ARG). The call allocates nothing: no hipMalloc, hipMallocAsync or
 * hipFree, and no memset.
 *
 * Limits: B * G <= 65536, and at most 32 MiB of split partials (gqa_decode_workspace_size()
 * minus the counter bytes bounds what a call needs); larger calls return GQA_ERR_WORKSPACE
 * before any HIP call. Each GPU the library runs on holds its own 32.25 MiB array until the
 * process ends. The first call on a device looks up the array's address there and zero-fills
 * its counters on `stream`; every completed call leaves them at zero again.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's partials: calls
 * that overlap in time on one GPU (on different streams, or from different threads without
 * ordering) race and may give wrong results. Calls ordered on one stream are safe.
 */
gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *seq_lens, void *out, int B, int H, int G, int D,
                              float scale, hipStream_t stream, const gqa_opts *opts);

/*
 * Single-token decode over a paged KV cache: the same computation as gqa_decode, with the
 * cache rows of each sequence held in fixed-size pages that a block table maps ["GQA
 * revolution ...", section on split-KV block computation, whose work-split heuristic takes a
 * page size and an is-paged flag; the pages say nothing more of the layout, so the layout
 * below is this library's reading].
 *
 *   k_pages, v_pages [num_pages, G, page_size, D]   kv_dtype; page p holds page_size
 *                                                   consecutive rows of every KV head
 *   block_table      [B, pages_per_seq] int32 (device)
 *
 * Row t of sequence b and KV head g is k_pages[block_table[b][t / page_size]][g][t % page_size]
 * (likewise v). The capacity is pages_per_seq * page_size rows per sequence and replaces
 * opts->kv_capacity; seq_lens are read as in gqa_decode against that capacity. page_size is a
 * power of two from 16 to 2^20. Only the table entries that cover rows 0 .. seq_lens[b]-1 are
 * used for the result (later entries of the row may be read, so all pages_per_seq entries must
 * be allocated, whatever they hold); entries outside 0 .. num_pages-1 are clamped into that
 * range (no out-of-bounds access; the result is then unspecified). Pages may be shared or
 * unused.
 *
 * Every option of gqa_decode applies (dtypes, fp8 scales per (sequence, KV head), workspace
 * of gqa_decode_workspace_size() for kv_capacity = pages_per_seq * page_size, layout, cache
 * append through opts->k_new / v_new, which writes the row's page). Kernel family: matrix
 * cores only (bf16 q with a bf16, fp8 or INT4 cache, D = 128); other paths and dtypes return
 * GQA_ERR_UNSUPPORTED.
 */
gqa_status gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                            const int32_t *seq_lens, void *out, int B, int H, int G, int D, float scale,
                            int page_size, int pages_per_seq, int num_pages, hipStream_t stream,
                            const gqa_opts *opts);

/*
 * Prefill: attention of every position of a sequence over the same sequence's keys
 * (compute-bound [GQA paper digest page, introduction and section "QA"]).
 *
 *   q   [B, H, T, D]   q_dtype
 *   k   [B, G, T, D]   kv_dtype (must equal q_dtype)
 *   v   [B, G, T, D]
 *   out [B, H, T, D]   q_dtype
 *
 * causal = 1: position i attends to keys 0..i (keys above the diagonal are masked,
 * "LLM principles -- code ...", section 3); causal = 0: to all T keys.
 * opts may be NULL (BF16 everywhere). Supported dtypes: F32 or BF16. D in 1..256.
 */
gqa_status gqa_prefill(const void *q, const void *k, const void *v, void *out, int B, int T,
                       int H, int G, int D, float scale, int causal, hipStream_t stream,
                       const gqa_opts *opts);

/*
 * Prefill of a chunk of Tq new positions against a KV cache (chunked prefill; Tq = 1 is
 * decode): the generalisation of ["LLM principles -- code ...", sections 3 and 5], where the
 * new keys and values are concatenated to the cache and the causal mask hides later keys.
 *
 *   q        [B, H, Tq, D]        q_dtype, the chunk's queries
 *   k_cache  [B, G, T_cap, D]     kv_dtype, T_cap = opts->kv_capacity (required)
 *   v_cache  [B, G, T_cap, D]
 *   seq_lens [B] int32 (device)   valid rows of sequence b, the chunk's own rows included
 *   out      [B, H, Tq, D]        q_dtype
 *
 * The caller has written the chunk's keys and values at rows seq_lens[b]-Tq .. seq_lens[b]-1.
 * Query i of sequence b sits at position p = seq_lens[b] - Tq + i. causal = 1: it attends to
 * rows 0 .. p; causal = 0: to rows 0 .. seq_lens[b]-1. seq_lens is read as in gqa_decode (a
 * value above T_cap is T_cap, below 0 is 0); a query with p < 0 sees no row and its output is
 * zero. Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16) and (BF16, FP8_E4M3FN) with
 * opts->k_scale / v_scale as in gqa_decode; the bf16 and fp8 caches run on the matrix cores
 * for D = 128 and R up to 64, everything else on the generic family. D in 1..256.
 */
gqa_status gqa_prefill_cached(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                              void *out, int B, int Tq, int H, int G, int D, float scale, int causal,
                              hipStream_t stream, const gqa_opts *opts);

/*
 * Chunk against a paged cache: gqa_prefill_cached with the cache rows in pages, laid out as
 * for gqa_decode_paged (pools [num_pages, G, page_size, D], int32 block_table
 * [B, pages_per_seq] in device memory; row t of (b, g) is row t mod page_size of page
 * block_table[b][t / page_size]; capacity pages_per_seq * page_size replaces
 * opts->kv_capacity). The chunk's rows are written into their pages by the caller first.
 * page_size: a power of two from 16 to 2^20. Only table entries covering rows below
 * seq_lens[b] are used for the result (later entries of the row may be read, so all
 * pages_per_seq entries must be allocated); entries outside [0, num_pages) are clamped
 * (memory-safe, result unspecified). Kernel family: matrix cores only (bf16 q with a bf16 or fp8 cache,
 * D = 128, R up to 64); anything else returns GQA_ERR_UNSUPPORTED.
 */
gqa_status gqa_prefill_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, void *out, int B, int Tq, int H, int G, int D, float scale,
                             int causal, int page_size, int pages_per_seq, int num_pages, hipStream_t stream,
                             const gqa_opts *opts);

/* Key ranges per (sequence, KV head) -- with the flat layout, the most partial results one
 * query head can have -- that gqa_decode uses for these sizes with path and layout AUTO
 * (num_splits 0 = the library's own choice, which depends only on these arguments). Returns 0
 * for invalid sizes. */
int gqa_decode_num_splits(int B, int H, int G, int D, int kv_capacity, int kv_dtype,
                          int num_splits);

/* Bytes of device workspace gqa_decode needs for these sizes, enough for every path and
 * layout; 0 when it needs none (one split). Returns SIZE_MAX for invalid sizes. */
size_t gqa_decode_workspace_size(int B, int H, int G, int D, int kv_capacity, int kv_dtype,
                                 int num_splits);

/* Static, NUL-terminated name of a status code. */
const char *gqa_status_string(gqa_status status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
