// Internal declarations shared by the host layer and the kernel sources of libgqa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_INT4 = 3 };

// Everything one attention launch needs. Pointers are device pointers.
struct AttnArgs {
    const void *q;            // decode [B,H,D]; prefill [B,H,T,D]
    const void *k;            // decode [B,G,T_cap,D], or paged [num_pages][G][page_size][D];
    const void *v;            //   prefill [B,G,T,D]
    void *out;                // same shape and type as q
    const int32_t *seq_lens;  // decode only
    const float *k_scale;     // fp8 only, [B*G]
    const float *v_scale;
    float *part_acc;          // split partials, [B*H][S][D] (unnormalised)
    float *part_ml;           // split partials, [B*H][S][2] = (running max, running sum)
    const void *k_new;        // decode with append: the current token's key [B*G][D] (q's dtype)
    const void *v_new;        //   and value; both null without append
    const int32_t *block_table;  // paged decode: [B][pages_per_seq] page ids, else null
    int ps_log2;              // paged decode: log2(rows per page)
    int pages_per_seq;        // paged decode: block-table row length (T_cap = pages_per_seq << ps_log2)
    int num_pages;            // paged decode: pages in each pool
    int *counters;            // split arrival counters, [B*G], zero between calls
    int fuse_combine;         // 1: the last workgroup of each (b, g) merges the partials
    int B, H, G, D;
    int Tq;                   // query rows per (b, h): 1 for decode, T for prefill
    int Tk;                   // key rows allocated per (b, g): T_cap or T
    int causal;               // prefill: 1 = keys j <= i only
    int decode;               // 1 = keys limited by seq_lens[b], query at row L-1
    int cached;               // prefill against a cache: keys limited by seq_lens[b], query i at
                              // position seq_lens[b] - Tq + i (Tk = T_cap); 0 = plain prefill
    int num_splits;           // decode: key ranges per (b, g) (1 = write out directly); with the
                              // flat layout, the partial slots per query head
    int split_len;            // decode, uniform layout: keys per range
    int flat;                 // decode: 1 = flat layout of a ragged batch (splitkv.h)
    int flat_nw;              // flat layout: workgroups of the decode kernel
    int flat_cmin;            // flat layout: fewest rows per workgroup
    int flat_pad;             // flat layout: rows of no work in front of each non-empty segment
    float scale_log2;         // scale * log2(e): scores are kept in the base-2 domain
    int q_dtype, kv_dtype;
};

hipError_t launch_generic(const AttnArgs &a, hipStream_t stream);
hipError_t launch_combine(const AttnArgs &a, hipStream_t stream);
hipError_t launch_decode_valu(const AttnArgs &a, hipStream_t stream);
hipError_t launch_decode_mfma(const AttnArgs &a, hipStream_t stream);
hipError_t launch_prefill_mfma(const AttnArgs &a, hipStream_t stream);
hipError_t launch_kv_append(const AttnArgs &a, hipStream_t stream);
hipError_t launch_zero_ints(int *p, int n, hipStream_t stream);

// Shape limits of the fast kernels (checked on the host before launch).
bool decode_valu_supports(const AttnArgs &a);
bool decode_mfma_supports(const AttnArgs &a);
bool prefill_mfma_supports(const AttnArgs &a);

}  // namespace gqa
