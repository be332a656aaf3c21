// Host-side launch interface between the C ABI (api.hip) and the kernels.
// Arguments reaching these functions have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// ---------------------------------------------------------------- decode
// Work split of one decode call: the attended rows [w0, total_seq) of every
// (sequence, KV head, head chunk) unit are cut into n_split contiguous row
// ranges of rows_per_split rows, one workgroup each.
struct DecodePlan {
    uint32_t head_chunk;      // Q heads handled per workgroup (<= 8)
    uint32_t n_chunks;        // head chunks per KV head
    uint32_t units;           // batch * kv_heads * n_chunks
    uint32_t n_split;         // workgroups per unit
    uint32_t rows_per_split;  // multiple of the rows one workgroup step covers
    uint32_t w0;              // first attended row
    size_t part_floats;       // partial-state floats in the workspace
    size_t part_offset;       // bytes before them: the units' arrival counters
    size_t workspace_bytes;   // counters + partial states (the whole workspace)
};

// With `append`, the split pass covers [w0, total_seq - 1) and the last row
// comes from the new K/V rows instead (n_split may then be 0).
DecodePlan plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window,
                       bool append = false, bool varlen = false);

// New K/V rows for attn_decode_append: written at `position` = total_seq - 1;
// with cos/sin ([D/2] for that position) q and the new K rows are rotated.
// Per-sequence lengths for a batch of mixed lengths: T_b = lens[b] + len_add
// (len_add 1 when lens are the append positions), each at most seq_bound.
struct DecodeVarlen {
    const uint32_t *lens;
    uint32_t len_add;
    uint32_t seq_bound;
    uint32_t window;
};

struct DecodeAppend {
    const float *k_new;
    const float *v_new;
    float *k_cache;
    float *v_cache;
    const float *cos_t = nullptr;
    const float *sin_t = nullptr;
    uint32_t cs_stride = 0;  // floats between sequences' tables (0: one shared table)
};

hipError_t launch_decode(const DecodePlan &plan, const float *q, const float *k_cache,
                         const float *v_cache, float *out, uint32_t num_heads,
                         uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                         uint32_t total_seq, float scale, void *workspace,
                         const DecodeAppend *append, hipStream_t stream,
                         const DecodeVarlen *varlen = nullptr);

// ---------------------------------------------------------------- prefill
hipError_t launch_prefill(const float *q, const float *k, const float *v, float *o,
                          uint32_t m, uint32_t q_stride, uint32_t kv_stride,
                          uint32_t num_q_heads, uint32_t heads_per_kv,
                          uint32_t head_dim, hipStream_t stream);

// ---------------------------------------------------------------- append
// With cos_t/sin_t ([head_dim/2]) the K rows are rotated (rotate-half) first.
// With positions ([batch], device) each sequence writes its own row, and
// `position` is their exclusive bound (rows at or past it are skipped).
hipError_t launch_kv_append(const float *k_src, const float *v_src, float *k_cache,
                            float *v_cache, uint32_t batch, uint32_t kv_heads,
                            uint32_t head_dim, uint32_t max_seq, uint32_t position,
                            hipStream_t stream, const float *cos_t = nullptr,
                            const float *sin_t = nullptr,
                            const uint32_t *positions = nullptr, uint32_t cs_stride = 0);

// Rows [0, m) of packed K/V ([m, kv_stride]) into [kv_heads, max_seq, d]
// caches from row `position` on.
hipError_t launch_kv_append_rows(const float *k_src, const float *v_src, float *k_cache,
                                 float *v_cache, uint32_t m, uint32_t kv_stride,
                                 uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                                 uint32_t position, hipStream_t stream);

}  // namespace attn
