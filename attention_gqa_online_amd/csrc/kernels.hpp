// Host-side launch interface between the C ABI (api.hip) and the kernels.
// Arguments reaching these functions have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.hpp"

namespace attn {

// Compute units of the current device, queried once per device and cached
// (kMaxCus where the query fails). Plans are made for this count.
uint32_t device_cus();

// ---------------------------------------------------------------- decode
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
hipError_t launch_prefill(const PrefillPlan &plan, const float *q, const float *k,
                          const float *v, float *o, uint32_t m, uint32_t q_stride,
                          uint32_t kv_stride, uint32_t num_q_heads, uint32_t heads_per_kv,
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
