// KV-cache appends: one row per (sequence, KV head), and the bulk append
// of a prefill pass's rows. The single-row append writes K and V in one launch (glia honeycrisp "attention.rs"
// page: the KV-append and KV-append-both kernels). Element (b, g, e) of each
// source row goes to cache[b, g, position, e]; one lane moves 16 bytes of K
// and 16 bytes of V. With cos/sin tables the K row is rotated (rotate-half
// rotary embedding at `position`) on its way in.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const float *__restrict__ k_src, const float *__restrict__ v_src, float *__restrict__ k_cache,
    float *__restrict__ v_cache, const float *__restrict__ cos_t, const float *__restrict__ sin_t,
    const uint32_t *__restrict__ positions, uint32_t cs_stride, uint32_t kv_heads, uint32_t n4,
    uint32_t d4, uint32_t max_seq, uint32_t position) {
    const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
    if (idx >= n4) return;
    const uint32_t bg = idx / d4;  // b * kv_heads + g
    const uint32_t c = idx % d4;
    if (positions != nullptr) {  // per-sequence rows; `position` bounds them
        const uint32_t p = positions[bg / kv_heads];
        if (p >= position) return;
        position = p;
    }
    const size_t dst = ((size_t)bg * max_seq + position) * (size_t)(4 * d4) + 4 * c;
    float4 kx = ld4(k_src + 4 * (size_t)idx);
    if (cos_t != nullptr) {
        const uint32_t h4 = d4 / 2;  // half a row, in float4 units
        const bool lo = c < h4;
        const float4 xp = ld4(k_src + 4 * (size_t)(lo ? idx + h4 : idx - h4));
        const size_t i = (size_t)(bg / kv_heads) * cs_stride + 4 * (lo ? c : c - h4);
        kx = rope_half(kx, xp, ld4(cos_t + i), ld4(sin_t + i), lo);
    }
    st4(k_cache + dst, kx);
    st4(v_cache + dst, ld4(v_src + 4 * (size_t)idx));
}

}  // namespace

hipError_t launch_kv_append(const float *k_src, const float *v_src, float *k_cache,
                            float *v_cache, uint32_t batch, uint32_t kv_heads,
                            uint32_t head_dim, uint32_t max_seq, uint32_t position,
                            hipStream_t stream, const float *cos_t, const float *sin_t,
                            const uint32_t *positions, uint32_t cs_stride) {
    const uint32_t d4 = head_dim / 4;
    const uint32_t n4 = batch * kv_heads * d4;  // bounded by the caller
    const uint32_t grid = (n4 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(kThreads), 0, stream, k_src, v_src,
                       k_cache, v_cache, cos_t, sin_t, positions, cs_stride, kv_heads, n4, d4,
                       max_seq, position);
    return hipGetLastError();
}

// Bulk append of a prefill pass's rows: thread (g, j, c) moves float4 c of
// row j of KV head g, K and V. Threads of a workgroup run along (j, c), so
// each cache write is a contiguous stretch of the head's [max_seq, d] plane
// and each source read covers the row's d contiguous floats of head g.
__global__ __launch_bounds__(kThreads) void kv_append_rows_kernel(
    const float *__restrict__ k_src, const float *__restrict__ v_src, float *__restrict__ k_cache,
    float *__restrict__ v_cache, uint32_t n4, uint32_t d4, uint32_t kv_stride, uint32_t max_seq,
    uint32_t position) {
    const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;  // over (j, c) of head g
    if (idx >= n4) return;
    const uint32_t g = blockIdx.y;
    const uint32_t j = idx / d4;
    const uint32_t c = idx % d4;
    const size_t src = (size_t)j * kv_stride + (size_t)g * 4 * d4 + 4 * c;
    const size_t dst = ((size_t)g * max_seq + position) * (size_t)(4 * d4) + 4 * (size_t)idx;
    const float4 k = ld4_stream(k_src + src);
    const float4 v = ld4_stream(v_src + src);
    st4(k_cache + dst, k);
    st4(v_cache + dst, v);
}

hipError_t launch_kv_append_rows(const float *k_src, const float *v_src, float *k_cache,
                                 float *v_cache, uint32_t m, uint32_t kv_stride,
                                 uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                                 uint32_t position, hipStream_t stream) {
    const uint32_t d4 = head_dim / 4;
    const uint32_t n4 = m * d4;  // bounded by the caller (< 2^31)
    const uint32_t grid = (n4 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(kv_append_rows_kernel, dim3(grid, kv_heads), dim3(kThreads), 0, stream,
                       k_src, v_src, k_cache, v_cache, n4, d4, kv_stride, max_seq, position);
    return hipGetLastError();
}

}  // namespace attn
