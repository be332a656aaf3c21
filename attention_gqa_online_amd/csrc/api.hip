// C ABI of libattn.so (declared in include/attn.h): argument checks on the
// host, then one kernel launch on the caller's stream. No check below makes a
// HIP call, so an invalid call returns before touching the device. The only
// HIP calls made before a launch, after the checks, are the compute-unit
// query (hipGetDevice per call, the attribute once per device) and, for the
// no-allocation decode step, the lookup of the scratch array (once per device).
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "attn.h"
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_cus[kMaxDevices];  // 0: not queried yet

// ATTN_GQA_CUS=n: plan for at most n compute units (read once; 0 if unset or
// not a positive number).
uint32_t env_cus_limit() {
    static const uint32_t limit = [] {
        const char *v = getenv("ATTN_GQA_CUS");
        if (v == nullptr) return 0u;
        char *end = nullptr;
        const unsigned long n = strtoul(v, &end, 10);
        return end != v && *end == '\0' && n > 0 && n <= kMaxCus ? (uint32_t)n : 0u;
    }();
    return limit;
}
}  // namespace

uint32_t device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kMaxCus;
    if (dev < kMaxDevices) {
        const uint32_t c = g_cus[dev].load(std::memory_order_relaxed);
        if (c != 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return kMaxCus;
    uint32_t c = (uint32_t)n < kMaxCus ? (uint32_t)n : kMaxCus;
    const uint32_t limit = env_cus_limit();
    if (limit != 0 && limit < c) c = limit;
    if (dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
    return c;
}

}  // namespace attn

namespace {

// ---- the decode workspace of attn_decode_append_noalloc: one array per GPU
// (each device holds its own copy of this file-scope array from the moment
// the library's code is loaded on it until the process ends). Layout as any
// decode workspace: the fixed block of arrival counters (which every
// complete call leaves at zero), then partial states. Calls on one GPU all
// use it, so calls that overlap on one GPU race.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, per device, and only that
// address is ever passed to a kernel.
struct ScratchSlot {
    bool ready;
    void *ptr;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kScratchDevices];

__global__ void clear_words_kernel(uint32_t *p, uint32_t n) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// This GPU's scratch address. On the first call on a device (with it
// current) the address is looked up and the counter block cleared on
// `stream`, ahead of the call's own kernel (static device memory starts at
// zero as well; the clear makes that explicit). Nothing is allocated.
hipError_t scratch_address(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchSlot &slot = g_scratch[dev];
    if (!slot.ready) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        constexpr uint32_t words = attn::kCounterBlock / sizeof(uint32_t);
        hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t *>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        slot.ptr = p;
        slot.ready = true;
    }
    *out = slot.ptr;
    return hipSuccess;
}

bool head_dim_multiple_of_32(uint32_t d) { return d != 0 && d % 32 == 0; }
bool head_dim_built(uint32_t d) { return d >= 32 && d <= 256 && d % 32 == 0; }
bool aligned16(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Host checks use the plan for kMaxCus compute units (plain arithmetic, no
// HIP call); it needs at least the workspace and the workgroups of the plan
// for any smaller count. Once they pass, the launch uses the plan for the
// device's own count.
attn::DecodePlan device_plan(const attn::DecodePlan &checked, uint32_t batch,
                             uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                             uint32_t total_seq, uint32_t window, bool append, bool varlen) {
    const uint32_t cus = attn::device_cus();
    if (cus >= attn::kMaxCus) return checked;
    return attn::plan_decode(batch, num_heads, kv_heads, head_dim, total_seq, window, append,
                             varlen, cus);
}

}  // namespace

extern "C" {

const char *attn_status_string(attn_status s) {
    switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID: argument breaks the attn.h contract";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: valid but not built (head_dim)";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: the HIP runtime refused the launch";
    }
    return "unknown attn_status";
}

attn_status attn_prefill_causal(const float *q, const float *k, const float *v, float *o,
                                uint32_t m, uint32_t q_stride, uint32_t kv_stride,
                                uint32_t num_q_heads, uint32_t heads_per_kv,
                                uint32_t head_dim, hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim) || heads_per_kv == 0) return ATTN_ERR_INVALID;
    if (num_q_heads % heads_per_kv != 0) return ATTN_ERR_INVALID;
    const uint64_t kv_heads = num_q_heads / heads_per_kv;
    if ((uint64_t)q_stride < (uint64_t)num_q_heads * head_dim) return ATTN_ERR_INVALID;
    if ((uint64_t)kv_stride < kv_heads * head_dim) return ATTN_ERR_INVALID;
    if (q_stride % 4 != 0 || kv_stride % 4 != 0) return ATTN_ERR_INVALID;
    if (!head_dim_built(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (m == 0 || num_q_heads == 0) return ATTN_OK;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID;
    // grid = kv_heads * ceil(heads_per_kv * ceil(m/32) / waves) workgroups,
    // waves 8 or 4
    const uint64_t pairs = (uint64_t)heads_per_kv * ((m + 31u) / 32u);
    if (kv_heads * ((pairs + 3) / 4) > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    const attn::PrefillPlan plan =
        attn::plan_prefill(m, num_q_heads, heads_per_kv, head_dim, attn::device_cus());
    return from_hip(attn::launch_prefill(plan, q, k, v, o, m, q_stride, kv_stride, num_q_heads,
                                         heads_per_kv, head_dim, stream));
}

size_t attn_decode_workspace_bytes(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                                   uint32_t head_dim, uint32_t total_seq, uint32_t window) {
    if (!head_dim_multiple_of_32(head_dim) || !head_dim_built(head_dim)) return 0;
    if (kv_heads == 0 || num_heads % kv_heads != 0 || total_seq == 0) return 0;
    if (batch == 0 || num_heads == 0) return 0;
    if ((uint64_t)batch * kv_heads * num_heads > 0x7fffffffu) return 0;
    // large enough for every decode entry point's plan of these shapes on
    // any gfx950 device (plans on fewer compute units need no more)
    size_t need = 0;
    for (int append = 0; append < 2; ++append)
        for (int varlen = 0; varlen < 2; ++varlen) {
            const size_t n = attn::plan_decode(batch, num_heads, kv_heads, head_dim, total_seq,
                                               window, append != 0, varlen != 0, attn::kMaxCus)
                                 .workspace_bytes;
            need = n > need ? n : need;
        }
    return need;
}

attn_status attn_decode(const float *q, const float *k_cache, const float *v_cache, float *out,
                        uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                        uint32_t head_dim, uint32_t max_seq, uint32_t total_seq,
                        uint32_t window, float scale, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim) || kv_heads == 0) return ATTN_ERR_INVALID;
    if (num_heads % kv_heads != 0) return ATTN_ERR_INVALID;
    if (total_seq == 0 || total_seq > max_seq) return ATTN_ERR_INVALID;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!head_dim_built(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || num_heads == 0) return ATTN_OK;
    if ((uint64_t)batch * kv_heads * num_heads > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return ATTN_ERR_INVALID;
    const attn::DecodePlan chk = attn::plan_decode(batch, num_heads, kv_heads, head_dim,
                                                   total_seq, window, false, false, attn::kMaxCus);
    if (!aligned16(workspace) || workspace_bytes < chk.workspace_bytes) return ATTN_ERR_INVALID;
    if ((uint64_t)chk.units * chk.n_split > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    const attn::DecodePlan plan = device_plan(chk, batch, num_heads, kv_heads, head_dim,
                                              total_seq, window, false, false);
    return from_hip(attn::launch_decode(plan, q, k_cache, v_cache, out, num_heads, kv_heads,
                                        head_dim, max_seq, total_seq, scale, workspace,
                                        nullptr, stream));
}

}  // extern "C"

namespace {

attn_status decode_step(const float *q, const float *k_new, const float *v_new,
                        const float *cos_t, const float *sin_t, float *k_cache,
                        float *v_cache, float *out, uint32_t batch, uint32_t num_heads,
                        uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                        uint32_t position, uint32_t window, float scale, void *workspace,
                        size_t workspace_bytes, hipStream_t stream, bool use_scratch = false);

}  // namespace

extern "C" {

attn_status attn_decode_append(const float *q, const float *k_new, const float *v_new,
                               float *k_cache, float *v_cache, float *out, uint32_t batch,
                               uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                               uint32_t max_seq, uint32_t position, uint32_t window,
                               float scale, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return decode_step(q, k_new, v_new, nullptr, nullptr, k_cache, v_cache, out, batch,
                       num_heads, kv_heads, head_dim, max_seq, position, window, scale,
                       workspace, workspace_bytes, stream);
}

attn_status attn_decode_rope_append(const float *q_raw, const float *k_raw,
                                    const float *v_raw, const float *cos_t,
                                    const float *sin_t, float *k_cache, float *v_cache,
                                    float *out, uint32_t batch, uint32_t num_heads,
                                    uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                                    uint32_t position, uint32_t window, float scale,
                                    void *workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (batch != 0 && (!aligned16(cos_t) || !aligned16(sin_t))) return ATTN_ERR_INVALID;
    return decode_step(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache, v_cache, out, batch,
                       num_heads, kv_heads, head_dim, max_seq, position, window, scale,
                       workspace, workspace_bytes, stream);
}

attn_status attn_decode_append_noalloc(const float *q, const float *k_new, const float *v_new,
                                       float *k_cache, float *v_cache, float *out,
                                       uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                                       uint32_t head_dim, uint32_t max_seq, uint32_t position,
                                       uint32_t window, float scale, hipStream_t stream) {
    return decode_step(q, k_new, v_new, nullptr, nullptr, k_cache, v_cache, out, batch,
                       num_heads, kv_heads, head_dim, max_seq, position, window, scale, nullptr,
                       0, stream, true);
}

}  // extern "C"

namespace {

// use_scratch: the workspace is this GPU's scratch array (above) instead of
// the caller's buffer; shapes whose plan needs more than it holds, or more
// arrival counters than its fixed counter block, are ATTN_ERR_UNSUPPORTED.
attn_status decode_step(const float *q, const float *k_new, const float *v_new,
                        const float *cos_t, const float *sin_t, float *k_cache,
                        float *v_cache, float *out, uint32_t batch, uint32_t num_heads,
                        uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                        uint32_t position, uint32_t window, float scale, void *workspace,
                        size_t workspace_bytes, hipStream_t stream, bool use_scratch) {
    if (!head_dim_multiple_of_32(head_dim) || kv_heads == 0) return ATTN_ERR_INVALID;
    if (num_heads % kv_heads != 0) return ATTN_ERR_INVALID;
    if (position >= max_seq) return ATTN_ERR_INVALID;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!head_dim_built(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (batch == 0) return ATTN_OK;
    if ((uint64_t)batch * kv_heads * num_heads > 0x7fffffffu ||
        (uint64_t)batch * kv_heads * (head_dim / 4) > 0x7fffffffu)
        return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_INVALID;
    if (num_heads == 0) {  // nothing to attend: the append alone
        return from_hip(attn::launch_kv_append(k_new, v_new, k_cache, v_cache, batch, kv_heads,
                                               head_dim, max_seq, position, stream, cos_t,
                                               sin_t));
    }
    const uint32_t total_seq = position + 1;
    const attn::DecodePlan chk = attn::plan_decode(batch, num_heads, kv_heads, head_dim,
                                                   total_seq, window, true, false, attn::kMaxCus);
    attn::DecodeAppend app{k_new, v_new, k_cache, v_cache, cos_t, sin_t};
    if (!aligned16(q) || !aligned16(out)) return ATTN_ERR_INVALID;
    if (use_scratch) {
        if (chk.workspace_bytes > kScratchBytes || chk.part_offset > attn::kCounterBlock)
            return ATTN_ERR_UNSUPPORTED;
    } else if (chk.workspace_bytes > 0 &&
               (!aligned16(workspace) || workspace_bytes < chk.workspace_bytes)) {
        return ATTN_ERR_INVALID;
    }
    if ((uint64_t)chk.units * chk.n_split > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    if (use_scratch && chk.workspace_bytes > 0) {
        const hipError_t e = scratch_address(stream, &workspace);
        if (e != hipSuccess) return ATTN_ERR_HIP;
    }
    const attn::DecodePlan plan = device_plan(chk, batch, num_heads, kv_heads, head_dim,
                                              total_seq, window, true, false);
    return from_hip(attn::launch_decode(plan, q, k_cache, v_cache, out, num_heads, kv_heads,
                                        head_dim, max_seq, total_seq, scale, workspace, &app,
                                        stream));
}

}  // namespace

extern "C" {

attn_status kv_append(const float *k_src, const float *v_src, float *k_cache, float *v_cache,
                      uint32_t batch, uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                      uint32_t position, hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim)) return ATTN_ERR_INVALID;
    if (position >= max_seq) return ATTN_ERR_INVALID;
    if (batch == 0 || kv_heads == 0) return ATTN_OK;
    if ((uint64_t)batch * kv_heads * (head_dim / 4) > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_INVALID;
    return from_hip(attn::launch_kv_append(k_src, v_src, k_cache, v_cache, batch, kv_heads,
                                           head_dim, max_seq, position, stream));
}

attn_status kv_append_rows(const float *k_src, const float *v_src, float *k_cache,
                           float *v_cache, uint32_t m, uint32_t kv_stride, uint32_t kv_heads,
                           uint32_t head_dim, uint32_t max_seq, uint32_t position,
                           hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim)) return ATTN_ERR_INVALID;
    if ((uint64_t)position + m > max_seq) return ATTN_ERR_INVALID;
    if (m == 0 || kv_heads == 0) return ATTN_OK;
    if (kv_stride % 4 != 0 || (uint64_t)kv_stride < (uint64_t)kv_heads * head_dim)
        return ATTN_ERR_INVALID;
    if ((uint64_t)m * (head_dim / 4) > 0x7fffffffu || kv_heads > 65535u)
        return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_cache) || !aligned16(v_cache))
        return ATTN_ERR_INVALID;
    return from_hip(attn::launch_kv_append_rows(k_src, v_src, k_cache, v_cache, m, kv_stride,
                                                kv_heads, head_dim, max_seq, position, stream));
}

attn_status attn_decode_varlen(const float *q, const float *k_cache, const float *v_cache,
                               float *out, const uint32_t *seq_lens, uint32_t batch,
                               uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                               uint32_t max_seq, uint32_t seq_bound, uint32_t window,
                               float scale, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim) || kv_heads == 0) return ATTN_ERR_INVALID;
    if (num_heads % kv_heads != 0) return ATTN_ERR_INVALID;
    if (seq_bound == 0 || seq_bound > max_seq) return ATTN_ERR_INVALID;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!head_dim_built(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || num_heads == 0) return ATTN_OK;
    if ((uint64_t)batch * kv_heads * num_heads > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        !aligned4(seq_lens))
        return ATTN_ERR_INVALID;
    const attn::DecodePlan chk = attn::plan_decode(batch, num_heads, kv_heads, head_dim,
                                                   seq_bound, window, false, true, attn::kMaxCus);
    if (!aligned16(workspace) || workspace_bytes < chk.workspace_bytes) return ATTN_ERR_INVALID;
    if ((uint64_t)chk.units * chk.n_split > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    const attn::DecodePlan plan = device_plan(chk, batch, num_heads, kv_heads, head_dim,
                                              seq_bound, window, false, true);
    const attn::DecodeVarlen vl{seq_lens, 0, seq_bound, window};
    return from_hip(attn::launch_decode(plan, q, k_cache, v_cache, out, num_heads, kv_heads,
                                        head_dim, max_seq, seq_bound, scale, workspace,
                                        nullptr, stream, &vl));
}

}  // extern "C"

namespace {

attn_status decode_step_varlen(const float *q, const float *k_new, const float *v_new,
                               const float *cos_t, const float *sin_t, float *k_cache,
                               float *v_cache, float *out, const uint32_t *positions,
                               uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                               uint32_t head_dim, uint32_t max_seq, uint32_t seq_bound,
                               uint32_t window, float scale, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (!head_dim_multiple_of_32(head_dim) || kv_heads == 0) return ATTN_ERR_INVALID;
    if (num_heads % kv_heads != 0) return ATTN_ERR_INVALID;
    if (seq_bound == 0 || seq_bound > max_seq) return ATTN_ERR_INVALID;
    if (!isfinite(scale)) return ATTN_ERR_INVALID;
    if (!head_dim_built(head_dim)) return ATTN_ERR_UNSUPPORTED;
    if (batch == 0) return ATTN_OK;
    if ((uint64_t)batch * kv_heads * num_heads > 0x7fffffffu ||
        (uint64_t)batch * kv_heads * (head_dim / 4) > 0x7fffffffu)
        return ATTN_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned4(positions))
        return ATTN_ERR_INVALID;
    const uint32_t cs_stride = cos_t != nullptr ? head_dim / 2 : 0;  // one table per sequence
    if (num_heads == 0) {  // nothing to attend: the appends alone
        return from_hip(attn::launch_kv_append(k_new, v_new, k_cache, v_cache, batch, kv_heads,
                                               head_dim, max_seq, seq_bound, stream, cos_t,
                                               sin_t, positions, cs_stride));
    }
    if (!aligned16(q) || !aligned16(out)) return ATTN_ERR_INVALID;
    const attn::DecodePlan chk = attn::plan_decode(batch, num_heads, kv_heads, head_dim,
                                                   seq_bound, window, true, true, attn::kMaxCus);
    if (chk.workspace_bytes > 0 && (!aligned16(workspace) || workspace_bytes < chk.workspace_bytes))
        return ATTN_ERR_INVALID;
    if ((uint64_t)chk.units * chk.n_split > 0x7fffffffu) return ATTN_ERR_UNSUPPORTED;
    const attn::DecodePlan plan = device_plan(chk, batch, num_heads, kv_heads, head_dim,
                                              seq_bound, window, true, true);
    const attn::DecodeAppend app{k_new, v_new, k_cache, v_cache, cos_t, sin_t, cs_stride};
    const attn::DecodeVarlen vl{positions, 1, seq_bound, window};
    return from_hip(attn::launch_decode(plan, q, k_cache, v_cache, out, num_heads, kv_heads,
                                        head_dim, max_seq, seq_bound, scale, workspace, &app,
                                        stream, &vl));
}

}  // namespace

extern "C" {

attn_status attn_decode_append_varlen(const float *q, const float *k_new, const float *v_new,
                                      float *k_cache, float *v_cache, float *out,
                                      const uint32_t *positions, uint32_t batch,
                                      uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                                      uint32_t max_seq, uint32_t seq_bound, uint32_t window,
                                      float scale, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    return decode_step_varlen(q, k_new, v_new, nullptr, nullptr, k_cache, v_cache, out,
                              positions, batch, num_heads, kv_heads, head_dim, max_seq,
                              seq_bound, window, scale, workspace, workspace_bytes, stream);
}

attn_status attn_decode_rope_append_varlen(const float *q_raw, const float *k_raw,
                                           const float *v_raw, const float *cos_t,
                                           const float *sin_t, float *k_cache,
                                           float *v_cache, float *out,
                                           const uint32_t *positions, uint32_t batch,
                                           uint32_t num_heads, uint32_t kv_heads,
                                           uint32_t head_dim, uint32_t max_seq,
                                           uint32_t seq_bound, uint32_t window, float scale,
                                           void *workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
    if (batch != 0 && (!aligned16(cos_t) || !aligned16(sin_t))) return ATTN_ERR_INVALID;
    return decode_step_varlen(q_raw, k_raw, v_raw, cos_t, sin_t, k_cache, v_cache, out,
                              positions, batch, num_heads, kv_heads, head_dim, max_seq,
                              seq_bound, window, scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
