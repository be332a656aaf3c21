// Decode work plan and dispatch (kernel template in decode_kernel.hpp).
#include "decode_kernel.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

// One launch per call. With a single split per unit and no appended row
// each workgroup writes its unit's normalised output itself; otherwise the
// last workgroup of each unit to finish merges the units' partial states
// and the appended row (kMergeFused). With no row before the appended one
// (n_split 0) every unit gets one workgroup over an empty range, which only
// folds in the new row. With per-sequence lengths the grid holds the
// proportional splits and one more workgroup per unit, so the units with no
// rows in the split pass (idle, only the new row, invalid) get one each.
template <int D, int HC>
hipError_t launch_hc(DecodeArgs args, uint32_t units, uint32_t n_split, uint32_t g_target,
                     hipStream_t stream) {
    constexpr int LPR = lanes_per_row(D);
    args.units = units;
    if (n_split == 1 && args.k_new == nullptr) {
        if (args.lens != nullptr)
            hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves, kPrefetch, kMergeDirect, true>),
                               dim3(units), dim3(kDecodeWaves * 64), 0, stream, args);
        else
            hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves, kPrefetch, kMergeDirect, false>),
                               dim3(units), dim3(kDecodeWaves * 64), 0, stream, args);
        return hipGetLastError();
    }
    if (args.lens == nullptr) {
        if (n_split == 0) {  // only the appended row
            args.n_split = 1;
            args.rows_per_split = 0;
            n_split = 1;
        }
        hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves, kPrefetch, kMergeFused, false>),
                           dim3(units * n_split), dim3(kDecodeWaves * 64), 0, stream, args);
        return hipGetLastError();
    }
    args.g_target = g_target;
    args.min_rows = kDecodeWaves * kMinRowsPerWave;
    args.rows_step = kDecodeWaves * (64 / LPR);
    hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves, kPrefetch, kMergeFused, true>),
                       dim3(args.g_target + units), dim3(kDecodeWaves * 64), 0, stream, args);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(uint32_t hc, const DecodeArgs &args, uint32_t units, uint32_t n_split,
                    uint32_t g_target, hipStream_t stream) {
    // head chunks beyond max_head_chunk(D) are never planned (nor built)
    switch (hc) {
    case 1: return launch_hc<D, 1>(args, units, n_split, g_target, stream);
    case 2: return launch_hc<D, 2>(args, units, n_split, g_target, stream);
    case 3: return launch_hc<D, 3>(args, units, n_split, g_target, stream);
    case 4: return launch_hc<D, 4>(args, units, n_split, g_target, stream);
    case 5:
        if constexpr (max_head_chunk(D) >= 5) return launch_hc<D, 5>(args, units, n_split, g_target, stream);
        return hipErrorInvalidValue;
    case 6:
        if constexpr (max_head_chunk(D) >= 6) return launch_hc<D, 6>(args, units, n_split, g_target, stream);
        return hipErrorInvalidValue;
    case 7:
        if constexpr (max_head_chunk(D) >= 7) return launch_hc<D, 7>(args, units, n_split, g_target, stream);
        return hipErrorInvalidValue;
    case 8:
        if constexpr (max_head_chunk(D) >= 8) return launch_hc<D, 8>(args, units, n_split, g_target, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodePlan &plan, const float *q, const float *k_cache,
                         const float *v_cache, float *out, uint32_t num_heads,
                         uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                         uint32_t total_seq, float scale, void *workspace,
                         const DecodeAppend *append, hipStream_t stream,
                         const DecodeVarlen *varlen) {
    DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.cnt = static_cast<uint32_t *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + plan.part_offset);
    a.num_heads = num_heads;
    a.kv_heads = kv_heads;
    a.hpk = num_heads / kv_heads;
    a.n_chunks = plan.n_chunks;
    a.max_seq = max_seq;
    a.w0 = plan.w0;
    a.total_seq = append ? total_seq - 1 : total_seq;  // end of the split pass
    a.n_split = plan.n_split;
    a.rows_per_split = plan.rows_per_split;
    a.qscale = scale * kLog2e;
    if (append) {
        a.k_new = append->k_new;
        a.v_new = append->v_new;
        a.k_dst = append->k_cache;
        a.v_dst = append->v_cache;
        a.position = total_seq - 1;
        a.cos_t = append->cos_t;
        a.sin_t = append->sin_t;
        a.cs_stride = append->cs_stride;
    }
    if (varlen) {  // total_seq is then the bound the plan was made for
        a.lens = varlen->lens;
        a.len_add = varlen->len_add;
        a.seq_bound = varlen->seq_bound;
        a.window = varlen->window;
    }
    const uint32_t hc = plan.head_chunk, u = plan.units, ns = plan.n_split, gt = plan.g_target;
    switch (head_dim) {
    case 32: return launch_d<32>(hc, a, u, ns, gt, stream);
    case 64: return launch_d<64>(hc, a, u, ns, gt, stream);
    case 96: return launch_d<96>(hc, a, u, ns, gt, stream);
    case 128: return launch_d<128>(hc, a, u, ns, gt, stream);
    case 160: return launch_d<160>(hc, a, u, ns, gt, stream);
    case 192: return launch_d<192>(hc, a, u, ns, gt, stream);
    case 224: return launch_d<224>(hc, a, u, ns, gt, stream);
    case 256: return launch_d<256>(hc, a, u, ns, gt, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
