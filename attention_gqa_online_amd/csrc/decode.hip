// Decode work plan and dispatch (kernel template in decode_kernel.hpp).
#include "decode_kernel.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kDecodeWaves = 4;          // waves per workgroup
constexpr int kPrefetch = 2;             // row steps in flight per wave
constexpr int kTargetWorkgroups = 256;   // one workgroup per CU, streaming long ranges
// Per-sequence lengths are only known on the device: each workgroup of the
// split pass evaluates the proportional table (a unit's share of the splits
// follows its rows, so every split holds about the same number of rows).
// The split counts are rounded up per unit, which adds about units / 2
// splits: the target leaves room for them, so the splits holding rows still
// fit one workgroup per CU.
constexpr uint32_t kTargetWorkgroupsVarlen(uint32_t units) {
    return units / 2 + 64 < (uint32_t)kTargetWorkgroups ? kTargetWorkgroups - units / 2 : 64;
}
constexpr int kMinRowsPerWave = 32;
constexpr size_t kCounterBlock = 65536;  // bytes of arrival counters: 16384 units

// Lanes that hold one K/V row. Short rows (head_dim 32, 64) take d / 8
// lanes, two float4 chunks each, as head_dim 128 does with 16: with one chunk
// per lane the per-row work (the lane-group sum, exp, running sums) would be
// paid for half the bytes and bound the loop by the vector ALU. Otherwise 16,
// or 8 where a lane's share of the row would not be whole float4 chunks
// (head_dim / 4 not a multiple of 16).
constexpr int lanes_per_row(int d) {
    return d == 32 ? 4 : d == 64 ? 8 : (d / 4) % 16 == 0 ? 16 : 8;
}

// Largest head chunk (at most 8) whose row-slot accumulators, [slots][HC][d]
// floats, fit the 160 KiB of LDS next to the kernel's other arrays, and whose
// registers (q and acc: about 10 per float4 of a lane's row share and head,
// the ring 16 per float4, about 100 more) fit the 512 a lane has at one wave
// per SIMD without spilling to scratch memory.
constexpr int max_head_chunk(int d) {
    const int slots = kDecodeWaves * (64 / lanes_per_row(d));
    const int lds_hc = (160 * 1024 - 4096) / (slots * d * 4);
    const int nf4 = d / lanes_per_row(d) / 4;  // float4 of a lane's row share
    const int reg_hc = (500 - 100 - 16 * nf4) / (10 * nf4);
    const int hc = lds_hc < reg_hc ? lds_hc : reg_hc;
    return hc < 8 ? hc : 8;
}

// One launch per call. With a single split per unit and no appended row
// each workgroup writes its unit's normalised output itself; otherwise the
// last workgroup of each unit to finish merges the units' partial states
// and the appended row (kMergeFused). With no row before the appended one
// (n_split 0) every unit gets one workgroup over an empty range, which only
// folds in the new row. With per-sequence lengths the grid holds the
// proportional splits and one more workgroup per unit, so the units with no
// rows in the split pass (idle, only the new row, invalid) get one each.
template <int D, int HC>
hipError_t launch_hc(DecodeArgs args, uint32_t units, uint32_t n_split, hipStream_t stream) {
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
    args.g_target = kTargetWorkgroupsVarlen(units);
    args.min_rows = kDecodeWaves * kMinRowsPerWave;
    args.rows_step = kDecodeWaves * (64 / LPR);
    hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves, kPrefetch, kMergeFused, true>),
                       dim3(args.g_target + units), dim3(kDecodeWaves * 64), 0, stream, args);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(uint32_t hc, const DecodeArgs &args, uint32_t units, uint32_t n_split,
                    hipStream_t stream) {
    // head chunks beyond max_head_chunk(D) are never planned (nor built)
    switch (hc) {
    case 1: return launch_hc<D, 1>(args, units, n_split, stream);
    case 2: return launch_hc<D, 2>(args, units, n_split, stream);
    case 3: return launch_hc<D, 3>(args, units, n_split, stream);
    case 4: return launch_hc<D, 4>(args, units, n_split, stream);
    case 5:
        if constexpr (max_head_chunk(D) >= 5) return launch_hc<D, 5>(args, units, n_split, stream);
        return hipErrorInvalidValue;
    case 6:
        if constexpr (max_head_chunk(D) >= 6) return launch_hc<D, 6>(args, units, n_split, stream);
        return hipErrorInvalidValue;
    case 7:
        if constexpr (max_head_chunk(D) >= 7) return launch_hc<D, 7>(args, units, n_split, stream);
        return hipErrorInvalidValue;
    case 8:
        if constexpr (max_head_chunk(D) >= 8) return launch_hc<D, 8>(args, units, n_split, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

inline uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

}  // namespace

DecodePlan plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window, bool append,
                       bool varlen) {
    DecodePlan p{};
    if (kv_heads == 0 || num_heads < kv_heads) return p;  // no head: no work, no workspace
    const uint32_t hpk = num_heads / kv_heads;
    uint32_t max_hc = 8;
    switch (head_dim) {  // the built head sizes (see max_head_chunk)
    case 32: max_hc = max_head_chunk(32); break;
    case 64: max_hc = max_head_chunk(64); break;
    case 96: max_hc = max_head_chunk(96); break;
    case 128: max_hc = max_head_chunk(128); break;
    case 160: max_hc = max_head_chunk(160); break;
    case 192: max_hc = max_head_chunk(192); break;
    case 224: max_hc = max_head_chunk(224); break;
    case 256: max_hc = max_head_chunk(256); break;
    default: break;
    }
    p.n_chunks = ceil_div(hpk, max_hc);
    p.head_chunk = ceil_div(hpk, p.n_chunks);
    p.units = batch * kv_heads * p.n_chunks;
    p.w0 = (window > 0 && total_seq > window) ? total_seq - window : 0;
    const uint32_t len = total_seq - p.w0 - (append ? 1 : 0);  // rows of the split pass
    if (len == 0) {  // only the appended row: no split pass
        p.n_split = 0;
        p.rows_per_split = 0;
        p.part_floats = 0;
        p.workspace_bytes = 0;
        return p;
    }
    const uint32_t rpt = 64 / lanes_per_row((int)head_dim);
    const uint32_t step = kDecodeWaves * rpt;
    const uint32_t max_split = ceil_div(len, (uint64_t)kDecodeWaves * kMinRowsPerWave);
    uint32_t n_split = ceil_div(kTargetWorkgroups, p.units);
    n_split = n_split > max_split ? max_split : n_split;
    n_split = n_split > (uint32_t)kMaxSplit ? (uint32_t)kMaxSplit : n_split;
    n_split = n_split < 1 ? 1 : n_split;
    uint32_t rows = ceil_div(len, n_split);
    rows = ceil_div(rows, step) * step;
    p.rows_per_split = rows;
    p.n_split = ceil_div(len, rows);
    // per-sequence lengths: the proportional table has at most
    // target + units splits (used unless the plan has a single split and no
    // appended row)
    const size_t slots = varlen && !(p.n_split == 1 && !append)
                             ? (size_t)kTargetWorkgroupsVarlen(p.units) + p.units
                             : (size_t)p.units * p.n_split;
    p.part_floats = slots * p.head_chunk * (head_dim + 4);  // kPartStride
    // arrival counters of the fused merge first (one per unit), then the
    // partial states. The counter block has one size for every shape up to
    // kCounterBlock / 4 units, so calls of different shapes can share a
    // workspace without one call's partial states landing on another's
    // counters.
    const size_t cnt_bytes = ((size_t)p.units * sizeof(uint32_t) + 255) / 256 * 256;
    p.part_offset = cnt_bytes > kCounterBlock ? cnt_bytes : kCounterBlock;
    p.workspace_bytes = p.part_offset + p.part_floats * sizeof(float);
    return p;
}

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
    const uint32_t hc = plan.head_chunk, u = plan.units, ns = plan.n_split;
    switch (head_dim) {
    case 32: return launch_d<32>(hc, a, u, ns, stream);
    case 64: return launch_d<64>(hc, a, u, ns, stream);
    case 96: return launch_d<96>(hc, a, u, ns, stream);
    case 128: return launch_d<128>(hc, a, u, ns, stream);
    case 160: return launch_d<160>(hc, a, u, ns, stream);
    case 192: return launch_d<192>(hc, a, u, ns, stream);
    case 224: return launch_d<224>(hc, a, u, ns, stream);
    case 256: return launch_d<256>(hc, a, u, ns, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
