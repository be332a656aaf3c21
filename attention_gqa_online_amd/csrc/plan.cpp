// Work plans of the decode and prefill launches (declared in plan.hpp).
#include "plan.hpp"

namespace attn {
namespace {

inline uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

uint32_t clamp_cus(uint32_t cus) { return cus < 1 ? 1 : cus > kMaxCus ? kMaxCus : cus; }

}  // namespace

DecodePlan plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window, bool append,
                       bool varlen, uint32_t cus) {
    DecodePlan p{};
    if (kv_heads == 0 || num_heads < kv_heads) return p;  // no head: no work, no workspace
    cus = clamp_cus(cus);
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
    p.g_target = target_workgroups_varlen(p.units, cus);
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
    uint32_t n_split = ceil_div(cus, p.units);  // about one workgroup per compute unit
    n_split = n_split > max_split ? max_split : n_split;
    n_split = n_split > (uint32_t)kMaxSplit ? (uint32_t)kMaxSplit : n_split;
    n_split = n_split < 1 ? 1 : n_split;
    uint32_t rows = ceil_div(len, n_split);
    rows = ceil_div(rows, step) * step;
    p.rows_per_split = rows;
    p.n_split = ceil_div(len, rows);
    // per-sequence lengths: the proportional table has at most
    // g_target + units splits (used unless the plan has a single split and no
    // appended row)
    const size_t slots = varlen && !(p.n_split == 1 && !append)
                             ? (size_t)p.g_target + p.units
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

PrefillPlan plan_prefill(uint32_t m, uint32_t num_q_heads, uint32_t heads_per_kv,
                         uint32_t head_dim, uint32_t cus) {
    PrefillPlan p{};
    if (heads_per_kv == 0) return p;
    if (m <= (uint32_t)kSmallRows) {
        p.small = 1;
        p.waves = 4;
        p.grid = (num_q_heads + 3) / 4;
        return p;
    }
    cus = clamp_cus(cus);
    const uint32_t kv_heads = num_q_heads / heads_per_kv;
    p.n_rb = (m + kPrefillRows - 1) / kPrefillRows;
    p.n_pairs = heads_per_kv * p.n_rb;
    p.waves = 8;
    if (head_dim >= (uint32_t)kMinDim4Waves &&
        (uint64_t)(p.n_pairs + 3) / 4 * kv_heads >= 2ull * cus)
        p.waves = 4;
    p.wg_per_group = (p.n_pairs + p.waves - 1) / p.waves;
    // a grid under two workgroups per compute unit is bound by its heaviest
    // workgroup: pair short and long row blocks instead
    p.nsub = (heads_per_kv + p.waves / 2 - 1) / (p.waves / 2);
    if ((uint64_t)p.wg_per_group * kv_heads < 2ull * cus) {
        p.zigzag = 1;
        p.wg_per_group = (p.n_rb + 1) / 2 * p.nsub;
        if (head_dim >= (uint32_t)kMinDim4Waves && head_dim % 64 == 0 && p.waves == 8) {
            // 16-row blocks, a pair per wave: equal work for every wave, and
            // half the registers of a 32-row block (the 8-wave 32-row kernel
            // spills at these head sizes)
            p.rows16 = 1;
            p.n_rb16 = (m + 15) / 16;
            p.n_tasks16 = (p.n_rb16 + 1) / 2 * heads_per_kv;
            p.wg_per_group = (p.n_tasks16 + 7) / 8;
        }
    }
    p.grid = p.wg_per_group * kv_heads;
    return p;
}

}  // namespace attn
