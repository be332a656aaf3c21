// Test-only C wrapper of the launch plans (attention_gqa_online_amd/csrc/
// plan.hpp). tests/test_plan.py builds it with plan.cpp using the host
// compiler: the plans are plain arithmetic, so they are checked on the CPU
// at any compute-unit count.
#include <stdint.h>

#include "plan.hpp"

extern "C" {

// out: head_chunk, n_chunks, units, n_split, rows_per_split, w0, g_target,
// part_floats, part_offset, workspace_bytes
void probe_plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window, int append,
                       int varlen, uint32_t cus, uint64_t *out) {
    const attn::DecodePlan p = attn::plan_decode(batch, num_heads, kv_heads, head_dim,
                                                 total_seq, window, append != 0, varlen != 0,
                                                 cus);
    out[0] = p.head_chunk;
    out[1] = p.n_chunks;
    out[2] = p.units;
    out[3] = p.n_split;
    out[4] = p.rows_per_split;
    out[5] = p.w0;
    out[6] = p.g_target;
    out[7] = p.part_floats;
    out[8] = p.part_offset;
    out[9] = p.workspace_bytes;
}

// out: waves, n_rb, n_pairs, zigzag, nsub, wg_per_group, grid, rows16, n_rb16,
// n_tasks16, small
void probe_plan_prefill(uint32_t m, uint32_t num_q_heads, uint32_t heads_per_kv,
                        uint32_t head_dim, uint32_t cus, uint64_t *out) {
    const attn::PrefillPlan p =
        attn::plan_prefill(m, num_q_heads, heads_per_kv, head_dim, cus);
    out[0] = p.waves;
    out[1] = p.n_rb;
    out[2] = p.n_pairs;
    out[3] = p.zigzag;
    out[4] = p.nsub;
    out[5] = p.wg_per_group;
    out[6] = p.grid;
    out[7] = p.rows16;
    out[8] = p.n_rb16;
    out[9] = p.n_tasks16;
    out[10] = p.small;
}

uint32_t probe_max_cus(void) { return attn::kMaxCus; }

}  // extern "C"
