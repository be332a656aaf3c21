// Work plans of the decode and prefill launches: plain host arithmetic (no
// HIP call, no device code), shared by the C ABI, the launchers and the
// kernels' compile-time constants, and testable on any host.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace attn {

// Most compute units a gfx950 device has (a whole MI355X: 8 XCDs of 32).
// Plans follow the device's own count, clamped to this; the decode workspace
// size is computed for it, which covers every smaller count (a plan never
// needs more workspace on fewer compute units).
constexpr uint32_t kMaxCus = 256;

// ---------------------------------------------------------------- decode
constexpr int kDecodeWaves = 4;       // waves per workgroup
constexpr int kPrefetch = 2;          // row steps in flight per wave
constexpr int kMinRowsPerWave = 32;   // shortest range worth a workgroup, per wave
constexpr size_t kCounterBlock = 65536;  // bytes of arrival counters: 16384 units
constexpr int kMaxSplit = 1024;       // most splits per unit

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

// Per-sequence lengths are only known on the device: each workgroup of the
// split pass evaluates the proportional table (a unit's share of the splits
// follows its rows, so every split holds about the same number of rows).
// The split counts are rounded up per unit, which adds about units / 2
// splits: the target leaves room for them, so the splits holding rows still
// fit one workgroup per compute unit.
constexpr uint32_t target_workgroups_varlen(uint32_t units, uint32_t cus) {
    return units / 2 + 64 < cus ? cus - units / 2 : 64;
}

// Work split of one decode call: the attended rows [w0, total_seq) of every
// (sequence, KV head, head chunk) unit are cut into n_split contiguous row
// ranges of rows_per_split rows, one workgroup each, so that the grid is
// about one workgroup per compute unit.
struct DecodePlan {
    uint32_t head_chunk;      // Q heads handled per workgroup (<= 8)
    uint32_t n_chunks;        // head chunks per KV head
    uint32_t units;           // batch * kv_heads * n_chunks
    uint32_t n_split;         // workgroups per unit
    uint32_t rows_per_split;  // multiple of the rows one workgroup step covers
    uint32_t w0;              // first attended row
    uint32_t g_target;        // per-sequence lengths: workgroups of the proportional table
    size_t part_floats;       // partial-state floats in the workspace
    size_t part_offset;       // bytes before them: the units' arrival counters
    size_t workspace_bytes;   // counters + partial states (the whole workspace)
};

// With `append`, the split pass covers [w0, total_seq - 1) and the last row
// comes from the new K/V rows instead (n_split may then be 0). With
// `varlen`, total_seq is the bound of the per-sequence lengths. `cus` is the
// device's compute-unit count (clamped to [1, kMaxCus]).
DecodePlan plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window, bool append,
                       bool varlen, uint32_t cus);

// ---------------------------------------------------------------- prefill
constexpr int kPrefillRows = 32;       // query rows per wave (one MFMA block)
constexpr int kMinDim4Waves = 192;     // head_dim from which large grids use 4-wave workgroups
constexpr int kSmallRows = 16;         // m up to this: one wave per Q head, no LDS (small)

// Grid of one prefill call. Prompts of at most kSmallRows rows take the
// small kernel (one wave per Q head reads its Q, K and V rows straight into
// registers). Otherwise workgroups of `waves` waves share one KV head;
// row-block-major (wave w of workgroup i owns (row block, head) pair
// i*waves + w of its group), or, on grids under two workgroups per compute
// unit, zigzag (the first half of the waves take row block u, the second
// half row block n_rb-1-u, nsub workgroups per pair of row blocks). Zigzag
// grids of head_dim 192 or 256 use 16-row blocks instead (rows16): every
// wave takes the 16-row blocks u and n_rb16-1-u of one head, one after the
// other, so all waves carry the same work; task t = u * heads_per_kv + head
// of a KV head's list goes to wave t mod 8 of its workgroup t / 8.
struct PrefillPlan {
    uint32_t waves;         // 8, or 4 for head_dim >= kMinDim4Waves on large grids
    uint32_t n_rb;          // ceil(m / 32)
    uint32_t n_pairs;       // heads_per_kv * n_rb
    uint32_t zigzag;        // 1: row blocks u and n_rb-1-u share a workgroup
    uint32_t nsub;          // zigzag: workgroups per row-block pair
    uint32_t wg_per_group;  // workgroups per KV head
    uint32_t grid;          // wg_per_group * kv_heads
    uint32_t rows16;        // 1: the 16-row kernel (then the fields below)
    uint32_t n_rb16;        // ceil(m / 16)
    uint32_t n_tasks16;     // ceil(n_rb16 / 2) * heads_per_kv per KV head
    uint32_t small;         // 1: m <= kSmallRows, one wave per Q head in 4-wave
                            // workgroups (grid = ceil(num_q_heads / 4)); the
                            // fields above are then unused
};

PrefillPlan plan_prefill(uint32_t m, uint32_t num_q_heads, uint32_t heads_per_kv,
                         uint32_t head_dim, uint32_t cus);

}  // namespace attn
