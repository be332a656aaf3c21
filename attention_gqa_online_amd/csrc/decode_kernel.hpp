// Single-query GQA decode kernel (template). Included by decode.hip, which
// holds the work plan and the dispatch over head_dim and heads per chunk.
//
// What is computed follows the decode module of the glia honeycrisp
// "attention.rs" page (module doc, Params struct, window_start rule): for each
// head h, softmax over positions s in [w0, total_seq) of scale * <q[h], K[g, s]>
// weights the V rows of KV head g = h / repeat.
//
// Work decomposition (MI355X design; the page's kernel is one 32-lane SIMD
// group walking every position of one head in sequence):
//   unit  = (sequence b, KV head g, chunk of <= 8 Q heads of that group)
//   split = a contiguous range of attended rows; one workgroup of NW waves
//           (with per-sequence lengths, each unit gets splits in proportion
//           to its rows: prop_split)
//   wave  = every NW-th step of the split's range, RPT = 64/LPR rows per step
//   lane  = (row slot r, d-chunk c): LPR lanes cover one row's head_dim; lane
//           c holds float4 chunks c, c+LPR, ... so each global_load_dwordx4
//           of a row is LPR*16 contiguous bytes.
// Each K row is read from HBM once and used for all Q heads of the chunk (the
// GQA reuse the pages leave to L2). Loads run P steps ahead of the arithmetic
// through a register ring, so every wave keeps P*RPT rows of K and V in
// flight. The q.K dot of a row is reduced over its LPR lanes with DPP
// butterflies; every lane keeps its own online-softmax state for its row
// slot, so a step needs no cross-row reduction. The reference value m of a
// slot is fixed from its first step instead of being raised row by row: the
// result acc / l is the same for any m, so the loop carries no rescale (no
// branch, no multiply of the accumulators); it only tracks the largest
// score, and the rare wave whose scores climb more than kMaxHeadroom above m
// re-streams its rows once with m = that maximum.
// The row slots and waves of a workgroup merge through LDS into one partial
// state (m, l, acc[d]) per head, written to the workspace; the last
// workgroup of each unit to finish (an arrival counter per unit) folds the
// partial states of its heads with a running log-sum-exp and writes the
// normalised output (decode_fused_merge), all in one launch. When the call
// also appends the current token (attn_decode_append), the
// split pass covers the rows before it and the merge folds the new row in as
// one more partial state, scored from the new K row itself, and writes the
// new K and V rows into the caches (rotated first when the call applies
// rotary embedding; the split pass then rotates q as it loads it).
#pragma once

#include "common.hpp"

namespace attn {

constexpr float kMaxHeadroom = 64.0f;  // log2 units: p = 2^(s - m) <= 2^64
constexpr float kMinRef = -1.0e30f;    // reference floor for slots with no row

struct DecodeArgs {
    const float *q;
    const float *k;
    const float *v;
    float *out;
    uint32_t *cnt;    // [units] arrival counters of the fused merge: zero between calls
    float *part;      // [splits][HC][D + 4]: acc[D], m, l, 2 pad; split s of unit u at s * units + u
                      // (per-sequence lengths: proportional splits numbered unit by unit)
    // fused append (the merging workgroups): new rows [B, Hkv, D], or null
    const float *k_new;
    const float *v_new;
    float *k_dst;     // the caches, written at the appended row (`position`, or per sequence)
    float *v_dst;
    uint32_t position;
    // rotary embedding of the current token (rotate-half), or null:
    // cos/sin [D/2] for `position`, applied to q and to the new K rows;
    // sequence b's table starts cs_stride * b floats in (0: one shared table)
    const float *cos_t;
    const float *sin_t;
    uint32_t cs_stride;
    // per-sequence lengths, or null (then every sequence has the rows
    // [w0, total_seq) before the appended one): sequence b then has
    // T_b = lens[b] + len_add rows, valid when T_b <= seq_bound; with an
    // append (len_add = 1, lens = positions) the new row is row T_b - 1
    const uint32_t *lens;
    uint32_t len_add, seq_bound, window;
    // with per-sequence lengths the split pass gives each unit a share of
    // g_target workgroups in proportion to its rows (prop_split)
    uint32_t units, g_target, min_rows, rows_step;
    uint32_t num_heads, kv_heads, hpk, n_chunks, max_seq;
    uint32_t w0, total_seq, n_split, rows_per_split;
    float qscale;     // scale * log2(e): scores come out in log2 units
};

// Rows of sequence b: the split pass covers [w0, hi); `pos` is the appended
// row. An invalid per-sequence length (past seq_bound) gives valid = false
// and an empty range.
struct SeqRange {
    uint32_t w0, hi, pos;
    bool valid;
};

// The same from sequence b's per-sequence length value `len` (lens[b]).
__device__ __forceinline__ SeqRange seq_range_len(const DecodeArgs &a, uint32_t len) {
    const uint64_t t = (uint64_t)len + a.len_add;
    const bool valid = t <= a.seq_bound;
    const uint32_t T = valid ? (uint32_t)t : 0;
    const uint32_t w0 = (a.window > 0 && T > a.window) ? T - a.window : 0;
    return {w0, T > 0 ? T - a.len_add : 0, T > 0 ? T - 1 : 0, valid};
}

__device__ __forceinline__ SeqRange seq_range(const DecodeArgs &a, uint32_t b) {
    if (a.lens == nullptr) return {a.w0, a.total_seq, a.position, true};
    return seq_range_len(a, a.lens[b]);
}

// Rows of the split pass of unit u (per-sequence lengths).
__device__ __forceinline__ uint32_t unit_rows(const DecodeArgs &a, uint32_t u) {
    const SeqRange r = seq_range(a, (u / a.n_chunks) / a.kv_heads);
    return r.hi > r.w0 ? r.hi - r.w0 : 0;
}

// Split of a unit with L of the batch's T rows: n splits of `rows` rows, n
// about L * g_target / T (at least 1, at most one per min_rows rows), rows a
// multiple of rows_step. Both passes evaluate it identically.
struct PropSplit {
    uint32_t n, rows;
};

__device__ __forceinline__ PropSplit prop_split(const DecodeArgs &a, uint32_t L, uint64_t T) {
    if (L == 0) return {0, 0};
    const uint64_t want = ((uint64_t)L * a.g_target + T - 1) / T;
    const uint64_t cap = ((uint64_t)L + a.min_rows - 1) / a.min_rows;
    const uint32_t n0 = (uint32_t)(want < cap ? want : cap);
    uint32_t rows = (L + n0 - 1) / n0;
    rows = (rows + a.rows_step - 1) / a.rows_step * a.rows_step;
    return {(L + rows - 1) / rows, rows};
}

// The proportional split table is evaluated by each wave on its own (the
// waves of a workgroup compute it redundantly: no LDS, no barrier), over W
// active lanes (64, or 32 for a 32-thread workgroup). Lane l takes units
// l, l + W, ...; splits are numbered unit by unit.
template <int W>
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, W);
    return x;
}

template <int W>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, W);
        if (lane >= o) x += y;
    }
    return x;
}

// The batch's rows of the split pass.
template <int W>
__device__ __forceinline__ uint64_t prop_total(const DecodeArgs &a, int lane) {
    uint64_t t = 0;
    for (uint32_t u = lane; u < a.units; u += W) t += unit_rows(a, u);
    return wave_sum_u64<W>(t);
}

struct PropHit {
    uint32_t unit, first, n, rows;
    bool found;
    uint32_t len;  // the unit's per-sequence length value
};

// Workgroup w of the split pass: the unit holding split index w, first = its
// first split index, n its split count. The workgroups past the last split
// (S splits in all) take the units with no rows in the split pass, in unit
// order: workgroup S + k the k-th such unit (n = 0), which then has only its
// appended row, or is idle, or has an invalid length. With at most W units
// (the usual case) each lane loads its unit's length once and the table is
// one scan: a single dependent global load before the split pass can issue
// its first K/V loads.
template <int W>
__device__ __forceinline__ PropHit prop_locate(const DecodeArgs &a, uint32_t w, int lane) {
    if (a.units > W) {
        const uint64_t T = prop_total<W>(a, lane);
        uint32_t carry = 0;  // splits before this chunk
        for (uint32_t base = 0; base < a.units; base += W) {
            const uint32_t u = base + lane;
            const PropSplit ps = u < a.units ? prop_split(a, unit_rows(a, u), T) : PropSplit{0, 0};
            const uint32_t incl = wave_incl_scan<W>(ps.n, lane);
            const uint32_t S = carry + incl - ps.n;
            const unsigned long long mask = __ballot(ps.n != 0 && S <= w && w - S < ps.n);
            if (mask != 0) {
                const int src = __ffsll((long long)mask) - 1;
                const uint32_t un = (uint32_t)__shfl((int)u, src);
                return {un, (uint32_t)__shfl((int)S, src), (uint32_t)__shfl((int)ps.n, src),
                        (uint32_t)__shfl((int)ps.rows, src), true,
                        a.lens[(un / a.n_chunks) / a.kv_heads]};
            }
            carry += (uint32_t)__shfl((int)incl, W - 1);
        }
        uint32_t k = w - carry;  // past the last split: the k-th unit with no rows
        for (uint32_t base = 0; base < a.units; base += W) {
            const uint32_t u = base + lane;
            const bool z = u < a.units && unit_rows(a, u) == 0;
            const unsigned long long zm = __ballot(z);
            const uint32_t cnt = (uint32_t)__popcll(zm);
            if (k < cnt) {
                const uint32_t rank = (uint32_t)__popcll(zm & ((1ull << lane) - 1ull));
                const unsigned long long hm = __ballot(z && rank == k);
                const uint32_t un = base + (uint32_t)(__ffsll((long long)hm) - 1);
                return {un, 0, 0, 0, true, a.lens[(un / a.n_chunks) / a.kv_heads]};
            }
            k -= cnt;
        }
        return {0, 0, 0, 0, false, 0};
    }
    const uint32_t u = lane;
    const bool in = u < a.units;
    const uint32_t len = in ? a.lens[(u / a.n_chunks) / a.kv_heads] : 0;
    const SeqRange r = seq_range_len(a, len);
    const uint32_t L = in && r.hi > r.w0 ? r.hi - r.w0 : 0;
    const uint64_t T1 = wave_sum_u64<W>(L);
    const PropSplit ps = in ? prop_split(a, L, T1) : PropSplit{0, 0};
    const uint32_t incl = wave_incl_scan<W>(ps.n, lane);
    const uint32_t S = incl - ps.n;
    unsigned long long mask = __ballot(in && ps.n != 0 && S <= w && w - S < ps.n);
    if (mask == 0) {
        // past the last split: the k-th unit with no rows
        const uint32_t total = (uint32_t)__shfl((int)incl, W - 1);
        const uint32_t k = w - total;
        const bool z = in && ps.n == 0;
        const unsigned long long zm = __ballot(z);
        const uint32_t rank = (uint32_t)__popcll(zm & ((1ull << lane) - 1ull));
        mask = __ballot(z && rank == k);
        if (mask == 0) return {0, 0, 0, 0, false, 0};
        const int src = __ffsll((long long)mask) - 1;
        return {(uint32_t)src, 0, 0, 0, true, (uint32_t)__shfl((int)len, src)};
    }
    const int src = __ffsll((long long)mask) - 1;
    return {(uint32_t)__shfl((int)u, src), (uint32_t)__shfl((int)S, src),
            (uint32_t)__shfl((int)ps.n, src), (uint32_t)__shfl((int)ps.rows, src), true,
            (uint32_t)__shfl((int)len, src)};
}

// Floats per (split, head) partial state: acc[D], m, l and two floats of
// padding, so every state starts on a 16-byte boundary (float4 stores).
template <int D>
constexpr int kPartStride = D + 4;

// kMergeFused: every workgroup writes one partial state per head, and the
// last workgroup of a unit to finish folds every split's state (and the
// appended row) and writes out. kMergeDirect: a single split per unit and no
// appended row, so each workgroup writes its unit's normalised output.
enum DecodeMerge { kMergeFused = 2, kMergeDirect = 3 };

// Partial states that another workgroup of the same launch reads back go
// through agent-scope (relaxed) atomic stores and loads, 8 bytes each.
//
// Why the merge needs no fence. The LLVM AMDGPU backend's user guide
// (AMDGPUUsage, "Memory Model GFX942", whose code sequences the backend also
// uses for gfx950) gives, for global memory at agent scope:
//   - load atomic monotonic      -> global_load   ... sc1=1
//   - store atomic monotonic     -> global_store  ... sc1=1
//   - atomicrmw monotonic        -> global_atomic ... sc1=1
//   - fence release              -> buffer_wbl2 sc1=1; s_waitcnt vmcnt(0)
//   - fence acquire              -> s_waitcnt vmcnt(0); buffer_inv sc1=1
// So an sc1 store is by itself coherent at agent scope (written through the
// XCD's L2, and complete only once every XCD can see it), and an sc1 load by
// itself reads the agent-coherent value (it never takes a line another XCD
// may have changed). The release fence's buffer_wbl2 writes back what plain
// stores left in the L2, and the acquire's buffer_inv drops what plain loads
// could find stale there; the partial states are written and read only with
// the sc1 accesses above, so neither is needed, and neither is issued (they
// act on the XCD's whole L2 and measured 2-5x slower). What remains of the
// release is its s_waitcnt vmcnt(0): every state store of the workgroup is
// complete before the arrival counter moves (decode_fused_merge). What
// remains of the acquire: the merging workgroup issues its state loads only
// after the counter's returned value has arrived and passed through a
// barrier, in program order. The compiler is kept from moving the accesses
// across those points by signal fences (code-free compiler barriers). The
// tests that poison the workspace before each call and that compare
// repeated calls bit for bit guard this at run time.
__device__ __forceinline__ void st_dev2(float *p, float x, float y) {
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, x) |
                       ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float *p) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__builtin_bit_cast(float, (uint32_t)v),
                       __builtin_bit_cast(float, (uint32_t)(v >> 32)));
}

// Merge of the split pass (kMergeFused), run by every workgroup after its
// slot merge. Each workgroup holds its own partial state in registers, one
// (head, 4 consecutive d) item per thread (two for the largest head chunks).
// With several splits per unit it stores that state, waits until the stores
// are acknowledged, and one thread counts the split in on the unit's
// arrival counter; the workgroup that brings the count to n_split is the
// last and the only one to go on (it also returns the counter to 0 for the
// next call). That workgroup folds, with a running log-sum-exp (M, num, den)
// per item: the appended row (state m = its score, l = 1, acc = v_new; the
// score is summed over the items of a head in LDS), then every split's state
// in index order, and writes acc / l. It also writes the new K and V rows
// into the caches (chunk 0 of each KV head).
// Where a unit's partial states live: ns splits, split s at slot
// slot0 + s * sstride, this workgroup's at `mine`; `pos` is the sequence's
// appended row and valid = false marks an invalid per-sequence length.
struct MergeSlots {
    uint32_t ns;
    size_t slot0, sstride, mine;
    uint32_t pos;
    bool valid;
};

template <int D, int HC, int NW, typename SlotMerge>
__device__ __forceinline__ void decode_fused_merge(const DecodeArgs &a, SlotMerge &slot_merge,
                                                   int tid, uint32_t unit, const MergeSlots &ms,
                                                   uint32_t b, uint32_t bg, uint32_t h0,
                                                   uint32_t hl0, int nh) {
    constexpr int NT = NW * 64;
    constexpr int NV = HC * D / 4;  // items
    constexpr int NITEM = (NV + NT - 1) / NT;
    constexpr int PS = kPartStride<D>;
    __shared__ __attribute__((aligned(16))) float s_dot[HC][D / 4];
    __shared__ uint32_t s_last;

    // item it of this thread; threads past NV repeat the last item and
    // store nothing
    int hv[NITEM], dv[NITEM];
    bool own[NITEM];
    float4 num[NITEM];
    float M[NITEM], den[NITEM];
#pragma unroll
    for (int it = 0; it < NITEM; ++it) {
        const int v0 = tid + it * NT;
        own[it] = v0 < NV;
        const int v = own[it] ? v0 : NV - 1;
        hv[it] = v / (D / 4);
        dv[it] = 4 * (v % (D / 4));
        slot_merge(v, num[it], M[it], den[it], true);
    }

    if (!ms.valid) {  // an invalid length: NaN output, nothing appended
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            if (!own[it] || hv[it] >= nh) continue;
            const float nan = __builtin_nanf("");
            st4(a.out + ((size_t)b * a.num_heads + h0 + hv[it]) * D + dv[it],
                make_float4(nan, nan, nan, nan));
        }
        return;
    }
    const uint32_t ns = ms.ns;
    if (ns > 1) {
        float *mypart = a.part + ms.mine * HC * PS;
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            if (!own[it]) continue;
            float *ph = mypart + hv[it] * PS;
            st_dev2(ph + dv[it], num[it].x, num[it].y);
            st_dev2(ph + dv[it] + 2, num[it].z, num[it].w);
            if (dv[it] == 0) st_dev2(ph + D, M[it], den[it]);
        }
        // The release half (see st_dev2): every thread's sc1 stores are
        // complete (s_waitcnt vmcnt(0)) before the barrier, and the count
        // goes up only after it. The signal fences keep the compiler from
        // moving a store below the wait or the counter above it.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) {
            const uint32_t prev =
                __hip_atomic_fetch_add(a.cnt + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = prev == ns - 1;
            if (last) __hip_atomic_store(a.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last ? 1u : 0u;
        }
        __syncthreads();
        // The acquire half: the state loads below (sc1) issue only after
        // the counter's value came back and every thread saw it; the fence
        // keeps the compiler from hoisting them above this point.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (s_last == 0) return;
    }

    // Fold in a fixed order, whichever workgroup merges (run-to-run
    // deterministic): the appended row first, then the splits by index, all
    // read back from the workspace (this workgroup's own state too), eight
    // per round as independent loads; entries of a round past ns re-read the
    // last split with weight 0. With a single split its state is still in
    // registers.
    float4 xo[NITEM];
    float Mo[NITEM], Lo[NITEM];
#pragma unroll
    for (int it = 0; it < NITEM; ++it) {
        xo[it] = num[it];
        Mo[it] = M[it];
        Lo[it] = den[it];
        num[it] = make_float4(0.f, 0.f, 0.f, 0.f);
        M[it] = kNegInf;
        den[it] = 0.f;
    }
    float2 ml[NITEM][8];
    float4 xs[NITEM][8];
    auto load_round = [&](uint32_t s0) {
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sp = min(s0 + i, ns - 1);
                const float *ps = a.part + (ms.slot0 + sp * ms.sstride) * HC * PS + hv[it] * PS;
                ml[it][i] = ld_dev2(ps + D);
                const float2 lo = ld_dev2(ps + dv[it]);
                const float2 hi = ld_dev2(ps + dv[it] + 2);
                xs[it][i] = make_float4(lo.x, lo.y, hi.x, hi.y);
                if (s0 + i >= ns) ml[it][i].x = kNegInf;
            }
        }
    };
    auto fold_round = [&](int n) {
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            float Mn = M[it];
            for (int i = 0; i < n; ++i) Mn = fmaxf(Mn, ml[it][i].x);
            const float c = M[it] == kNegInf ? 0.f : fast_exp2(M[it] - Mn);
            num[it] = num[it] * c;
            den[it] *= c;
            for (int i = 0; i < n; ++i) {
                const float w = ml[it][i].x == kNegInf ? 0.f : fast_exp2(ml[it][i].x - Mn);
                num[it].x += xs[it][i].x * w;
                num[it].y += xs[it][i].y * w;
                num[it].z += xs[it][i].z * w;
                num[it].w += xs[it][i].w * w;
                den[it] += ml[it][i].y * w;
            }
            M[it] = Mn;
        }
    };
    if (ns > 1) load_round(0);  // in flight while the new row is scored

    if (a.k_new != nullptr) {
        float4 kn[NITEM], vn[NITEM];
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            const int hh = hv[it], d = dv[it];
            const int hq = hh < nh ? hh : nh - 1;  // heads past nh: in bounds, never stored
            const float *qp = a.q + ((size_t)b * a.num_heads + h0 + hq) * D + d;
            const float *kp = a.k_new + (size_t)bg * D + d;
            float4 qd = ld4(qp);
            kn[it] = ld4(kp);
            vn[it] = ld4(a.v_new + (size_t)bg * D + d);
            if (a.cos_t != nullptr) {  // rotate-half: q and the new K row
                const bool lo = d < D / 2;
                const int off = lo ? D / 2 : -D / 2;
                const size_t ci = (size_t)b * a.cs_stride + (d % (D / 2));
                const float4 cc = ld4(a.cos_t + ci);
                const float4 ss = ld4(a.sin_t + ci);
                kn[it] = rope_half(kn[it], ld4(kp + off), cc, ss, lo);
                qd = rope_half(qd, ld4(qp + off), cc, ss, lo);
            }
            if (own[it]) s_dot[hh][d / 4] = dot4(qd * a.qscale, kn[it]);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            // the new row's state: m = its score (log2 units), l = 1, acc = v_new
            float sc = 0.f;
#pragma unroll
            for (int j = 0; j < D / 4; j += 4) {
                const float4 y = ld4(&s_dot[hv[it]][j]);
                sc += (y.x + y.y) + (y.z + y.w);
            }
            M[it] = sc;
            num[it] = vn[it];
            den[it] = 1.f;
            if (hl0 == 0 && hv[it] == 0 && own[it]) {  // one writer per (sequence, KV head)
                const size_t dst = ((size_t)bg * a.max_seq + ms.pos) * D + dv[it];
                st4(a.k_dst + dst, kn[it]);
                st4(a.v_dst + dst, vn[it]);
            }
        }
    }

    if (ns > 1) {
        fold_round(8);
        for (uint32_t s0 = 8; s0 < ns; s0 += 8) {
            load_round(s0);
            fold_round(8);
        }
    } else {
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            ml[it][0] = make_float2(Mo[it], Lo[it]);
            xs[it][0] = xo[it];
        }
        fold_round(1);
    }
#pragma unroll
    for (int it = 0; it < NITEM; ++it) {
        if (!own[it] || hv[it] >= nh) continue;
        // den is 0 only for an idle sequence (no rows, nothing appended): 0
        const bool zero = !(den[it] > 0.f);
        const float4 o = zero ? make_float4(0.f, 0.f, 0.f, 0.f)
                              : make_float4(num[it].x / den[it], num[it].y / den[it],
                                            num[it].z / den[it], num[it].w / den[it]);
        st4(a.out + ((size_t)b * a.num_heads + h0 + hv[it]) * D + dv[it], o);
    }
}

// VARLEN: per-sequence lengths (a.lens set); without, the code for them is not
// compiled in, so the uniform kernel carries none of its registers.
template <int D, int HC, int LPR, int NW, int P, int MERGE, bool VARLEN>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
    constexpr int VPL = D / LPR;   // floats per lane per row
    constexpr int NF4 = VPL / 4;   // float4 per lane per row
    constexpr int RPT = 64 / LPR;  // rows per wave step (row slots)
    constexpr int NSLOT = NW * RPT;
    static_assert(VPL % 4 == 0 && LPR * VPL == D, "lane tiling");

    __shared__ __attribute__((aligned(16))) float s_acc[NSLOT][HC][D];  // per row slot accumulators
    __shared__ float s_m[HC][NSLOT];       // per row slot reference m and sum l
    __shared__ float s_l[HC][NSLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane / LPR;
    const int c = lane % LPR;
    const int slot = wave * RPT + r;

    // split-major numbering: the splits of a unit are units apart, so with
    // units a multiple of 8 they land on one XCD (workgroups go round-robin
    // over the 8 XCDs)
    uint32_t split = blockIdx.x / a.units;
    uint32_t unit = blockIdx.x % a.units;
    uint32_t rps = a.rows_per_split;
    bool have_len = false;  // the unit's length value is already in `len`
    uint32_t len = 0;
    MergeSlots msl{a.n_split, unit, a.units, blockIdx.x, a.position, true};
    if constexpr (MERGE == kMergeFused && VARLEN) {
        {
            // per-sequence lengths: workgroup w is split w - first(u) of the
            // unit u whose splits include w (proportional table), or takes a
            // unit with no rows (an empty range, then only the merge)
            const PropHit ph = prop_locate<64>(a, blockIdx.x, lane);
            if (!ph.found) return;  // past the last unit (uniform)
            unit = ph.unit;
            split = ph.n != 0 ? blockIdx.x - ph.first : 0;
            rps = ph.rows;
            len = ph.len;
            have_len = true;
            msl = MergeSlots{ph.n != 0 ? ph.n : 1u, ph.first, 1, blockIdx.x, 0, true};
        }
    }
    const uint32_t chunk = unit % a.n_chunks;
    const uint32_t bg = unit / a.n_chunks;  // b * kv_heads + g
    const uint32_t g = bg % a.kv_heads;
    const uint32_t b = bg / a.kv_heads;
    const uint32_t hl0 = chunk * HC;
    const int nh = min(HC, (int)(a.hpk - hl0));
    const uint32_t h0 = g * a.hpk + hl0;

    // rows of this workgroup, then of this wave: every NW-th step of the
    // workgroup's range, so the workgroup streams one contiguous region
    const SeqRange sr = !VARLEN ? SeqRange{a.w0, a.total_seq, a.position, true}
                        : have_len ? seq_range_len(a, len)
                                   : seq_range(a, b);
    msl.pos = sr.pos;
    msl.valid = sr.valid;
    const uint32_t ws0 = sr.w0 + split * rps;
    const uint32_t ws1 = min(ws0 + rps, sr.hi);
    const uint32_t ra = ws0 + wave * RPT;
    const uint32_t rb = ws1;
    constexpr uint32_t kStride = NW * RPT;  // rows between a wave's steps
    const uint32_t ntile = rb > ra ? (rb - ra + kStride - 1) / kStride : 0;

    const size_t cache_base = (size_t)bg * a.max_seq * D + 4 * c;
    const float *kb = a.k + cache_base;
    const float *vb = a.v + cache_base;

    // Online softmax state of this lane's row slot, per head: reference m,
    // l = sum 2^(s - m), acc = sum 2^(s - m) V, and the largest score seen.
    // m is fixed from the slot's first step (floored at kMinRef, so masked
    // rows, score -inf, give 2^(s - m) = 0 and never NaN) and is not raised
    // in the loop: exact for any m, and p stays finite while scores stay
    // below m + kMaxHeadroom. A wave whose scores ever exceed that redoes
    // its range with m = the true maximum (a second pass that cannot overflow).
    float m[HC], mx[HC], l[HC];
    float4 acc[HC][NF4];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
        m[hh] = kMinRef;
        mx[hh] = kNegInf;
        l[hh] = 0.f;
#pragma unroll
        for (int t = 0; t < NF4; ++t) acc[hh][t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    if (ntile > 0) {
        // ring of P row steps in flight, issued first so that the q loads
        // below wait under them; rows past rb are clamped to rb - 1 (in
        // bounds, masked out of the softmax)
        float4 kf[P][NF4], vf[P][NF4];
#pragma unroll
        for (int s = 0; s < P; ++s) {
            if (s > 0 && s >= (int)ntile) break;  // a ring slot no step uses: no load
            const size_t off = (size_t)min(ra + s * kStride + r, rb - 1) * D;
#pragma unroll
            for (int t = 0; t < NF4; ++t) kf[s][t] = ld4_stream(kb + off + 4 * LPR * t);
#pragma unroll
            for (int t = 0; t < NF4; ++t) vf[s][t] = ld4_stream(vb + off + 4 * LPR * t);
        }

        // q of every head of the chunk, pre-scaled (zero for heads past nh;
        // those re-read the last valid head so the load stays in bounds)
        float4 qv[HC][NF4];
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
            const int hq = hh < nh ? hh : nh - 1;
            const float *qh = a.q + ((size_t)b * a.num_heads + h0 + hq) * D + 4 * c;
            const float qs = hh < nh ? a.qscale : 0.f;
#pragma unroll
            for (int t = 0; t < NF4; ++t) qv[hh][t] = ld4(qh + 4 * LPR * t);
            if (a.cos_t != nullptr) {
                // rotate-half rotary embedding of this head's q: element d0
                // pairs with d0 +- D/2 and turns by cos/sin[d0 mod D/2]
#pragma unroll
                for (int t = 0; t < NF4; ++t) {
                    const int d0 = 4 * (c + LPR * t);
                    const bool lo = d0 < D / 2;
                    const float4 xp = ld4(qh + 4 * LPR * t + (lo ? D / 2 : -D / 2));
                    const size_t ci = (size_t)b * a.cs_stride + (d0 % (D / 2));
                    const float4 cc = ld4(a.cos_t + ci);
                    const float4 ss = ld4(a.sin_t + ci);
                    qv[hh][t] = rope_half(qv[hh][t], xp, cc, ss, lo);
                }
            }
#pragma unroll
            for (int t = 0; t < NF4; ++t) qv[hh][t] = qv[hh][t] * qs;
        }

        // one row step: scores of `row` from kf, softmax weights, V accumulate.
        // Rows past rb (only in a range's last step) get score -inf: the
        // penalty seeds the dot product, so masking costs no extra op.
        auto step = [&](const float4 (&kf)[NF4], const float4 (&vf)[NF4], uint32_t row) {
            const float pen = row < rb ? 0.f : kNegInf;
            float sc[HC];
#pragma unroll
            for (int hh = 0; hh < HC; ++hh) {
                sc[hh] = pen;
#pragma unroll
                for (int t = 0; t < NF4; ++t) sc[hh] = fma4(sc[hh], qv[hh][t], kf[t]);
            }
            group_sum_n<LPR>(sc);
#pragma unroll
            for (int hh = 0; hh < HC; ++hh) {
                mx[hh] = fmaxf(mx[hh], sc[hh]);
                const float p = fast_exp2(sc[hh] - m[hh]);
                l[hh] += p;
#pragma unroll
                for (int t = 0; t < NF4; ++t) {
                    acc[hh][t].x += p * vf[t].x;
                    acc[hh][t].y += p * vf[t].y;
                    acc[hh][t].z += p * vf[t].z;
                    acc[hh][t].w += p * vf[t].w;
                }
            }
        };

        {
            // reference m from the first step's scores
            {
                const float pen = ra + r < rb ? 0.f : kNegInf;
                float sc[HC];
#pragma unroll
                for (int hh = 0; hh < HC; ++hh) {
                    sc[hh] = pen;
#pragma unroll
                    for (int t = 0; t < NF4; ++t) sc[hh] = fma4(sc[hh], qv[hh][t], kf[0][t]);
                }
                group_sum_n<LPR>(sc);
#pragma unroll
                for (int hh = 0; hh < HC; ++hh) m[hh] = fmaxf(sc[hh], kMinRef);
            }
            // Steady state: groups of P steps, each refilling its ring slot
            // with the step P ahead. The last P steps load nothing: a load no
            // step consumes would still hold its registers, and the first
            // reuse of them after the loop would wait for its HBM round trip.
            const uint32_t nref = ntile > (uint32_t)P ? ntile - P : 0;  // steps that refill
            uint32_t base = 0;
            for (; base + P <= nref; base += P) {
#pragma unroll
                for (int s = 0; s < P; ++s) {
                    const uint32_t row = ra + (base + s) * kStride + r;
                    step(kf[s], vf[s], row);
                    const size_t off = (size_t)min(row + P * kStride, rb - 1) * D;
#pragma unroll
                    for (int t = 0; t < NF4; ++t) kf[s][t] = ld4_stream(kb + off + 4 * LPR * t);
#pragma unroll
                    for (int t = 0; t < NF4; ++t) vf[s][t] = ld4_stream(vb + off + 4 * LPR * t);
                }
            }
            // tail: the remaining (fewer than 2P) steps, refilling only while a
            // step P ahead exists (uniform branches)
#pragma unroll
            for (int s = 0; s < 2 * P - 1; ++s) {
                if (base + s < ntile) {
                    const uint32_t row = ra + (base + s) * kStride + r;
                    step(kf[s % P], vf[s % P], row);
                    if (base + s + P < ntile) {
                        const size_t off = (size_t)min(row + P * kStride, rb - 1) * D;
#pragma unroll
                        for (int t = 0; t < NF4; ++t)
                            kf[s % P][t] = ld4_stream(kb + off + 4 * LPR * t);
#pragma unroll
                        for (int t = 0; t < NF4; ++t)
                            vf[s % P][t] = ld4_stream(vb + off + 4 * LPR * t);
                    }
                }
            }
        }

        bool ovf = false;
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) ovf |= mx[hh] > m[hh] + kMaxHeadroom;
        if (__any(ovf)) {
            // rare: redo this wave's range against the exact per-slot maximum
#pragma unroll
            for (int hh = 0; hh < HC; ++hh) {
                m[hh] = fmaxf(mx[hh], kMinRef);
                l[hh] = 0.f;
#pragma unroll
                for (int t = 0; t < NF4; ++t) acc[hh][t] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (uint32_t i = 0; i < ntile; ++i) {
                const uint32_t row = ra + i * kStride + r;
                const size_t off = (size_t)min(row, rb - 1) * D;
                float4 kf[NF4], vf[NF4];
#pragma unroll
                for (int t = 0; t < NF4; ++t) kf[t] = ld4(kb + off + 4 * LPR * t);
#pragma unroll
                for (int t = 0; t < NF4; ++t) vf[t] = ld4(vb + off + 4 * LPR * t);
                step(kf, vf, row);
            }
        }
    }

    // The row slots merge in LDS with one barrier: every slot stores its
    // state (acc, m, l) as it is; a thread then takes the per-head maximum M
    // of the slots' m and sums 2^(m - M) acc over the slots, four consecutive
    // d at a time, with every LDS read in flight at once.
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
#pragma unroll
        for (int t = 0; t < NF4; ++t) st4(&s_acc[slot][hh][4 * (c + LPR * t)], acc[hh][t]);
        if (c == 0) {
            s_m[hh][slot] = m[hh];
            s_l[hh][slot] = l[hh];
        }
    }
    __syncthreads();

    // one (head hh, four consecutive d) item of this workgroup's partial
    // state: acc[d..d+3], the slots' maximum M and L = sum 2^(m - M) l
    auto slot_merge = [&](int v, float4 &x, float &M, float &lsum, bool want_l) {
        const int hh = v / (D / 4);
        const int d = 4 * (v % (D / 4));
        float ws[NSLOT];
        M = kNegInf;
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) {
            ws[sl] = s_m[hh][sl];
            M = fmaxf(M, ws[sl]);
        }
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) ws[sl] = fast_exp2(ws[sl] - M);  // m, M >= kMinRef: no NaN
        x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) {
            const float4 y = ld4(&s_acc[sl][hh][d]);
            x.x += ws[sl] * y.x;
            x.y += ws[sl] * y.y;
            x.z += ws[sl] * y.z;
            x.w += ws[sl] * y.w;
        }
        lsum = 0.f;
        if (want_l) {
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) lsum += ws[sl] * s_l[hh][sl];
        }
    };

    if constexpr (MERGE == kMergeFused) {
        decode_fused_merge<D, HC, NW>(a, slot_merge, tid, unit, msl, b, bg, h0, hl0, nh);
        return;
    }

    // a single split and no appended row: the normalised output directly
    for (int v = tid; v < HC * D / 4; v += NW * 64) {
        const int hh = v / (D / 4);
        const int d = 4 * (v % (D / 4));
        float4 x;
        float M, lsum;
        slot_merge(v, x, M, lsum, true);
        // no rows (an idle sequence): 0; an invalid length: NaN
        const bool nan = !sr.valid, zero = !(lsum > 0.f);
        float4 o;
        o.x = nan ? __builtin_nanf("") : zero ? 0.f : x.x / lsum;
        o.y = nan ? __builtin_nanf("") : zero ? 0.f : x.y / lsum;
        o.z = nan ? __builtin_nanf("") : zero ? 0.f : x.z / lsum;
        o.w = nan ? __builtin_nanf("") : zero ? 0.f : x.w / lsum;
        if (hh < nh) st4(a.out + ((size_t)b * a.num_heads + h0 + hh) * D + d, o);
    }
}

}  // namespace attn
