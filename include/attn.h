/*
 * attn.h -- fused grouped-query attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so: three operations, the decode step that combines the
 * last two, and their serving forms. Every entry point is one kernel launch
 * on the caller's stream (decode merges its splits inside that launch):
 *
 *   attn_prefill_causal   causal self-attention over a packed projection output
 *   attn_decode           single-query attention over a KV cache, optional
 *                         sliding window
 *   kv_append             write one new K row and V row per (sequence, KV head)
 *                         into the caches
 *   attn_decode_append    kv_append + attn_decode of the same token in one launch
 *   attn_decode_rope_append
 *                         the same decode step with rotary position embedding
 *                         applied to q and to the new K rows on the way in
 *   attn_decode_append_noalloc
 *                         attn_decode_append without a workspace argument,
 *                         for callers that cannot allocate
 *   kv_append_rows        write a prefill pass's K and V rows into a
 *                         sequence's caches (prefill -> decode hand-over)
 *   attn_decode_varlen    attn_decode with one length per sequence
 *   attn_decode_append_varlen
 *                         attn_decode_append with one position per sequence
 *   attn_decode_rope_append_varlen
 *                         attn_decode_rope_append with one position (and one
 *                         rotary table) per sequence
 *
 * Common rules
 *   - Every tensor is fp32, row-major. Every pointer is a DEVICE pointer owned
 *     by the caller; the library allocates nothing and keeps no state across
 *     calls apart from the decode workspace the caller passes in.
 *   - Grouped-query head map: Q head h reads KV head h / heads_per_kv
 *     (integer division), so consecutive Q heads share a KV head.
 *   - Calls are asynchronous on `stream` (0 = the default stream). They
 *     return after the launch; errors inside the kernel surface at the
 *     caller's next synchronisation. All argument checks run on the host
 *     before any HIP call, so an invalid call launches nothing. The work
 *     split follows the current device's compute-unit count, queried once
 *     per device and kept for the life of the process; the environment
 *     variable ATTN_GQA_CUS=n (read once) caps it at n, for a GPU shared
 *     with other work. Results do not depend on it beyond fp32 rounding.
 *   - Outputs must not overlap inputs. Concurrent calls must not share an
 *     output buffer or a decode workspace.
 *   - Pointers must be 16-byte aligned; strides are in elements and must be
 *     multiples of 4 (every row starts 16-byte aligned).
 *   - head_dim must be a multiple of 32 (ATTN_ERR_INVALID otherwise); this
 *     build supports every multiple of 32 from 32 to 256 (ATTN_ERR_UNSUPPORTED
 *     above 256).
 *
 * The softmax is evaluated in one pass with a running maximum, a correction
 * factor and a running sum (online softmax), so no score matrix is stored;
 * results match plain softmax attention up to fp32 rounding.
 */
#ifndef ATTN_GQA_ATTN_H
#define ATTN_GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,              /* launched (or nothing to do)                    */
    ATTN_ERR_INVALID = 1,     /* an argument breaks the contract above          */
    ATTN_ERR_UNSUPPORTED = 2, /* valid, but outside what this build implements  */
    ATTN_ERR_HIP = 3          /* the HIP runtime refused the launch             */
} attn_status;

/*
 * Causal prefill (aprender-gpu 0.32.0 "prefill_fused.rs" page: the module doc,
 * the PrefillAttentionKernel constructor and the kernel parameter list).
 *
 *   q  [m, q_stride]   Q head h at columns [h*head_dim, (h+1)*head_dim)
 *   k  [m, kv_stride]  KV head g at columns [g*head_dim, (g+1)*head_dim)
 *   v  [m, kv_stride]  same layout as k
 *   o  [m, q_stride]   written at the same columns as q; other columns untouched
 *
 * For every Q head h < num_q_heads and row i < m:
 *   O[i, h] = sum_{j <= i} softmax_j( scale * <Q[i, h], K[j, g]> ) V[j, g],
 *   g = h / heads_per_kv, scale = 1.0f / sqrtf((float)head_dim).
 * Rows may be slices of a fused [m, (Hq + 2*Hkv)*head_dim] projection output
 * (q_stride = kv_stride = that row length, k and v offset into the row).
 *
 * Errors: ATTN_ERR_INVALID if head_dim % 32 != 0, heads_per_kv == 0,
 * num_q_heads % heads_per_kv != 0, q_stride < num_q_heads*head_dim,
 * kv_stride < (num_q_heads/heads_per_kv)*head_dim, a stride not a multiple
 * of 4, or a null / misaligned pointer. m == 0 or num_q_heads == 0 returns
 * ATTN_OK without a launch.
 */
attn_status attn_prefill_causal(const float *q, const float *k, const float *v,
                                float *o, uint32_t m, uint32_t q_stride,
                                uint32_t kv_stride, uint32_t num_q_heads,
                                uint32_t heads_per_kv, uint32_t head_dim,
                                hipStream_t stream);

/*
 * Size in bytes of the decode workspace for these shapes (glia honeycrisp
 * "attention.rs" page: the decode module doc and its Params struct). Pure
 * host function (no HIP call); 0 if the shapes are invalid. The size covers
 * every decode entry point's work split on any gfx950 device (the split
 * follows the device's compute units, at most 256). Any device buffer at least this
 * large serves, provided it was zero-filled before its first use (hipMemset,
 * a fill kernel, torch.zeros): it begins with a block of 32-bit arrival
 * counters, one per work unit, which every call leaves at zero again: the
 * first 65536 bytes, or 4 * batch * num_heads bytes rounded up to a multiple
 * of 256 where that is more. The rest holds partial states, scratch that
 * need not be cleared. Calls that run concurrently need separate workspaces.
 * Calls ordered on one stream may share one whatever their shapes while
 * batch * num_heads <= 16384 (all of them then have the same counter block);
 * beyond that, only calls of the same batch, num_heads, kv_heads and
 * head_dim, unless the workspace is zero-filled again in between. A call
 * that does not run to completion (a device fault) can leave counters set:
 * zero-fill the workspace again before reusing it.
 */
size_t attn_decode_workspace_bytes(uint32_t batch, uint32_t num_heads,
                                   uint32_t kv_heads, uint32_t head_dim,
                                   uint32_t total_seq, uint32_t window);

/*
 * Single-query decode with optional sliding window (glia honeycrisp
 * "attention.rs" page: the decode module doc, the Params struct and the
 * window_start rule of the flash-decode kernel).
 *
 *   q        [batch, num_heads, head_dim]
 *   k_cache  [batch, kv_heads, max_seq, head_dim]   rows >= total_seq unused
 *   v_cache  same layout as k_cache
 *   out      [batch, num_heads, head_dim]
 *
 * With repeat = num_heads / kv_heads and
 *   w0 = (window > 0 && total_seq > window) ? total_seq - window : 0,
 * for every sequence b and head h:
 *   out[b, h] = sum_{w0 <= s < total_seq}
 *               softmax_s( scale * <q[b, h], K[b, h/repeat, s]> ) V[b, h/repeat, s].
 * Rows before w0 are never read. The current token is expected to be in the
 * cache already (kv_append at position total_seq - 1 first).
 *
 * workspace: device buffer of at least attn_decode_workspace_bytes(...) bytes,
 * zero-filled before its first use (see above). The attended range is split
 * over many workgroups of one launch; each writes its partial (max, sum,
 * accumulator) state per head into the workspace and counts itself in on its
 * unit's arrival counter, and the last workgroup of each unit merges the
 * partial states of its heads and writes out.
 *
 * Errors: ATTN_ERR_INVALID if head_dim % 32 != 0, kv_heads == 0,
 * num_heads % kv_heads != 0, total_seq == 0, total_seq > max_seq,
 * workspace_bytes too small, scale not finite, or a null / misaligned pointer.
 * batch == 0 or num_heads == 0 returns ATTN_OK without a launch.
 */
attn_status attn_decode(const float *q, const float *k_cache,
                        const float *v_cache, float *out, uint32_t batch,
                        uint32_t num_heads, uint32_t kv_heads,
                        uint32_t head_dim, uint32_t max_seq,
                        uint32_t total_seq, uint32_t window, float scale,
                        void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * One decode step: append the current token's K and V rows, then attend
 * (the two calls kv_append(position) and attn_decode(total_seq = position + 1)
 * in one: glia honeycrisp "attention.rs" page, the fused append + decode
 * kernel's doc, which removes the separate append dispatch and the wait
 * between the two; rotary embedding is not applied here).
 *
 *   q                 [batch, num_heads, head_dim]
 *   k_new, v_new      [batch, kv_heads, head_dim]   the current token's rows
 *   k_cache, v_cache  [batch, kv_heads, max_seq, head_dim]
 *   out               [batch, num_heads, head_dim]
 *
 * Writes k_cache[b, g, position, :] = k_new[b, g, :] (same for V) and
 *   out[b, h] = sum_{w0 <= s <= position} softmax_s( scale * <q[b, h], K[b, h/repeat, s]> )
 *               V[b, h/repeat, s],   w0 from total_seq = position + 1 as in attn_decode,
 * where row `position` is the new row. Cache rows other than `position` are
 * only read. The current token's contribution is computed from k_new/v_new,
 * not read back from the cache. Sources must not overlap the caches.
 *
 * workspace: at least attn_decode_workspace_bytes(batch, num_heads, kv_heads,
 * head_dim, position + 1, window) bytes, zero-filled before its first use
 * (may be null when that size is 0).
 *
 * Errors: as attn_decode (with total_seq = position + 1), plus position >=
 * max_seq, and ATTN_ERR_UNSUPPORTED past kv_append's size bound. batch == 0
 * returns ATTN_OK without a launch; num_heads == 0 only appends.
 */
attn_status attn_decode_append(const float *q, const float *k_new, const float *v_new,
                               float *k_cache, float *v_cache, float *out,
                               uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                               uint32_t head_dim, uint32_t max_seq, uint32_t position,
                               uint32_t window, float scale, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step with rotary position embedding (glia honeycrisp
 * "attention.rs" page, the fused RoPE + KV-append + flash-decode kernel's
 * doc): rotate the current token's raw q and K rows, append the rotated K row
 * and the raw V row at `position`, then attend over [w0, position] as in
 * attn_decode_append. The pages run one sequence and head_dim 128; here any
 * batch and every built head_dim, one cos/sin table shared by the batch (all
 * sequences decode the same position).
 *
 *   q_raw             [batch, num_heads, head_dim]  before rotation
 *   k_raw, v_raw      [batch, kv_heads, head_dim]   the current token's rows,
 *                                                   K before rotation
 *   cos_t, sin_t      [head_dim / 2]   cos and sin of pair i's angle at
 *                                      `position` (the caller's frequency
 *                                      table; not range-checked)
 *   k_cache, v_cache  [batch, kv_heads, max_seq, head_dim]
 *   out               [batch, num_heads, head_dim]
 *
 * Rotation (rotate-half): element i < head_dim/2 pairs with i + head_dim/2;
 *   x'[i]              = x[i] cos_t[i] - x[i + head_dim/2] sin_t[i]
 *   x'[i + head_dim/2] = x[i] sin_t[i] + x[i + head_dim/2] cos_t[i]
 * applied to every q_raw head and every k_raw row. Then
 *   k_cache[b, g, position, :] = k'[b, g, :],  v_cache[b, g, position, :] = v_raw[b, g, :]
 * and out is the attention of q' over cache rows [w0, position], the new
 * row scored from k' in registers. Cache rows other than `position` are only
 * read and must already hold rotated keys.
 *
 * workspace, errors and zero-work cases: as attn_decode_append; cos_t and
 * sin_t must also be non-null and 16-byte aligned (ATTN_ERR_INVALID).
 * num_heads == 0 only appends (the K rows still rotated).
 */
attn_status attn_decode_rope_append(const float *q_raw, const float *k_raw,
                                    const float *v_raw, const float *cos_t,
                                    const float *sin_t, float *k_cache,
                                    float *v_cache, float *out, uint32_t batch,
                                    uint32_t num_heads, uint32_t kv_heads,
                                    uint32_t head_dim, uint32_t max_seq,
                                    uint32_t position, uint32_t window,
                                    float scale, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_append for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops and harnesses that forbid hipMalloc.
 * The same step and kernels, with the decode workspace taken from a 16 MiB
 * array inside the library instead of a caller's buffer.
 *
 * Arguments and results: as attn_decode_append, without workspace and
 * workspace_bytes. The array is per GPU: each device the library runs on
 * holds its own copy until the process ends. The first call on a device
 * looks up that device's copy and clears its arrival counters on `stream`;
 * no call allocates or frees memory.
 *
 * Every call on one GPU uses that GPU's array (and leaves its counters at
 * zero), so calls that overlap on one GPU race: order them on one stream. A
 * call that does not run to completion (a device fault) leaves the array
 * unusable for the rest of the process.
 *
 * Errors: as attn_decode_append, plus ATTN_ERR_UNSUPPORTED when the step's
 * work split needs more than the 16 MiB (the batch of 32 sequences x 12 Q /
 * 2 KV heads of 128 needs under 1 MiB at any position) or more than 16384
 * work units (batch * kv_heads * ceil(num_heads / kv_heads / 8)), and
 * ATTN_ERR_HIP if the array's device address cannot be looked up.
 */
attn_status attn_decode_append_noalloc(const float *q, const float *k_new,
                                       const float *v_new, float *k_cache,
                                       float *v_cache, float *out, uint32_t batch,
                                       uint32_t num_heads, uint32_t kv_heads,
                                       uint32_t head_dim, uint32_t max_seq,
                                       uint32_t position, uint32_t window, float scale,
                                       hipStream_t stream);

/*
 * KV-cache append of K and V in one launch (glia honeycrisp "attention.rs"
 * page: the KV-append and KV-append-both kernels).
 *
 *   k_src, v_src      [batch, kv_heads, head_dim]
 *   k_cache, v_cache  [batch, kv_heads, max_seq, head_dim]
 *
 * k_cache[b, g, position, :] = k_src[b, g, :] and the same for V; no other
 * element is written. Sources must not overlap the caches.
 *
 * Errors: ATTN_ERR_INVALID if head_dim % 32 != 0, position >= max_seq, or a
 * null / misaligned pointer; ATTN_ERR_UNSUPPORTED if
 * batch*kv_heads*head_dim/4 >= 2^31. batch == 0 or kv_heads == 0 returns
 * ATTN_OK without a launch.
 */
attn_status kv_append(const float *k_src, const float *v_src, float *k_cache,
                      float *v_cache, uint32_t batch, uint32_t kv_heads,
                      uint32_t head_dim, uint32_t max_seq, uint32_t position,
                      hipStream_t stream);

/*
 * Bulk append of a prefill pass's K and V rows into one sequence's caches
 * (glia honeycrisp "attention.rs" page, the KV-append kernels, taken over the
 * m rows of the packed K/V layout of aprender-gpu 0.32.0 "prefill_fused.rs"
 * page, the kernel's buffer parameters), so that decode can follow prefill.
 *
 *   k_src, v_src      [m, kv_stride]   KV head g at columns g*head_dim ..
 *                                      (the layout attn_prefill_causal reads)
 *   k_cache, v_cache  [kv_heads, max_seq, head_dim]  one sequence's caches
 *                     (for a batch slot b of [batch, kv_heads, max_seq,
 *                     head_dim] caches, pass the slot's base address)
 *
 * k_cache[g, position + j, :] = k_src[j, g*head_dim : (g+1)*head_dim] for
 * j < m and every g, the same for V; no other element is written. One
 * launch. Sources must not overlap the caches.
 *
 * Errors: ATTN_ERR_INVALID if head_dim % 32 != 0, position + m > max_seq,
 * kv_stride < kv_heads*head_dim or not a multiple of 4, or a null /
 * misaligned pointer; ATTN_ERR_UNSUPPORTED if m*head_dim/4 >= 2^31 or
 * kv_heads > 65535. m == 0 or kv_heads == 0 returns ATTN_OK without a launch.
 */
attn_status kv_append_rows(const float *k_src, const float *v_src, float *k_cache,
                           float *v_cache, uint32_t m, uint32_t kv_stride,
                           uint32_t kv_heads, uint32_t head_dim, uint32_t max_seq,
                           uint32_t position, hipStream_t stream);

/*
 * Decode of a batch whose sequences have their own lengths (the decode
 * Params struct of glia honeycrisp "attention.rs" page carries one
 * total_seq; here there is one per sequence, read by the kernels from
 * device memory, so a serving loop can change them without a host sync).
 *
 *   seq_lens   [batch] uint32, DEVICE memory: T_b, the rows of sequence b
 *   seq_bound  host-side bound on every T_b, 1 <= seq_bound <= max_seq; the
 *              work split and the workspace are sized for it
 *   other arguments as attn_decode.
 *
 * Sequence b attends rows [w0_b, T_b), w0_b = (window > 0 && T_b > window)
 * ? T_b - window : 0. Device-side lengths cannot be checked before the
 * launch, so the kernels define the rest: T_b == 0 (an idle batch slot)
 * gives out[b] = 0, and T_b > seq_bound gives out[b] = NaN with no cache
 * row read.
 *
 * workspace: at least attn_decode_workspace_bytes(batch, num_heads,
 * kv_heads, head_dim, seq_bound, window) bytes, zero-filled before its
 * first use as for attn_decode.
 *
 * Errors: as attn_decode with total_seq replaced by seq_bound, plus a null
 * or misaligned (4-byte) seq_lens. batch == 0 or num_heads == 0 returns
 * ATTN_OK without a launch.
 */
attn_status attn_decode_varlen(const float *q, const float *k_cache,
                               const float *v_cache, float *out,
                               const uint32_t *seq_lens, uint32_t batch,
                               uint32_t num_heads, uint32_t kv_heads,
                               uint32_t head_dim, uint32_t max_seq,
                               uint32_t seq_bound, uint32_t window, float scale,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * One decode step of a batch whose sequences sit at their own positions:
 * sequence b appends its new K and V rows at positions[b] and attends rows
 * [w0_b, positions[b]] (T_b = positions[b] + 1, window rule as above); the
 * batched form of attn_decode_append.
 *
 *   positions  [batch] uint32, DEVICE memory
 *   seq_bound  host-side bound: every positions[b] + 1 <= seq_bound <= max_seq
 *   other arguments as attn_decode_append.
 *
 * A sequence with positions[b] + 1 > seq_bound gets out[b] = NaN and no
 * cache write. workspace: at least attn_decode_workspace_bytes(batch,
 * num_heads, kv_heads, head_dim, seq_bound, window) bytes (may be null when
 * that size is 0).
 *
 * Errors: as attn_decode_append with position + 1 replaced by seq_bound,
 * plus a null or misaligned (4-byte) positions. batch == 0 returns ATTN_OK
 * without a launch; num_heads == 0 only appends.
 */
attn_status attn_decode_append_varlen(const float *q, const float *k_new,
                                      const float *v_new, float *k_cache,
                                      float *v_cache, float *out,
                                      const uint32_t *positions, uint32_t batch,
                                      uint32_t num_heads, uint32_t kv_heads,
                                      uint32_t head_dim, uint32_t max_seq,
                                      uint32_t seq_bound, uint32_t window,
                                      float scale, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * The rotary decode step of a batch whose sequences sit at their own
 * positions: attn_decode_rope_append per sequence, with sequence b's table
 * for its own position positions[b] (the fused kernel of glia honeycrisp
 * "attention.rs" page, which serves one sequence, taken over a batch as in
 * attn_decode_append_varlen).
 *
 *   cos_t, sin_t  [batch, head_dim / 2]  row b: cos and sin of pair i's angle
 *                                        at positions[b]
 *   other arguments as attn_decode_append_varlen (q_raw, k_raw, v_raw as in
 *   attn_decode_rope_append).
 *
 * Errors and zero-work cases: as attn_decode_append_varlen, plus null or
 * misaligned (16-byte) cos_t / sin_t.
 */
attn_status attn_decode_rope_append_varlen(const float *q_raw, const float *k_raw,
                                           const float *v_raw, const float *cos_t,
                                           const float *sin_t, float *k_cache,
                                           float *v_cache, float *out,
                                           const uint32_t *positions, uint32_t batch,
                                           uint32_t num_heads, uint32_t kv_heads,
                                           uint32_t head_dim, uint32_t max_seq,
                                           uint32_t seq_bound, uint32_t window,
                                           float scale, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char *attn_status_string(attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GQA_ATTN_H */
