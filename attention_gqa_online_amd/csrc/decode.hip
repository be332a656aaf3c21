// Single-query GQA decode over a KV cache, split across wavefronts and
// workgroups, with an online softmax per split and a log-sum-exp merge.
//
// What is computed follows the decode module of the glia honeycrisp
// "attention.rs" page (module doc, Params struct, window_start rule): for each
// head h, softmax over positions s in [w0, total_seq) of scale * <q[h], K[g, s]>
// weights the V rows of KV head g = h / repeat.
//
// Work decomposition (MI355X design, not the page's one-SIMD-group loop):
//   unit  = (sequence b, KV head g, chunk of <= 8 Q heads of that group)
//   split = a contiguous range of attended rows; one workgroup of NW waves
//   wave  = a contiguous sub-range, streamed 64/LPR rows per step
//   lane  = (row slot r, d-chunk c): LPR lanes cover one row's head_dim, each
//           holding head_dim/LPR consecutive-in-float4 elements, so one
//           global_load_dwordx4 per lane reads LPR*16 contiguous bytes per row.
// Each K row is read from HBM once and used for all Q heads of the chunk (the
// GQA reuse the pages leave to L2). The q.K dot of one row is reduced over
// its LPR lanes with DPP butterflies; every lane then keeps its own online
// softmax state for its row slot, so a step needs no cross-row reduction.
// The running max is only raised when a score exceeds it by more than
// kRescaleSlack (log2 units): p = 2^(s - m) stays below 2^kRescaleSlack and
// the accumulator is rescaled rarely, which is exact since any reference
// value m gives the same acc / l.
// At the end, the row slots of a wave merge through lane shuffles, the waves
// of a workgroup through LDS, and the workgroups of a unit through the
// workspace: the last workgroup to arrive (atomic counter) merges all splits
// and writes the normalised output, then resets its counter to zero.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kDecodeWaves = 4;          // waves per workgroup
constexpr int kTargetWorkgroups = 1024;  // enough to fill 256 CUs several times
constexpr int kMinRowsPerWave = 32;
constexpr float kRescaleSlack = 8.0f;

struct DecodeArgs {
    const float *q;
    const float *k;
    const float *v;
    float *out;
    float *part;        // [units][n_split][HC][D + 2]: acc[D], m, l
    uint32_t *count;    // [units]
    uint32_t num_heads, kv_heads, hpk, n_chunks, max_seq;
    uint32_t w0, total_seq, n_split, rows_per_split;
    float qscale;       // scale * log2(e): scores come out in log2 units
};

constexpr int lanes_per_row(int d) { return d == 32 ? 8 : 16; }

template <int D, int HC, int LPR, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
    constexpr int VPL = D / LPR;  // floats per lane per row
    constexpr int NF4 = VPL / 4;  // float4 per lane per row
    constexpr int RPT = 64 / LPR; // rows per wave step
    static_assert(VPL % 4 == 0 && LPR * VPL == D, "lane tiling");

    __shared__ float s_acc[NW][HC][D];
    __shared__ float s_m[NW][HC];
    __shared__ float s_l[NW][HC];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane / LPR;
    const int c = lane % LPR;

    const uint32_t split = blockIdx.x % a.n_split;
    const uint32_t unit = blockIdx.x / a.n_split;
    const uint32_t chunk = unit % a.n_chunks;
    const uint32_t bg = unit / a.n_chunks;  // b * kv_heads + g
    const uint32_t g = bg % a.kv_heads;
    const uint32_t b = bg / a.kv_heads;
    const uint32_t hl0 = chunk * HC;
    const int nh = min(HC, (int)(a.hpk - hl0));
    const uint32_t h0 = g * a.hpk + hl0;

    // rows of this workgroup, then of this wave
    const uint32_t ws0 = a.w0 + split * a.rows_per_split;
    const uint32_t ws1 = min(ws0 + a.rows_per_split, a.total_seq);
    const uint32_t per_wave = a.rows_per_split / NW;
    const uint32_t ra = min(ws0 + wave * per_wave, ws1);
    const uint32_t rb = min(ra + per_wave, ws1);

    // q of every head of the chunk, pre-scaled (zero for heads past nh)
    float4 qv[HC][NF4];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
        // heads past nh re-read the last valid head (in bounds) and are zeroed
        const int hq = hh < nh ? hh : nh - 1;
        const float *qh = a.q + ((size_t)b * a.num_heads + h0 + hq) * D + 4 * c;
        const float qs = hh < nh ? a.qscale : 0.f;
#pragma unroll
        for (int t = 0; t < NF4; ++t) qv[hh][t] = ld4(qh + 4 * LPR * t) * qs;
    }

    float m[HC], l[HC];
    float4 acc[HC][NF4];
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
        m[hh] = kNegInf;
        l[hh] = 0.f;
#pragma unroll
        for (int t = 0; t < NF4; ++t) acc[hh][t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const size_t cache_base = (size_t)bg * a.max_seq * D + 4 * c;
    const float *kb = a.k + cache_base;
    const float *vb = a.v + cache_base;

    for (uint32_t row0 = ra; row0 < rb; row0 += RPT) {
        const uint32_t row = row0 + r;
        const bool valid = row < rb;
        const size_t off = (size_t)(valid ? row : rb - 1) * D;
        float4 kf[NF4], vf[NF4];
#pragma unroll
        for (int t = 0; t < NF4; ++t) kf[t] = ld4(kb + off + 4 * LPR * t);
#pragma unroll
        for (int t = 0; t < NF4; ++t) vf[t] = ld4(vb + off + 4 * LPR * t);

        float s[HC];
        bool need = false;
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
            float part = 0.f;
#pragma unroll
            for (int t = 0; t < NF4; ++t) part += dot4(qv[hh][t], kf[t]);
            const float tot = group_sum<LPR>(part);  // all lanes active here
            s[hh] = valid ? tot : kNegInf;
            need |= s[hh] > m[hh] + kRescaleSlack;
        }
        if (__any(need)) {
#pragma unroll
            for (int hh = 0; hh < HC; ++hh) {
                if (s[hh] > m[hh] + kRescaleSlack) {
                    const float cf = fast_exp2(m[hh] - s[hh]);
                    l[hh] *= cf;
#pragma unroll
                    for (int t = 0; t < NF4; ++t) acc[hh][t] = acc[hh][t] * cf;
                    m[hh] = s[hh];
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < HC; ++hh) {
            const float p = valid ? fast_exp2(s[hh] - m[hh]) : 0.f;
            l[hh] += p;
#pragma unroll
            for (int t = 0; t < NF4; ++t) {
                acc[hh][t].x += p * vf[t].x;
                acc[hh][t].y += p * vf[t].y;
                acc[hh][t].z += p * vf[t].z;
                acc[hh][t].w += p * vf[t].w;
            }
        }
    }

    // merge the RPT row slots of this wave (lanes c, c+LPR, c+2LPR, ...)
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) {
        float mx = m[hh];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const float f = m[hh] == kNegInf ? 0.f : fast_exp2(m[hh] - mx);
        float lw = l[hh] * f;
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) lw += __shfl_xor(lw, o);
#pragma unroll
        for (int t = 0; t < NF4; ++t) {
            float4 x = acc[hh][t] * f;
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) {
                x.x += __shfl_xor(x.x, o);
                x.y += __shfl_xor(x.y, o);
                x.z += __shfl_xor(x.z, o);
                x.w += __shfl_xor(x.w, o);
            }
            if (r == 0) st4(&s_acc[wave][hh][4 * (c + LPR * t)], x);
        }
        if (lane == 0) {
            s_m[wave][hh] = mx;
            s_l[wave][hh] = lw;
        }
    }
    __syncthreads();

    // merge the waves; write this workgroup's partial state
    float *mypart = a.part + ((size_t)unit * a.n_split + split) * HC * (D + 2);
    for (int idx = tid; idx < HC * D; idx += NW * 64) {
        const int hh = idx / D;
        const int d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hh]);
        float x = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = s_m[w][hh];
            const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
            x += s_acc[w][hh][d] * f;
            lsum += s_l[w][hh] * f;
        }
        mypart[hh * (D + 2) + d] = x;
        if (d == 0) {
            mypart[hh * (D + 2) + D] = M;
            mypart[hh * (D + 2) + D + 1] = lsum;
        }
    }

    // publish; the last workgroup of the unit merges every split
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(a.count + unit, 1u);
        s_last = prev == a.n_split - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const float *up = a.part + (size_t)unit * a.n_split * HC * (D + 2);
    for (int idx = tid; idx < nh * D; idx += NW * 64) {
        const int hh = idx / D;
        const int d = idx % D;
        float M = kNegInf;
        for (uint32_t sp = 0; sp < a.n_split; ++sp)
            M = fmaxf(M, __hip_atomic_load(up + (sp * HC + hh) * (D + 2) + D, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
        float num = 0.f, den = 0.f;
        for (uint32_t sp = 0; sp < a.n_split; ++sp) {
            const float *ps = up + (sp * HC + hh) * (D + 2);
            const float ms = __hip_atomic_load(ps + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float f = ms == kNegInf ? 0.f : fast_exp2(ms - M);
            num += __hip_atomic_load(ps + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * f;
            den += __hip_atomic_load(ps + D + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) * f;
        }
        a.out[((size_t)b * a.num_heads + h0 + hh) * D + d] = num / den;
    }
    if (tid == 0) a.count[unit] = 0;
}

template <int D, int HC>
hipError_t launch_hc(const DecodeArgs &args, uint32_t grid, hipStream_t stream) {
    constexpr int LPR = lanes_per_row(D);
    hipLaunchKernelGGL((decode_kernel<D, HC, LPR, kDecodeWaves>), dim3(grid),
                       dim3(kDecodeWaves * 64), 0, stream, args);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(uint32_t hc, const DecodeArgs &args, uint32_t grid, hipStream_t stream) {
    switch (hc) {
    case 1: return launch_hc<D, 1>(args, grid, stream);
    case 2: return launch_hc<D, 2>(args, grid, stream);
    case 3: return launch_hc<D, 3>(args, grid, stream);
    case 4: return launch_hc<D, 4>(args, grid, stream);
    case 5: return launch_hc<D, 5>(args, grid, stream);
    case 6: return launch_hc<D, 6>(args, grid, stream);
    case 7: return launch_hc<D, 7>(args, grid, stream);
    case 8: return launch_hc<D, 8>(args, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

inline uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

}  // namespace

DecodePlan plan_decode(uint32_t batch, uint32_t num_heads, uint32_t kv_heads,
                       uint32_t head_dim, uint32_t total_seq, uint32_t window) {
    DecodePlan p{};
    const uint32_t hpk = num_heads / kv_heads;
    p.n_chunks = ceil_div(hpk, 8);
    p.head_chunk = ceil_div(hpk, p.n_chunks);
    p.units = batch * kv_heads * p.n_chunks;
    p.w0 = (window > 0 && total_seq > window) ? total_seq - window : 0;
    const uint32_t len = total_seq - p.w0;
    const uint32_t rpt = 64 / lanes_per_row((int)head_dim);
    const uint32_t step = kDecodeWaves * rpt;
    const uint32_t max_split = ceil_div(len, (uint64_t)kDecodeWaves * kMinRowsPerWave);
    uint32_t n_split = ceil_div(kTargetWorkgroups, p.units);
    n_split = n_split < 1 ? 1 : (n_split > max_split ? max_split : n_split);
    uint32_t rows = ceil_div(len, n_split);
    rows = ceil_div(rows, step) * step;
    p.rows_per_split = rows;
    p.n_split = ceil_div(len, rows);
    p.part_floats = (size_t)p.units * p.n_split * p.head_chunk * (head_dim + 2);
    const size_t count_bytes = ((size_t)p.units * sizeof(uint32_t) + 255) & ~(size_t)255;
    p.workspace_bytes = count_bytes + p.part_floats * sizeof(float);
    return p;
}

hipError_t launch_decode(const DecodePlan &plan, const float *q, const float *k_cache,
                         const float *v_cache, float *out, uint32_t batch,
                         uint32_t num_heads, uint32_t kv_heads, uint32_t head_dim,
                         uint32_t max_seq, uint32_t total_seq, float scale,
                         void *workspace, hipStream_t stream) {
    (void)batch;
    DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    const size_t count_bytes = ((size_t)plan.units * sizeof(uint32_t) + 255) & ~(size_t)255;
    a.count = static_cast<uint32_t *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + count_bytes);
    a.num_heads = num_heads;
    a.kv_heads = kv_heads;
    a.hpk = num_heads / kv_heads;
    a.n_chunks = plan.n_chunks;
    a.max_seq = max_seq;
    a.w0 = plan.w0;
    a.total_seq = total_seq;
    a.n_split = plan.n_split;
    a.rows_per_split = plan.rows_per_split;
    a.qscale = scale * kLog2e;
    const uint32_t grid = plan.units * plan.n_split;
    switch (head_dim) {
    case 32: return launch_d<32>(plan.head_chunk, a, grid, stream);
    case 64: return launch_d<64>(plan.head_chunk, a, grid, stream);
    case 128: return launch_d<128>(plan.head_chunk, a, grid, stream);
    case 256: return launch_d<256>(plan.head_chunk, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
