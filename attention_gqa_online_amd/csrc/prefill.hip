// Causal GQA prefill on fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// What is computed follows the aprender-gpu "prefill_fused.rs" page (module
// doc "Algorithm", constructor and kernel parameter list): Q head h, row i,
// attends keys j <= i of KV head h / heads_per_kv with scale 1/sqrt(d) in f32;
// rows are strided (q_stride, kv_stride) so Q, K and V may be slices of one
// fused projection output, and O is written with Q's stride.
//
// MI355X design (the page's one-warp-per-head kernel with K/V through L2 is
// prior art only):
//   workgroup = 8 waves sharing one KV head g. Wave w of workgroup i owns the
//               (row block, head) pair i*8 + w of the group, enumerated row
//               block major, so the waves of a workgroup sit in at most a few
//               consecutive 32-row blocks.
//   K/V tiles of 64 keys are staged once in LDS and used by all 8 waves
//   (every Q head of the group reads the same tile; the GQA reuse is explicit).
//   Per wave and tile:
//     S^T[64 keys x 32 rows] = K_tile . Q^T        (2 x D/2 MFMAs, A = K from LDS,
//                                                 B = Q^T held in registers)
//     online softmax per query row (column of S^T), masked on diagonal tiles
//     O^T[D x 32 rows] += V_tile^T . P^T             (D/32 x 32 MFMAs, A = V from LDS,
//                                                 B = P^T straight from the S^T
//                                                 accumulator registers)
//   Operand layouts: for 32x32x2 f32, lane l supplies A[l%32][l/32] and
//   B[l/32][l%32] and receives C[8(v/4) + 4(l/32) + v%4][l%32] in register v.
//   The contraction index of each MFMA may be any permutation as long as A
//   and B agree, which is used twice: the d index of QK^T is chosen so a lane
//   reads 4 consecutive K floats with one ds_read_b128, and the key index of
//   P.V is chosen so the S^T accumulator register v is exactly the P^T
//   operand of k-step v (no shuffle between the two products). The output d
//   index of a lane's A row i is D/32*i + block, so a lane reads D/32
//   consecutive V floats per key and stores D/32 consecutive O floats.
//   Scores are kept in log2 units (Q pre-scaled by scale*log2 e); exp is
//   v_exp_f32. Workgroups are issued heaviest (last row blocks) first.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kWaves = 8;
constexpr int kBr = 32;  // query rows per wave
constexpr int kBc = 64;  // keys per LDS tile

struct PrefillArgs {
    const float *q;
    const float *k;
    const float *v;
    float *o;
    uint32_t m, q_stride, kv_stride, hpk, kv_heads;
    uint32_t n_pairs;      // hpk * ceil(m / 32)
    uint32_t wg_per_group; // ceil(n_pairs / 8)
    float qscale;          // (1/sqrt(d) in f32) * log2(e)
};

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void prefill_kernel(PrefillArgs a) {
    constexpr int KS = D + 4;   // LDS row stride (floats), padded against bank conflicts
    constexpr int NQ = D / 8;   // float4 chunks of the Q^T operand per lane
    constexpr int NMD = D / 32; // 32-row blocks of O^T (= floats per lane per V row)
    constexpr int D4 = D / 4;
    __shared__ float sK[kBc * KS];
    __shared__ float sV[kBc * KS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;    // query column of this lane
    const int half = lane >> 5; // which of the two keys of a k-step

    const uint32_t g = blockIdx.x % a.kv_heads;
    const uint32_t wi = a.wg_per_group - 1 - blockIdx.x / a.kv_heads;  // heavy first
    const uint32_t pair = wi * kWaves + wave;
    const bool active = pair < a.n_pairs;
    const uint32_t rb = pair / a.hpk;
    const uint32_t h = g * a.hpk + pair % a.hpk;
    const uint32_t qr0 = rb * kBr;
    const uint32_t qi = qr0 + j;
    const bool qvalid = active && qi < a.m;

    // keys this workgroup needs: [0, kend)
    const uint32_t last_pair = min(wi * kWaves + kWaves - 1, a.n_pairs - 1);
    const uint32_t kend = min((last_pair / a.hpk) * kBr + kBr, a.m);
    const uint32_t ntiles = (kend + kBc - 1) / kBc;
    const uint32_t my_kend = active ? min(qr0 + kBr, a.m) : 0;
    const uint32_t my_ntiles = (my_kend + kBc - 1) / kBc;

    // Q^T operand: lane (j, half) holds Q[qi][8u + 4half + 0..3] for u < D/8
    float4 qt[NQ];
    {
        const float *qrow = a.q + (size_t)(qvalid ? qi : 0) * a.q_stride + (size_t)(active ? h : 0) * D;
        const float qs = qvalid ? a.qscale : 0.f;
#pragma unroll
        for (int u = 0; u < NQ; ++u) qt[u] = ld4(qrow + 8 * u + 4 * half) * qs;
    }

    floatx16 acc[NMD];
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[md][e] = 0.f;
    float mrow = kNegInf, lrow = 0.f;

    const float *kg = a.k + (size_t)g * D;
    const float *vg = a.v + (size_t)g * D;

    for (uint32_t kt = 0; kt < ntiles; ++kt) {
        __syncthreads();  // previous tile fully consumed
        for (int idx = tid; idx < kBc * D4; idx += kWaves * 64) {
            const int row = idx / D4;
            const int c4 = idx % D4;
            const uint32_t key = kt * kBc + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < a.m) {
                kx = ld4(kg + (size_t)key * a.kv_stride + 4 * c4);
                vx = ld4(vg + (size_t)key * a.kv_stride + 4 * c4);
            }
            st4(&sK[row * KS + 4 * c4], kx);
            st4(&sV[row * KS + 4 * c4], vx);
        }
        __syncthreads();
        if (kt >= my_ntiles) continue;  // wave-uniform: beyond this wave's diagonal

        // S^T = K_tile . Q^T, two 32-key blocks
        floatx16 s0, s1;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const float4 ka = *reinterpret_cast<const float4 *>(&sK[j * KS + 8 * u + 4 * half]);
            const float4 kb = *reinterpret_cast<const float4 *>(&sK[(32 + j) * KS + 8 * u + 4 * half]);
            s0 = mfma32(ka.x, qt[u].x, s0);
            s1 = mfma32(kb.x, qt[u].x, s1);
            s0 = mfma32(ka.y, qt[u].y, s0);
            s1 = mfma32(kb.y, qt[u].y, s1);
            s0 = mfma32(ka.z, qt[u].z, s0);
            s1 = mfma32(kb.z, qt[u].z, s1);
            s0 = mfma32(ka.w, qt[u].w, s0);
            s1 = mfma32(kb.w, qt[u].w, s1);
        }

        // causal mask on tiles that reach past this wave's first row
        if (kt * kBc + kBc - 1 > qr0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t key = kt * kBc + 8 * (e / 4) + 4 * half + (e % 4);
                if (key > qi) s0[e] = kNegInf;
                if (key + 32 > qi) s1[e] = kNegInf;
            }
        }

        // online softmax for query row qi (this lane and lane ^ 32 share it)
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow, mx);
        const float cf = fast_exp2(mrow - mnew);
        mrow = mnew;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s0[e] = fast_exp2(s0[e] - mnew);
            s1[e] = fast_exp2(s1[e] - mnew);
            ls += s0[e] + s1[e];
        }
        lrow = lrow * cf + ls;
#pragma unroll
        for (int md = 0; md < NMD; ++md)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[md][e] *= cf;

        // O^T += V_tile^T . P^T; k-step (block mb, register e) uses key
        // 32mb + 8(e/4) + 4half + e%4, the key register e of S^T holds
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key0 = 8 * (e / 4) + 4 * half + (e % 4);
            const float *v0 = &sV[key0 * KS + NMD * j];
            const float *v1 = &sV[(32 + key0) * KS + NMD * j];
            float va[NMD], vb[NMD];
#pragma unroll
            for (int md = 0; md < NMD; ++md) { va[md] = v0[md]; vb[md] = v1[md]; }
#pragma unroll
            for (int md = 0; md < NMD; ++md) acc[md] = mfma32(va[md], s0[e], acc[md]);
#pragma unroll
            for (int md = 0; md < NMD; ++md) acc[md] = mfma32(vb[md], s1[e], acc[md]);
        }
    }

    // normalise and store: register e of block md is O[qi][NMD*(8(e/4)+4half+e%4) + md]
    lrow += __shfl_xor(lrow, 32);
    if (qvalid) {
        const float inv = 1.0f / lrow;
        float *orow = a.o + (size_t)qi * a.q_stride + (size_t)h * D;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 8 * (e / 4) + 4 * half + (e % 4);
#pragma unroll
            for (int md = 0; md < NMD; ++md) orow[NMD * i + md] = acc[md][e] * inv;
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs &args, uint32_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((prefill_kernel<D>), dim3(grid), dim3(kWaves * 64), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const float *q, const float *k, const float *v, float *o,
                          uint32_t m, uint32_t q_stride, uint32_t kv_stride,
                          uint32_t num_q_heads, uint32_t heads_per_kv,
                          uint32_t head_dim, hipStream_t stream) {
    PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.m = m;
    a.q_stride = q_stride;
    a.kv_stride = kv_stride;
    a.hpk = heads_per_kv;
    a.kv_heads = num_q_heads / heads_per_kv;
    const uint32_t n_rb = (m + kBr - 1) / kBr;
    a.n_pairs = heads_per_kv * n_rb;
    a.wg_per_group = (a.n_pairs + kWaves - 1) / kWaves;
    a.qscale = (1.0f / sqrtf((float)head_dim)) * kLog2e;
    const uint32_t grid = a.wg_per_group * a.kv_heads;
    switch (head_dim) {
    case 32: return launch_d<32>(a, grid, stream);
    case 64: return launch_d<64>(a, grid, stream);
    case 128: return launch_d<128>(a, grid, stream);
    case 256: return launch_d<256>(a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
