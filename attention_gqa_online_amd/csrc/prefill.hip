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
//   workgroup = NW waves sharing one KV head g (NW = 8, or 4 for head_dim
//               >= 192 on large grids: see kMinDim4Waves). Wave w of workgroup i owns the
//               (row block, head) pair i*NW + w of the group, enumerated row
//               block major, so the waves of a workgroup sit in at most a few
//               consecutive 32-row blocks. Grids too small to fill the chip
//               twice pair row blocks u and n-1-u instead (first / second
//               half of the waves, NW/2 heads each), balancing the causal
//               work per workgroup.
//   K/V tiles of 64 keys are staged once in LDS and used by all the waves
//   (every Q head of the group reads the same tile; the GQA reuse is explicit).
//   Tiles go global -> LDS directly (no registers) into two buffers, so the
//   next tile's loads run under the current tile's matrix work; one barrier
//   per tile.
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

// Waves per workgroup: 8 (two per SIMD, so one wave's matrix work fills the
// other's waits on LDS reads, barriers and dependent instructions; vector
// instructions themselves do not run under fp32 MFMAs, whichever wave issues
// them), or, for head_dim >= 192 on grids that fill the chip
// twice, 4: there Q^T and the O^T accumulators of a 32-row block alone take
// head_dim registers, and with one wave per SIMD a lane has 512 registers
// instead of 256, so nothing goes to scratch memory. (On smaller grids the
// 4-wave workgroups would need two rounds of the CUs.)
// (kMinDim4Waves and the grid itself: plan_prefill in plan.cpp)
constexpr int kBr = kPrefillRows;  // query rows per wave
constexpr int kBc = 64;  // keys per LDS tile
constexpr float kLazyRescale = 8.0f;  // log2 units

struct PrefillArgs {
    const float *q;
    const float *k;
    const float *v;
    float *o;
    uint32_t m, q_stride, kv_stride, hpk, kv_heads;
    uint32_t n_pairs;      // hpk * ceil(m / 32)
    uint32_t wg_per_group; // workgroups per KV head
    uint32_t n_rb;         // ceil(m / 32)
    uint32_t zigzag;       // 1: waves 0-3 / 4-7 take row blocks u / n_rb-1-u
    uint32_t nsub;         // zigzag: workgroups per row-block pair (ceil(hpk / (waves / 2)))
    uint32_t n_rb16;       // 16-row kernel: ceil(m / 16)
    uint32_t n_tasks16;    // 16-row kernel: ceil(n_rb16 / 2) * hpk per KV head
    float qscale;          // (1/sqrt(d) in f32) * log2(e)
};

// max of three scores in one instruction. Written out because fmaxf on
// matrix-core results is preceded by a canonicalising max per operand (the
// compiler cannot assume they are quieted); scores here are finite or -inf.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max of lane l and lane l ^ 32: v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second, so with both equal
// to x the two results hold x and its partner in every lane
__device__ __forceinline__ float max_lane_pair(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum of lane l and lane l ^ 32 (the same exchange as max_lane_pair)
__device__ __forceinline__ float sum_lane_pair(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 16-byte chunk index of a K/V element row inside an LDS tile row, XOR-
// swizzled by the row so that the 32 lanes of an MFMA operand read (one row
// each, same logical chunk) land in different LDS banks without padding.
// Width of the XOR swizzle: the largest of 16, 8, 4 that divides the row's
// chunk count, so a swizzled chunk stays inside its row.
constexpr int swz_width(int d) { return (d / 4) % 16 == 0 ? 16 : (d / 4) % 8 == 0 ? 8 : 4; }

template <int D>
__device__ __forceinline__ int swz_chunk(int row, int chunk) {
    constexpr int SW = swz_width(D);
    return chunk ^ (row & (SW - 1));
}

// Copy one 64-row tile of K and of V for KV head g into LDS with direct
// global->LDS loads (global_load_lds_dwordx4): each instruction moves 64
// lanes x 16 bytes to consecutive LDS addresses; the lane picks which global
// chunk fills its LDS slot, which is how the swizzle is applied. Rows past
// m re-read row m - 1 (in bounds); the causal mask removes them.
template <int D, int NW>
__device__ __forceinline__ void load_tile_lds(const PrefillArgs &a, uint32_t g, uint32_t kt,
                                              float *sk, float *sv, int wave, int lane) {
    constexpr int CPR = D / 4;                    // 16-byte chunks per row
    constexpr int NI = kBc * CPR / (NW * 64);     // instructions per wave per tensor
    static_assert(NI >= 1 && kBc * CPR % (NW * 64) == 0, "tile split over waves");
    // opaque copy of the lane id: the per-lane source offsets below are then
    // formed at each call instead of being hoisted out of the tile loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int l = (wave * NI + i) * 64 + ln;  // LDS chunk slot of this lane
        const int row = l / CPR;
        const int c = swz_chunk<D>(row, l % CPR);  // global chunk stored there
        const uint32_t key = min(kt * kBc + row, a.m - 1);
        const size_t goff = (size_t)key * a.kv_stride + (size_t)g * D + 4 * c;
        const int loff = (wave * NI + i) * 64 * 4;  // floats; lane offset added by hardware
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(a.k + goff),
            (__attribute__((address_space(3))) void *)(sk + loff), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(a.v + goff),
            (__attribute__((address_space(3))) void *)(sv + loff), 16, 0, 0);
    }
}

// The same copy for a tile whose 64 rows all lie below m, for head sizes
// whose row holds a power-of-two number of chunks (32, 64, 128). Instruction
// i covers rows R_i .. R_i + 64 / CPR - 1 (R_i = (wave * NI + i) * 64 / CPR,
// a multiple of 64 / CPR), so the swizzled chunk of lane l is
// (l mod CPR) ^ ((l / CPR) mod SW) ^ (R_i mod SW): a per-lane constant lx
// XOR a uniform value. The source is a uniform row address plus a 32-bit
// per-lane offset (ly = the lane's row within the instruction, in bytes,
// plus 16 * chunk): two vector instructions per copy.
template <int D>
constexpr bool kFastCopy = D == 32 || D == 64 || D == 128;

template <int D, int NW>
__device__ __forceinline__ void load_tile_lds_full(const PrefillArgs &a, uint32_t g, uint32_t kt,
                                                   float *sk, float *sv, int wave, uint32_t lx,
                                                   uint32_t ly) {
    constexpr int CPR = D / 4;
    constexpr int NI = kBc * CPR / (NW * 64);
    constexpr int SW = swz_width(D);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint32_t ri = (uint32_t)(wave * NI + i) * (64 / CPR);  // uniform
        const size_t row0 = ((size_t)kt * kBc + ri) * a.kv_stride + (size_t)g * D;
        const uint32_t off = ly + 16u * (lx ^ (ri & (SW - 1)));
        const char *kb = reinterpret_cast<const char *>(a.k + row0);
        const char *vb = reinterpret_cast<const char *>(a.v + row0);
        const int loff = (wave * NI + i) * 64 * 4;  // floats; lane offset added by hardware
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(kb + off),
            (__attribute__((address_space(3))) void *)(sk + loff), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(vb + off),
            (__attribute__((address_space(3))) void *)(sv + loff), 16, 0, 0);
    }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
    constexpr int HW = NW / 2;  // zigzag: waves per row block of the pair
    constexpr int NQ = D / 8;   // float4 chunks of the Q^T operand per lane
    constexpr int NMD = D / 32; // 32-row blocks of O^T (= floats per lane per V row)
    constexpr int NBUF = D <= 128 ? 2 : 1;  // double-buffered tiles when LDS allows
    constexpr int TILE = kBc * D;           // floats per tile and tensor
    __shared__ __attribute__((aligned(16))) float sK0[TILE];
    __shared__ __attribute__((aligned(16))) float sV0[TILE];
    __shared__ __attribute__((aligned(16))) float sK1[NBUF == 2 ? TILE : 4];
    __shared__ __attribute__((aligned(16))) float sV1[NBUF == 2 ? TILE : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index in a scalar register: everything derived from it (pair,
    // head, LDS load slots) stays out of the vector register file
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;    // query column of this lane
    const int half = lane >> 5; // which of the two keys of a k-step

    const uint32_t g = blockIdx.x % a.kv_heads;
    const uint32_t wi = a.wg_per_group - 1 - blockIdx.x / a.kv_heads;  // heavy first
    bool active;
    uint32_t rb, hl, rb_last;  // this wave's row block and head; the workgroup's last block
    if (a.zigzag) {
        // small grids: the first half of the waves take heads of row block
        // u, the second half the same heads of block n_rb-1-u, so each SIMD
        // runs one short and one long wave (8 waves) and every workgroup has
        // about the same work
        //
        // The sub-workgroup index of a pair is rotated by a term that grows
        // with u, so that workgroups with fewer heads (the last sub-workgroup
        // when heads_per_kv is not a multiple of NW / 2) are spread over the
        // XCDs instead of all landing on the XCDs (blockIdx mod 8) of one
        // parity: an XCD whose compute units all run four busy SIMDs ends
        // later than one that runs three. gx = gcd(8, kv_heads); over the
        // blocks of one XCD, u / (8 / (nsub * gx)) steps once per such
        // period. Within a pair's nsub workgroups it is a rotation, so every
        // (u, sub) is still taken exactly once.
        const uint32_t u = wi / a.nsub;
        const uint32_t gx = min(a.kv_heads & (~a.kv_heads + 1u), 8u);
        const uint32_t sub = (wi % a.nsub + u * a.nsub * gx / 8) % a.nsub;
        hl = sub * HW + (wave % HW);
        const uint32_t lo = u, hi = a.n_rb - 1 - u;
        rb = wave < HW ? lo : hi;
        active = hl < a.hpk && (wave < HW || hi > lo);
        rb_last = hi;
    } else {
        // row-block-major pairs: workgroup wi owns pairs wi*NW .. wi*NW+NW-1
        const uint32_t pair = wi * NW + wave;
        active = pair < a.n_pairs;
        rb = pair / a.hpk;
        hl = pair % a.hpk;
        rb_last = min(wi * NW + NW - 1, a.n_pairs - 1) / a.hpk;
    }
    const uint32_t h = g * a.hpk + (active ? hl : 0);
    const uint32_t qr0 = rb * kBr;
    const uint32_t qi = qr0 + j;
    const bool qvalid = active && qi < a.m;

    // keys this workgroup needs: [0, kend)
    const uint32_t kend = min(rb_last * kBr + kBr, a.m);
    const uint32_t ntiles = (kend + kBc - 1) / kBc;
    const uint32_t my_kend = active ? min(qr0 + kBr, a.m) : 0;
    const uint32_t my_ntiles = (my_kend + kBc - 1) / kBc;

    // tiles whose rows all lie below m take the cheaper copy when its 32-bit
    // per-lane offsets hold (a tile's rows span under 4 GiB: kv_stride < 2^24)
    constexpr int CPR = D / 4;
    const uint32_t lx = (uint32_t)((lane % CPR) ^ ((lane / CPR) & (swz_width(D) - 1)));
    const uint32_t ly = (uint32_t)(lane / CPR) * a.kv_stride * 4u;
    const uint32_t nfull = kFastCopy<D> && a.kv_stride < (1u << 24) ? a.m / kBc : 0;
    auto load_tile = [&](uint32_t kt, float *sk, float *sv) __attribute__((always_inline)) {
        if (kFastCopy<D> && kt < nfull) {
            // opaque per copy: the offsets are formed here, not hoisted out
            // of the tile loop and held in registers
            uint32_t x = lx, y = ly;
            asm volatile("" : "+v"(x), "+v"(y));
            load_tile_lds_full<D, NW>(a, g, kt, sk, sv, wave, x, y);
        } else {
            load_tile_lds<D, NW>(a, g, kt, sk, sv, wave, lane);
        }
    };
    load_tile(0, sK0, sV0);

    // Q^T operand: lane (j, half) holds Q[qi][8u + 4half + 0..3] for u < D/8
    float4 qt[NQ];
    {
        const float *qrow = a.q + (size_t)(qvalid ? qi : 0) * a.q_stride + (size_t)h * D;
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

    // matrix work of one tile (sk, sv in LDS) for this wave
    auto tile = [&](const float *sk, const float *sv, uint32_t kt) {
        if (kt < my_ntiles) {  // wave-uniform: not yet past this wave's diagonal
            // this lane's swizzle key, made opaque per tile so the swizzled
            // LDS addresses are formed where they are used instead of being
            // hoisted out of the loop and held in registers
            int xj = j;
            asm volatile("" : "+v"(xj));

            // S^T = K_tile . Q^T, two 32-key blocks. The K operands of step
            // u + 1 are read from LDS while the MFMAs of step u run (two
            // register sets), so the matrix pipe does not wait on LDS.
            floatx16 s0, s1;
#pragma unroll
            for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
            // chunk 2u + half of row j sits at (2u + half) ^ (j mod SW) =
            // 2u ^ xh: one XOR with a constant per step, no per-step register
            constexpr int SW = swz_width(D);
            int xh = (j & (SW - 1)) ^ half;
            asm volatile("" : "+v"(xh));
            const float *krow = sk + j * D;
            // a wave in a matrix phase gets issue priority (measured faster;
            // vector instructions do not run under fp32 MFMAs here, so this
            // orders the two waves' issue rather than hiding the softmax)
            __builtin_amdgcn_s_setprio(1);
            float4 ka[2], kb[2];
            ka[0] = ld4(krow + 4 * xh);
            kb[0] = ld4(krow + 4 * xh + 32 * D);  // row 32 + j: same swizzle
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                if (u + 1 < NQ) {
                    const float *kp = krow + 4 * ((2 * (u + 1)) ^ xh);
                    ka[(u + 1) & 1] = ld4(kp);
                    kb[(u + 1) & 1] = ld4(kp + 32 * D);
                }
                const float4 a0 = ka[u & 1], b0 = kb[u & 1];
                s0 = mfma32(a0.x, qt[u].x, s0);
                s1 = mfma32(b0.x, qt[u].x, s1);
                s0 = mfma32(a0.y, qt[u].y, s0);
                s1 = mfma32(b0.y, qt[u].y, s1);
                s0 = mfma32(a0.z, qt[u].z, s0);
                s1 = mfma32(b0.z, qt[u].z, s1);
                s0 = mfma32(a0.w, qt[u].w, s0);
                s1 = mfma32(b0.w, qt[u].w, s1);
            }
            // keep that order through scheduling: the reads of step u + 1
            // go ahead of the 8 MFMAs of step u
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads of steps 0, 1
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // MFMAs of step u
                if (u + 2 < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // reads of u + 2
            }

            __builtin_amdgcn_s_setprio(0);

            // causal mask on tiles that reach past this wave's first row (also
            // removes the re-read rows past m: their keys exceed every query)
            if (kt * kBc + kBc - 1 > qr0) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t key = kt * kBc + 8 * (e / 4) + 4 * half + (e % 4);
                    if (key > qi) s0[e] = kNegInf;
                    if (key + 32 > qi) s1[e] = kNegInf;
                }
            }

            // online softmax for query row qi (this lane and lane ^ 32 share it)
            // two chains of v_max3 over the 32 scores (no canonicalising of
            // the MFMA results, which fmaxf would add), then the partner
            // lane's maximum through a lane-half swap
            float ma = vmax3(s0[0], s0[1], s1[0]), mb = vmax3(s1[1], s0[2], s1[2]);
#pragma unroll
            for (int e = 3; e < 15; e += 2) {
                ma = vmax3(ma, s0[e], s1[e]);
                mb = vmax3(mb, s0[e + 1], s1[e + 1]);
            }
            ma = vmax3(ma, s0[15], s1[15]);
            float mx = fmaxf(ma, mb);
            mx = max_lane_pair(mx);
            // The reference max is raised (and O, l rescaled) only when some
            // row of the wave sees a score more than kLazyRescale above it;
            // otherwise the weights 2^(s - m) stay below 2^kLazyRescale and
            // O / l is the same for any reference. Every processed tile has
            // an unmasked key per row, so mx is finite; the first tile always
            // raises m from -inf.
            if (__any(mx > mrow + kLazyRescale)) {  // wave-uniform branch
                const float mnew = fmaxf(mrow, mx);
                const float cf = fast_exp2(mrow - mnew);
                mrow = mnew;
                lrow *= cf;
#pragma unroll
                for (int md = 0; md < NMD; ++md)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[md][e] *= cf;
            }
            float ls = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                s0[e] = fast_exp2(s0[e] - mrow);
                s1[e] = fast_exp2(s1[e] - mrow);
                ls += s0[e] + s1[e];
            }
            lrow += ls;

            __builtin_amdgcn_s_setprio(1);
            // O^T += V_tile^T . P^T; k-step (block mb, register e) uses key
            // 32mb + 8(e/4) + 4half + e%4, the key register e of S^T holds
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key0 = 8 * (e / 4) + 4 * half + (e % 4);
                float va[NMD], vb[NMD];
                if constexpr (NMD % 4 == 0) {
                    // NMD consecutive floats = whole 16-byte chunks: ds_read_b128
#pragma unroll
                    for (int q4 = 0; q4 < NMD / 4; ++q4) {
                        const int cchunk = NMD / 4 * xj + q4;
                        const float *vp = sv + key0 * D + 4 * swz_chunk<D>(key0, cchunk);
                        const float4 x = ld4(vp);
                        const float4 y = ld4(vp + 32 * D);  // row 32 + key0: same swizzle
                        va[4 * q4 + 0] = x.x; va[4 * q4 + 1] = x.y;
                        va[4 * q4 + 2] = x.z; va[4 * q4 + 3] = x.w;
                        vb[4 * q4 + 0] = y.x; vb[4 * q4 + 1] = y.y;
                        vb[4 * q4 + 2] = y.z; vb[4 * q4 + 3] = y.w;
                    }
                } else if constexpr (NMD == 2) {
                    // two consecutive floats, half a 16-byte chunk: ds_read_b64
                    const int f = 2 * xj;
                    const float *vp = sv + key0 * D + 4 * swz_chunk<D>(key0, f / 4) + f % 4;
                    const float2 x = *reinterpret_cast<const float2 *>(vp);
                    const float2 y = *reinterpret_cast<const float2 *>(vp + 32 * D);
                    va[0] = x.x; va[1] = x.y;
                    vb[0] = y.x; vb[1] = y.y;
                } else {
#pragma unroll
                    for (int md = 0; md < NMD; ++md) {
                        const int f = NMD * xj + md;  // float index in the V row
                        const float *vp = sv + key0 * D + 4 * swz_chunk<D>(key0, f / 4) + f % 4;
                        va[md] = vp[0];
                        vb[md] = vp[32 * D];  // row 32 + key0 has the same swizzle
                    }
                }
#pragma unroll
                for (int md = 0; md < NMD; ++md) acc[md] = mfma32(va[md], s0[e], acc[md]);
#pragma unroll
                for (int md = 0; md < NMD; ++md) acc[md] = mfma32(vb[md], s1[e], acc[md]);
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    if constexpr (NBUF == 2) {
        // two static buffers, tiles alternate between them: every LDS read
        // and every direct load names its buffer, so the compiler can see
        // the next tile's loads do not touch the tile being read
        for (uint32_t kt = 0; kt < ntiles; kt += 2) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt landed
            __syncthreads();  // every wave's loads landed; buffer 1 is free
            if (kt + 1 < ntiles) load_tile(kt + 1, sK1, sV1);
            tile(sK0, sV0, kt);
            if (kt + 1 >= ntiles) break;
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();  // buffer 0 is free
            if (kt + 2 < ntiles) load_tile(kt + 2, sK0, sV0);
            tile(sK1, sV1, kt + 1);
        }
    } else {
        for (uint32_t kt = 0; kt < ntiles; ++kt) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            tile(sK0, sV0, kt);
            if (kt + 1 < ntiles) {
                __syncthreads();  // single buffer: everyone done before it is refilled
                load_tile(kt + 1, sK0, sV0);
            }
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

// ---------------------------------------------------------------------------
// 16-row variant for grids under two workgroups per CU at head_dim 192 and
// 256 (v_mfma_f32_16x16x4_f32).
//
// There the 8-wave 32-row kernel needs head_dim registers per lane for Q^T
// and O^T alone and spills to scratch; a 16-row block needs half. The zigzag
// pairs of that kernel (short and long block on one SIMD) also leave the
// long wave running alone for the last tiles. Here a wave owns the 16-row
// blocks u and n_rb16-1-u of one head and runs them one after the other, so
// every wave carries the same number of tile steps and both waves of a SIMD
// stay busy to the end. The 8 waves of a workgroup take 8 consecutive tasks
// (u, head) of one KV head, so their row blocks differ by at most one tile
// and they still share every K/V tile in LDS: the workgroup streams the
// tiles of the first blocks, then, from tile 0 again, those of the second.
//
// Operand layouts of 16x16x4 f32: lane l supplies A[l%16][l/16] and
// B[l/16][l%16] and receives C[4(l/16) + v][l%16] in register v. With
// i = j = l%16 and kq = l/16:
//   S^T[64 keys x 16 rows] = K_tile . Q^T: four 16-key blocks kb; k-step
//     (g, c) uses d = 16g + 4kq + c, so a lane reads K[key][16g+4kq .. +3]
//     with one ds_read_b128 and holds Q[row j][16g+4kq .. +3] in registers.
//     Register v of block kb holds S^T[16kb + 4kq + v][row j].
//   O^T[D x 16 rows] += V_tile^T . P^T: k-step (kb, v) takes keys
//     16kb + 4kq + v, so its B operand is S^T register (kb, v) as it is; output
//     block mb = 4q + c holds d = 64q + 4i + c, so a lane reads the 16-byte
//     chunks i and 16 + i, ... of a V row (16 lanes: 256 contiguous bytes).
// Needs head_dim a multiple of 64. (At head_dim 128 it measured slower than
// the 32-row kernel: its per-step overheads weigh twice as much per FLOP.)
template <int D>
__global__ __launch_bounds__(512) void prefill16_kernel(PrefillArgs a) {
    constexpr int NW = 8;
    constexpr int NG = D / 16;   // float4 of the Q^T operand per lane
    constexpr int NQ4 = D / 64;  // 16-byte V chunks per lane per key
    constexpr int NMB = D / 16;  // 16-row blocks of O^T
    constexpr int NBUF = D <= 128 ? 2 : 1;
    constexpr int TILE = kBc * D;
    static_assert(D % 64 == 0, "head_dim a multiple of 64");
    __shared__ __attribute__((aligned(16))) float sK0[TILE];
    __shared__ __attribute__((aligned(16))) float sV0[TILE];
    __shared__ __attribute__((aligned(16))) float sK1[NBUF == 2 ? TILE : 4];
    __shared__ __attribute__((aligned(16))) float sV1[NBUF == 2 ? TILE : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;   // query row of this lane (and A-operand row i)
    const int kq = lane >> 4;  // k lane group

    const uint32_t g = blockIdx.x % a.kv_heads;
    const uint32_t wi = blockIdx.x / a.kv_heads;
    const uint32_t t = wi * NW + wave;
    const bool active = t < a.n_tasks16;
    const uint32_t tt = active ? t : a.n_tasks16 - 1;  // idle waves: in bounds, no store
    const uint32_t u = tt / a.hpk;
    const uint32_t h = g * a.hpk + tt % a.hpk;
    const uint32_t rbA = u, rbB = a.n_rb16 - 1 - u;  // rbB == rbA: the middle block, once

    // 64-key tiles a 16-row block needs: keys [0, min(16 rb + 16, m))
    auto tiles_of = [&](uint32_t rb) { return (min(16 * rb + 16, a.m) + kBc - 1) / kBc; };
    const uint32_t t_first = wi * NW;
    const uint32_t t_last = min(t_first + NW - 1, a.n_tasks16 - 1);
    const uint32_t uA = t_last / a.hpk;  // largest first block of the workgroup
    const uint32_t uB = t_first / a.hpk; // largest second block: a.n_rb16 - 1 - uB
    const uint32_t ntA = tiles_of(uA);
    const uint32_t ntB = a.n_rb16 - 1 - uB != uB ? tiles_of(a.n_rb16 - 1 - uB) : 0;
    const uint32_t my_ntA = active ? tiles_of(rbA) : 0;
    const uint32_t my_ntB = active && rbB != rbA ? tiles_of(rbB) : 0;

    float4 qt[NG];
    floatx4 acc[NMB];
    float mrow, lrow;
    uint32_t qr0 = 0, my_nt = 0;

    // start a block: Q^T operand (pre-scaled; zero past m), cleared state
    auto begin = [&](uint32_t rb, uint32_t nt) {
        qr0 = rb * 16;
        my_nt = nt;
        const uint32_t qi = qr0 + j;
        const bool ok = nt > 0 && qi < a.m;
        const float *qrow = a.q + (size_t)(ok ? qi : 0) * a.q_stride + (size_t)h * D + 4 * kq;
        const float qs = ok ? a.qscale : 0.f;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) qt[gg] = ld4(qrow + 16 * gg) * qs;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mb][v] = 0.f;
        mrow = kNegInf;
        lrow = 0.f;
    };
    // finish a block: normalise and store rows qr0 + j < m
    auto finish = [&]() {
        if (my_nt == 0) return;
        float l = lrow + __shfl_xor(lrow, 16);
        l += __shfl_xor(l, 32);
        const uint32_t qi = qr0 + j;
        if (qi >= a.m) return;
        const float inv = 1.0f / l;
        float *orow = a.o + (size_t)qi * a.q_stride + (size_t)h * D + 16 * kq;
#pragma unroll
        for (int q = 0; q < NQ4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                st4(orow + 64 * q + 4 * v,
                    make_float4(acc[4 * q + 0][v] * inv, acc[4 * q + 1][v] * inv,
                                acc[4 * q + 2][v] * inv, acc[4 * q + 3][v] * inv));
    };

    // matrix work of one tile (sk, sv in LDS) for this wave's current block
    auto tile = [&](const float *sk, const float *sv, uint32_t kt) {
        if (kt >= my_nt) return;  // wave-uniform
        int xj = j;
        asm volatile("" : "+v"(xj));  // swizzle key formed at each use, not held
        floatx4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) s[kb][v] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        {
            // step gg: the four 16-key blocks' K chunks (rows 16kb + i, whose
            // swizzle key is i), read one step ahead; the four accumulator
            // chains interleave so no MFMA waits on the one before it
            const float *krow = sk + xj * D;
            float4 ka[2][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                ka[0][kb] = ld4(krow + 16 * kb * D + 4 * swz_chunk<D>(xj, kq));
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                if (gg + 1 < NG) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
                        ka[(gg + 1) & 1][kb] =
                            ld4(krow + 16 * kb * D + 4 * swz_chunk<D>(xj, 4 * (gg + 1) + kq));
                }
                const float4 *kc = ka[gg & 1];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[kb].x, qt[gg].x, s[kb], 0, 0, 0);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[kb].y, qt[gg].y, s[kb], 0, 0, 0);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[kb].z, qt[gg].z, s[kb], 0, 0, 0);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[kb].w, qt[gg].w, s[kb], 0, 0, 0);
            }
            // keep that order through scheduling: the reads of step gg + 1
            // go ahead of the 16 MFMAs of step gg
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads of steps 0, 1
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // MFMAs of step gg
                if (gg + 2 < NG) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // reads of gg + 2
            }
        }
        __builtin_amdgcn_s_setprio(0);

        const uint32_t qi = qr0 + j;
        // causal mask on tiles that reach past this block's first row (also
        // removes the re-read rows past m: their keys exceed every query)
        if (kt * kBc + kBc - 1 > qr0) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (kt * kBc + 16 * kb + 4 * kq + v > qi) s[kb][v] = kNegInf;
        }
        // online softmax for row qi: its 64 scores sit in lanes j, j+16,
        // j+32, j+48, 16 each; every processed tile has an unmasked key per row
        // v_max3 over the 16 scores (as in prefill_kernel), then the other
        // lane groups of the row
        float mx = vmax3(s[0][0], s[0][1], s[0][2]);
        mx = vmax3(mx, s[0][3], s[1][0]);
        mx = vmax3(mx, s[1][1], s[1][2]);
        mx = vmax3(mx, s[1][3], s[2][0]);
        mx = vmax3(mx, s[2][1], s[2][2]);
        mx = vmax3(mx, s[2][3], s[3][0]);
        mx = vmax3(mx, s[3][1], s[3][2]);
        mx = fmaxf(mx, s[3][3]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = max_lane_pair(mx);
        if (__any(mx > mrow + kLazyRescale)) {  // wave-uniform, as in prefill_kernel
            const float mnew = fmaxf(mrow, mx);
            const float cf = fast_exp2(mrow - mnew);
            mrow = mnew;
            lrow *= cf;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mb][v] *= cf;
        }
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                s[kb][v] = fast_exp2(s[kb][v] - mrow);
                ls += s[kb][v];
            }
        lrow += ls;

        __builtin_amdgcn_s_setprio(1);
        {
            // k-step e = (kb, v) takes keys 16kb + 4kq + v; its V chunks are
            // read one step ahead of its MFMAs
            auto vload = [&](int e, float4 (&vv)[NQ4]) {
                const int key = 16 * (e >> 2) + 4 * kq + (e & 3);
                const float *vrow = sv + key * D;
#pragma unroll
                for (int q = 0; q < NQ4; ++q) vv[q] = ld4(vrow + 4 * swz_chunk<D>(key, 16 * q + xj));
            };
            float4 vv[2][NQ4];
            vload(0, vv[0]);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (e + 1 < 16) vload(e + 1, vv[(e + 1) & 1]);
                const float p = s[e >> 2][e & 3];
#pragma unroll
                for (int q = 0; q < NQ4; ++q) {
                    const float4 x = vv[e & 1][q];
                    acc[4 * q + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, p, acc[4 * q + 0], 0, 0, 0);
                    acc[4 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, p, acc[4 * q + 1], 0, 0, 0);
                    acc[4 * q + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, p, acc[4 * q + 2], 0, 0, 0);
                    acc[4 * q + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, p, acc[4 * q + 3], 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * NQ4, 0);  // reads of k-steps 0, 1
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * NQ4, 0);  // MFMAs of k-step e
                if (e + 2 < 16) __builtin_amdgcn_sched_group_barrier(0x100, NQ4, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // the workgroup's tile stream: it = 0 .. ntA-1 are tiles 0.. of the
    // first blocks, it = ntA .. ntA+ntB-1 tiles 0.. of the second blocks
    const uint32_t nit = ntA + ntB;
    auto kt_of = [&](uint32_t it) { return it < ntA ? it : it - ntA; };
    begin(rbA, my_ntA);
    if (nit > 0) load_tile_lds<D, NW>(a, g, 0, sK0, sV0, wave, lane);
    auto step = [&](uint32_t it, const float *sk, const float *sv) {
        if (it == ntA) {  // second blocks start
            finish();
            begin(rbB, my_ntB);
        }
        tile(sk, sv, kt_of(it));
    };
    if constexpr (NBUF == 2) {
        for (uint32_t it = 0; it < nit; it += 2) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile it landed
            __syncthreads();                     // every wave's loads landed; buffer 1 is free
            if (it + 1 < nit) load_tile_lds<D, NW>(a, g, kt_of(it + 1), sK1, sV1, wave, lane);
            step(it, sK0, sV0);
            if (it + 1 >= nit) break;
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();  // buffer 0 is free
            if (it + 2 < nit) load_tile_lds<D, NW>(a, g, kt_of(it + 2), sK0, sV0, wave, lane);
            step(it + 1, sK1, sV1);
        }
    } else {
        for (uint32_t it = 0; it < nit; ++it) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            step(it, sK0, sV0);
            if (it + 1 < nit) {
                __syncthreads();  // single buffer: everyone done before it is refilled
                load_tile_lds<D, NW>(a, g, kt_of(it + 1), sK0, sV0, wave, lane);
            }
        }
    }
    finish();  // the second blocks (or the first, in a workgroup without second blocks)
}

// ---------------------------------------------------------------------------
// Prompts of at most kSmallRows (16) rows: one wave per Q head h computes the
// whole problem on v_mfma_f32_16x16x4_f32 with its operands read straight
// from global memory into registers (no LDS, no barrier; each head of a KV
// group reads the group's few K and V rows, from L2 after the first).
// Lane l = (i, kk), i = l % 16, kk = l / 16. Operand layouts of 16x16x4: lane
// l supplies A[i][kk] and B[kk][i] and receives C[4kk + v][i] in register v.
//   S^T[key][row] = sum_d K[key][d] Q[row][d]: k-step s of lane group kk
//     contracts d = kk * D/4 + s, so a lane reads D/4 consecutive floats of
//     its K row and of its Q row (row i; rows past m re-read row m - 1).
//   Lane (i, kk) then holds the scores of keys 4kk + v for row i; keys above
//     the row (which include those past m) are masked, and the row's maximum
//     and sum combine the four lane groups with two exchanges. Key 0 is never
//     masked, so every maximum is finite.
//   O^T[d][row] += V^T[d][key] P^T[key][row] for output blocks b: A row i' is
//     d = b + (D/16) i', and k-step t of lane group kk takes key 4kk + t, so
//     the B operand is register t of the score accumulator and a lane reads
//     D/16 consecutive floats of V row 4kk + t per k-step.
template <int D>
__global__ __launch_bounds__(256) void prefill_small_kernel(PrefillArgs a) {
    constexpr int NS = D / 4;   // QK^T k-steps per lane group
    constexpr int NB = D / 16;  // 16-row blocks of O^T = floats of a V row per lane
    static_assert(NS % 4 == 0 && NB % 2 == 0, "whole float4 / float2 reads");
    const int lane = threadIdx.x & 63;
    const uint32_t h = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (h >= a.kv_heads * a.hpk) return;  // wave-uniform: past the last head
    const uint32_t g = h / a.hpk;
    const int i = lane & 15, kk = lane >> 4;
    const uint32_t r = min((uint32_t)i, a.m - 1);  // this lane's Q row and K row

    // V operands first: nothing they feed depends on the scores' arrival
    float vv[4][NB];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t rv = min((uint32_t)(4 * kk + t), a.m - 1);
        const float *vrow = a.v + (size_t)rv * a.kv_stride + (size_t)g * D + NB * i;
        if constexpr (NB % 4 == 0) {
#pragma unroll
            for (int c = 0; c < NB / 4; ++c) {
                const float4 x = ld4(vrow + 4 * c);
                vv[t][4 * c] = x.x; vv[t][4 * c + 1] = x.y;
                vv[t][4 * c + 2] = x.z; vv[t][4 * c + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < NB / 2; ++c) {
                const float2 x = *reinterpret_cast<const float2 *>(vrow + 2 * c);
                vv[t][2 * c] = x.x; vv[t][2 * c + 1] = x.y;
            }
        }
    }

    const float *qrow = a.q + (size_t)r * a.q_stride + (size_t)h * D + kk * NS;
    const float *krow = a.k + (size_t)r * a.kv_stride + (size_t)g * D + kk * NS;
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NS / 4; ++c) {
        const float4 q4 = ld4(qrow + 4 * c) * a.qscale;
        const float4 k4 = ld4(krow + 4 * c);
        s = mfma16(k4.x, q4.x, s);
        s = mfma16(k4.y, q4.y, s);
        s = mfma16(k4.z, q4.z, s);
        s = mfma16(k4.w, q4.w, s);
    }

#pragma unroll
    for (int v = 0; v < 4; ++v)
        if (4 * kk + v > i) s[v] = kNegInf;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = max_lane_pair(mx);
    float p[4], l = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        p[v] = fast_exp2(s[v] - mx);
        l += p[v];
    }
    l += __shfl_xor(l, 16);
    l = sum_lane_pair(l);

    floatx4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma16(vv[t][b], p[t], acc[b]);

    // register v of block b is O[i][b + NB (4kk + v)]: NB consecutive floats per v
    if ((uint32_t)i < a.m) {
        const float inv = 1.0f / l;
        float *orow = a.o + (size_t)i * a.q_stride + (size_t)h * D;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float *op = orow + NB * (4 * kk + v);
            if constexpr (NB % 4 == 0) {
#pragma unroll
                for (int c = 0; c < NB / 4; ++c)
                    *reinterpret_cast<float4 *>(op + 4 * c) =
                        make_float4(acc[4 * c][v] * inv, acc[4 * c + 1][v] * inv,
                                    acc[4 * c + 2][v] * inv, acc[4 * c + 3][v] * inv);
            } else {
#pragma unroll
                for (int c = 0; c < NB / 2; ++c)
                    *reinterpret_cast<float2 *>(op + 2 * c) =
                        make_float2(acc[2 * c][v] * inv, acc[2 * c + 1][v] * inv);
            }
        }
    }
}

template <int D>
hipError_t launch_d(const PrefillArgs &args, uint32_t grid, uint32_t nw, bool rows16,
                    bool small, hipStream_t stream) {
    if (small) {
        hipLaunchKernelGGL((prefill_small_kernel<D>), dim3(grid), dim3(256), 0, stream, args);
        return hipGetLastError();
    }
    if constexpr (D >= kMinDim4Waves && D % 64 == 0) {  // the plan's rows16 head sizes
        if (rows16) {
            hipLaunchKernelGGL((prefill16_kernel<D>), dim3(grid), dim3(8 * 64), 0, stream, args);
            return hipGetLastError();
        }
    }
    if constexpr (D >= kMinDim4Waves) {
        if (nw == 4) {
            hipLaunchKernelGGL((prefill_kernel<D, 4>), dim3(grid), dim3(4 * 64), 0, stream, args);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((prefill_kernel<D, 8>), dim3(grid), dim3(8 * 64), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillPlan &plan, const float *q, const float *k,
                          const float *v, float *o, uint32_t m, uint32_t q_stride,
                          uint32_t kv_stride, uint32_t num_q_heads, uint32_t heads_per_kv,
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
    a.n_rb = plan.n_rb;
    a.n_pairs = plan.n_pairs;
    a.wg_per_group = plan.wg_per_group;
    a.zigzag = plan.zigzag;
    a.nsub = plan.nsub;
    a.n_rb16 = plan.n_rb16;
    a.n_tasks16 = plan.n_tasks16;
    a.qscale = (1.0f / sqrtf((float)head_dim)) * kLog2e;
    const uint32_t grid = plan.grid, nw = plan.waves;
    const bool r16 = plan.rows16 != 0, sm = plan.small != 0;
    switch (head_dim) {
    case 32: return launch_d<32>(a, grid, nw, r16, sm, stream);
    case 64: return launch_d<64>(a, grid, nw, r16, sm, stream);
    case 96: return launch_d<96>(a, grid, nw, r16, sm, stream);
    case 128: return launch_d<128>(a, grid, nw, r16, sm, stream);
    case 160: return launch_d<160>(a, grid, nw, r16, sm, stream);
    case 192: return launch_d<192>(a, grid, nw, r16, sm, stream);
    case 224: return launch_d<224>(a, grid, nw, r16, sm, stream);
    case 256: return launch_d<256>(a, grid, nw, r16, sm, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
