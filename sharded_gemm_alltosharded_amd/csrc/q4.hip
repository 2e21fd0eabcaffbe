// 4-bit affine weight-streaming GEMM for few tokens (M <= 32): the quantized
// all-to-sharded / sharded-to-all layers of "MLX 张量并行实战指南" sections 2.3
// and 6 (group_size 64, bits 4, mode affine), HBM-bound at 4.5 bits/weight.
//
// Per quantization group g of 64 inputs of weight row n:
//     sum_k w[n,k] x[t,k] = s[n,g] * sum_k q[n,k] x[t,k] + b[n,g] * sum_k x[t,k]
// The codes stay exact: a mask-and-or turns eight 4-bit codes into eight
// 16-bit numbers c + q with c = 128 (bf16) or 1024 (fp16), so the MFMA forms
// acc = sum (c + q) x = sum q x + c * xs, and the epilogue of the group adds
//     s * acc + (b - c * s) * xs,
// where xs = sum_k x[t,k] comes from one more MFMA of the token fragments
// against an all-ones operand (same register layout as acc, no shuffles).
//
// MFMA v_mfma_f32_32x32x16: the tokens are the row operand (32 token slots),
// 32 weight rows the column operand, so each lane owns one weight row and
// needs one (scale, bias) pair per group.  Lane (row j, half h) loads 16 bytes
// = codes of chunks 4h .. 4h+3 of the group; MFMA step u of the group uses
// chunk 4h + u, and the token fragment of step u holds the same chunk.
//
// Workgroup = 4 waves on RB blocks of 32 rows; each wave takes a contiguous
// quarter of the groups (in runs of 4, so scales and biases arrive 8 bytes at
// a time).  Wave partials are summed in LDS in wave order.  Sharded-to-all
// layers split by rank (grid.y = P) and reduce the rank partials in rank
// order in the last workgroup to arrive, as in the dense streaming kernel.
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// eight codes (stored in q4_nibble_pos order) -> eight (c + q) 16-bit numbers
template <bool F16>
__device__ __forceinline__ u32x4 unpack8(uint32_t w) {
    constexpr uint32_t magic = F16 ? 0x64006400u : 0x43004300u;
    u32x4 r;
    r[0] = (w & 0x000F000Fu) | magic;
    r[1] = ((w >> 4) & 0x000F000Fu) | magic;
    r[2] = ((w >> 8) & 0x000F000Fu) | magic;
    r[3] = ((w >> 12) & 0x000F000Fu) | magic;
    return r;
}

template <int TB, int RB, bool F16, bool SWIGLU, bool SPLIT>
__global__ __launch_bounds__(256) void q4_kernel(Problem p) {
    constexpr int ROWS = SWIGLU ? RB / 2 * 32 : RB * 32;  // logical columns per workgroup
    constexpr int NR = 4 * TB;                            // token registers in use
    constexpr int NV = RB * TB;                           // values per thread after reduction
    constexpr float C = F16 ? 1024.f : 128.f;
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    __shared__ float red[4][RB * NR][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = blockIdx.x;
    const int seg_lo = SPLIT ? blockIdx.y : 0;
    const int seg_cnt = SPLIT ? 1 : p.nseg;
    const int64_t base = (int64_t)rg * ROWS;
    const int h = lane >> 5;

    int64_t qoff[RB], goff[RB];
    bool wok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row;
        if constexpr (SWIGLU) {
            const int64_t j = base + (rb >> 1) * 32 + (lane & 31);
            wok[rb] = j < p.N;
            row = weight_row(p, wok[rb] ? j : 0, rb & 1);
        } else {
            const int64_t n = base + rb * 32 + (lane & 31);
            wok[rb] = n < p.N;
            row = wok[rb] ? n : 0;
        }
        qoff[rb] = row * p.ldq + h * 4;
        goff[rb] = row * p.ldg;
    }
    const int t = lane & 31;
    const bool xok = t < p.M;
    const int64_t xoff = (int64_t)(xok ? t : 0) * p.lda + h * 32;

    const u32x4 ones = F16 ? u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                           : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const u32x4 zero = {0u, 0u, 0u, 0u};

    f32x16 y[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) y[rb][r] = 0.f;

    const int G = p.Kseg / 64;  // groups per segment (a multiple of 4)
    const int runs = G / 4;
    const int r_lo = wave * runs / 4, r_hi = (wave + 1) * runs / 4;
    for (int s = seg_lo; s < seg_lo + seg_cnt; ++s) {
        const uint32_t* Qb = p.wq + s * p.q_seg;
        const uint16_t* Sb = p.qs + s * p.g_seg;
        const uint16_t* Bb = p.qb + s * p.g_seg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg;
        for (int run = r_lo; run < r_hi; ++run) {
            const int g0 = run * 4;
            u32x4 wv[4][RB];
            u32x2 sv[RB], bv[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int gi = 0; gi < 4; ++gi)
                    wv[gi][rb] = wok[rb] ? *(const u32x4*)(Qb + qoff[rb] + (g0 + gi) * 8) : zero;
                sv[rb] = *(const u32x2*)(Sb + goff[rb] + g0);
                bv[rb] = *(const u32x2*)(Bb + goff[rb] + g0);
            }
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                u32x4 xf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    xf[u] = xok ? *(const u32x4*)(Ab + xoff + (g0 + gi) * 64 + u * 8) : zero;
                f32x16 xs;
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[r] = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u) xs = mfma32<F16>(xf[u], ones, xs);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x16 acc;
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc = mfma32<F16>(xf[u], unpack8<F16>(wv[gi][rb][u]), acc);
                    const uint32_t sw = sv[rb][gi >> 1], bw = bv[rb][gi >> 1];
                    const float sc = f16_to_f32((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                    const float bi = f16_to_f32((uint16_t)((gi & 1) ? (bw >> 16) : (bw & 0xFFFFu)));
                    const float bp = fmaf(-C, sc, bi);
#pragma unroll
                    for (int r = 0; r < NR; ++r) y[rb][r] = fmaf(sc, acc[r], fmaf(bp, xs[r], y[rb][r]));
                }
            }
        }
    }

    // ---- wave partials -> workgroup result (wave order)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < NR; ++r) red[wave][rb * NR + r][lane] = y[rb][r];
    __syncthreads();
    // thread owns register index R = 4 i + tid / 64 (R = rb * NR + r) at lane tid % 64
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int R = 4 * i + (tid >> 6), ln = tid & 63;
        v[i] = ((red[0][R][ln] + red[1][R][ln]) + red[2][R][ln]) + red[3][R][ln];
    }

    if constexpr (SPLIT) {
        const int nrg = gridDim.x;
        const int64_t slab = (int64_t)nrg * NV * 256;
        float* mine = p.ws + blockIdx.y * slab + (int64_t)rg * NV * 256;
#pragma unroll
        for (int i = 0; i < NV; ++i) mine[i * 256 + tid] = v[i];
        __threadfence();
        __syncthreads();
        __shared__ int last;
        if (tid == 0) {
            const unsigned prev = atomicAdd(&p.counters[rg], 1u);
            last = prev == (unsigned)p.nseg - 1;
            if (last) p.counters[rg] = 0u;
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = 0.f;
        for (int s = 0; s < p.nseg; ++s) {  // rank order
            const float* src = p.ws + s * slab + (int64_t)rg * NV * 256;
#pragma unroll
            for (int i = 0; i < NV; ++i) v[i] += src[i * 256 + tid];
        }
    }

    // ---- epilogue
    const int ln = tid & 63;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int R = 4 * i + (tid >> 6);
        const int rb = R / NR, r = R % NR;
        if constexpr (SWIGLU) {
            if (rb & 1) continue;
        }
        const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
        const int64_t n = SWIGLU ? base + (rb >> 1) * 32 + (ln & 31) : base + rb * 32 + (ln & 31);
        if (m >= p.M || n >= p.N) continue;
        float x = SWIGLU ? silu_f32(v[i]) * v[i + TB] : v[i];
        if (p.bias) x += load_as_f32(p.bias, p.dtype, n);
        const int64_t o = out_index(p, m, n);
        if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
        store_from_f32(p.out, p.out_dtype, o, x);
    }
}

SplitLayout q4_split_layout(int M, int N, int nseg) {
    const size_t TB = (M + 7) / 8, RB = 2;
    const size_t nrg = (N + RB * 32 - 1) / (RB * 32);
    return {nseg * nrg * RB * TB * 256, nrg};
}

template <int TB, bool F16>
static hipError_t launch_tb(const Problem& p, hipStream_t s) {
    constexpr int RB = 2;
    if (p.swiglu) {
        const int nrg = (p.N + RB / 2 * 32 - 1) / (RB / 2 * 32);
        hipLaunchKernelGGL((q4_kernel<TB, RB, F16, true, false>), dim3(nrg), dim3(256), 0, s, p);
    } else {
        const int nrg = (p.N + RB * 32 - 1) / (RB * 32);
        if (p.split)
            hipLaunchKernelGGL((q4_kernel<TB, RB, F16, false, true>), dim3(nrg, p.nseg), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((q4_kernel<TB, RB, F16, false, false>), dim3(nrg), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <bool F16>
static hipError_t launch_f(const Problem& p, hipStream_t s) {
    switch ((p.M + 7) / 8) {
    case 1: return launch_tb<1, F16>(p, s);
    case 2: return launch_tb<2, F16>(p, s);
    case 3: return launch_tb<3, F16>(p, s);
    default: return launch_tb<4, F16>(p, s);
    }
}

hipError_t launch_q4(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    return p.dtype == SG_F16 ? launch_f<true>(p, s) : launch_f<false>(p, s);
}

// Reorder the eight codes of every word: forward (standard -> kernel order,
// code k moves from nibble k to nibble q4_nibble_pos(k)) or back.
__global__ void q4_repack_kernel(uint32_t* w, int64_t n, int forward) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t a = w[i];
    uint32_t r = 0;
    for (int k = 0; k < 8; ++k) {
        const int src = forward ? k : q4_nibble_pos(k);
        const int dst = forward ? q4_nibble_pos(k) : k;
        r |= ((a >> (4 * src)) & 0xFu) << (4 * dst);
    }
    w[i] = r;
}

hipError_t q4_repack(uint32_t* w, int64_t n, int forward, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(q4_repack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w, n, forward);
    return hipGetLastError();
}

}  // namespace sg
