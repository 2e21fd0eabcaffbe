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
// Workgroup = NW waves on RB blocks of 32 rows (a gate/up pair for SwiGLU)
// across every rank; a wave takes one (row block, rank, part) unit and walks
// that rank's groups in runs of 4 (so scales and biases arrive 8 bytes at a
// time), runs j, j + J, ...  Unit partials land in LDS slots and are summed in
// part order, then rank order -- the fused all_sum, as in the dense streaming
// kernel -- with no cross-workgroup traffic.
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

template <int TB, int RB, int NW, bool F16, bool SWIGLU>
__global__ __launch_bounds__(NW * 64) void q4_kernel(Problem p) {
    constexpr int ROWS = SWIGLU ? RB / 2 * 32 : RB * 32;  // logical columns per workgroup
    constexpr int NR = 4 * TB;                            // token registers in use
    constexpr int SLOT = NR * 64;                         // floats per unit slot
    constexpr float C = F16 ? 1024.f : 128.f;
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    extern __shared__ float slots[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    const int h = lane >> 5;
    const int per_rb = p.nseg >= NW / RB ? p.nseg : (NW / RB / p.nseg) * p.nseg;
    const int J = per_rb / p.nseg;  // waves per (row block, rank)
    const int units = RB * per_rb;
    const int G = p.Kseg / 64;      // groups per rank (a multiple of 4)
    const int runs = G / 4;

    const int t = lane & 31;
    const bool xok = t < p.M;
    const int64_t xoff = (int64_t)(xok ? t : 0) * p.lda + h * 32;
    const u32x4 ones = F16 ? u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                           : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const u32x4 zero = {0u, 0u, 0u, 0u};

    for (int u = wave; u < units; u += NW) {
        const int rb = u / per_rb, s = (u % per_rb) / J, j = u % J;
        int64_t row;
        bool wok;
        if constexpr (SWIGLU) {
            const int64_t jj = base + (rb >> 1) * 32 + (lane & 31);
            wok = jj < p.N;
            row = weight_row(p, wok ? jj : 0, rb & 1);
        } else {
            const int64_t n = base + rb * 32 + (lane & 31);
            wok = n < p.N;
            row = wok ? n : 0;
        }
        const uint32_t* Qb = p.wq + s * p.q_seg + row * p.ldq + h * 4;
        const uint16_t* Sb = p.qs + s * p.g_seg + row * p.ldg;
        const uint16_t* Bb = p.qb + s * p.g_seg + row * p.ldg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg + xoff;

        f32x16 y;
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = 0.f;
        for (int run = j; run < runs; run += J) {
            const int g0 = run * 4;
            u32x4 wv[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) wv[gi] = wok ? *(const u32x4*)(Qb + (g0 + gi) * 8) : zero;
            const u32x2 sv = *(const u32x2*)(Sb + g0);
            const u32x2 bv = *(const u32x2*)(Bb + g0);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                u32x4 xf[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xf[q] = xok ? *(const u32x4*)(Ab + (g0 + gi) * 64 + q * 8) : zero;
                f32x16 xs, acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[r] = acc[r] = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xs = mfma32<F16>(xf[q], ones, xs);
                    acc = mfma32<F16>(xf[q], unpack8<F16>(wv[gi][q]), acc);
                }
                const uint32_t sw = sv[gi >> 1], bw = bv[gi >> 1];
                const float sc = f16_to_f32((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                const float bi = f16_to_f32((uint16_t)((gi & 1) ? (bw >> 16) : (bw & 0xFFFFu)));
                const float bp = fmaf(-C, sc, bi);
#pragma unroll
                for (int r = 0; r < NR; ++r) y[r] = fmaf(sc, acc[r], fmaf(bp, xs[r], y[r]));
            }
        }
        float* slot = slots + (size_t)u * SLOT;
#pragma unroll
        for (int r = 0; r < NR; ++r) slot[r * 64 + lane] = y[r];
    }
    __syncthreads();

    // ---- reduction (parts of a rank in order, then ranks in order) + epilogue
    constexpr int NE = (SWIGLU ? RB / 2 : RB) * SLOT;
    for (int idx = tid; idx < NE; idx += NW * 64) {
        const int ln = idx & 63, r = (idx >> 6) % NR, rbo = (idx >> 6) / NR;
        const int rb = SWIGLU ? 2 * rbo : rbo;
        float v = 0.f, vu = 0.f;
        for (int s = 0; s < p.nseg; ++s) {
            float zs = 0.f, zu = 0.f;
            for (int jj = 0; jj < J; ++jj) {
                zs += slots[(size_t)(rb * per_rb + s * J + jj) * SLOT + r * 64 + ln];
                if constexpr (SWIGLU) zu += slots[(size_t)((rb + 1) * per_rb + s * J + jj) * SLOT + r * 64 + ln];
            }
            v += zs;
            vu += zu;
        }
        const int m = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
        const int64_t n = base + rbo * 32 + (ln & 31);
        if (m >= p.M || n >= p.N) continue;
        float x = SWIGLU ? silu_f32(v) * vu : v;
        if (p.bias) x += load_as_f32(p.bias, p.dtype, n);
        const int64_t o = out_index(p, m, n);
        if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
        store_from_f32(p.out, p.out_dtype, o, x);
    }
}

// Shape choice: RB row blocks of 32 per workgroup (a gate/up pair for
// SwiGLU), NW waves, several thousand waves on the chip.
Q4Shape q4_shape(int M, int N, int nseg, int swiglu) {
    Q4Shape sh;
    sh.TB = (M + 7) / 8;
    sh.RB = swiglu ? 2 : 1;
    const int rows = swiglu ? N * 2 : N;
    const int64_t wgs = ((int64_t)rows + sh.RB * 32 - 1) / (sh.RB * 32);
    int nw = 4;
    while (nw < 8 && (wgs * nw < 4096 || nw < sh.RB * nseg)) nw *= 2;
    sh.NW = nw;
    const int per_rb = nseg >= nw / sh.RB ? nseg : (nw / sh.RB / nseg) * nseg;
    sh.lds = (size_t)sh.RB * per_rb * 4 * sh.TB * 64 * sizeof(float);
    return sh;
}

template <int TB, int NW, bool F16>
static hipError_t launch_nw(const Problem& p, hipStream_t s, size_t lds) {
    if (p.swiglu) {
        const int nwg = (p.N + 31) / 32;
        hipLaunchKernelGGL((q4_kernel<TB, 2, NW, F16, true>), dim3(nwg), dim3(NW * 64), lds, s, p);
    } else {
        const int nwg = (p.N + 31) / 32;
        hipLaunchKernelGGL((q4_kernel<TB, 1, NW, F16, false>), dim3(nwg), dim3(NW * 64), lds, s, p);
    }
    return hipGetLastError();
}

template <int TB, bool F16>
static hipError_t launch_tb(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    switch (sh.NW) {
    case 4: return launch_nw<TB, 4, F16>(p, s, sh.lds);
    default: return launch_nw<TB, 8, F16>(p, s, sh.lds);
    }
}

template <bool F16>
static hipError_t launch_f(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    switch (sh.TB) {
    case 1: return launch_tb<1, F16>(p, s, sh);
    case 2: return launch_tb<2, F16>(p, s, sh);
    case 3: return launch_tb<3, F16>(p, s, sh);
    default: return launch_tb<4, F16>(p, s, sh);
    }
}

hipError_t launch_q4(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const Q4Shape sh = q4_shape(p.M, p.N, p.nseg, p.swiglu);
    return p.dtype == SG_F16 ? launch_f<true>(p, s, sh) : launch_f<false>(p, s, sh);
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
