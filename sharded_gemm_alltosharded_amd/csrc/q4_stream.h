// The 4-bit affine weight-streaming kernel (q4_kernel) and its launch
// templates, shared by q4.hip (1 to 16 tokens) and q4_wide.hip (17 to 32
// tokens, built with VGPR-form MFMAs).  The design is described in q4.hip.
#pragma once
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

// eight codes (stored in q4_nibble_pos order) -> eight (c + q) 16-bit numbers.
// mask = 0x000F000F and magic = the 16-bit pattern of c in both halves, held in
// registers so that each and-or is one v_and_or_b32 (gfx9's three-operand
// instructions take no literal constants).
__device__ __forceinline__ u32x4 unpack8(uint32_t w, uint32_t mask, uint32_t magic) {
    u32x4 r;
    r[0] = (w & mask) | magic;
    r[1] = ((w >> 4) & mask) | magic;
    r[2] = ((w >> 8) & mask) | magic;
    r[3] = ((w >> 12) & mask) | magic;
    return r;
}

// the fp32 MFMA of the bias term: D (32 x 32) += A (32 x 2) B (2 x 32), lane l
// holding A[l & 31][l >> 5] and B[l >> 5][l & 31]
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int TB, int RB, int NW, bool F16, bool SWIGLU, bool PF, bool XH>
__global__ __launch_bounds__(NW * 64) void q4_kernel(Problem p) {
    constexpr int ROWS = SWIGLU ? RB / 2 * 32 : RB * 32;  // logical columns per workgroup
    constexpr int NR = 4 * TB;                            // token registers in use
    constexpr int SLOT = RB * NR * 64;                    // floats per unit slot
    constexpr float C = F16 ? 1024.f : 128.f;
    // the bias term on the fp32 MFMA (MB) once the tokens fill most of the
    // accumulators; with up to 8 tokens its two FMAs per group touch only 4 of
    // them, and the MFMA's 16 live accumulators would cost registers instead
    constexpr bool MB = TB >= 2;
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    extern __shared__ float slots[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    const int h = lane >> 5;
    const int J = p.nseg >= NW ? 1 : NW / p.nseg;  // waves per rank
    const int units = p.nseg * J;
    const int G = p.Kseg / 64;                     // groups per rank (a multiple of 4)
    const int runs = G / 4;

    int64_t qoff[RB], goff[RB];
    bool wok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row;
        if constexpr (SWIGLU) {
            const int64_t jj = base + (rb >> 1) * 32 + (lane & 31);
            wok[rb] = jj < p.N;
            row = weight_row(p, wok[rb] ? jj : 0, rb & 1);
        } else {
            const int64_t n = base + rb * 32 + (lane & 31);
            wok[rb] = n < p.N;
            row = wok[rb] ? n : 0;
        }
        qoff[rb] = q4_word_offset(row, 4 * h, G);  // group g at + 256 g
        goff[rb] = q4_group_offset(row, 0, G);     // run r at + 128 r
    }
    // Rows past N and tokens past M read row / token 0 (never stored).  With MB
    // the loads take no branch; without, they are skipped and read as zero
    // (measured faster with up to 8 tokens, whose registers are nearly full).
    const int t = lane & 31;
    const bool xok = MB || t < p.M;
    const int64_t xoff = (int64_t)(t < p.M ? t : 0) * p.lda + h * 32;
    const u32x4 ones = F16 ? u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                           : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const f32x16 fzero = {};
    uint32_t mask = 0x000F000Fu, magic = F16 ? 0x64006400u : 0x43004300u;
    if constexpr (MB) {
        asm("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
        asm("v_mov_b32 %0, %1" : "=v"(magic) : "i"(F16 ? 0x64006400 : 0x43004300));
    }
    const int hs = 16 * h;  // this lane's half of a scale word: group 2p + h of pair p

    for (int u = wave; u < units; u += NW) {
        const int s = u / J, j = u % J;
        const uint32_t* Qb = p.wq + s * p.q_seg;
        const uint16_t* Sb = p.qs + s * p.g_seg;
        const uint16_t* Bb = p.qb + s * p.g_seg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg + xoff;
        f32x16 y[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) y[rb] = fzero;
        // codes, scales and biases of a run of 4 groups; with PF the next run's
        // are in flight while this one is computed (register double buffer)
        constexpr int NB = PF ? 2 : 1;
        u32x4 wv[NB][4][RB];
        u32x2 sv[NB][RB], bv[NB][RB];
        auto load = [&](int buf, int run) {
            const uint32_t* qr = Qb + (int64_t)run * 1024;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int gi = 0; gi < 4; ++gi)
                    wv[buf][gi][rb] = (MB || wok[rb]) ? __builtin_nontemporal_load((const u32x4*)(qr + qoff[rb] + gi * 256))
                                                      : zero;
                sv[buf][rb] = *(const u32x2*)(Sb + goff[rb] + (int64_t)run * 128);
                bv[buf][rb] = *(const u32x2*)(Bb + goff[rb] + (int64_t)run * 128);
            }
        };
        auto compute = [&](int buf, int run) {
            const int g0 = run * 4;
            // XH: the run's activation fragments are loaded up front (one L2
            // round trip per run instead of one per group)
            u32x4 xr[XH ? 4 : 1][4];
            if constexpr (XH) {
#pragma unroll
                for (int gi = 0; gi < 4; ++gi)
#pragma unroll
                    for (int q = 0; q < 4; ++q) xr[gi][q] = xok ? *(const u32x4*)(Ab + (g0 + gi) * 64 + q * 8) : zero;
            }
            float xa = 0.f;  // A operand of the pair's bias MFMA: xs[token t][group 2p + h]
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                u32x4 xf[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xf[q] = XH ? xr[XH ? gi : 0][q] : (xok ? *(const u32x4*)(Ab + (g0 + gi) * 64 + q * 8) : zero);
                // MB: ones (A) x tokens (B), every register of lane l holds xs of
                // token l & 31; else tokens (A) x ones (B), xs in acc's layout
                f32x16 xs = fzero;
#pragma unroll
                for (int q = 0; q < 4; ++q) xs = MB ? mfma32<F16>(ones, xf[q], xs) : mfma32<F16>(xf[q], ones, xs);
                if constexpr (MB) xa = (gi & 1) ? (h ? xs[0] : xa) : xs[0];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x16 acc = fzero;
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = mfma32<F16>(xf[q], unpack8(wv[buf][gi][rb][q], mask, magic), acc);
                    const uint32_t sw = sv[buf][rb][gi >> 1];
                    const float sc = f16_to_f32((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                    if constexpr (MB) {
#pragma unroll
                        for (int r = 0; r < NR; ++r) y[rb][r] = fmaf(sc, acc[r], y[rb][r]);
                    } else {
                        const uint32_t bw = bv[buf][rb][gi >> 1];
                        const float bi = f16_to_f32((uint16_t)((gi & 1) ? (bw >> 16) : (bw & 0xFFFFu)));
                        const float bp = fmaf(-C, sc, bi);
#pragma unroll
                        for (int r = 0; r < NR; ++r) y[rb][r] = fmaf(sc, acc[r], fmaf(bp, xs[r], y[rb][r]));
                    }
                }
                if (MB && (gi & 1)) {
                    // bias term of groups gi - 1, gi: lane (row, h) supplies (b - c s) of group gi - 1 + h
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const float sc = f16_to_f32((uint16_t)(sv[buf][rb][gi >> 1] >> hs));
                        const float bi = f16_to_f32((uint16_t)(bv[buf][rb][gi >> 1] >> hs));
                        y[rb] = mfma32_f32(xa, fmaf(-C, sc, bi), y[rb]);
                    }
                }
            }
        };
        if constexpr (PF) {
            int run = j;
            if (run < runs) load(0, run);
            for (; run + J < runs; run += 2 * J) {
                load(1, run + J);
                compute(0, run);
                if (run + 2 * J < runs) load(0, run + 2 * J);
                compute(1, run + J);
            }
            if (run < runs) compute(0, run);
        } else {
            for (int run = j; run < runs; run += J) {
                load(0, run);
                compute(0, run);
            }
        }
        float* slot = slots + (size_t)u * SLOT;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < NR; ++r) slot[(rb * NR + r) * 64 + lane] = y[rb][r];
    }
    __syncthreads();

    // ---- reduction (parts of a rank in order, then ranks in order) + epilogue
    constexpr int NE = (SWIGLU ? RB / 2 : RB) * NR * 64;
    for (int idx = tid; idx < NE; idx += NW * 64) {
        const int ln = idx & 63, r = (idx >> 6) % NR, rbo = (idx >> 6) / NR;
        const int rb = SWIGLU ? 2 * rbo : rbo;
        const int off = (rb * NR + r) * 64 + ln;
        float v = 0.f, vu = 0.f;
        for (int s = 0; s < p.nseg; ++s) {
            float zs = 0.f, zu = 0.f;
            for (int jj = 0; jj < J; ++jj) {
                const float* sl = slots + (size_t)(s * J + jj) * SLOT;
                zs += sl[off];
                if constexpr (SWIGLU) zu += sl[off + NR * 64];
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

template <int TB, int RB, int NW, bool F16, bool PF = false, bool XH = false>
hipError_t launch_q4_variant(const Problem& p, hipStream_t s, size_t lds) {
    if (p.swiglu) {
        if constexpr (RB % 2 == 0) {
            const int nwg = (p.N + RB / 2 * 32 - 1) / (RB / 2 * 32);
            launch(q4_kernel<TB, RB, NW, F16, true, PF, XH>, dim3(nwg), dim3(NW * 64), lds, s, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        const int nwg = (p.N + RB * 32 - 1) / (RB * 32);
        launch(q4_kernel<TB, RB, NW, F16, false, PF, XH>, dim3(nwg), dim3(NW * 64), lds, s, p);
    }
    return hipGetLastError();
}

template <int TB, int RB, bool F16>
static hipError_t launch_rb(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    // up to 16 tokens the run's activation fragments are hoisted (measured
    // faster); beyond that their registers cost more than the latency saved
    constexpr bool XH = TB <= 2;
    return sh.NW == 4 ? launch_q4_variant<TB, RB, 4, F16, false, XH>(p, s, sh.lds)
                      : launch_q4_variant<TB, RB, 8, F16, false, XH>(p, s, sh.lds);
}

template <int TB, bool F16>
static hipError_t launch_tb(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    switch (sh.RB) {
    case 1: return launch_rb<TB, 1, F16>(p, s, sh);
    case 2: return launch_rb<TB, 2, F16>(p, s, sh);
    default: return launch_rb<TB, 4, F16>(p, s, sh);
    }
}

// the launches for 17 to 32 tokens (three or four 8-token blocks), q4_wide.hip
template <bool F16>
hipError_t launch_q4_wide(const Problem& p, hipStream_t s, const Q4Shape& sh);

}  // namespace sg
