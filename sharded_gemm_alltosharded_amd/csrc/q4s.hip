// 4-bit affine weight streaming on 16-row blocks: the quantized layers of
// "MLX 张量并行实战指南" sections 2.3 and 6 (group_size 64, bits 4, affine) for
// few tokens, reading the same stored codes, scales and biases as q4.hip.
//
// q4.hip's v_mfma_f32_32x32x16 owns 32 weight rows per block, so a layer with
// 4096 outputs (the down projection of the MLP) gives only 128 workgroups for
// 256 CUs.  Here v_mfma_f32_16x16x32 takes 16 weight rows per block: the
// activations are the A operand (16 token rows), the weights the B operand (16
// columns = weight rows), so each lane owns one weight row for 4 tokens and
// needs one (scale, bias) pair per group, as in q4.hip.
//
// k order.  An MFMA sums over its 32 k positions in any order the two operands
// agree on.  For group g (64 inputs) and step u in {0, 1}, the lane with chunk
// slot c = lane >> 4 supplies k = 64 g + 16 c + 8 u + (0..7): the weight lane
// takes code word 2c + u of its row's group (eight codes in one word, stored
// so that a mask-and-or gives them in k order), the activation lane the eight
// values x[t, 64 g + 16 c + 8 u ..].  A lane's two words (2c, 2c + 1) are 8
// contiguous bytes of the stored fragment, so one wave-wide load brings a
// group's 16 rows (512 bytes), and a lane's activations are 32 contiguous
// bytes.  The affine terms are as in q4.hip: acc = sum (C + q) x, xs = sum x
// from an MFMA against an all-ones operand, and per group
//     y += s * acc + (b - C s) * xs.
//
// Workgroup = NW waves on RB blocks of 16 rows (gate/up pairs for SwiGLU)
// across every rank of the layer; units (rank s, part j) walk runs of 4 groups
// (scales and biases arrive 8 bytes at a time) j, j + J, ...; unit partials
// land in LDS slots and are summed in part order, then rank order, then the
// bias once -- the fused all_sum.  Rows past N and tokens past M read a valid
// row or token (the loads need no branch); their results are never stored.
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// eight codes (stored in q4_nibble_pos order) -> eight (C + q) 16-bit numbers
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

}  // namespace

template <int MT, int RB, int NW, bool F16, bool SWIGLU>
__global__ __launch_bounds__(NW * 64) void q4s_kernel(Problem p) {
    constexpr int ROWS = SWIGLU ? RB / 2 * 16 : RB * 16;  // logical columns per workgroup
    constexpr int SLOT = RB * MT * 4 * 64;                 // floats per unit slot
    constexpr float C = F16 ? 1024.f : 128.f;
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    extern __shared__ float slots[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    const int c = lane >> 4;
    const int J = p.nseg >= NW ? 1 : NW / p.nseg;  // waves per rank
    const int units = p.nseg * J;
    const int G = p.Kseg / 64;  // groups per rank (a multiple of 4)
    const int runs = G / 4;

    int64_t qoff[RB], goff[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row;
        if constexpr (SWIGLU) {
            const int64_t jj = base + (rb >> 1) * 16 + (lane & 15);
            row = weight_row(p, jj < p.N ? jj : 0, rb & 1);
        } else {
            const int64_t n = base + rb * 16 + (lane & 15);
            row = n < p.N ? n : 0;
        }
        qoff[rb] = q4_word_offset(row, 2 * c, G);  // group g at + 256 g (u32)
        goff[rb] = q4_group_offset(row, 0, G);     // run r at + 128 r (halves)
    }
    int64_t xoff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = mt * 16 + (lane & 15);
        // row-major: group g at + 64 g (steps u = 0, 1 at + 0, + 8); fragment-major
        // (act_frag_offset_q4): group g at + 1024 g (steps at + 0, + 512)
        xoff[mt] = p.xfrag ? act_frag_offset_q4(t, 16 * c, p.Kseg / 32) : (int64_t)(t < p.M ? t : 0) * p.lda + 16 * c;
    }
    const int64_t xg = p.xfrag ? 1024 : 64, xu = p.xfrag ? 512 : 8;  // elements per group, per step
    const u32x4 ones = F16 ? u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                           : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    for (int u = wave; u < units; u += NW) {
        const int s = u / J, j = u - s * J;
        const uint32_t* Qb = p.wq + s * p.q_seg;
        const uint16_t* Sb = p.qs + s * p.g_seg;
        const uint16_t* Bb = p.qb + s * p.g_seg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg;
        f32x4 y[RB][MT];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) y[rb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // codes, scales and biases of a run of 4 groups; the next run's are in
        // flight while this one is computed (register double buffer)
        u32x2 cw[2][4][RB], sv[2][RB], bv[2][RB];
        auto load = [&](int buf, int run) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int gi = 0; gi < 4; ++gi)
                    cw[buf][gi][rb] = __builtin_nontemporal_load((const u32x2*)(Qb + qoff[rb] + (int64_t)(run * 4 + gi) * 256));
                sv[buf][rb] = *(const u32x2*)(Sb + goff[rb] + (int64_t)run * 128);
                bv[buf][rb] = *(const u32x2*)(Bb + goff[rb] + (int64_t)run * 128);
            }
        };
        auto compute = [&](int buf, int run) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int g = run * 4 + gi;
                u32x4 xf[MT][2];
                f32x4 xs[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xf[mt][0] = *(const u32x4*)(Ab + xoff[mt] + g * xg);
                    xf[mt][1] = *(const u32x4*)(Ab + xoff[mt] + g * xg + xu);
                    xs[mt] = mfma16<F16>(xf[mt][0], ones, f32x4{0.f, 0.f, 0.f, 0.f});
                    xs[mt] = mfma16<F16>(xf[mt][1], ones, xs[mt]);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint32_t sw = sv[buf][rb][gi >> 1], bw = bv[buf][rb][gi >> 1];
                    const float sc = f16_to_f32((uint16_t)((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                    const float bi = f16_to_f32((uint16_t)((gi & 1) ? (bw >> 16) : (bw & 0xFFFFu)));
                    const float bp = fmaf(-C, sc, bi);
                    const u32x4 w0 = unpack8<F16>(cw[buf][gi][rb][0]), w1 = unpack8<F16>(cw[buf][gi][rb][1]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        f32x4 acc = mfma16<F16>(xf[mt][0], w0, f32x4{0.f, 0.f, 0.f, 0.f});
                        acc = mfma16<F16>(xf[mt][1], w1, acc);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[rb][mt][e] = fmaf(sc, acc[e], fmaf(bp, xs[mt][e], y[rb][mt][e]));
                    }
                }
            }
        };
        int run = j;
        if (run < runs) load(0, run);
        for (; run + J < runs; run += 2 * J) {
            load(1, run + J);
            compute(0, run);
            if (run + 2 * J < runs) load(0, run + 2 * J);
            compute(1, run + J);
        }
        if (run < runs) compute(0, run);

        float* slot = slots + (size_t)u * SLOT;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) slot[((rb * MT + mt) * 4 + e) * 64 + lane] = y[rb][mt][e];
    }
    __syncthreads();

    // ---- reduction (parts of a rank in order, then ranks in order) + epilogue.
    // Element ((rb MT + mt) 4 + e) 64 + ln holds token mt 16 + 4 (ln >> 4) + e
    // of weight row rb 16 + (ln & 15).
    constexpr int NE = SWIGLU ? SLOT / 2 : SLOT;
    for (int idx = tid; idx < NE; idx += NW * 64) {
        const int ln = idx & 63, e = (idx >> 6) & 3, bm = idx >> 8;
        const int mt = bm % MT;
        const int rbo = bm / MT;  // row block (SwiGLU: pair index)
        const int eg = SWIGLU ? (((2 * rbo) * MT + mt) * 4 + e) * 64 + ln : idx;
        float v = 0.f, vu = 0.f;
        for (int s = 0; s < p.nseg; ++s) {
            float zs = 0.f, zu = 0.f;
            for (int jj = 0; jj < J; ++jj) {
                const float* sl = slots + (size_t)(s * J + jj) * SLOT;
                zs += sl[eg];
                if constexpr (SWIGLU) zu += sl[eg + MT * 256];
            }
            v += zs;
            vu += zu;
        }
        const int m = mt * 16 + 4 * (ln >> 4) + e;
        const int64_t n = base + rbo * 16 + (ln & 15);
        if (m >= p.M || n >= p.N) continue;
        float x = SWIGLU ? silu_f32(v) * vu : v;
        if (p.bias) x += load_as_f32(p.bias, p.dtype, n);
        const int64_t o = out_index(p, m, n);
        if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
        store_from_f32(p.out, p.out_dtype, o, x);
    }
}

// Shape choice: up to two 16-row blocks per wave (more spill: a block's double-
// buffered codes, scales and biases take 24 registers), as many as still leave
// about 1500 waves on the chip, the fewest waves per workgroup that reach that,
// at least one wave per rank, LDS slots within kMaxStreamLds.
SkinnyShape q4s_shape(int M, int N, int nseg, int swiglu) {
    SkinnyShape sh;
    sh.MT = M <= 16 ? 1 : 2;
    const int64_t rows = swiglu ? 2 * (int64_t)N : N;
    auto lds_of = [&](int rb, int nw) {
        const int J = nseg >= nw ? 1 : nw / nseg;
        return (size_t)nseg * J * rb * sh.MT * 4 * 64 * sizeof(float);
    };
    sh.RB = swiglu ? 2 : 1;
    sh.NW = 8;
    for (int rb : {2, 1}) {
        if (swiglu && rb < 2) break;
        const int64_t wgs = (rows + rb * 16 - 1) / (rb * 16);
        int nw = 2;
        while (nw < 8 && (wgs * nw < 1536 || nw < nseg || lds_of(rb, nw) > kMaxStreamLds)) nw *= 2;
        while (nw > 2 && lds_of(rb, nw) > kMaxStreamLds) nw /= 2;
        if ((wgs * nw >= 1536 && lds_of(rb, nw) <= kMaxStreamLds) || rb == (swiglu ? 2 : 1)) {
            sh.RB = rb;
            sh.NW = nw;
            break;
        }
    }
    sh.lds = lds_of(sh.RB, sh.NW);
    return sh;
}

template <int MT, int RB, int NW, bool F16>
static hipError_t launch_nw(const Problem& p, hipStream_t s, size_t lds) {
    if (p.swiglu) {
        if constexpr (RB % 2 == 0) {
            const int nwg = (p.N + RB / 2 * 16 - 1) / (RB / 2 * 16);
            launch((q4s_kernel<MT, RB, NW, F16, true>), dim3(nwg), dim3(NW * 64), lds, s, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        const int nwg = (p.N + RB * 16 - 1) / (RB * 16);
        launch((q4s_kernel<MT, RB, NW, F16, false>), dim3(nwg), dim3(NW * 64), lds, s, p);
    }
    return hipGetLastError();
}

template <int MT, int RB, bool F16>
static hipError_t launch_rb(const Problem& p, hipStream_t s, const SkinnyShape& sh) {
    switch (sh.NW) {
    case 2: return launch_nw<MT, RB, 2, F16>(p, s, sh.lds);
    case 4: return launch_nw<MT, RB, 4, F16>(p, s, sh.lds);
    default: return launch_nw<MT, RB, 8, F16>(p, s, sh.lds);
    }
}

template <int MT, bool F16>
static hipError_t launch_mt(const Problem& p, hipStream_t s, const SkinnyShape& sh) {
    return sh.RB == 1 ? launch_rb<MT, 1, F16>(p, s, sh) : launch_rb<MT, 2, F16>(p, s, sh);
}

hipError_t launch_q4s(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!p.qfrag || p.M > 32 || p.Kseg % 256) return hipErrorInvalidValue;
    const SkinnyShape sh = q4s_shape(p.M, p.N, p.nseg, p.swiglu);
    if (sh.lds > kMaxStreamLds) return hipErrorInvalidValue;
    if (p.dtype == SG_F16) return sh.MT == 1 ? launch_mt<1, true>(p, s, sh) : launch_mt<2, true>(p, s, sh);
    return sh.MT == 1 ? launch_mt<1, false>(p, s, sh) : launch_mt<2, false>(p, s, sh);
}

}  // namespace sg
