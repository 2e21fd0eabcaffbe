// Weight-streaming GEMM for few tokens (M <= 32): decode-shaped sharded
// layers and the vocabulary-parallel head.  HBM-bound: every weight byte is
// read once, so the kernel is organised around keeping enough 16-byte loads
// in flight, not around reuse.
//
// One workgroup (NW waves) owns a group of RB x 16 weight rows across every
// rank of the layer; each wave streams all RB row blocks for its part of k,
// so one activation fragment feeds RB MFMAs.  Dense 16-bit layers store their
// weights fragment-major (frag_offset): the 16 x 32 operand fragment of a row
// block and k step is one contiguous 1 KB, and each step is one fully
// coalesced wave-wide read per row block.  The work of that row group is cut into units (rank s,
// part j): J = max(1, NW / nseg) waves share one rank's k range, taking its
// 32-wide k steps round robin (step j, j + J, ...), so the waves of one rank
// read adjacent 64-byte pieces of the same rows at the same time.  Each step
// is one v_mfma_f32_16x16x32 per (row block, token block): 16 weight rows x
// 32 k (16 bytes per lane straight from HBM) as the row operand, the tokens
// as the column operand.  Loads of step t+1 are issued before the MFMAs of
// step t (register double buffering).  Weights are read once, so their loads
// are non-temporal (measured ~10% more HBM throughput than cached loads; the
// activations, reused by every workgroup, stay cached).
//
// Every unit's partial goes to its own LDS slot; the epilogue adds the parts
// of a rank in part order and the ranks in rank order, then the bias once --
// the all_sum of "MLX 张量并行实战指南" section 2.2, fused into the kernel,
// deterministic, with no cross-workgroup traffic.  All-to-sharded layers are
// the one-rank case; the SwiGLU variant pairs a 16-row gate block with the
// matching up block and stores silu(g) * u (sections 5.2-5.3).
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// MX FP8 weights (FP8): a step covers two 32-wide k steps; the lane's 16 code
// bytes of the pair are one load (mx_code_offset), its row's two E8M0 scales
// two bytes of one word; mx8_to_bf16 (internal.h) turns each 8 codes into the
// bf16 operand.

template <int MT, int RB, int NW, bool F16, bool SWIGLU, int U, bool FP8 = false>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(Problem p) {
    static_assert(!(FP8 && F16), "MX FP8 layers take bf16 activations");
    constexpr int ROWS = SWIGLU ? RB / 2 * 16 : RB * 16;  // logical columns per workgroup
    constexpr int SLOT = RB * MT * 4 * 64;                 // floats per unit slot
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    extern __shared__ float slots[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t base = (int64_t)blockIdx.x * ROWS;
    const int kq = (lane >> 4) * 8;
    const int J = p.nseg >= NW ? 1 : NW / p.nseg;  // waves per rank
    const int units = p.nseg * J;

    int64_t woff[RB], soff[RB];  // soff: FP8 scales (pair step st: the word at + (st >> 1) 64)
    bool wok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row;
        if constexpr (SWIGLU) {
            const int64_t j = base + (rb >> 1) * 16 + (lane & 15);
            wok[rb] = j < p.N;
            row = weight_row(p, wok[rb] ? j : 0, rb & 1);
        } else {
            const int64_t n = base + rb * 16 + (lane & 15);
            wok[rb] = n < p.N;
            row = wok[rb] ? n : 0;
        }
        // row-major: lane's 16 bytes of a step at row * ldw + k; fragment-major:
        // the block's 1 KB fragment, lane l at l * 8 (one coalesced read per step)
        woff[rb] = p.wfrag ? frag_offset(row, kq, p.wsteps) : row * p.ldw + kq;
        if constexpr (FP8) {
            woff[rb] = mx_code_offset(row, kq, p.wsteps);
            soff[rb] = mx_scale_offset(row, 0, p.wsteps);
        }
    }
    // elements (FP8: bytes) per step; an FP8 step is a pair of 32-wide k steps
    const int wstep = FP8 ? 1024 : (p.wfrag ? 512 : 32);
    constexpr int KS = FP8 ? 64 : 32;  // k per step
    constexpr int XF = FP8 ? 2 : 1;    // activation fragments per step
    // activations: row-major (lane's 16 bytes at m * lda + k), or fragment-major
    // (act_frag_offset: the 16 tokens x 32 inputs of a step are one 1 KB, lane l
    // at 8 l), elements per 32-wide k step xstep
    int64_t xoff[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        xok[mt] = m < p.M;
        xoff[mt] = p.xfrag ? act_frag_offset(mt * 16 + (lane & 15), kq, p.Kseg / 32)
                           : (int64_t)(xok[mt] ? m : 0) * p.lda + kq;
    }
    const int64_t xstep = p.xfrag ? 512 : 32;

    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int nsteps = (p.Kseg + KS - 1) / KS;

    for (int u = wave; u < units; u += NW) {
        const int s = u / J, j = u - s * J;
        const uint16_t* Wb = (const uint16_t*)p.W + s * p.w_seg;
        const uint8_t* Wb8 = (const uint8_t*)p.W + s * p.w_seg;
        const uint8_t* Sb8 = p.ms + s * p.ms_seg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg;
        f32x4 acc[RB][MT];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[rb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // this unit's steps: j, j + J, ...; U of them per batch, next batch prefetched
        const int my_steps = nsteps > j ? (nsteps - j + J - 1) / J : 0;
        const int batches = (my_steps + U - 1) / U;
        u32x4 wv[2][U][RB], xv[2][U][MT][XF];
        uint32_t wsc[2][U][RB];   // FP8: the step pair's two scale bytes
        auto load = [&](int buf, int b) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int idx = b * U + q;
                const int st = j + idx * J, k0 = st * KS;
                const bool ok = idx < my_steps && k0 + kq < p.Kseg;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if constexpr (FP8) {
                        wv[buf][q][rb] = (ok && wok[rb])
                                             ? __builtin_nontemporal_load((const u32x4*)(Wb8 + woff[rb] + (int64_t)st * wstep))
                                             : zero;
                        const uint32_t sw = (ok && wok[rb]) ? *(const uint32_t*)(Sb8 + soff[rb] + (int64_t)(st >> 1) * 64)
                                                            : 0x7F7F7F7Fu;
                        wsc[buf][q][rb] = (sw >> (16 * (st & 1))) & 0xFFFFu;
                    } else {
                        wv[buf][q][rb] = (ok && wok[rb])
                                             ? __builtin_nontemporal_load((const u32x4*)(Wb + woff[rb] + (int64_t)st * wstep))
                                             : zero;
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int f = 0; f < XF; ++f)
                        xv[buf][q][mt][f] = (ok && xok[mt]) ? *(const u32x4*)(Ab + xoff[mt] + (int64_t)(k0 / 32 + f) * xstep) : zero;
            }
        };
        auto compute = [&](int buf) {
#pragma unroll
            for (int q = 0; q < U; ++q)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if constexpr (FP8) {
                        const u32x4 c = wv[buf][q][rb];
                        const u32x4 w0 = mx8_to_bf16(u32x2{c[0], c[1]}, wsc[buf][q][rb] & 0xFFu);
                        const u32x4 w1 = mx8_to_bf16(u32x2{c[2], c[3]}, wsc[buf][q][rb] >> 8);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            acc[rb][mt] = mfma16<F16>(w0, xv[buf][q][mt][0], acc[rb][mt]);
                            acc[rb][mt] = mfma16<F16>(w1, xv[buf][q][mt][XF - 1], acc[rb][mt]);
                        }
                    } else {
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[rb][mt] = mfma16<F16>(wv[buf][q][rb], xv[buf][q][mt][0], acc[rb][mt]);
                    }
                }
        };
        if (batches > 0) load(0, 0);
        int b = 0;
        for (; b + 1 < batches; b += 2) {
            load(1, b + 1);
            compute(0);
            if (b + 2 < batches) load(0, b + 2);
            compute(1);
        }
        if (b < batches) compute(0);

        float* slot = slots + (size_t)u * SLOT;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) slot[((rb * MT + mt) * 4 + e) * 64 + lane] = acc[rb][mt][e];
    }
    __syncthreads();

    // ---- reduction (parts of a rank in order, then ranks in order) + epilogue
    // element index: ((rb * MT + mt) * 4 + e) * 64 + ln
    constexpr int NE = SWIGLU ? SLOT / 2 : SLOT;  // outputs of this workgroup
    for (int idx = tid; idx < NE; idx += NW * 64) {
        const int ln = idx & 63, e = (idx >> 6) & 3, bm = idx >> 8;  // bm = rb * MT + mt (gate half for SwiGLU)
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
        const int m = mt * 16 + (ln & 15);
        const int rowin = 4 * (ln >> 4) + e;
        const int64_t n = base + rbo * 16 + rowin;
        if (m >= p.M || n >= p.N) continue;
        float x = SWIGLU ? silu_f32(v) * vu : v;
        if (p.bias) x += load_as_f32(p.bias, p.dtype, n);
        const int64_t o = out_index(p, m, n);
        if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
        store_from_f32(p.out, p.out_dtype, o, x);
    }
}

// Shape choice (from a sweep of RB, NW and U on the decode gate|up, down and
// vocabulary-head shapes): as many row blocks per wave as still leave about
// 1500 waves on the chip (each activation fragment then serves RB weight
// fragments) and workgroups for at least three quarters of the 256 CUs, the
// fewest waves per workgroup that reach that, at least one wave per rank, and
// LDS slots within kMaxStreamLds.  (Without the workgroup floor, one rank's
// share of the vocabulary head -- 6284 rows -- ran 99 workgroups of 8 waves:
// 95.6 us, against 66.8 us on 197 of 4.)
SkinnyShape skinny_shape(int M, int N, int nseg, int swiglu) {
    SkinnyShape sh;
    sh.MT = M <= 16 ? 1 : 2;
    const int64_t rows = swiglu ? 2 * (int64_t)N : N;
    // two token tiles hold twice the accumulators: fewer, longer streams per
    // workgroup measured faster (vocabulary head: two waves per workgroup
    // instead of four, 236 -> 224 us)
    const int64_t target = sh.MT == 2 ? 768 : 1536;
    auto lds_of = [&](int rb, int nw) {
        const int J = nseg >= nw ? 1 : nw / nseg;
        return (size_t)nseg * J * rb * sh.MT * 4 * 64 * sizeof(float);
    };
    sh.RB = swiglu ? 2 : 1;
    sh.NW = 8;
    for (int rb : {8, 4, 2, 1}) {
        if (swiglu && rb < 2) break;
        const int64_t wgs = (rows + rb * 16 - 1) / (rb * 16);
        int nw = 2;
        while (nw < 8 && (wgs * nw < target || nw < nseg || lds_of(rb, nw) > kMaxStreamLds)) nw *= 2;
        while (nw > 2 && lds_of(rb, nw) > kMaxStreamLds) nw /= 2;
        if ((wgs * nw >= target && wgs >= 192 && lds_of(rb, nw) <= kMaxStreamLds) || rb == (swiglu ? 2 : 1)) {
            sh.RB = rb;
            sh.NW = nw;
            break;
        }
    }
    sh.lds = lds_of(sh.RB, sh.NW);
    return sh;
}

template <int MT, int RB, int NW, bool F16, bool FP8 = false>
static hipError_t launch_nw(const Problem& p, hipStream_t s, size_t lds) {
    constexpr int U = (FP8 || (MT == 2 && RB >= 8)) ? 1 : 2;  // an FP8 step already spans 64 k
    if (p.swiglu) {
        if constexpr (RB % 2 == 0) {
            const int nwg = (p.N + RB / 2 * 16 - 1) / (RB / 2 * 16);
            launch((skinny_kernel<MT, RB, NW, F16, true, U, FP8>), dim3(nwg), dim3(NW * 64), lds, s, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        const int nwg = (p.N + RB * 16 - 1) / (RB * 16);
        launch((skinny_kernel<MT, RB, NW, F16, false, U, FP8>), dim3(nwg), dim3(NW * 64), lds, s, p);
    }
    return hipGetLastError();
}

template <int MT, int RB, bool F16, bool FP8>
static hipError_t launch_rb(const Problem& p, hipStream_t s, const SkinnyShape& sh) {
    switch (sh.NW) {
    case 2: return launch_nw<MT, RB, 2, F16, FP8>(p, s, sh.lds);
    case 4: return launch_nw<MT, RB, 4, F16, FP8>(p, s, sh.lds);
    default: return launch_nw<MT, RB, 8, F16, FP8>(p, s, sh.lds);
    }
}

template <int MT, bool F16, bool FP8 = false>
static hipError_t launch_mt(const Problem& p, hipStream_t s, const SkinnyShape& sh) {
    switch (sh.RB) {
    case 1: return launch_rb<MT, 1, F16, FP8>(p, s, sh);
    case 2: return launch_rb<MT, 2, F16, FP8>(p, s, sh);
    case 4: return launch_rb<MT, 4, F16, FP8>(p, s, sh);
    default: return launch_rb<MT, 8, F16, FP8>(p, s, sh);
    }
}

hipError_t launch_skinny(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const SkinnyShape sh = skinny_shape(p.M, p.N, p.nseg, p.swiglu);
    if (p.fp8) {
        // fragment-major codes and scales, bf16 activations, 4-step scale runs
        if (!p.wfrag || p.dtype != SG_BF16 || p.wsteps % 4) return hipErrorInvalidValue;
        SkinnyShape f = sh;
        if (f.MT == 2 && f.RB == 8 && f.NW == 8) {  // two token tiles would spill at 8 waves
            f.NW = 4;
            const int J = p.nseg >= 4 ? 1 : 4 / p.nseg;
            f.lds = (size_t)p.nseg * J * f.RB * f.MT * 4 * 64 * sizeof(float);
        }
        return f.MT == 1 ? launch_mt<1, false, true>(p, s, f) : launch_mt<2, false, true>(p, s, f);
    }
    if (p.dtype == SG_F16) return sh.MT == 1 ? launch_mt<1, true>(p, s, sh) : launch_mt<2, true>(p, s, sh);
    return sh.MT == 1 ? launch_mt<1, false>(p, s, sh) : launch_mt<2, false>(p, s, sh);
}

}  // namespace sg
