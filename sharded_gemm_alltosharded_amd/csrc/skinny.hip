// Weight-streaming GEMM for few tokens (M <= 32): decode-shaped sharded
// layers and the vocabulary-parallel head.  HBM-bound: every weight byte is
// read once, so the kernel is organised around keeping enough 16-byte loads
// in flight, not around reuse.
//
// Workgroup = 4 waves on one group of weight rows (RB blocks of 16 rows);
// the waves interleave over 32-wide k steps (wave w takes steps w, w+4, ...)
// so that at any moment the four waves read adjacent 64-byte pieces of the
// same rows.  Each step is one v_mfma_f32_16x16x32 per (row block, token
// block): the weight block is the MFMA's row operand (16 rows x 32 k, 16
// bytes per lane straight from HBM) and the tokens are its column operand.
// The four wave partials are added in LDS in wave order.
//
// Sharded-to-all layers: the workgroups of one row group split by rank
// (grid.y = P); each forms its rank's partial, writes it to the workspace,
// and the last workgroup to arrive adds the P partials in rank order, then
// the bias once -- the all_sum of "MLX 张量并行实战指南" section 2.2 as a
// fused, deterministic epilogue.  All-to-sharded layers need no reduction;
// the SwiGLU variant pairs a 16-row gate block with the matching up block so
// the epilogue can store silu(g) * u directly (sections 5.2-5.3).
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int MT, int RB, bool F16, bool SWIGLU, bool SPLIT, int U>
__global__ __launch_bounds__(256) void skinny_kernel(Problem p) {
    constexpr int ROWS = SWIGLU ? RB / 2 * 16 : RB * 16;  // logical columns per workgroup
    constexpr int NV = RB * MT;                            // values per thread after reduction
    static_assert(!SWIGLU || RB % 2 == 0, "gate/up blocks come in pairs");
    __shared__ float red[4][NV * 4][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = blockIdx.x;
    const int seg_lo = SPLIT ? blockIdx.y : 0;
    const int seg_cnt = SPLIT ? 1 : p.nseg;
    const int64_t base = (int64_t)rg * ROWS;
    const int kq = (lane >> 4) * 8;

    int64_t woff[RB];
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
        woff[rb] = row * p.ldw + kq;
    }
    int64_t xoff[MT];
    bool xok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        xok[mt] = m < p.M;
        xoff[mt] = (int64_t)(xok[mt] ? m : 0) * p.lda + kq;
    }

    f32x4 acc[RB][MT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int nsteps = (p.Kseg + 31) / 32;
    for (int s = seg_lo; s < seg_lo + seg_cnt; ++s) {
        const uint16_t* Wb = (const uint16_t*)p.W + s * p.w_seg;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg;
        for (int st = wave; st < nsteps; st += 4 * U) {
            u32x4 wv[U][RB], xv[U][MT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k0 = (st + 4 * u) * 32;
                const bool ok = (st + 4 * u < nsteps) && (k0 + kq < p.Kseg);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    wv[u][rb] = (ok && wok[rb]) ? *(const u32x4*)(Wb + woff[rb] + k0) : zero;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    xv[u][mt] = (ok && xok[mt]) ? *(const u32x4*)(Ab + xoff[mt] + k0) : zero;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[rb][mt] = mfma16<F16>(wv[u][rb], xv[u][mt], acc[rb][mt]);
        }
    }

    // ---- wave partials -> workgroup result (wave order)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][(rb * MT + mt) * 4 + e][lane] = acc[rb][mt][e];
    __syncthreads();
    // thread tid now owns value i = rb * MT + mt of MFMA register e = tid / 64 at lane tid % 64
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int reg = 4 * i + (tid >> 6), ln = tid & 63;
        v[i] = ((red[0][reg][ln] + red[1][reg][ln]) + red[2][reg][ln]) + red[3][reg][ln];
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
    const int ln = tid & 63, e = tid >> 6;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int rb = i / MT, mt = i % MT;
        if constexpr (SWIGLU) {
            if (rb & 1) continue;
        }
        const int m = mt * 16 + (ln & 15);
        const int rowin = 4 * (ln >> 4) + e;
        const int64_t n = SWIGLU ? base + (rb >> 1) * 16 + rowin : base + rb * 16 + rowin;
        if (m >= p.M || n >= p.N) continue;
        float x = SWIGLU ? silu_f32(v[i]) * v[i + MT] : v[i];
        if (p.bias) x += load_as_f32(p.bias, p.dtype, n);
        const int64_t o = out_index(p, m, n);
        if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
        store_from_f32(p.out, p.out_dtype, o, x);
    }
}

SplitLayout skinny_split_layout(int M, int N, int nseg) {
    const size_t MT = M <= 16 ? 1 : 2, RB = 2;
    const size_t nrg = (N + RB * 16 - 1) / (RB * 16);
    return {nseg * nrg * RB * MT * 256, nrg};
}

template <int MT, int RB, bool F16>
static hipError_t launch_mt(const Problem& p, hipStream_t s) {
    constexpr int U = 4;
    if (p.swiglu) {
        const int nrg = (p.N + RB / 2 * 16 - 1) / (RB / 2 * 16);
        hipLaunchKernelGGL((skinny_kernel<MT, RB, F16, true, false, U>), dim3(nrg), dim3(256), 0, s, p);
    } else {
        const int nrg = (p.N + RB * 16 - 1) / (RB * 16);
        if (p.split)
            hipLaunchKernelGGL((skinny_kernel<MT, RB, F16, false, true, U>), dim3(nrg, p.nseg), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((skinny_kernel<MT, RB, F16, false, false, U>), dim3(nrg), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_skinny(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    const bool f16 = p.dtype == SG_F16;
    if (p.M <= 16) return f16 ? launch_mt<1, 2, true>(p, s) : launch_mt<1, 2, false>(p, s);
    return f16 ? launch_mt<2, 2, true>(p, s) : launch_mt<2, 2, false>(p, s);
}

}  // namespace sg
