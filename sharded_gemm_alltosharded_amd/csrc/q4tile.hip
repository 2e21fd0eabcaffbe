// 4-bit affine tile GEMM for many tokens (M > 32): the quantized
// all-to-sharded / sharded-to-all layers of "MLX 张量并行实战指南" sections 2.3
// and 6 (group_size 64, bits 4, affine) when the streaming kernels' token limit
// is passed.  Same factored arithmetic as q4.hip, exact in the codes: per
// quantization group g of weight row n,
//     sum_k w[n,k] x[t,k] = s[n,g] * sum_k (C + q[n,k]) x[t,k] + (b[n,g] - C s[n,g]) * sum_k x[t,k],
// the first sum and sum_k x[t,k] on the matrix cores; the scale term is one
// fp32 FMA per accumulator per group, and the bias term
// sum_g (b - C s)[n,g] xs[t,g], itself a product over the groups, runs on the
// fp32 MFMA per pair of groups into the same accumulators.
//
// Workgroup: 4 waves (2 x 2) on 64 or 128 tokens x 128 weight rows (SwiGLU:
// 64 gate rows and the 64 matching up rows, 64 outputs), one k tile per
// quantization group (64 inputs).  v_mfma_f32_32x32x16 with the tokens as the
// row operand and the weight rows as the column operand gives each lane one
// weight row per 32-row block, so each lane needs one (scale, bias) per group.
// The lane's four MFMA steps of a group use input chunks 4h + u (h = lane / 32,
// u = 0..3): its 16 bytes of the group's fragment-major codes (q4_word_offset)
// arrive straight from global memory (one coalesced 1 KB per 32-row block),
// and the matching activation chunks come from LDS (register-staged, double
// buffered, 16-byte chunks XOR-swizzled by (row ^ row >> 3) & 7).  The group
// sum of the activations is one more MFMA per step, of an all-ones operand
// against the token fragments.  Ranks of a sharded-to-all layer are the K
// segments of the loop, summed in order in registers, or (SPLIT, when the
// output gives too few tiles to fill the chip) one workgroup per rank and
// tile, the partial tiles stored in the caller's workspace and added in rank
// order by the last of a tile's workgroups to arrive.  Two workgroups per CU
// (two waves per SIMD) so that one wave's loads and barrier waits overlap the
// other's matrix work.
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
}

// eight codes (stored in q4_nibble_pos order) -> eight (C + q) 16-bit numbers;
// mask and magic in registers, so each and-or is one v_and_or_b32
__device__ __forceinline__ u32x4 unpack8(uint32_t w, uint32_t mask, uint32_t magic) {
    u32x4 r;
    r[0] = (w & mask) | magic;
    r[1] = ((w >> 4) & mask) | magic;
    r[2] = ((w >> 8) & mask) | magic;
    r[3] = ((w >> 12) & mask) | magic;
    return r;
}

// fp32 MFMA: D (32 x 32) += A (32 x 2) B (2 x 32), lane l holding A[l & 31][l >> 5]
// and B[l >> 5][l & 31]
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

}  // namespace

template <bool F16, bool SWIGLU, bool SPLIT, int NMB>
__global__ __launch_bounds__(256, 2) void q4_tile_kernel(Problem p, int tiles_m, int tiles_n) {
    constexpr int BM = 64 * NMB, BN = 128, BK = 64;  // NMB 32-token blocks per wave
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;  // logical columns per tile
    constexpr float C = F16 ? 1024.f : 128.f;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 4;  // tile rows per group of the raster (shared weight panels)
    const int grp = tile / (GM * tiles_n), first_m = grp * GM, gsz = min(GM, tiles_m - first_m);
    const int tin = tile - grp * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;
    const int G = p.Kseg / 64;  // groups per segment
    // SPLIT: this workgroup takes segment blockIdx.y only (groups [g_lo, g_lo + G))
    const int g_lo = SPLIT ? (int)blockIdx.y * G : 0;
    const int ngroups = SPLIT ? G : G * p.nseg;

    // activation loader: thread -> rows lrow + 32 i, 16-byte chunk lch; tokens
    // past M read token 0 (no branch on the loads) and are never stored
    constexpr int NLD = BM / 32;
    const int lrow = tid >> 3, lch = tid & 7;
    int64_t aoff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int m = m0 + lrow + 32 * i;
        aoff[i] = (int64_t)(m < p.M ? m : 0) * p.lda + lch * 8;
    }
    // this lane's weight row in each of the wave's two 32-row blocks
    const int h = lane >> 5;
    int64_t qoff[2], goff[2];
    bool nok[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        int64_t row;
        if constexpr (SWIGLU) {
            const int64_t j = n0 + wave_n * 32 + (lane & 31);  // nb 0: gate row, 1: up row of output j
            nok[nb] = j < p.N;
            row = weight_row(p, nok[nb] ? j : 0, nb);
        } else {
            const int64_t n = n0 + wave_n * 64 + nb * 32 + (lane & 31);
            nok[nb] = n < p.N;
            row = nok[nb] ? n : 0;
        }
        // the stored layout spans ldg groups per row (a segment may be part of it)
        qoff[nb] = q4_word_offset(row, 4 * h, p.ldg);  // group g at + 256 g (u32)
        goff[nb] = q4_group_offset(row, 0, p.ldg);     // group g at + 128 (g / 4) + g % 4 (halves)
    }

    u32x4 ra[NLD];
    auto gload = [&](int gl) {
        const int gi = g_lo + gl, s = gi / G, g = gi - s * G;
        const uint16_t* Ab = (const uint16_t*)p.A + s * p.a_seg + g * 64;
#pragma unroll
        for (int i = 0; i < NLD; ++i) ra[i] = *(const u32x4*)(Ab + aoff[i]);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int row = lrow + 32 * i;
            *(u32x4*)(&sA[buf][row * BK + ((lch ^ swz(row)) << 3)]) = ra[i];
        }
    };
    // codes, scale and bias of group gi for the lane's two rows
    u32x4 cw[2];
    uint16_t sc16[2], bi16[2];
    auto wload = [&](int gl) {
        const int gi = g_lo + gl, s = gi / G, g = gi - s * G;
        const uint32_t* Qb = p.wq + s * p.q_seg;
        const uint16_t* Sb = p.qs + s * p.g_seg;
        const uint16_t* Bb = p.qb + s * p.g_seg;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            cw[nb] = *(const u32x4*)(Qb + qoff[nb] + (int64_t)g * 256);
            const int64_t go = goff[nb] + (int64_t)(g >> 2) * 128 + (g & 3);
            sc16[nb] = Sb[go];
            bi16[nb] = Bb[go];
        }
    };

    f32x16 y[2][NMB];
    const f32x16 zero16 = {};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) y[nb][mb] = zero16;
    const u32x4 ones = F16 ? u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                           : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    uint32_t mask, magic;
    asm("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
    asm("v_mov_b32 %0, %1" : "=v"(magic) : "i"(F16 ? 0x64006400 : 0x43004300));
    const int frow = lane & 31;

    if (ngroups > 0) {
        gload(0);
        sstore(0);
        wload(0);
    }
    __syncthreads();
    // The bias term sum_g (b - C s)[n,g] xs[t,g] runs on the fp32 MFMA per pair
    // of groups (its 2 k = the pair): lane (l & 31, h) supplies xs of token
    // l & 31 and (b - C s) of its row, both of group 2 p + h.
    float xa[NMB] = {}, bq[2] = {0.f, 0.f};
    for (int gi = 0; gi < ngroups; ++gi) {
        const int buf = gi & 1;
        const u32x4 cwc[2] = {cw[0], cw[1]};
        const float sc[2] = {f16_to_f32(sc16[0]), f16_to_f32(sc16[1])};
        const float bi[2] = {f16_to_f32(bi16[0]), f16_to_f32(bi16[1])};
        if (gi + 1 < ngroups) {
            gload(gi + 1);
            wload(gi + 1);
        }
        // activation chunks 4h + u of the wave's two token blocks
        const uint16_t* a = sA[buf];
        u32x4 xf[NMB][4];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const int row = wave_m * (32 * NMB) + mb * 32 + frow;
#pragma unroll
            for (int u = 0; u < 4; ++u) xf[mb][u] = *(const u32x4*)(a + row * BK + (((4 * h + u) ^ swz(row)) << 3));
        }
        // ones (A) x tokens (B): every register of lane l holds xs of token l & 31
        const bool mine = (gi & 1) == h;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            f32x16 xs = zero16;
#pragma unroll
            for (int u = 0; u < 4; ++u) xs = mfma32<F16>(ones, xf[mb][u], xs);
            xa[mb] = mine ? xs[0] : xa[mb];
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            bq[nb] = mine ? fmaf(-C, sc[nb], bi[nb]) : bq[nb];
            u32x4 wf[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) wf[u] = unpack8(cwc[nb][u], mask, magic);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                f32x16 acc = zero16;
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = mfma32<F16>(xf[mb][u], wf[u], acc);
#pragma unroll
                for (int r = 0; r < 16; ++r) y[nb][mb][r] = fmaf(sc[nb], acc[r], y[nb][mb][r]);
            }
        }
        // the pair's bias term once both groups are in (or the last, odd group:
        // the lanes of the missing group then hold its xs = 0 contribution)
        if ((gi & 1) || gi + 1 == ngroups) {
            if (!(gi & 1)) {  // last group of an odd count: no partner group
                if (h) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) xa[mb] = 0.f;
                }
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) y[nb][mb] = mfma32_f32(xa[mb], bq[nb], y[nb][mb]);
        }
        if (gi + 1 < ngroups) sstore(buf ^ 1);
        __syncthreads();
    }

    // cross-segment reduction (split by rank): every workgroup stores its
    // partial tile; the last of a tile's nseg to arrive adds them in rank order
    if constexpr (SPLIT) {
        const int ntiles = tiles_m * tiles_n;
        const int64_t slab = (int64_t)ntiles * BM * BN;  // floats per segment
        f32x4* mine = (f32x4*)(p.ws + blockIdx.y * slab + (int64_t)tile * BM * BN);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mine[((nb * NMB + mb) * 4 + q) * 256 + tid] =
                        f32x4{y[nb][mb][4 * q], y[nb][mb][4 * q + 1], y[nb][mb][4 * q + 2], y[nb][mb][4 * q + 3]};
        __threadfence();
        __syncthreads();
        __shared__ int last;
        if (tid == 0) {
            const unsigned prev = atomicAdd(&p.counters[tile], 1u);
            last = prev == (unsigned)p.nseg - 1;
            if (last) p.counters[tile] = 0u;  // ready for the next call
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) y[nb][mb] = zero16;
        for (int sr = 0; sr < p.nseg; ++sr) {  // rank order
            const f32x4* src = (const f32x4*)(p.ws + sr * slab + (int64_t)tile * BM * BN);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = src[((nb * NMB + mb) * 4 + q) * 256 + tid];
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[nb][mb][4 * q + e] += v[e];
                    }
        }
    }

    // epilogue: lane l of a 32 x 32 block holds weight row l & 31 (column) and
    // tokens 8 j + 4 (l >> 5) + e (rows)
    static_for<0, NMB>([&](auto mc) {
        constexpr int mb = decltype(mc)::value;
        static_for<0, 16>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const int m = m0 + wave_m * (32 * NMB) + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m >= p.M) return;
            if constexpr (SWIGLU) {
                const int64_t n = n0 + wave_n * 32 + (lane & 31);
                if (!nok[0]) return;
                const float v = silu_f32(y[0][mb][r]) * y[1][mb][r];
                store_from_f32(p.out, p.out_dtype, out_index(p, m, n), v);
            } else {
                static_for<0, 2>([&](auto nc) {
                    constexpr int nb = decltype(nc)::value;
                    const int64_t n = n0 + wave_n * 64 + nb * 32 + (lane & 31);
                    if (!nok[nb]) return;
                    float v = y[nb][mb][r];
                    if (p.bias) v += load_as_f32(p.bias, p.dtype, n);
                    const int64_t o = out_index(p, m, n);
                    if (p.accumulate && p.out_dtype == SG_F32) v += ((const float*)p.out)[o];
                    store_from_f32(p.out, p.out_dtype, o, v);
                });
            }
        });
    });
}

// fragment-major codes (rows % 32 == 0, groups per segment % 4 == 0), 16-byte
// activation rows
bool q4_tile_fits(const Problem& p) {
    return p.qfrag && !p.xfrag && p.Kseg % 256 == 0 && p.lda % 8 == 0 && p.a_seg % 8 == 0 &&
           (p.out_map == OUT_ROWMAJOR || p.out_map == OUT_SHARDED) && !(p.split && p.swiglu);
}

// Token tile, 64 (one 32-token block per wave: half the accumulators, three
// workgroups per CU) or 128, measured on the decode MLP shapes from 40 to 1024
// tokens: the gate|up layer is faster on 64-token tiles up to 192 tokens
// (128 tokens: 85 against 97 us); the down layer (4096 outputs) on 128-token
// tiles split by rank from 65 to 256 tokens (256 tokens: 158 against 208 us)
// and on 64-token tiles beyond, where they fill the chip without the split
// (512 tokens: 184 against 269 us).
static int q4_tile_bm(int M, bool swiglu) {
    if (swiglu) return M <= 192 ? 64 : 128;
    return (M > 64 && M <= 256) ? 128 : 64;
}

int q4_tile_count(int M, int N) {
    const int bm = q4_tile_bm(M, false);
    return ((M + bm - 1) / bm) * ((N + 127) / 128);
}
int q4_tile_rows(int M) { return q4_tile_bm(M, false); }

template <bool F16, bool SWIGLU, bool SPLIT>
static void launch_nmb(const Problem& p, hipStream_t s, dim3 grid, int tm, int tn) {
    if (q4_tile_bm(p.M, SWIGLU) == 64) launch(q4_tile_kernel<F16, SWIGLU, SPLIT, 1>, grid, dim3(256), 0, s, p, tm, tn);
    else launch(q4_tile_kernel<F16, SWIGLU, SPLIT, 2>, grid, dim3(256), 0, s, p, tm, tn);
}

hipError_t launch_q4_tile(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!q4_tile_fits(p)) return hipErrorInvalidValue;
    const int nout = p.swiglu ? 64 : 128, bm = q4_tile_bm(p.M, p.swiglu);
    const int tm = (p.M + bm - 1) / bm, tn = (p.N + nout - 1) / nout;
    const dim3 grid(tm * tn, p.split ? p.nseg : 1);
    const bool f16 = p.dtype == SG_F16;
    if (p.swiglu) {
        if (f16) launch_nmb<true, true, false>(p, s, grid, tm, tn);
        else launch_nmb<false, true, false>(p, s, grid, tm, tn);
    } else if (p.split) {
        if (f16) launch_nmb<true, false, true>(p, s, grid, tm, tn);
        else launch_nmb<false, false, true>(p, s, grid, tm, tn);
    } else {
        if (f16) launch_nmb<true, false, false>(p, s, grid, tm, tn);
        else launch_nmb<false, false, false>(p, s, grid, tm, tn);
    }
    return hipGetLastError();
}

}  // namespace sg
