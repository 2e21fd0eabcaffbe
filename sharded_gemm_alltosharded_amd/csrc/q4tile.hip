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
// order by a second kernel (q4_split_reduce_kernel).  Two workgroups per CU
// (two waves per SIMD) so that one wave's loads and barrier waits overlap the
// other's matrix work.  q4_tile_dma_kernel below is the same tile with every
// operand staged by direct-to-LDS loads several groups ahead; it runs whenever
// its 32-bit buffer offsets reach every operand.
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// direct-to-LDS loads (each lane's bytes land at the wave's LDS base + size x
// lane) through buffer resources, and LDS reads issued as inline assembly so
// that the compiler's wait insertion does not hold them behind the loads still
// in flight (the caller waits for them with wait_lgkm, which ties the registers)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ u32x4 lds16(const void* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
__device__ __forceinline__ u32x2 lds8(const void* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
// s_waitcnt vmcnt(N) (N <= 63), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

}  // namespace

// The stores of a finished tile, or (split by rank) of its partial tile.
template <bool SWIGLU, bool SPLIT, int NMB>
__device__ __forceinline__ void q4_tile_finish(const Problem& p, f32x16 (&y)[2][NMB], int tiles_m, int tiles_n,
                                               int tile, int m0, int64_t n0, int wave_m, int wave_n,
                                               const bool (&nok)[2]) {
    constexpr int BM = 64 * NMB, BN = 128;
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
    if constexpr (SPLIT) {
        // this segment's partial tile: thread tid's float4 v = (nb NMB + mb) 4 + q
        // (y[nb][mb][4q .. 4q + 3]) at float4 index v * 256 + tid of the tile's
        // slab; q4_split_reduce_kernel adds the segments in rank order
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * tiles_m * tiles_n + tile) * (BM * BN));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mine[((nb * NMB + mb) * 4 + q) * 256 + tid] =
                        f32x4{y[nb][mb][4 * q], y[nb][mb][4 * q + 1], y[nb][mb][4 * q + 2], y[nb][mb][4 * q + 3]};
        return;
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

    q4_tile_finish<SWIGLU, SPLIT, NMB>(p, y, tiles_m, tiles_n, tile, m0, n0, wave_m, wave_n, nok);
}

// The same tile with its operands staged by direct-to-LDS loads in a ring of
// NS group stages (activations BM x 64, the four 32-row blocks' 1 KB code
// fragments), issued NS - 1 groups ahead, and each run's scales and biases
// (2 x 4 blocks x 256 bytes) in two run buffers: the register-staged kernel
// above prefetches one group ahead and waits on its code loads at every group.
// Every wave issues the same loads in the same order (dummy loads of the last
// group or run past the end), so the waits are compile-time counts.
template <bool F16, bool SWIGLU, bool SPLIT, int NMB>
__global__ __launch_bounds__(256, 2) void q4_tile_dma_kernel(Problem p, int tiles_m, int tiles_n) {
    constexpr int BM = 64 * NMB, BN = 128;
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    constexpr float C = F16 ? 1024.f : 128.f;
    constexpr int NS = NMB == 1 ? 4 : 3;       // group stages
    constexpr int SA = BM * 128, ST = SA + 4096;  // activation / stage bytes
    constexpr int NA = BM / 32;                // activation loads per wave per group
    constexpr int L = NA + 1;                  // loads per wave per group (+ codes)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * ST + 2 * 2048];
    uint8_t* const sscale = smem + NS * ST;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave >> 1, wave_n = wave & 1, h = lane >> 5;
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 4;
    const int grp = tile / (GM * tiles_n), first_m = grp * GM, gsz = min(GM, tiles_m - first_m);
    const int tin = tile - grp * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;
    const int G = p.Kseg / 64;
    const int g_lo = SPLIT ? (int)blockIdx.y * G : 0;
    const int ngroups = SPLIT ? G : G * p.nseg;  // a multiple of 4
    const int nruns = ngroups / 4;

    // rows of the wave's blocks (for the stores) and the block whose fragments
    // and scales this wave loads: slot w = (w >> 1) wave_n, (w & 1) nb
    bool nok[2];
    int64_t bw;
    {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t j = SWIGLU ? n0 + wave_n * 32 + (lane & 31) : n0 + wave_n * 64 + nb * 32 + (lane & 31);
            nok[nb] = j < p.N;
        }
        const int sn = wave >> 1, snb = wave & 1;
        const int64_t j0 = SWIGLU ? n0 + sn * 32 : n0 + sn * 64 + snb * 32;
        const int64_t jc = j0 < p.N ? j0 : 0;
        bw = (SWIGLU ? weight_row(p, jc, snb) : jc) >> 5;
    }
    const int64_t rows = SWIGLU ? 2 * (int64_t)p.N : p.N;
    const int64_t nblk = (rows + 31) / 32;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.A, 0, (int)((((int64_t)p.nseg - 1) * p.a_seg + (int64_t)(p.M - 1) * p.lda + p.Kseg) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.wq, 0, (int)((((int64_t)p.nseg - 1) * p.q_seg + nblk * p.ldg * 256) * 4), 0x00020000);
    const int sext = (int)((((int64_t)p.nseg - 1) * p.g_seg + nblk * (p.ldg / 4) * 128) * 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)p.qs, 0, sext, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)p.qb, 0, sext, 0x00020000);

    // per-lane byte offsets: activation load j covers tile rows (w + 4 j) 8 ..
    // + 8, lane -> row lane >> 3, 16-byte chunk lane & 7 (stored at chunk
    // (lane & 7) ^ swz8(row) of the row); the code fragment 1 KB, lane at 16
    // lane; the scale run 256 bytes, lane at 4 lane
    uint32_t aoffd[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int row = (wave + 4 * j) * 8 + (lane >> 3);
        const int m = min(m0 + row, p.M - 1);
        aoffd[j] = (uint32_t)(((int64_t)m * p.lda + (((lane & 7) ^ swz8(row)) << 3)) * 2);
    }
    const uint32_t coff = (uint32_t)(bw * p.ldg * 256 * 4 + lane * 16);
    const uint32_t soffl = (uint32_t)(bw * (p.ldg / 4) * 128 * 2 + lane * 4);

    // group gl's loads into stage gu % NS (gu = the unclamped slot index)
    auto issue_group = [&](int gu) {
        const int gl = min(gu, ngroups - 1), gi = g_lo + gl, s = gi / G, g = gi - s * G;
        uint8_t* st = smem + (gu % NS) * ST;
        const uint32_t as = (uint32_t)((s * p.a_seg + (int64_t)g * 64) * 2);
#pragma unroll
        for (int j = 0; j < NA; ++j) dma16(ra, aoffd[j], as, st + (wave + 4 * j) * 1024);
        dma16(rq, coff, (uint32_t)((s * p.q_seg + (int64_t)g * 256) * 4), st + SA + wave * 1024);
    };
    auto issue_scales = [&](int ru) {
        const int r = min(ru, nruns - 1), gi = g_lo + 4 * r, s = gi / G, g = gi - s * G;
        uint8_t* b = sscale + (ru & 1) * 2048;
        const uint32_t so = (uint32_t)((s * p.g_seg + (int64_t)(g >> 2) * 128) * 2);
        dma4(rs, soffl, so, b + wave * 256);
        dma4(rb, soffl, so, b + 1024 + wave * 256);
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

    // prologue: groups 0 .. NS - 2 (each run's scales just before its first group)
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
        if (u % 4 == 0) issue_scales(u / 4);
        issue_group(u);
    }
    float xa[NMB] = {}, bq[2] = {0.f, 0.f};
    u32x2 sv[2], bv[2];
    for (int base = 0; base < ngroups; base += 4) {
        static_for<0, 4>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int gl = base + q;
            // this wave's loads of group gl (and of its run's scales) have landed
            // once at most the later groups' batches are outstanding
            constexpr int extra = (NS == 4) ? ((q == 2 || q == 3) ? 2 : 0) : (q == 3 ? 2 : 0);
            wait_vm<(NS - 2) * L + extra>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // stage (gl - 1) % NS and the other run buffer are free: everyone
            // finished reading them before this barrier
            if ((gl + NS - 1) % 4 == 0) issue_scales((gl + NS - 1) / 4);
            issue_group(gl + NS - 1);
            const uint8_t* st = smem + (gl % NS) * ST;
            u32x4 xf[NMB][4], cw[2];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const int row = wave_m * (32 * NMB) + mb * 32 + frow;
#pragma unroll
                for (int u = 0; u < 4; ++u) xf[mb][u] = lds16(st + row * 128 + (((4 * h + u) ^ swz8(row)) << 4));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) cw[nb] = lds16(st + SA + (wave_n * 2 + nb) * 1024 + lane * 16);
            if constexpr (q == 0) {
                const uint8_t* b = sscale + ((gl >> 2) & 1) * 2048;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    sv[nb] = lds8(b + (wave_n * 2 + nb) * 256 + frow * 8);
                    bv[nb] = lds8(b + 1024 + (wave_n * 2 + nb) * 256 + frow * 8);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sv[0]), "+v"(sv[1]), "+v"(bv[0]), "+v"(bv[1]));
            }
            if constexpr (NMB == 1)
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(xf[0][0]), "+v"(xf[0][1]), "+v"(xf[0][2]), "+v"(xf[0][3]), "+v"(cw[0]), "+v"(cw[1]));
            else
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(xf[0][0]), "+v"(xf[0][1]), "+v"(xf[0][2]), "+v"(xf[0][3]),
                               "+v"(xf[NMB - 1][0]), "+v"(xf[NMB - 1][1]), "+v"(xf[NMB - 1][2]), "+v"(xf[NMB - 1][3]),
                               "+v"(cw[0]), "+v"(cw[1]));
            float sc[2], bi[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const uint32_t sw = sv[nb][q >> 1], bw2 = bv[nb][q >> 1];
                sc[nb] = f16_to_f32((uint16_t)((q & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                bi[nb] = f16_to_f32((uint16_t)((q & 1) ? (bw2 >> 16) : (bw2 & 0xFFFFu)));
            }
            // ones (A) x tokens (B): every register of lane l holds xs of token l & 31
            const bool mine = (q & 1) == h;
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
                for (int u = 0; u < 4; ++u) wf[u] = unpack8(cw[nb][u], mask, magic);
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    f32x16 acc = zero16;
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc = mfma32<F16>(xf[mb][u], wf[u], acc);
#pragma unroll
                    for (int r = 0; r < 16; ++r) y[nb][mb][r] = fmaf(sc[nb], acc[r], y[nb][mb][r]);
                }
            }
            if constexpr (q & 1) {  // the pair's bias term
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) y[nb][mb] = mfma32_f32(xa[mb], bq[nb], y[nb][mb]);
            }
        });
    }
    // no load may still be writing this workgroup's LDS when it ends
    wait_vm<0>();
    q4_tile_finish<SWIGLU, SPLIT, NMB>(p, y, tiles_m, tiles_n, tile, m0, n0, wave_m, wave_n, nok);
}

// Sum of a split product's partial tiles (no SwiGLU): workgroup (tile, y)
// takes float4 indices RV y .. RV y + RV - 1 of every thread of the tile
// kernels' partial layout, adds the segments' partials in rank order and
// stores them with the bias.  A second kernel rather than the last workgroup
// of a tile to arrive: the kernel boundary orders the partial stores before
// the loads (an in-kernel handoff needs a device-scope release per
// workgroup), and the sums are spread over every compute unit.
template <int NMB, int RV>
__global__ __launch_bounds__(256) void q4_split_reduce_kernel(Problem p, int tiles_m, int tiles_n) {
    constexpr int BM = 64 * NMB, BN = 128;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
    const int wave_m = wave >> 1, wave_n = wave & 1;
    const int tile = blockIdx.x;
    constexpr int GM = 4;  // the tile -> (m0, n0) map of the tile kernels
    const int grp = tile / (GM * tiles_n), first_m = grp * GM, gsz = min(GM, tiles_m - first_m);
    const int tin = tile - grp * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * BN;
    const int v0 = blockIdx.y * RV;
    f32x4 sum[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) sum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < p.nseg; ++g) {  // rank order
        const f32x4* src = (const f32x4*)(p.ws + ((int64_t)g * tiles_m * tiles_n + tile) * (BM * BN));
        f32x4 v[RV];
#pragma unroll
        for (int r = 0; r < RV; ++r) v[r] = src[(v0 + r) * 256 + tid];
#pragma unroll
        for (int r = 0; r < RV; ++r) sum[r] += v[r];
    }
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        const int v = v0 + r, nb = v / (NMB * 4), mb = (v / 4) % NMB, q = v % 4;
        const int64_t n = n0 + wave_n * 64 + nb * 32 + (lane & 31);
        if (n >= p.N) continue;
        const float bias = p.bias ? load_as_f32(p.bias, p.dtype, n) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + wave_m * (32 * NMB) + mb * 32 + 8 * q + 4 * h + e;
            if (m >= p.M) continue;
            float x = sum[r][e];
            if (p.bias) x += bias;
            const int64_t o = out_index(p, m, n);
            if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[o];
            store_from_f32(p.out, p.out_dtype, o, x);
        }
    }
}

// fragment-major codes (rows % 32 == 0, groups per segment % 4 == 0), 16-byte
// activation rows
bool q4_tile_fits(const Problem& p) {
    return p.qfrag && !p.xfrag && p.Kseg % 256 == 0 && p.lda % 8 == 0 && p.a_seg % 8 == 0 &&
           (p.out_map == OUT_ROWMAJOR || p.out_map == OUT_SHARDED) && !(p.split && p.swiglu);
}

// Token tile, 64 (one 32-token block per wave: half the accumulators, three
// workgroups per CU) or 128, measured with the direct-to-LDS kernel on the
// decode MLP shapes from 40 to 512 tokens: 64-token tiles win or tie
// everywhere (gate|up at 64 tokens 43 against 80 us, at 512 tokens 191
// against 203 us; the down layer at 512 tokens 130 against 220 us); 128-token
// tiles are kept beyond 512 tokens for the SwiGLU layer, where they halve the
// weight re-reads.
static int q4_tile_bm(int M, bool swiglu) { return (swiglu && M > 512) ? 128 : 64; }

int q4_tile_count(int M, int N) {
    const int bm = q4_tile_bm(M, false);
    return ((M + bm - 1) / bm) * ((N + 127) / 128);
}
int q4_tile_rows(int M) { return q4_tile_bm(M, false); }

// the direct-to-LDS form addresses every operand through 32-bit buffer
// offsets, and reads a SwiGLU layer's gate and up rows as whole 32-row blocks
static bool q4_tile_dma_fits(const Problem& p) {
    if (p.swiglu && p.floc % 32) return false;
    const int64_t rows = p.swiglu ? 2 * (int64_t)p.N : p.N, nblk = (rows + 31) / 32;
    const int64_t a = (((int64_t)p.nseg - 1) * p.a_seg + (int64_t)(p.M - 1) * p.lda + p.Kseg) * 2;
    const int64_t q = (((int64_t)p.nseg - 1) * p.q_seg + nblk * p.ldg * 256) * 4;
    const int64_t g = (((int64_t)p.nseg - 1) * p.g_seg + nblk * (p.ldg / 4) * 128) * 2;
    return a < (1LL << 31) && q < (1LL << 31) && g < (1LL << 31) && p.ldg % 4 == 0;
}

template <bool F16, bool SWIGLU, bool SPLIT>
static void launch_nmb(const Problem& p, hipStream_t s, dim3 grid, int tm, int tn) {
    const bool nmb1 = q4_tile_bm(p.M, SWIGLU) == 64;
    if (q4_tile_dma_fits(p)) {
        if (nmb1) launch(q4_tile_dma_kernel<F16, SWIGLU, SPLIT, 1>, grid, dim3(256), 0, s, p, tm, tn);
        else launch(q4_tile_dma_kernel<F16, SWIGLU, SPLIT, 2>, grid, dim3(256), 0, s, p, tm, tn);
    } else {
        if (nmb1) launch(q4_tile_kernel<F16, SWIGLU, SPLIT, 1>, grid, dim3(256), 0, s, p, tm, tn);
        else launch(q4_tile_kernel<F16, SWIGLU, SPLIT, 2>, grid, dim3(256), 0, s, p, tm, tn);
    }
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
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        constexpr int RV = 4;  // 8 float4 per thread (one 32-token block per wave)
        if (bm != 64) return hipErrorInvalidValue;
        launch(q4_split_reduce_kernel<1, RV>, dim3(tm * tn, 8 / RV), dim3(256), 0, s, p, tm, tn);
    } else {
        if (f16) launch_nmb<true, false, false>(p, s, grid, tm, tn);
        else launch_nmb<false, false, false>(p, s, grid, tm, tn);
    }
    return hipGetLastError();
}

}  // namespace sg
