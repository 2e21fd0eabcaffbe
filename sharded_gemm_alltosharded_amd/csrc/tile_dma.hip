// MFMA tile GEMM for gfx950 with direct global -> LDS loads (prefill-shaped
// sharded GEMMs).  Same product and epilogues as tile.hip's NT / SWIGLU modes;
// what differs is the feed:
//
//  * global_load_lds_dwordx4: each lane's 16 bytes go straight from memory to
//    LDS slot (M0 + 16 lane) with no staging registers and no ds_write, so the
//    LDS can hold a 4-stage pipeline (BK = 32, 32 KB per stage): three k tiles
//    are in flight while the MFMAs consume the fourth, which covers the global
//    latency a single register-staged prefetch could not.
//  * each wave-wide load fills 16 tile rows x 64 bytes; a lane picks its
//    global chunk so that the row's four 16-byte chunks land XOR-swizzled by
//    (row >> 1) & 3, which keeps the MFMA fragment reads conflict-free.  With
//    fragment-major weights those 16 rows x 64 bytes are one contiguous 1 KB.
//  * the k loop is unrolled over the 4 stages so every LDS buffer is a
//    distinct array (the waits before a stage's reads then cover only that
//    stage's loads); one barrier per k tile.
//
// Rows past M or N read a clamped valid row (their outputs are never
// stored); K must be a multiple of 32.
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
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int swz4(int row) { return (row >> 1) & 3; }

__device__ __forceinline__ void dma16(const uint16_t* g, uint16_t* lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// LDS fragment read issued as inline assembly: the compiler's wait insertion
// cannot tell these reads from the direct-to-LDS loads still in flight and
// would otherwise wait for all of them (vmcnt(0)) before each read.  The
// caller waits for the reads with wait_lds, which also ties the registers.
__device__ __forceinline__ u32x4 lds_read16(const uint16_t* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
}

template <int NWF, int NXF>
__device__ __forceinline__ void wait_lds(u32x4 (&w)[NWF], u32x4 (&x)[NXF]) {
    static_assert(NXF == 4 && (NWF == 4 || NWF == 2), "fragments of one k step");
    if constexpr (NWF == 4)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// s_waitcnt vmcnt(n) (n <= 63), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void store4(const Problem& p, int m, int64_t n, float (&v)[4]) {
    if (n >= p.N) return;
    if (p.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) v[e] += load_as_f32(p.bias, p.dtype, n + e);
    }
    const bool full = n + 3 < p.N && (p.out_map == OUT_ROWMAJOR ? (p.ldo % 4 == 0) : (p.nloc % 4 == 0));
    const int64_t o = out_index(p, m, n);
    if (full && !p.accumulate && p.out_dtype != SG_F32) {
        u32x2 w;
        if (p.out_dtype == SG_BF16) {
            w[0] = f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            w[1] = f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        } else {
            w[0] = f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
            w[1] = f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
        }
        *(u32x2*)((uint16_t*)p.out + o) = w;
    } else if (full && p.out_dtype == SG_F32) {
        f32x4* dst = (f32x4*)((float*)p.out + o);
        f32x4 r = {v[0], v[1], v[2], v[3]};
        if (p.accumulate) r += *dst;
        *dst = r;
    } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) {
            const int64_t oe = out_index(p, m, n + e);
            float x = v[e];
            if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[oe];
            store_from_f32(p.out, p.out_dtype, oe, x);
        }
    }
}

}  // namespace

template <bool F16, bool SWIGLU, int NW>
__global__ __launch_bounds__(NW * 64) void tile_dma_kernel(Problem p, int tiles_m, int tiles_n) {
    constexpr int BM = 256, BN = 256, BK = 32;
    // NW = 4: 2 x 2 waves of 128 x 128; NW = 8: 2 x 4 waves of 128 x 64 (two
    // waves per SIMD, so one wave's barrier or LDS wait overlaps the other's MFMAs)
    constexpr int WN = NW / 2;
    constexpr int WTM = BM / 2, WTN = BN / WN, NBM = WTM / 32, NBN = WTN / 32;
    constexpr int LPT = 1024 / (NW * 64);  // 16-byte loads per thread per operand and stage
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    constexpr int TILE = BM * BK;  // elements of one operand stage (16 KB)
    __shared__ __attribute__((aligned(1024))) uint16_t sA0[TILE], sA1[TILE], sA2[TILE], sA3[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sB0[TILE], sB1[TILE], sB2[TILE], sB3[TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WN, wave_n = wave % WN;

    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int group = tile / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - group * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;

    // ---- load descriptors: instruction i of this wave fills tile rows
    // (NW i + wave) * 16 .. +16; lane -> (row lr, LDS chunk lc)
    const int lr = lane >> 2, lc = lane & 3;
    int64_t aoff[LPT], boff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int row = (NW * i + wave) * 16 + lr;
        const int ch = lc ^ swz4(row);
        const int m = min(m0 + row, p.M - 1);
        aoff[i] = (int64_t)m * p.lda + ch * 8;
        int64_t wrow;
        if constexpr (SWIGLU) {
            const int64_t j = min(n0 + (row >> 6) * 32 + (row & 31), (int64_t)p.N - 1);
            wrow = weight_row(p, j, (row >> 5) & 1);
        } else {
            wrow = min(n0 + row, (int64_t)p.N - 1);
        }
        boff[i] = p.wfrag ? frag_offset(wrow, ch * 8, p.Kseg / 32) : wrow * p.ldw + ch * 8;
    }
    const int bk_step = p.wfrag ? 16 : 1;  // elements of W per element of k
    const uint16_t* Ag = (const uint16_t*)p.A;
    const uint16_t* Wg = (const uint16_t*)p.W;
    const int ktiles_seg = p.Kseg / BK;
    const int nkt = ktiles_seg * p.nseg;

    auto issue = [&](int kt, uint16_t* a, uint16_t* b) {
        const int s = kt / ktiles_seg;
        const int k0 = (kt - s * ktiles_seg) * BK;
        const uint16_t* Ab = Ag + s * p.a_seg + k0;
        const uint16_t* Wb = Wg + s * p.w_seg + (int64_t)k0 * bk_step;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            dma16(Ab + aoff[i], a + (NW * i + wave) * 16 * BK);
            dma16(Wb + boff[i], b + (NW * i + wave) * 16 * BK);
        }
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane & 31, fch = lane >> 5;
    auto compute = [&](const uint16_t* a, const uint16_t* b) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + fch;
            u32x4 wf[NBN], xf[NBM];
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
                const int row = wave_n * WTN + i * 32 + frow;
                wf[i] = lds_read16(b + row * BK + ((c ^ swz4(row)) << 3));
            }
#pragma unroll
            for (int j = 0; j < NBM; ++j) {
                const int row = wave_m * WTM + j * 32 + frow;
                xf[j] = lds_read16(a + row * BK + ((c ^ swz4(row)) << 3));
            }
            wait_lds(wf, xf);
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(wf[i], xf[j], acc[i][j]);
        }
    };

    // stage t: wait for its loads (2 LPT per thread per stage; up to two later
    // stages may stay in flight), barrier, refill the buffer consumed in the
    // previous iteration with stage t + 3, compute stage t.
    auto step = [&](int t, const uint16_t* a, const uint16_t* b, uint16_t* na, uint16_t* nb) {
        const int later = min(2, nkt - 1 - t);
        if (later >= 2) wait_vm<4 * LPT>();
        else if (later == 1) wait_vm<2 * LPT>();
        else wait_vm<0>();
        // every wave has its own loads of stage t in LDS; a plain barrier (no
        // release fence, which would wait for the later stages too) publishes them
        __builtin_amdgcn_s_barrier();
        if (t + 3 < nkt) issue(t + 3, na, nb);
        compute(a, b);
    };

    if (nkt > 0) issue(0, sA0, sB0);
    if (nkt > 1) issue(1, sA1, sB1);
    if (nkt > 2) issue(2, sA2, sB2);
    for (int kt = 0; kt < nkt; kt += 4) {
        step(kt, sA0, sB0, sA3, sB3);
        if (kt + 1 < nkt) step(kt + 1, sA1, sB1, sA0, sB0);
        if (kt + 2 < nkt) step(kt + 2, sA2, sB2, sA1, sB1);
        if (kt + 3 < nkt) step(kt + 3, sA3, sB3, sA2, sB2);
    }

    // ---- epilogue (as tile.hip)
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (SWIGLU) {
                    const int blk32 = wave_n * NBN + i;
                    n = n0 + (blk32 >> 1) * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i + 1][j][4 * blk + e];
                } else {
                    n = n0 + wave_n * WTN + i * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * blk + e];
                }
                store4(p, m, n, v);
            });
        });
    });
}

template <int NW>
hipError_t launch_tile_dma_nw(const Problem& p, hipStream_t s) {
    const int nout = p.swiglu ? 128 : 256;
    const int tm = (p.M + 255) / 256, tn = (p.N + nout - 1) / nout;
    const bool f16 = p.dtype == SG_F16;
    const dim3 grid(tm * tn), block(NW * 64);
    if (p.swiglu) {
        if (f16) launch(tile_dma_kernel<true, true, NW>, grid, block, 0, s, p, tm, tn);
        else launch(tile_dma_kernel<false, true, NW>, grid, block, 0, s, p, tm, tn);
    } else {
        if (f16) launch(tile_dma_kernel<true, false, NW>, grid, block, 0, s, p, tm, tn);
        else launch(tile_dma_kernel<false, false, NW>, grid, block, 0, s, p, tm, tn);
    }
    return hipGetLastError();
}
template hipError_t launch_tile_dma_nw<4>(const Problem& p, hipStream_t s);

hipError_t launch_tile_dma(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.Kseg % 32 || p.nn || p.split) return hipErrorInvalidValue;
    return launch_tile_dma_nw<4>(p, s);
}

}  // namespace sg
