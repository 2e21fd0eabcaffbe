// MFMA tile GEMM for gfx950 (prefill-shaped sharded GEMMs and SUMMA).
//
// C[m][n] = sum over segments s (ranks of a sharded-to-all layer, or the q
// steps of SUMMA) of A_s W_s^T, bf16 / fp16 operands, fp32 accumulation in
// v_mfma_f32_32x32x16_{bf16,f16}.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid; block tile BM tokens x BN
// weight rows x 64 k; each wave owns (BM/2) x (BN/2) outputs as 32 x 32 MFMA
// blocks.  The weight tile feeds the MFMA's row operand and the activation
// tile its column operand, so each lane ends with four consecutive output
// columns per block and the store is an 8-byte vector.
//
// Pipeline: global -> registers (tile k+1) while the MFMAs consume tile k
// from LDS, then registers -> the other LDS buffer; one barrier per k-tile.
// LDS rows are 128 bytes (64 bf16) with the 16-byte chunk index XOR-swizzled
// by (row ^ row >> 3) & 7, which keeps the MFMA fragment reads, the row
// stores and the transposed SUMMA stores free of bank conflicts.
//
// Operand modes:
//  NT      W is (N, K): weight rows, K contiguous (the MLX layout).
//  SWIGLU  W holds [gate; up] rank blocks; the tile interleaves 32 gate rows
//          and the 32 matching up rows so the pair lands in one lane and the
//          epilogue writes silu(g) * u ("MLX 张量并行实战指南" 5.2-5.3).
//  NN      W is (K, N) (SUMMA's A operand, "ColossalAI 2D 张量并行", SUMMA
//          section): each thread loads an 8 x 8 block and transposes it in
//          registers before the LDS store.
//
// Cross-segment sum: either in registers (the K loop walks rank 0's slice,
// then rank 1's, ...) or split by segment, where each workgroup forms one
// rank's partial tile, writes it to the workspace and the last of the nseg
// workgroups of a tile adds the partials in rank order (deterministic).
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { WM_NT = 0, WM_SWIGLU = 1, WM_NN = 2 };
constexpr int BK = 64;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 x 8 transpose of 16-bit elements: in[i] holds row i (8 values as 4
// words), out[j] receives column j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
#pragma unroll
        for (int q = 0; q < 4; ++q)
            out[j][q] = __builtin_amdgcn_perm(in[2 * q + 1][w], in[2 * q][w], sel);
    }
}

// Store four consecutive logical columns n .. n+3 of row m (bias, output
// map, dtype conversion, fp32 accumulate); vector store when they are
// contiguous and aligned.
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

// FP8: MX FP8 weights (E4M3 codes, one E8M0 scale per 32 inputs of a row), each
// 8-code chunk turned into the bf16 operand in registers before the LDS store
// (exact: 4 significant bits times a power of two), so the MFMAs and the rest
// of the pipeline are the dense ones.
template <int BM, int BN, bool F16, int WMODE, bool SPLIT, bool FP8 = false>
__global__ __launch_bounds__(256) void tile_kernel(Problem p, int tiles_m, int tiles_n) {
    static_assert(!FP8 || (!F16 && WMODE != WM_NN), "MX FP8 weights: bf16 activations, (out, in) weights");
    constexpr int WTM = BM / 2, WTN = BN / 2;  // per-wave outputs
    constexpr int NBM = WTM / 32, NBN = WTN / 32;
    constexpr int CA = BM / 32, CB = BN / 32;  // 16-byte chunks per thread
    constexpr int NOUT = (WMODE == WM_SWIGLU) ? BN / 2 : BN;  // logical columns per tile
    static_assert(NBN % 2 == 0 || WMODE != WM_SWIGLU, "gate/up blocks pair within a wave");
    static_assert(WMODE != WM_NN || BN == 256, "transposing loader covers 256 columns");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];
    uint16_t* sA = smem;                 // [2][BM][BK]
    uint16_t* sB = smem + 2 * BM * BK;   // [2][BN][BK]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave >> 1, wave_n = wave & 1;

    // ---- tile coordinates: XCD-contiguous ranges, groups of GM tile rows
    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int group = tile / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - group * GM * tiles_n;
    const int tm = first_m + tin % gsz, tn = tin / gsz;
    const int m0 = tm * BM;
    const int64_t n0 = (int64_t)tn * NOUT;
    // split: workgroup (tile, y) takes group y of gridDim.y groups of consecutive segments
    const int seg_cnt = SPLIT ? p.nseg / (int)gridDim.y : p.nseg;
    const int seg_lo = SPLIT ? (int)blockIdx.y * seg_cnt : 0;

    const uint16_t* Ag = (const uint16_t*)p.A;
    const uint16_t* Wg = (const uint16_t*)p.W;

    // ---- per-thread global load descriptors
    const int lrow = tid >> 3, lch = tid & 7;  // row-chunk loader (A, NT weights)
    int64_t aoff[CA];
    bool aok[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int m = m0 + lrow + 32 * i;
        aok[i] = m < p.M;
        aoff[i] = (int64_t)(aok[i] ? m : 0) * p.lda + lch * 8;
    }
    int64_t woff[CB];
    int64_t wrow[CB];  // FP8: the weight row of each chunk
    bool wok[CB];
    const int tkb = tid >> 5, tnb = tid & 31;  // transposing loader (NN)
    if constexpr (WMODE == WM_NN) {
        const int64_t n = n0 + tnb * 8;
        wok[0] = n < p.N;
        woff[0] = (int64_t)tkb * 8 * p.ldw + (wok[0] ? n : 0);
    } else {
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            int64_t row;
            if constexpr (WMODE == WM_SWIGLU) {
                const int64_t j = n0 + (i >> 1) * 32 + lrow;  // logical column
                wok[i] = j < p.N;
                row = weight_row(p, wok[i] ? j : 0, i & 1);
            } else {
                const int64_t n = n0 + lrow + 32 * i;
                wok[i] = n < p.N;
                row = wok[i] ? n : 0;
            }
            woff[i] = p.wfrag ? frag_offset(row, lch * 8, p.wsteps) : row * p.ldw + lch * 8;
            wrow[i] = row;
        }
    }
    // advancing k by one 64-wide tile moves 64 elements (row-major) or two
    // 512-element fragments (fragment-major)
    const int wk = p.wfrag ? 1024 / BK : 1;

    const int ktiles_seg = (p.Kseg + BK - 1) / BK;
    const int nkt = ktiles_seg * seg_cnt;

    u32x4 ra[CA], rb[(WMODE == WM_NN) ? 8 : CB];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int kt) {
        const int s = seg_lo + kt / ktiles_seg;
        const int k0 = (kt % ktiles_seg) * BK;
        const uint16_t* Ab = Ag + s * p.a_seg + k0;
        const uint16_t* Wb = Wg + s * p.w_seg;
        const bool kok = k0 + lch * 8 < p.Kseg;
#pragma unroll
        for (int i = 0; i < CA; ++i)
            ra[i] = (aok[i] && kok) ? *(const u32x4*)(Ab + aoff[i]) : zero;
        if constexpr (WMODE == WM_NN) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = wok[0] && (k0 + tkb * 8 + e < p.Kseg);
                rb[e] = ok ? *(const u32x4*)(Wb + (int64_t)(k0 + e) * p.ldw + woff[0]) : zero;
            }
        } else if constexpr (FP8) {
            const uint8_t* W8 = (const uint8_t*)p.W + s * p.w_seg;
            const uint8_t* S8 = p.ms + s * p.ms_seg;
            const int k = k0 + lch * 8;
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                if (wok[i] && kok) {
                    const int64_t ci = p.wfrag ? mx_code_offset(wrow[i], k, p.wsteps) : wrow[i] * p.ldw + k;
                    const int64_t si = p.wfrag ? mx_scale_offset(wrow[i], k >> 5, p.wsteps) : wrow[i] * (p.ldw >> 5) + (k >> 5);
                    rb[i] = mx8_to_bf16(*(const u32x2*)(W8 + ci), S8[si]);
                } else {
                    rb[i] = zero;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CB; ++i)
                rb[i] = (wok[i] && kok) ? *(const u32x4*)(Wb + woff[i] + (int64_t)k0 * wk) : zero;
        }
    };
    auto sstore = [&](int buf) {
        uint16_t* a = sA + buf * BM * BK;
        uint16_t* b = sB + buf * BN * BK;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int row = lrow + 32 * i;
            *(u32x4*)(a + row * BK + ((lch ^ swz(row)) << 3)) = ra[i];
        }
        if constexpr (WMODE == WM_NN) {
            u32x4 cols[8];
            transpose8x8(rb, cols);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = tnb * 8 + j;
                *(u32x4*)(b + row * BK + ((tkb ^ swz(row)) << 3)) = cols[j];
            }
        } else {
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const int row = lrow + 32 * i;
                *(u32x4*)(b + row * BK + ((lch ^ swz(row)) << 3)) = rb[i];
            }
        }
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // fragment read positions
    const int frow = lane & 31, fch = lane >> 5;

    if (nkt > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        const uint16_t* a = sA + buf * BM * BK;
        const uint16_t* b = sB + buf * BN * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + fch;
            u32x4 wf[NBN], xf[NBM];
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
                const int row = wave_n * WTN + i * 32 + frow;
                wf[i] = *(const u32x4*)(b + row * BK + ((c ^ swz(row)) << 3));
            }
#pragma unroll
            for (int j = 0; j < NBM; ++j) {
                const int row = wave_m * WTM + j * 32 + frow;
                xf[j] = *(const u32x4*)(a + row * BK + ((c ^ swz(row)) << 3));
            }
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(wf[i], xf[j], acc[i][j]);
        }
        if (kt + 1 < nkt) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- rank split: this segment's partial tile to the workspace (thread
    // tid's float4 v = (i NBM + j) 4 + q at float4 index v * 256 + tid of the
    // tile's slab); split_reduce_kernel adds the segments in rank order
    if constexpr (SPLIT) {
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * ntiles + tile) * (BM * BN));
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    mine[((i * NBM + j) * 4 + q) * 256 + tid] = v;
                }
        return;
    }

    // ---- epilogue
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (WMODE == WM_SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (WMODE == WM_SWIGLU) {
                    const int blk32 = wave_n * NBN + i;
                    n = n0 + (blk32 >> 1) * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i | 1][j][4 * blk + e];  // i even: i | 1 = i + 1
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

// Sum of a split product's partial tiles (NT or NN weights, no SwiGLU):
// partial g of tile t is the BM x BN floats at (g ntiles + t) BM BN of the
// workspace, holding thread tid's float4 v (its accumulator acc[i][j][4q ..
// 4q + 3], v = (i NBM + j) 4 + q) at float4 index v NT + tid.  Workgroup
// (t, y) takes float4 indices RV y .. RV y + RV - 1 of every thread, adds the
// groups' partials in group (rank) order and stores them through the
// epilogue (bias, output layout and dtype).  A second kernel rather than the
// last workgroup of a tile to arrive: the kernel boundary orders the partial
// stores before the loads, where an in-kernel handoff needs a device-scope
// release per workgroup, and the sum is spread over every compute unit.
// MLOW: the product kernel's wave w covers rows (w mod 2) WTM (the ping-pong
// kernel) rather than (w / 2) WTM.
template <int BM, int BN, int WTM, int WTN, int NT, bool MLOW, int RV>
__global__ __launch_bounds__(NT) void split_reduce_kernel(Problem p, int tiles_m, int tiles_n, int groups) {
    constexpr int NBM = WTM / 32, NWN = BN / WTN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = MLOW ? wave % (BM / WTM) : wave / NWN;
    const int wave_n = MLOW ? wave / (BM / WTM) : wave % NWN;
    const int hi = lane >> 5;
    const int ntiles = tiles_m * tiles_n;
    const int tile = blockIdx.x;
    constexpr int GM = 4;  // the tile -> (m0, n0) map of the product kernels
    const int gidx = tile / (GM * tiles_n);
    const int first_m = gidx * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - gidx * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * BN;

    const int v0 = blockIdx.y * RV;
    f32x4 sum[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) sum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < groups; ++g) {  // rank order
        const f32x4* src = (const f32x4*)(p.ws + ((int64_t)g * ntiles + tile) * (BM * BN));
        f32x4 v[RV];
#pragma unroll
        for (int r = 0; r < RV; ++r) v[r] = src[(v0 + r) * NT + tid];
#pragma unroll
        for (int r = 0; r < RV; ++r) sum[r] += v[r];
    }
#pragma unroll
    for (int r = 0; r < RV; ++r) {
        const int v = v0 + r, i = v / (NBM * 4), j = (v / 4) % NBM, q = v % 4;
        const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
        if (m >= p.M) continue;
        const int64_t n = n0 + wave_n * WTN + i * 32 + 8 * q + 4 * hi;
        float o[4] = {sum[r][0], sum[r][1], sum[r][2], sum[r][3]};
        store4(p, m, n, o);
    }
}

hipError_t launch_split_reduce(const Problem& p, int tiles_m, int tiles_n, int groups, int layout, hipStream_t s) {
    constexpr int RV = 4;
    const int ntiles = tiles_m * tiles_n;
    switch (layout) {
    case 0:  // ping-pong 256 x 256, 8 waves of 128 x 64: 32 float4 per thread
        launch((split_reduce_kernel<256, 256, 128, 64, 512, true, RV>), dim3(ntiles, 32 / RV), dim3(512), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    case 1:  // register-staged 128 x 128, 4 waves of 64 x 64: 16 float4 per thread
        launch((split_reduce_kernel<128, 128, 64, 64, 256, false, RV>), dim3(ntiles, 16 / RV), dim3(256), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    case 2:  // register-staged 256 x 256, 4 waves of 128 x 128: 64 float4 per thread
        launch((split_reduce_kernel<256, 256, 128, 128, 256, false, RV>), dim3(ntiles, 64 / RV), dim3(256), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    case 3:  // few-token 64 x 128, 4 waves of 32 x 64: 8 float4 per thread
        launch((split_reduce_kernel<64, 128, 32, 64, 256, true, RV>), dim3(ntiles, 8 / RV), dim3(256), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    case 4:  // few-token 128 x 128, 4 waves of 64 x 64: 16 float4 per thread
        launch((split_reduce_kernel<128, 128, 64, 64, 256, true, RV>), dim3(ntiles, 16 / RV), dim3(256), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    default:  // few-token 256 x 128, 4 waves of 128 x 64: 32 float4 per thread
        launch((split_reduce_kernel<256, 128, 128, 64, 256, true, RV>), dim3(ntiles, 32 / RV), dim3(256), 0, s, p,
               tiles_m, tiles_n, groups);
        break;
    }
    return hipGetLastError();
}

// variant 0: 256 x 256 tiles; variant 1: 128 x 128 tiles
int tile_count(int M, int N, int variant) {
    const int bm = variant == 0 ? 256 : 128;
    return ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
}

int device_cus() {
    static int cus = -1;
    if (cus < 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        cus = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
                  ? prop.multiProcessorCount
                  : 256;
    }
    return cus;
}

int split_groups(int tiles, int nseg) {
    const int cus = device_cus();
    for (int d = 1; d < nseg; ++d)
        if (nseg % d == 0 && tiles * d >= cus) return d;
    return nseg;
}

int tile_pp_groups(int M, int N, int nseg) { return split_groups(tile_count(M, N, 0), nseg); }

// variant 0 splits into tile_pp_groups groups, variant 1 into nseg
SplitLayout tile_split_layout(int M, int N, int nseg, int variant) {
    const size_t t = (size_t)tile_count(M, N, variant), bm = variant == 0 ? 256 : 128;
    const size_t groups = variant == 0 ? (size_t)tile_pp_groups(M, N, nseg) : (size_t)nseg;
    return {t * bm * bm * groups, t};
}

template <int BM, int BN, bool F16, int WMODE, bool SPLIT, bool FP8 = false>
static hipError_t launch_one(const Problem& p, hipStream_t s) {
    const int nout = WMODE == WM_SWIGLU ? BN / 2 : BN;
    const int tm = (p.M + BM - 1) / BM, tn = (p.N + nout - 1) / nout;
    // the split groups tile_split_layout sizes the workspace for
    const int groups = !SPLIT ? 1 : BM == 256 ? tile_pp_groups(p.M, p.N, p.nseg) : p.nseg;
    dim3 grid(tm * tn, groups);
    launch((tile_kernel<BM, BN, F16, WMODE, SPLIT, FP8>), grid, dim3(256), 0, s, p, tm, tn);
    if constexpr (SPLIT) {
        static_assert(WMODE != WM_SWIGLU, "no split with SwiGLU");
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_split_reduce(p, tm, tn, groups, BM == 128 ? 1 : 2, s);
    }
    return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_fp8(const Problem& p, hipStream_t s) {
    if (p.dtype != SG_BF16 || p.nn) return hipErrorInvalidValue;
    if (p.swiglu) return launch_one<BM, BN, false, WM_SWIGLU, false, true>(p, s);
    return p.split ? launch_one<BM, BN, false, WM_NT, true, true>(p, s) : launch_one<BM, BN, false, WM_NT, false, true>(p, s);
}

template <int BM, int BN, bool F16>
static hipError_t launch_mode(const Problem& p, hipStream_t s) {
    // transposed weights: no split (no caller splits them)
    if (p.nn) return p.split ? hipErrorInvalidValue : launch_one<BM, 256, F16, WM_NN, false>(p, s);
    if (p.swiglu) return launch_one<BM, BN, F16, WM_SWIGLU, false>(p, s);
    return p.split ? launch_one<BM, BN, F16, WM_NT, true>(p, s)
                   : launch_one<BM, BN, F16, WM_NT, false>(p, s);
}

hipError_t launch_tile_dma(const Problem& p, hipStream_t s);
bool tile_dma_fits(const Problem& p);

hipError_t launch_tile(const Problem& p, hipStream_t s, int variant) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    // 256 x 256 weight tiles: the direct-to-LDS pipeline (tile_dma.hip)
    if (variant == 0 && tile_dma_fits(p)) return launch_tile_dma(p, s);
    // MX FP8 weights: 128 x 128 tiles only (the 256 x 256 form with the FP8
    // loader spills its registers)
    if (p.fp8) return launch_fp8<128, 128>(p, s);
    const bool f16 = p.dtype == SG_F16;
    if (variant == 0) return f16 ? launch_mode<256, 256, true>(p, s) : launch_mode<256, 256, false>(p, s);
    return f16 ? launch_mode<128, 128, true>(p, s) : launch_mode<128, 128, false>(p, s);
}

}  // namespace sg
