// Backward of the sharded layers: the vector-Jacobian products of
// "MLX 张量并行实战指南" sections 2.1-2.2 (the sum_gradients wrapper of the
// all-to-sharded layer: its input is shared by every rank, so the input
// gradient is the all_sum of the rank gradients).
//
//  * all-to-sharded, Y_r = X W_r^T:  dX = sum_r dY_r W_r (ranks summed in
//    order, on chip), dW_r = dY_r^T X;
//  * sharded-to-all, Y = sum_r X_r W_r^T:  dX_r = dY W_r (stays sharded, no
//    reduction), dW_r = dY^T X_r.
//
// 16-bit layers whose shapes tile run their input gradients on the forward
// matrix-core kernels over a transposed copy of the shards, and their weight
// gradients on dw_small_kernel below (few tokens) or on the tile kernels over
// transposed operands.  This file also holds the vector-unit kernels that
// serve every other case (fp32 layers, unaligned shapes, many-token weight
// gradients without a workspace), with fp32 accumulation: the input gradient
// token-blocked with the K range split over the waves of a workgroup, the
// weight gradient a few elements per thread (its reduction runs over the B
// tokens only).  They read the weight in the layout the layer stores
// (fragment-major or row-major), element W_r[k][n] of rank r's (rows_r,
// cols_r) shard.
#include "internal.h"

namespace sg {

// operand element as fp32, the dtype fixed at compile time (no per-load branch,
// so the unrolled loops keep several loads in flight)
template <int DT>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    if constexpr (DT == SG_F32) return ((const float*)p)[i];
    else if constexpr (DT == SG_BF16) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    else return (float)((const _Float16*)p)[i];
}

// out[m][n] (reduce: the ranks summed in order) or out[s][m][n] =
// sum_k A_s[m][k] W_s[k][n], token-blocked: a workgroup of 16 waves owns CW output
// columns n and 16 tokens.  Lane l takes column l % CW and every (64 / CW)-th
// k of each staged chunk starting at l / CW, keeping the 16 tokens' sums for
// its column, so every weight element is loaded once for all of them.  The 16
// waves split each rank's K range; a wave stages its 64 x 16 chunk of A in its
// own LDS buffer and reads it back as broadcasts.  The partials (waves, then
// lane groups) are added in a fixed order after the one workgroup barrier,
// which every thread reaches (no early exit).  CW < 64 gives narrow outputs
// enough workgroups.  grid: (N / CW, M / 16, reduce ? 1 : nseg).
template <int DT, bool WFRAG, int CW>
__global__ __launch_bounds__(1024) void bwd_dxt_kernel(BwdDx p) {
    constexpr int NWV = 16, TB = 16, CH = 64, SUB = 64 / CW;
    __shared__ float stage[NWV][CH][TB];      // per wave: A chunk, [k][token]
    __shared__ float red[NWV][TB][64];        // per wave: partial sums, [token][lane]
    const int lane = threadIdx.x & 63, col = lane % CW, sub = lane / CW;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n = (int64_t)blockIdx.x * CW + col;
    const int64_t nc = n < p.N ? n : p.N - 1;  // clamped column for loads
    const int m0 = blockIdx.y * TB;
    const int so = blockIdx.z;
    const int s0 = p.reduce ? 0 : so, s1 = p.reduce ? p.nseg : so + 1;
    const int kp = (p.K + NWV - 1) / NWV, ks = min(p.K, wave * kp), ke = min(p.K, ks + kp);
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.f;
    for (int s = s0; s < s1; ++s) {  // ranks in order
        const int64_t r0 = p.stacked ? (int64_t)s * p.K : 0, wb = p.stacked ? 0 : s * p.w_seg;
        for (int c = ks; c < ke; c += CH) {
            // stage A[s][m0 + t][c + lane] (zero past ke or past M)
            const int k = c + lane;
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const bool ok = k < ke && m0 + t < p.M;
                stage[wave][lane][t] = ok ? ld<DT>(p.A, s * p.a_seg + (int64_t)(m0 + t) * p.lda + k) : 0.f;
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's stores are in LDS
            __builtin_amdgcn_wave_barrier();
            const int len = min(CH, ke - c);
            for (int kk = sub; kk < len; kk += SUB) {
                const int64_t kr = r0 + c + kk;
                const float w = ld<DT>(p.W, wb + (WFRAG ? frag_offset(kr, nc, p.wsteps) : kr * p.ldw + nc));
#pragma unroll
                for (int t = 0; t < TB; ++t) acc[t] = fmaf(stage[wave][kk][t], w, acc[t]);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();  // every lane has read the chunk before it is overwritten
        }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    // thread (wave, lane < CW): token m0 + wave, column n -- partials in order
    if (lane < CW) {
        float v = 0.f;
        for (int w = 0; w < NWV; ++w)
            for (int g = 0; g < SUB; ++g) v += red[w][wave][g * CW + col];
        const int m = m0 + wave;
        if (m < p.M && n < p.N) store_from_f32(p.out, p.out_dtype, ((int64_t)so * p.M + m) * p.N + n, v);
    }
}

template <int DT, bool WFRAG>
static void launch_dxt(const BwdDx& p, hipStream_t s) {
    const unsigned gy = (unsigned)((p.M + 15) / 16), gz = (unsigned)(p.reduce ? 1 : p.nseg);
    const dim3 block(1024);
    // the widest column group that still gives every CU a workgroup
    const int64_t per = (int64_t)gy * gz;
    if ((p.N + 63) / 64 * per >= 256)
        launch(bwd_dxt_kernel<DT, WFRAG, 64>, dim3((unsigned)((p.N + 63) / 64), gy, gz), block, 0, s, p);
    else if ((p.N + 31) / 32 * per >= 256)
        launch(bwd_dxt_kernel<DT, WFRAG, 32>, dim3((unsigned)((p.N + 31) / 32), gy, gz), block, 0, s, p);
    else
        launch(bwd_dxt_kernel<DT, WFRAG, 16>, dim3((unsigned)((p.N + 15) / 16), gy, gz), block, 0, s, p);
}

// out[s][o][i] = sum_m G_s[m][o] X_s[m][i]
template <int DT>
__global__ __launch_bounds__(256) void bwd_dw_kernel(BwdDw p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t plane = (int64_t)p.R * p.C;
    if (idx >= p.nseg * plane) return;
    const int s = (int)(idx / plane);
    const int64_t rem = idx - s * plane;
    const int64_t o = rem / p.C, i = rem - o * p.C;
    const int64_t gb = s * p.g_seg + o, xb = s * p.x_seg + i;
    float acc = 0.f;
#pragma unroll 8
    for (int m = 0; m < p.M; ++m) acc = fmaf(ld<DT>(p.G, gb + (int64_t)m * p.ldg), ld<DT>(p.X, xb + (int64_t)m * p.ldx), acc);
    store_from_f32(p.out, p.out_dtype, idx, acc);
}

// out[s][o][i .. i+3]: four adjacent outputs per thread share each G load and
// read X four elements (8 or 16 bytes) at a time; C % 4 == 0 and 16-bit or fp32
// rows aligned to 4 elements
template <int DT>
__global__ __launch_bounds__(256) void bwd_dw4_kernel(BwdDw p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t C4 = p.C / 4, plane = (int64_t)p.R * C4;
    if (idx >= p.nseg * plane) return;
    const int s = (int)(idx / plane);
    const int64_t rem = idx - s * plane;
    const int64_t o = rem / C4, i = (rem - o * C4) * 4;
    const int64_t gb = s * p.g_seg + o, xb = s * p.x_seg + i;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int m = 0; m < p.M; ++m) {
        const float g = ld<DT>(p.G, gb + (int64_t)m * p.ldg);
        const int64_t xi = xb + (int64_t)m * p.ldx;
        float x[4];
        if constexpr (DT == SG_F32) {
            const float4 v = *(const float4*)((const float*)p.X + xi);
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        } else {
            const uint2 v = *(const uint2*)((const uint16_t*)p.X + xi);
            const uint16_t h[4] = {(uint16_t)(v.x & 0xFFFFu), (uint16_t)(v.x >> 16), (uint16_t)(v.y & 0xFFFFu),
                                   (uint16_t)(v.y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = DT == SG_BF16 ? __uint_as_float((uint32_t)h[e] << 16) : (float)__builtin_bit_cast(_Float16, h[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(g, x[e], acc[e]);
    }
    const int64_t oi = (int64_t)s * p.R * p.C + o * p.C + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_from_f32(p.out, p.out_dtype, oi + e, acc[e]);
}

// Weight gradient with few tokens on the matrix cores, reading the caller's
// row-major upstream gradient and layer input directly:
//     out[o][i] = sum_b G(b, o) X(b, i),
// G(b, o) = G[(o / gl) g_seg + b ldg + o % gl] and X(b, i) likewise (the rank
// blocks of a sharded operand), out (O, I) row-major or, with nloc > 0, the
// sharded (I / nloc, O, nloc).  A workgroup (4 waves) owns 128 o x 128 i: it
// stages both operands' 128 x Bp slices in LDS transposed (token-contiguous,
// tokens past B zero; 16-byte global reads of 8 consecutive o or i), then each
// wave runs v_mfma_f32_32x32x16 on 64 x 64 outputs with the rows o as the row
// operand and the inputs i as the column operand.  Each accumulator register
// then holds 32 consecutive i of one row across lanes 0-31 (and of the row 4
// further down across lanes 32-63), so every store writes two contiguous
// 128-byte row pieces -- the kernel is bound by these fp32 writes.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ f32x16_t mfma32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
}

// stage rows [r0, r0 + 128) of the transposed operand T(row, b) = S(b, row)
// into lds[row - r0][b], b < Bp (zero past B and past rows)
__device__ __forceinline__ void stage_t(uint16_t* lds, int ldl, const uint16_t* S, int64_t gl, int64_t seg,
                                        int64_t ld, int r0, int rows, int B, int Bp) {
    const int chunks = 16 * Bp;  // (b, 8-row chunk) pairs
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        const int b = c >> 4, rr = (c & 15) * 8;
        const int row = r0 + rr;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (b < B && row < rows) {
            const int64_t g = row / gl;
            v = *(const u32x4_t*)(S + g * seg + (int64_t)b * ld + (row - g * gl));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lds[(rr + 2 * e) * ldl + b] = (uint16_t)(v[e] & 0xFFFFu);
            lds[(rr + 2 * e + 1) * ldl + b] = (uint16_t)(v[e] >> 16);
        }
    }
}

template <bool F16>
__global__ __launch_bounds__(256) void dw_small_kernel(BwdDwSmall p) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const int ldl = p.Bp + 8;  // LDS row: Bp tokens + 16 bytes of padding
    uint16_t* sA = smem;
    uint16_t* sB = smem + 128 * ldl;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ob = blockIdx.y * 128, ib = blockIdx.x * 128;
    stage_t(sA, ldl, (const uint16_t*)p.G, p.gl, p.g_seg, p.ldg, ob, p.O, p.B, p.Bp);
    stage_t(sB, ldl, (const uint16_t*)p.X, p.xl, p.x_seg, p.ldx, ib, p.I, p.B, p.Bp);
    __syncthreads();
    const int wo = (wave >> 1) * 64, wi = (wave & 1) * 64;
    const int r = lane & 31, kh = (lane >> 5) * 8;
    f32x16_t acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;
    for (int k = 0; k < p.Bp; k += 16) {
        u32x4_t a[2], b[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            a[x] = *(const u32x4_t*)(sA + (wo + x * 32 + r) * ldl + k + kh);
            b[x] = *(const u32x4_t*)(sB + (wi + x * 32 + r) * ldl + k + kh);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = mfma32x16<F16>(a[x], b[y], acc[x][y]);
    }
    // lane l of a 32 x 32 block: column l & 31, rows 8 j + 4 (l >> 5) + e
    static_for<0, 2>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        static_for<0, 2>([&](auto yc) {
            constexpr int y = decltype(yc)::value;
            const int i = ib + wi + y * 32 + (lane & 31);
            if (i >= p.I) return;
            int64_t col = i, base = 0, ld = p.I;
            if (p.nloc > 0) {
                const int64_t rk = i / p.nloc;
                col = i - rk * p.nloc;
                base = rk * (int64_t)p.O * p.nloc;
                ld = p.nloc;
            }
            static_for<0, 16>([&](auto ec) {
                constexpr int e = decltype(ec)::value;
                const int o = ob + wo + x * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (o >= p.O) return;
                const int64_t at = base + (int64_t)o * ld + col;
                // written once, never read back here: streaming stores (measured ~10%
                // faster on the decode-MLP gradients than cached ones)
                if (p.out_dtype == SG_F32) __builtin_nontemporal_store(acc[x][y][e], (float*)p.out + at);
                else store_from_f32(p.out, p.out_dtype, at, acc[x][y][e]);
            });
        });
    });
}

size_t dw_small_lds(int Bp) { return (size_t)2 * 128 * (Bp + 8) * sizeof(uint16_t); }

hipError_t launch_dw_small(const BwdDwSmall& p, hipStream_t s) {
    if (p.O == 0 || p.I == 0 || p.B == 0) return hipSuccess;
    if (p.Bp % 16 || p.Bp < p.B || p.Bp > kDwSmallMaxTokens || (p.dtype != SG_BF16 && p.dtype != SG_F16) || p.gl % 8 ||
        p.xl % 8 || p.ldg % 8 || p.ldx % 8 || p.g_seg % 8 || p.x_seg % 8 || p.O % 8 || p.I % 8)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((p.I + 127) / 128), (unsigned)((p.O + 127) / 128)), block(256);
    const size_t lds = dw_small_lds(p.Bp);
    if (p.dtype == SG_F16) launch(dw_small_kernel<true>, grid, block, lds, s, p);
    else launch(dw_small_kernel<false>, grid, block, lds, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdDx& p, hipStream_t s) {
    const int64_t total = (p.reduce ? 1 : p.nseg) * (int64_t)p.M * p.N;
    if (total == 0) return hipSuccess;
    if (p.dtype == SG_F32 && p.wfrag) return hipErrorInvalidValue;  // fp32 layers are stored row-major
    if (p.dtype == SG_F32) launch_dxt<SG_F32, false>(p, s);
    else if (p.dtype == SG_BF16 && p.wfrag) launch_dxt<SG_BF16, true>(p, s);
    else if (p.dtype == SG_BF16) launch_dxt<SG_BF16, false>(p, s);
    else if (p.wfrag) launch_dxt<SG_F16, true>(p, s);
    else launch_dxt<SG_F16, false>(p, s);
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const BwdDw& p, hipStream_t s) {
    const int64_t total = p.nseg * (int64_t)p.R * p.C;
    if (total == 0) return hipSuccess;
    const int esz = p.dtype == SG_F32 ? 4 : 2;
    const bool vec = p.C % 4 == 0 && p.ldx % 4 == 0 && p.x_seg % 4 == 0 && ((uintptr_t)p.X % (4 * esz)) == 0;
    if (vec) {
        const dim3 grid((unsigned)((total / 4 + 255) / 256)), block(256);
        if (p.dtype == SG_F32) launch(bwd_dw4_kernel<SG_F32>, grid, block, 0, s, p);
        else if (p.dtype == SG_BF16) launch(bwd_dw4_kernel<SG_BF16>, grid, block, 0, s, p);
        else launch(bwd_dw4_kernel<SG_F16>, grid, block, 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (p.dtype == SG_F32) launch(bwd_dw_kernel<SG_F32>, grid, block, 0, s, p);
    else if (p.dtype == SG_BF16) launch(bwd_dw_kernel<SG_BF16>, grid, block, 0, s, p);
    else launch(bwd_dw_kernel<SG_F16>, grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace sg
