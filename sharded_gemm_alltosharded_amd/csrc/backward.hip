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
// fp32 accumulation on the vector units (the products are not on the matrix
// cores yet): the input gradient token-blocked with the K range split over the
// waves of a workgroup, the weight gradient one thread per element (its
// reduction runs over the B tokens only).  The weight is read in the layout the
// layer stores (fragment-major or row-major), element W_r[k][n] of rank r's
// (rows_r, cols_r) shard.
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
