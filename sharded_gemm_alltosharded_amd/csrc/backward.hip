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
// First implementation: one thread per output element with fp32 accumulation
// (the products are not yet on the matrix cores).  The weight is read in the
// layout the layer stores (fragment-major or row-major), element W_r[k][n] of
// rank r's (rows_r, cols_r) shard.
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

// out[m][n] (reduce) or out[s][m][n] = sum_k A_s[m][k] W_s[k][n]
template <int DT, bool WFRAG>
__global__ __launch_bounds__(256) void bwd_dx_kernel(BwdDx p) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t plane = (int64_t)p.M * p.N;
    if (idx >= (p.reduce ? 1 : p.nseg) * plane) return;
    const int so = (int)(idx / plane);
    const int64_t rem = idx - so * plane;
    const int m = (int)(rem / p.N);
    const int64_t n = rem - (int64_t)m * p.N;
    const int s0 = p.reduce ? 0 : so, s1 = p.reduce ? p.nseg : so + 1;
    float tot = 0.f;
    for (int s = s0; s < s1; ++s) {  // ranks in order: the all_sum
        // all-to-sharded ranks are stacked rows of one matrix (a fragment-major
        // layout spans the stack, rank s's row k being row s K + k);
        // sharded-to-all ranks are separate matrices w_seg apart
        const int64_t ab = s * p.a_seg + (int64_t)m * p.lda;
        const int64_t r0 = p.stacked ? (int64_t)s * p.K : 0, wb = p.stacked ? 0 : s * p.w_seg;
        float part = 0.f;
#pragma unroll 8
        for (int k = 0; k < p.K; ++k) {
            const int64_t wi = wb + (WFRAG ? frag_offset(r0 + k, n, p.wsteps) : (r0 + k) * p.ldw + n);
            part = fmaf(ld<DT>(p.A, ab + k), ld<DT>(p.W, wi), part);
        }
        tot += part;
    }
    store_from_f32(p.out, p.out_dtype, idx, tot);
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

hipError_t launch_bwd_dx(const BwdDx& p, hipStream_t s) {
    const int64_t total = (p.reduce ? 1 : p.nseg) * (int64_t)p.M * p.N;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (p.dtype == SG_F32) {
        if (p.wfrag) return hipErrorInvalidValue;  // fp32 layers are stored row-major
        launch(bwd_dx_kernel<SG_F32, false>, grid, block, 0, s, p);
    } else if (p.dtype == SG_BF16) {
        if (p.wfrag) launch(bwd_dx_kernel<SG_BF16, true>, grid, block, 0, s, p);
        else launch(bwd_dx_kernel<SG_BF16, false>, grid, block, 0, s, p);
    } else {
        if (p.wfrag) launch(bwd_dx_kernel<SG_F16, true>, grid, block, 0, s, p);
        else launch(bwd_dx_kernel<SG_F16, false>, grid, block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const BwdDw& p, hipStream_t s) {
    const int64_t total = p.nseg * (int64_t)p.R * p.C;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (p.dtype == SG_F32) launch(bwd_dw_kernel<SG_F32>, grid, block, 0, s, p);
    else if (p.dtype == SG_BF16) launch(bwd_dw_kernel<SG_BF16>, grid, block, 0, s, p);
    else launch(bwd_dw_kernel<SG_F16>, grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace sg
