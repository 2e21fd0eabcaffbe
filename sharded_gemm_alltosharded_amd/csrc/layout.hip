// Layout transforms: row-major <-> fragment-major weights (one-time, at layer
// construction and shard copy-out; see frag_offset in internal.h), and SUMMA's
// (K, N) right operand into fragment-major transposed blocks (per call).
#include "internal.h"

namespace sg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one thread per 16-byte chunk (8 elements along k)
__global__ void frag_transform_kernel(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t K,
                                      int64_t chunks, int forward) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks) return;
    const int64_t per = rows * (K / 8);
    const int64_t mat = c / per, rem = c - mat * per;
    const int64_t row = rem / (K / 8), k = (rem - row * (K / 8)) * 8;
    const int64_t lin = mat * rows * K + row * K + k;
    const int64_t frg = mat * rows * K + frag_offset(row, k, K / 32);
    if (forward)
        *(u32x4*)(dst + frg) = *(const u32x4*)(src + lin);
    else
        *(u32x4*)(dst + lin) = *(const u32x4*)(src + frg);
}

hipError_t frag_transform(void* dst, const void* src, int P, int64_t rows, int64_t K, int forward, hipStream_t s) {
    const int64_t chunks = (int64_t)P * rows * (K / 8);
    if (chunks == 0) return hipSuccess;
    launch(frag_transform_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)src, (uint16_t*)dst, rows, K, chunks, forward);
    return hipGetLastError();
}

__global__ void q4_words_kernel(const uint32_t* src, uint32_t* dst, int64_t rows, int64_t words, int64_t total,
                                int forward) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t per = rows * words, mat = i / per, rem = i - mat * per;
    const int64_t row = rem / words, w = rem - row * words;
    const int64_t lin = mat * per + row * words + w;
    const int64_t frg = mat * per + q4_word_offset(row, w, words / 8);
    if (forward)
        dst[frg] = src[lin];
    else
        dst[lin] = src[frg];
}

__global__ void q4_groups_kernel(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t groups, int64_t total,
                                 int forward) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t per = rows * groups, mat = i / per, rem = i - mat * per;
    const int64_t row = rem / groups, g = rem - row * groups;
    const int64_t lin = mat * per + row * groups + g;
    const int64_t frg = mat * per + q4_group_offset(row, g, groups);
    if (forward)
        dst[frg] = src[lin];
    else
        dst[lin] = src[frg];
}

hipError_t q4_transform(uint32_t* dst_w, const uint32_t* src_w, uint16_t* dst_g, const uint16_t* src_g, int P,
                        int64_t rows, int64_t K, int forward, hipStream_t s) {
    if (dst_w) {
        const int64_t total = (int64_t)P * rows * (K / 8);
        if (total) launch(q4_words_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src_w, dst_w, rows,
                          K / 8, total, forward);
    }
    if (dst_g) {
        const int64_t total = (int64_t)P * rows * (K / 64);
        if (total) launch(q4_groups_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src_g, dst_g, rows,
                          K / 64, total, forward);
    }
    return hipGetLastError();
}

// SUMMA's A (K, N) row-major -> q fragment-major matrices B_t = A_t^T, where
// A_t holds rows [t bk, (t + 1) bk) of A: element (n, kk) of B_t goes to
// t N bk + frag_offset(n, kk, bk / 32).  The MFMA tile kernels then read the
// blocks exactly like the (out, in) weights of a linear layer.  One workgroup
// per 32 (k) x 64 (n) tile: 16-byte reads of 32 rows x 128 bytes into LDS, then
// each thread gathers the 8 k values of one fragment lane slot and writes them
// as 16 contiguous bytes.  Needs N % 16 == 0 and bk % 32 == 0.
__global__ __launch_bounds__(256) void nn_frag_kernel(const uint16_t* A, uint16_t* dst, int64_t N, int64_t bk) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[32][64 + 8];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 32;
    {
        const int r = tid >> 3, c = tid & 7;
        if (n0 + c * 8 < N) *(u32x4*)&tile[r][c * 8] = *(const u32x4*)(A + (k0 + r) * N + n0 + c * 8);
    }
    __syncthreads();
    const int b = tid >> 6, l = tid & 63;
    if (n0 + b * 16 >= N) return;
    const int n = b * 16 + (l & 15), kq = 8 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = tile[kq + 2 * i][n] | ((uint32_t)tile[kq + 2 * i + 1][n] << 16);
    const int64_t t = k0 / bk, kin = k0 - t * bk;
    const int64_t off = t * N * bk + (((n0 / 16 + b) * (bk / 32) + kin / 32) * 64 + l) * 8;
    *(u32x4*)(dst + off) = u32x4{w[0], w[1], w[2], w[3]};
}

hipError_t nn_to_frag(void* dst, const void* A, int64_t K, int64_t N, int q, hipStream_t s) {
    if (K == 0 || N == 0) return hipSuccess;
    if (q < 1 || K % q || (K / q) % 32 || N % 16) return hipErrorInvalidValue;
    // launched directly: a layout pass is never the kernel sg_time_next_launch times
    hipLaunchKernelGGL(nn_frag_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)(K / 32)), dim3(256), 0, s,
                       (const uint16_t*)A, (uint16_t*)dst, N, K / q);
    return hipGetLastError();
}

// P row-major (R, C) 16-bit matrices -> P row-major (C, Rp) transposes, the
// columns R .. Rp-1 of each zero-filled (a padded contraction dimension adds
// nothing).  One workgroup per 64 x 64 tile: 16-byte row reads into LDS, then
// each thread gathers 8 values of one output row and writes them as 16
// contiguous bytes.  Needs C % 8 == 0 and Rp % 8 == 0.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* src, uint16_t* dst, int64_t R, int64_t C,
                                                          int64_t Rp) {
    __shared__ uint16_t tile[64][64 + 2];
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
    const uint16_t* S = src + (int64_t)blockIdx.z * R * C;
    uint16_t* D = dst + (int64_t)blockIdx.z * C * Rp;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (tid >> 3) + 32 * i, c = (tid & 7) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r0 + r < R && c0 + c < C) v = *(const u32x4*)(S + (r0 + r) * C + c0 + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[r][c + 2 * e] = (uint16_t)(v[e] & 0xFFFFu);
            tile[r][c + 2 * e + 1] = (uint16_t)(v[e] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = (tid >> 3) + 32 * i, r = (tid & 7) * 8;
        if (c0 + c >= C || r0 + r >= Rp) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = tile[r + 2 * e][c] | ((uint32_t)tile[r + 2 * e + 1][c] << 16);
        *(u32x4*)(D + (c0 + c) * Rp + r0 + r) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

hipError_t transpose16(void* dst, const void* src, int P, int64_t R, int64_t C, int64_t Rp, hipStream_t s) {
    if (P == 0 || C == 0 || Rp == 0) return hipSuccess;
    if (C % 8 || Rp % 8 || Rp < R) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((Rp + 63) / 64), (unsigned)P),
                       dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst, R, C, Rp);
    return hipGetLastError();
}

// P row-major (R, C) 16-bit matrices -> one fragment-major matrix of P C rows
// and Rp k: element (p C + c, r) = src[p][r][c], zero for r >= R (the
// transposes stacked, as the MFMA kernels read a weight operand).  Same tile
// scheme as nn_frag_kernel.  Needs C % 16 == 0 and Rp % 32 == 0.
__global__ __launch_bounds__(256) void t_frag_kernel(const uint16_t* src, uint16_t* dst, int64_t R, int64_t C,
                                                     int64_t Rp) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[32][64 + 8];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 32;
    const int64_t mat = blockIdx.z;
    const uint16_t* S = src + mat * R * C;
    {
        const int r = tid >> 3, c = tid & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k0 + r < R && n0 + c * 8 < C) v = *(const u32x4*)(S + (k0 + r) * C + n0 + c * 8);
        *(u32x4*)&tile[r][c * 8] = v;
    }
    __syncthreads();
    const int b = tid >> 6, l = tid & 63;
    if (n0 + b * 16 >= C) return;
    const int n = b * 16 + (l & 15), kq = 8 * (l >> 4);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = tile[kq + 2 * i][n] | ((uint32_t)tile[kq + 2 * i + 1][n] << 16);
    const int64_t row = mat * C + n0 + b * 16;  // first row of this 16-row block in the stack
    *(u32x4*)(dst + frag_offset(row + (l & 15), k0 + kq, Rp / 32)) = u32x4{w[0], w[1], w[2], w[3]};
}

hipError_t t_frag(void* dst, const void* src, int P, int64_t R, int64_t C, int64_t Rp, hipStream_t s) {
    if (P == 0 || C == 0 || Rp == 0) return hipSuccess;
    if (C % 16 || Rp % 32 || Rp < R) return hipErrorInvalidValue;
    hipLaunchKernelGGL(t_frag_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)(Rp / 32), (unsigned)P), dim3(256), 0,
                       s, (const uint16_t*)src, (uint16_t*)dst, R, C, Rp);
    return hipGetLastError();
}

// MX FP8 layers: P stacked (rows, K) byte matrices of E4M3 codes <-> the
// fragment-major byte layout (mx_code_offset), and their (rows, K/32) E8M0
// scales <-> mx_scale_offset.  One thread per 8 codes / per scale.
__global__ void mx_codes_kernel(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t K, int64_t chunks,
                                int forward) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= chunks) return;
    const int64_t per = rows * (K / 8);
    const int64_t mat = c / per, rem = c - mat * per;
    const int64_t row = rem / (K / 8), k = (rem - row * (K / 8)) * 8;
    const int64_t lin = mat * rows * K + row * K + k;
    const int64_t frg = mat * rows * K + mx_code_offset(row, k, K / 32);
    if (forward)
        *(uint64_t*)(dst + frg) = *(const uint64_t*)(src + lin);
    else
        *(uint64_t*)(dst + lin) = *(const uint64_t*)(src + frg);
}

__global__ void mx_scales_kernel(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t steps, int64_t total,
                                 int forward) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t per = rows * steps, mat = i / per, rem = i - mat * per;
    const int64_t row = rem / steps, st = rem - row * steps;
    const int64_t lin = mat * per + row * steps + st;
    const int64_t frg = mat * per + mx_scale_offset(row, st, steps);
    if (forward)
        dst[frg] = src[lin];
    else
        dst[lin] = src[frg];
}

hipError_t mx_transform(uint8_t* dst_codes, const uint8_t* src_codes, uint8_t* dst_scales,
                        const uint8_t* src_scales, int P, int64_t rows, int64_t K, int forward, hipStream_t s) {
    if (rows % 16 || K % 128) return hipErrorInvalidValue;
    if (dst_codes) {
        const int64_t chunks = (int64_t)P * rows * (K / 8);
        if (chunks)
            launch(mx_codes_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, src_codes, dst_codes,
                   rows, K, chunks, forward);
    }
    if (dst_scales) {
        const int64_t total = (int64_t)P * rows * (K / 32);
        if (total)
            launch(mx_scales_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src_scales, dst_scales,
                   rows, K / 32, total, forward);
    }
    return hipGetLastError();
}

}  // namespace sg
