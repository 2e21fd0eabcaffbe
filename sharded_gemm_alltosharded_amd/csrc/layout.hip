// Weight layout transforms (one-time, at layer construction and shard
// copy-out): row-major <-> fragment-major (see frag_offset in internal.h).
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

}  // namespace sg
