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
    hipLaunchKernelGGL(frag_transform_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)src, (uint16_t*)dst, rows, K, chunks, forward);
    return hipGetLastError();
}

}  // namespace sg
