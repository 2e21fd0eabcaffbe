// Generic sharded GEMM: one thread per output element, fp32 accumulation.
//
// Serves the fp32 layers (the plumbing case of the two-device worked
// example), shapes whose rows are not 16-byte aligned, and 4-bit and MX FP8
// layers with more tokens than the streaming kernels take.  Structure follows the
// method literally: each rank's partial product is formed over its own input
// slice, and the partials are summed in rank order before the bias is added
// once ("MLX 张量并行实战指南" section 2.2).
#include "internal.h"

namespace sg {

__device__ __forceinline__ float weight_at(const Problem& p, int s, int64_t row, int k) {
    if (p.wq) {
        const int64_t wi = p.qfrag ? q4_word_offset(row, k >> 3, p.ldg) : row * p.ldq + (k >> 3);
        uint32_t word = p.wq[s * p.q_seg + wi];
        float q = (float)((word >> (4 * q4_nibble_pos(k & 7))) & 0xFu);
        int64_t g = s * p.g_seg + (p.qfrag ? q4_group_offset(row, k >> 6, p.ldg) : row * p.ldg + (k >> 6));
        return fmaf(f16_to_f32(p.qs[g]), q, f16_to_f32(p.qb[g]));
    }
    if (p.fp8) {
        const int64_t ci = p.wfrag ? mx_code_offset(row, k, p.wsteps) : row * p.ldw + k;
        const int64_t si = p.wfrag ? mx_scale_offset(row, k >> 5, p.wsteps) : row * (p.ldw >> 5) + (k >> 5);
        return e8m0_to_f32(p.ms[s * p.ms_seg + si]) * e4m3_to_f32(((const uint8_t*)p.W)[s * p.w_seg + ci]);
    }
    if (p.nn) return load_as_f32(p.W, p.dtype, s * p.w_seg + (int64_t)k * p.ldw + row);
    if (p.wfrag) return load_as_f32(p.W, p.dtype, s * p.w_seg + frag_offset(row, k, p.wsteps));
    return load_as_f32(p.W, p.dtype, s * p.w_seg + row * p.ldw + k);
}

__global__ __launch_bounds__(256) void generic_kernel(Problem p) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)p.M * p.N) return;
    const int m = (int)(idx / p.N);
    const int64_t n = idx - (int64_t)m * p.N;
    float tot[2];
    const int halves = p.swiglu ? 2 : 1;
    for (int h = 0; h < halves; ++h) {
        const int64_t row = weight_row(p, n, h);
        float total = 0.f;
        for (int s = 0; s < p.nseg; ++s) {
            const int64_t abase = s * p.a_seg + (int64_t)m * p.lda;
            float part = 0.f;  // this rank's partial
            for (int k = 0; k < p.Kseg; ++k)
                part = fmaf(load_as_f32(p.A, p.dtype, abase + k), weight_at(p, s, row, k), part);
            total += part;  // all_sum in rank order
        }
        tot[h] = total;
    }
    float v = p.swiglu ? silu_f32(tot[0]) * tot[1] : tot[0];
    if (p.bias) v += load_as_f32(p.bias, p.dtype, n);
    const int64_t o = out_index(p, m, n);
    if (p.accumulate && p.out_dtype == SG_F32) v += ((const float*)p.out)[o];
    store_from_f32(p.out, p.out_dtype, o, v);
}

hipError_t launch_generic(const Problem& p, hipStream_t s) {
    int64_t total = (int64_t)p.M * p.N;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    launch(generic_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace sg
