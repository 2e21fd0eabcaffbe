// 4-bit affine weight-streaming GEMM for few tokens (M <= 32): the quantized
// all-to-sharded / sharded-to-all layers of "MLX 张量并行实战指南" sections 2.3
// and 6 (group_size 64, bits 4, mode affine), HBM-bound at 4.5 bits/weight.
//
// Per quantization group g of 64 inputs of weight row n:
//     sum_k w[n,k] x[t,k] = s[n,g] * sum_k q[n,k] x[t,k] + b[n,g] * sum_k x[t,k]
// The codes stay exact: a mask-and-or turns eight 4-bit codes into eight
// 16-bit numbers c + q with c = 128 (bf16) or 1024 (fp16), so the MFMA forms
// acc = sum (c + q) x = sum q x + c * xs per group, and the group adds
//     s * acc + (b - c * s) * xs,
// where xs = sum_k x[t,k] comes from one more MFMA against an all-ones
// operand.  With up to 8 tokens both terms are FMAs on the accumulators (xs in
// their layout).  Beyond 8 tokens (MB) the scale term stays one FMA per
// accumulator per group, while the bias term sum_g (b - c s)[n,g] xs[t,g] --
// itself a small product over the groups -- runs on the fp32 MFMA
// (v_mfma_f32_32x32x2f32) per pair of groups straight into the accumulators,
// which halves the vector-unit work of a group (the kernel is issue-bound on
// the vector unit, not on HBM).
//
// MFMA v_mfma_f32_32x32x16: the tokens are the row operand (32 token slots),
// 32 weight rows the column operand, so each lane owns one weight row and
// needs one (scale, bias) pair per group.  Lane (row j, half h) loads 16 bytes
// = codes of chunks 4h .. 4h+3 of the group; MFMA step u of the group uses
// chunk 4h + u, and the token fragment of step u holds the same chunk.  The
// layer stores codes, scales and biases fragment-major (q4_word_offset,
// q4_group_offset), so every one of these loads is a coalesced wave-wide read.
//
// Workgroup = NW waves on RB blocks of 32 rows (gate/up pairs for SwiGLU)
// across every rank; a wave takes one (rank, part) unit for all RB row blocks
// (one activation fragment serves RB of them; codes are read once, with
// non-temporal loads) and walks that rank's groups in runs of 4 (scales and
// biases arrive 8 bytes at a time), runs j, j + J, ...  Unit partials land in
// LDS slots and are summed in part order, then rank order -- the fused
// all_sum, as in the dense streaming kernel -- with no cross-workgroup traffic.
#include "q4_stream.h"

namespace sg {

// Shape choice: RB row blocks of 32 per wave (a gate/up pair for SwiGLU; more
// share each activation fragment), about 1500 waves on the chip, LDS slots
// within kMaxStreamLds.  Up to 8 tokens eight waves per workgroup; beyond,
// where the bias term runs on the MFMA and the kernel needs ~165 registers,
// four (measured on the gate|up layer of the decode MLP: 16 tokens 23.7 ->
// 21.7 us with the activations hoisted, 32 tokens 29.9 -> 28.2 us).  Four row
// blocks only up to 8 tokens (beyond that the token registers make them spill).
Q4Shape q4_shape(int M, int N, int nseg, int swiglu) {
    Q4Shape sh;
    sh.TB = (M + 7) / 8;
    const int64_t rows = swiglu ? 2 * (int64_t)N : N;
    auto lds_of = [&](int rb, int nw) {
        const int J = nseg >= nw ? 1 : nw / nseg;
        return (size_t)nseg * J * rb * 4 * sh.TB * 64 * sizeof(float);
    };
    sh.RB = swiglu ? 2 : 1;
    sh.NW = 8;
    for (int rb : {4, 2, 1}) {
        if (swiglu && rb < 2) break;
        if (rb == 4 && sh.TB > 1) continue;
        const int64_t wgs = (rows + rb * 32 - 1) / (rb * 32);
        const int nw = (sh.TB == 1 && lds_of(rb, 8) <= kMaxStreamLds) ? 8 : 4;
        if ((wgs * nw >= 1536 && lds_of(rb, nw) <= kMaxStreamLds) || rb == (swiglu ? 2 : 1)) {
            sh.RB = rb;
            sh.NW = nw;
            break;
        }
    }
    sh.lds = lds_of(sh.RB, sh.NW);
    return sh;
}

template <bool F16>
static hipError_t launch_f(const Problem& p, hipStream_t s, const Q4Shape& sh) {
    switch (sh.TB) {
    case 1: return launch_tb<1, F16>(p, s, sh);
    case 2: return launch_tb<2, F16>(p, s, sh);
    default: return launch_q4_wide<F16>(p, s, sh);
    }
}

bool q4s_takes(const Problem& p) {
    return !p.swiglu && p.M <= 32 && p.Kseg % 256 == 0 && q4s_shape(p.M, p.N, p.nseg, 0).lds <= kMaxStreamLds;
}

hipError_t launch_q4(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!p.qfrag) return hipErrorInvalidValue;  // the streaming kernel reads the fragment layout
    // Layers without the SwiGLU pairing (the down projection: few output rows,
    // many ranks) run on 16-row blocks (q4s.hip), which give twice the
    // workgroups; measured on the 4-bit MLP shapes, the gate|up layer is faster
    // on 32-row blocks and the down layer on 16-row blocks.
    if (q4s_takes(p)) return launch_q4s(p, s);
    if (p.xfrag) return hipErrorInvalidValue;  // fragment-major activations: the 16-row kernel only
    const Q4Shape sh = q4_shape(p.M, p.N, p.nseg, p.swiglu);
    return p.dtype == SG_F16 ? launch_f<true>(p, s, sh) : launch_f<false>(p, s, sh);
}

// Reorder the eight codes of every word: forward (standard -> kernel order,
// code k moves from nibble k to nibble q4_nibble_pos(k)) or back.
__global__ void q4_repack_kernel(uint32_t* w, int64_t n, int forward) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t a = w[i];
    uint32_t r = 0;
    for (int k = 0; k < 8; ++k) {
        const int src = forward ? k : q4_nibble_pos(k);
        const int dst = forward ? q4_nibble_pos(k) : k;
        r |= ((a >> (4 * src)) & 0xFu) << (4 * dst);
    }
    w[i] = r;
}

hipError_t q4_repack(uint32_t* w, int64_t n, int forward, hipStream_t s) {
    if (n == 0) return hipSuccess;
    launch(q4_repack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, w, n, forward);
    return hipGetLastError();
}

}  // namespace sg
