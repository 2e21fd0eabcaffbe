// Internal declarations shared by the host entry points (api.cpp) and the
// gfx950 kernels.  Nothing here is part of the public C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/shardgemm.h"

namespace sg {

// ---------------------------------------------------------------------------
// one GEMM-shaped problem:  C[m][n] = sum_s sum_k A_s[m][k] * W_s[n][k]
//
//  * A_s: activations of segment s (a rank's input slice), row-major
//    M x Kseg:  A + s * a_seg + m * lda + k.
//  * W_s: weights.  NT: row-major N_w x Kseg  (W + s * w_seg + n * ldw + k);
//    NN: row-major Kseg x N  (W + s * w_seg + k * ldw + n), used by SUMMA.
//  * segments are the ranks of a sharded-to-all layer (nseg = P); the sum over
//    s is the all_sum.  nseg = 1 otherwise.
//  * swiglu: W holds P rank blocks of [gate rows (floc); up rows (floc)];
//    logical output column j (0 .. N-1, N = P * floc) pairs gate row and up row
//    of rank j / floc, and the kernel stores silu(g) * u.
// ---------------------------------------------------------------------------
enum OutMap { OUT_ROWMAJOR = 0, OUT_SHARDED = 1, OUT_FRAG = 2, OUT_FRAG_Q4 = 3 };

struct Problem {
    const void* A;
    int64_t lda, a_seg;
    const void* W;
    int64_t ldw, w_seg;
    // 4-bit weights (when quantized): packed (rows, ldq u32), scales / biases (rows, ldg)
    const uint32_t* wq;
    const uint16_t* qs;
    const uint16_t* qb;
    int64_t ldq, ldg, q_seg, g_seg;  // per-segment offsets in u32 / group units
    int M, N, Kseg, nseg;
    int dtype;      // sg_dtype of A and W
    int nn;         // W is K x N (SUMMA)
    int wfrag;      // W is stored fragment-major (frag_offset), Kseg % 32 == 0
    int64_t wsteps; // fragment-major W: 32-wide k steps per stored row (frag_offset's nsteps)
    // MX FP8 weights (fp8): W holds E4M3 codes, one byte each, in the dense
    // layouts above; ms their E8M0 scales, one per 32 inputs of a row
    // (fragment-major: mx_scale_offset; row-major: row * ldw / 32 + k / 32)
    int fp8;
    const uint8_t* ms;
    int64_t ms_seg;
    int qfrag;      // 4-bit codes / scales / biases stored fragment-major (q4 offsets)
    int xfrag;      // A is a fragment-major sharded activation in the reading kernel's order
                    // (act_frag_offset for skinny.hip, act_frag_offset_q4 for q4s.hip)
    int swiglu;     // fused gate/up pairs
    int64_t floc;   // rank width of the swiglu output (rows per gate block)
    // epilogue
    void* out;
    int out_dtype;
    int out_map;    // OutMap
    int64_t ldo;    // OUT_ROWMAJOR row stride
    int64_t nloc;   // OUT_SHARDED / OUT_FRAG rank width: column n -> rank n / nloc
    const void* bias;  // per output column, dtype `dtype`; may be null
    int accumulate; // fp32 output only: out += result
    // cross-segment reduction through a workspace (split by segment): the
    // product kernel stores one partial slab per group of segments, a second
    // kernel adds them in order
    int split;
    float* ws;
};

// Fragment-major layout of a row-major (rows, K) weight, rows % 16 == 0 and
// K % 32 == 0: the 16 x 32 block (row block rb, k step st) is 512 contiguous
// elements ordered (rb, st) with st fastest; inside it lane l of a wave owns
// elements l * 8 .. l * 8 + 7 = W[16 rb + (l & 15)][32 st + 8 (l >> 4) + 0..7],
// exactly its operand fragment of a v_mfma_f32_16x16x32.  A wave streaming one
// k step of a row block then reads 1 KB contiguous.
__host__ __device__ inline int64_t frag_offset(int64_t row, int64_t k, int64_t nsteps) {
    return (((row >> 4) * nsteps + (k >> 5)) * 64 + (row & 15) + 16 * ((k >> 3) & 3)) * 8 + (k & 7);
}

// Fragment-major sharded activation (the h a fused MLP keeps between its two
// layers): rank r's (act_rows(M), nloc) block at r * act_rows(M) * nloc, laid
// out like a fragment-major weight with tokens as rows, so that the 16 tokens x
// 32 inputs a streaming wave feeds one MFMA are one contiguous 1 KB.  Token
// rows past M are padding (never stored, their results never kept).
__host__ __device__ inline int64_t act_rows(int64_t M) { return (M + 15) / 16 * 16; }
__host__ __device__ inline int64_t act_frag_offset(int64_t m, int64_t k, int64_t nsteps) {
    return frag_offset(m, k, nsteps);
}
// The same for the 16-row 4-bit kernel's k order: inside a group of 64 inputs
// the lane with chunk slot c feeds k = 16 c + 8 u + e to its MFMA step u, so
// input k is stored at k' = 32 u + 8 c + e of the group (two 1 KB fragments
// per 16 tokens and group, one per step).
__host__ __device__ inline int64_t act_frag_offset_q4(int64_t m, int64_t k, int64_t nsteps) {
    const int64_t kp = (k & ~(int64_t)63) | (((k >> 3) & 1) << 5) | (((k >> 4) & 3) << 3) | (k & 7);
    return frag_offset(m, kp, nsteps);
}

// E4M3 codes of a fragment-major MX FP8 layer: for each 16-row block and pair
// of 32-wide k steps, 1 KB in which lane l (row l & 15, chunk c = l >> 4) owns
// 16 bytes: its 8 codes of the even step, then its 8 codes of the odd step
// (k = 64 sp + 32 h + 8 c + e).  One 16-byte load per lane feeds two MFMAs.
__host__ __device__ inline int64_t mx_code_offset(int64_t row, int64_t k, int64_t nsteps) {
    return (((row >> 4) * (nsteps >> 1) + (k >> 6)) * 64 + (row & 15) + 16 * ((k >> 3) & 3)) * 16 +
           8 * ((k >> 5) & 1) + (k & 7);
}

// E8M0 scales of a fragment-major MX FP8 layer: for each 16-row block and run
// of 4 k steps, 16 rows x 4 bytes (a row's scales of the 4 steps adjacent).
__host__ __device__ inline int64_t mx_scale_offset(int64_t row, int64_t st, int64_t nsteps) {
    return (((row >> 4) * (nsteps >> 2) + (st >> 2)) * 16 + (row & 15)) * 4 + (st & 3);
}

// Events armed by sg_time_next_launch for the calling thread: the next kernel
// the library launches records them at its own start and end.
struct ArmedEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
ArmedEvents& armed_events();

#ifdef __HIPCC__
template <typename K, typename... Args>
inline void launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    ArmedEvents& ev = armed_events();
    if (ev.start || ev.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0, args...);
        ev = ArmedEvents{};
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    }
}
#endif

// Fragment-major layout of 4-bit layers, rows % 32 == 0 and G = K / 64 groups
// with G % 4 == 0.  Codes: the 32 rows x 8 words of (row block rb, group g)
// are 256 contiguous words; lane l of a wave owns words l * 4 .. l * 4 + 3 =
// words 4 (l >> 5) .. 4 (l >> 5) + 3 of group g of row 32 rb + (l & 31), its
// operand of one group in v_mfma_f32_32x32x16.  Scales and biases: the 32 rows
// x 4 groups of (rb, run g / 4) are 128 contiguous halves, row-major.
__host__ __device__ inline int64_t q4_word_offset(int64_t row, int64_t word, int64_t groups) {
    const int64_t g = word >> 3, wi = word & 7;
    return (((row >> 5) * groups + g) * 64 + (row & 31) + 32 * (wi >> 2)) * 4 + (wi & 3);
}
__host__ __device__ inline int64_t q4_group_offset(int64_t row, int64_t g, int64_t groups) {
    return (((row >> 5) * (groups >> 2) + (g >> 2)) * 32 + (row & 31)) * 4 + (g & 3);
}

// launchers (return hipError_t of the launch)
hipError_t launch_generic(const Problem& p, hipStream_t s);
hipError_t launch_tile(const Problem& p, hipStream_t s, int variant);
hipError_t launch_skinny(const Problem& p, hipStream_t s);
hipError_t launch_q4(const Problem& p, hipStream_t s);
hipError_t launch_q4s(const Problem& p, hipStream_t s);  // 16-row blocks, M <= 32, Kseg % 256 == 0
hipError_t launch_q4_tile(const Problem& p, hipStream_t s);  // 4-bit, many tokens (q4tile.hip)
bool q4_tile_fits(const Problem& p);
int q4_tile_count(int M, int N);  // output tiles of the 4-bit tile kernel (no SwiGLU): q4_tile_rows(M) x 128
int q4_tile_rows(int M);           // its token tile: 64 up to 64 tokens, else 128
// P stacked (rows, K) 16-bit matrices: row-major -> fragment-major (forward) or back
hipError_t frag_transform(void* dst, const void* src, int P, int64_t rows, int64_t K, int forward, hipStream_t s);
// SUMMA's A (K, N) -> q fragment-major blocks of A_t^T (N, K / q); N % 16 == 0, (K / q) % 32 == 0
hipError_t nn_to_frag(void* dst, const void* A, int64_t K, int64_t N, int q, hipStream_t s);
// P row-major (R, C) 16-bit matrices -> P row-major (C, Rp) transposes, columns
// R .. Rp-1 zero; C % 8 == 0, Rp % 8 == 0
hipError_t transpose16(void* dst, const void* src, int P, int64_t R, int64_t C, int64_t Rp, hipStream_t s);
// P row-major (R, C) 16-bit matrices -> their transposes stacked as one
// fragment-major (P C, Rp) matrix, k >= R zero; C % 16 == 0, Rp % 32 == 0
hipError_t t_frag(void* dst, const void* src, int P, int64_t R, int64_t C, int64_t Rp, hipStream_t s);
// MX FP8: P stacked (rows, K) code bytes and (rows, K/32) scales <-> fragment-major
// (either pair of pointers may be null); rows % 16 == 0, K % 128 == 0
hipError_t mx_transform(uint8_t* dst_codes, const uint8_t* src_codes, uint8_t* dst_scales,
                        const uint8_t* src_scales, int P, int64_t rows, int64_t K, int forward, hipStream_t s);
hipError_t q4_repack(uint32_t* w, int64_t n, int forward, hipStream_t s);
// P stacked 4-bit matrices (rows, K): codes (rows, K/8 words) and scales or
// biases (rows, K/64), row-major <-> fragment-major
hipError_t q4_transform(uint32_t* dst_w, const uint32_t* src_w, uint16_t* dst_g, const uint16_t* src_g, int P,
                        int64_t rows, int64_t K, int forward, hipStream_t s);

// Workspace of the split-by-segment reduction: `floats` partial values (one
// slab of `tiles` output tiles per group of segments), written before they
// are read by every call, so it needs no clearing.
struct SplitLayout {
    size_t floats;
    size_t tiles;
};
SplitLayout tile_split_layout(int M, int N, int nseg, int variant);
// compute units of the current device (queried once)
int device_cus();
// groups of consecutive segments the 256 x 256 tile kernel splits a
// sharded-to-all product into: the fewest that divide nseg and give every
// compute unit a workgroup
int tile_pp_groups(int M, int N, int nseg);
// the fewest groups of consecutive segments (dividing nseg) that give every
// compute unit a workgroup when each output tile runs once per group
int split_groups(int tiles, int nseg);
// second kernel of a split tile product: adds the groups' partial tiles in
// order and stores them; layout 0: ping-pong 256 x 256 tiles, 1: register-
// staged 128 x 128, 2: register-staged 256 x 256, 3, 4 and 5: few-token
// 64 x 128, 128 x 128 and 256 x 128
hipError_t launch_split_reduce(const Problem& p, int tiles_m, int tiles_n, int groups, int layout, hipStream_t s);
// few-token tile kernel (tile_dma.hip): up to 256 tokens, 64-, 128- or
// 256-token tiles (tile_nw_tm) of 128 weight rows; MX FP8 weights (fp8): any
// token count, 64- or 128-token tiles
int tile_nw_tm(int M, bool fp8 = false);
int tile_nw_count(int M, int N, int swiglu, bool fp8 = false);
bool tile_nw_fits(const Problem& p);
hipError_t launch_tile_nw(const Problem& p, hipStream_t s);

// launch shapes of the streaming kernels (dynamic LDS bytes included)
struct SkinnyShape {
    int MT, RB, NW;
    size_t lds;
};
struct Q4Shape {
    int TB, RB, NW;
    size_t lds;
};
SkinnyShape skinny_shape(int M, int N, int nseg, int swiglu);
Q4Shape q4_shape(int M, int N, int nseg, int swiglu);
SkinnyShape q4s_shape(int M, int N, int nseg, int swiglu);
bool q4s_takes(const Problem& p);  // launch_q4 runs p on the 16-row kernel (q4s.hip)

// Backward products (backward.hip).  BwdDx: out[m][n] (reduce: summed over the
// nseg ranks in order) or out[s][m][n] = sum_k A_s[m][k] W_s[k][n], W_s rank
// s's stored (rows, cols) shard read as its (K, N) operand.  BwdDw:
// out[s][o][i] = sum_m G_s[m][o] X_s[m][i].
struct BwdDx {
    const void* A;
    int64_t lda, a_seg;
    const void* W;
    int64_t ldw, w_seg, wsteps;
    int wfrag, dtype, M, N, K, nseg, reduce;
    int stacked;  // ranks are stacked rows of one matrix (all-to-sharded), else w_seg apart
    void* out;
    int out_dtype;
};
struct BwdDw {
    const void* G;
    int64_t ldg, g_seg;
    const void* X;
    int64_t ldx, x_seg;
    int dtype, M, R, C, nseg;
    void* out;
    int out_dtype;
};
// Weight gradient with few tokens (backward.hip): out[o][i] = sum_b G(b, o) X(b, i)
// with G(b, o) = G[(o / gl) g_seg + b ldg + o % gl], X likewise; out (O, I)
// row-major, or (I / nloc, O, nloc) when nloc > 0.  Bp = B rounded up to 16,
// at most kDwSmallMaxTokens; gl, xl, ldg, ldx, g_seg, x_seg multiples of 8.
constexpr int kDwSmallMaxTokens = 128;
struct BwdDwSmall {
    const void* G;
    int64_t gl, g_seg, ldg;
    const void* X;
    int64_t xl, x_seg, ldx;
    int dtype, O, I, B, Bp;
    void* out;
    int out_dtype;
    int64_t nloc;
};
hipError_t launch_dw_small(const BwdDwSmall& p, hipStream_t s);
hipError_t launch_bwd_dx(const BwdDx& p, hipStream_t s);
hipError_t launch_bwd_dw(const BwdDw& p, hipStream_t s);
constexpr size_t kMaxStreamLds = 64 * 1024;
int tile_count(int M, int N, int variant);
inline size_t split_workspace_bytes(SplitLayout s) { return s.floats * sizeof(float); }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
#ifdef __HIPCC__
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 v = (_Float16)f;  // round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &v, 2);
    return h;
}
__device__ __forceinline__ float load_as_f32(const void* p, int dtype, int64_t i) {
    if (dtype == SG_F32) return ((const float*)p)[i];
    uint16_t b = ((const uint16_t*)p)[i];
    return dtype == SG_BF16 ? bf16_to_f32(b) : f16_to_f32(b);
}
__device__ __forceinline__ void store_from_f32(void* p, int dtype, int64_t i, float v) {
    if (dtype == SG_F32)
        ((float*)p)[i] = v;
    else
        ((uint16_t*)p)[i] = dtype == SG_BF16 ? f32_to_bf16(v) : f32_to_f16(v);
}
// A 4-bit layer stores each uint32 with its eight codes reordered so that
// code k (0..7) of the word sits at nibble q4_nibble_pos(k): nibbles e and
// e + 4 then hold codes 2e and 2e + 1, and one mask-and-or turns a word into
// four 16-bit pairs in natural k order (see q4.hip).
__host__ __device__ __forceinline__ int q4_nibble_pos(int k) { return (k >> 1) | ((k & 1) << 2); }

// FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
// subnormal, 0x7F / 0xFF NaN) and E8M0 (2^(x - 127), 255 NaN), exact in fp32
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return __builtin_nanf("");
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return s ? -v : v;
}
__device__ __forceinline__ float e8m0_to_f32(uint32_t x) {
    if (x == 255u) return __builtin_nanf("");
    return x ? __uint_as_float(x << 23) : __uint_as_float(0x00400000u);  // 2^-127 is subnormal
}

// eight E4M3 codes (two words) times the E8M0 scale 2^(x - 127) -> eight bf16
// (four words, k order) with v_cvt_scalef32_pk_bf16_fp8; exact: an E4M3 value
// has 4 significant bits and the scale is a power of two
__device__ __forceinline__ uint32_t __attribute__((ext_vector_type(4)))
mx8_to_bf16(uint32_t __attribute__((ext_vector_type(2))) c, uint32_t scale_byte) {
    const float sc = scale_byte ? __uint_as_float(scale_byte << 23) : __uint_as_float(0x00400000u);
    uint32_t __attribute__((ext_vector_type(4))) r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], sc, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], sc, true));
    return r;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.  Used
// where register arrays are indexed, so indices stay static even when a loop
// body is too large for the unroller (a dynamic index would move the whole
// array to scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// output address of logical element (m, n)
__device__ __forceinline__ int64_t out_index(const Problem& p, int m, int64_t n) {
    if (p.out_map == OUT_FRAG || p.out_map == OUT_FRAG_Q4) {
        const int64_t r = n / p.nloc, c = n - r * p.nloc;
        return r * act_rows(p.M) * p.nloc +
               (p.out_map == OUT_FRAG ? act_frag_offset(m, c, p.nloc / 32) : act_frag_offset_q4(m, c, p.nloc / 32));
    }
    if (p.out_map == OUT_SHARDED) {
        int64_t r = n / p.nloc;
        return (r * p.M + m) * p.nloc + (n - r * p.nloc);
    }
    return (int64_t)m * p.ldo + n;
}

// weight row of logical column n (swiglu: `up` selects the up row of the pair)
__device__ __forceinline__ int64_t weight_row(const Problem& p, int64_t n, int up) {
    if (!p.swiglu) return n;
    int64_t r = n / p.floc;
    return r * 2 * p.floc + (up ? p.floc : 0) + (n - r * p.floc);
}

// Map a workgroup id to a tile id so that each of the 8 XCDs (which receive
// workgroups round-robin) works on one contiguous range of tiles: tiles that
// share operand panels then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
    const int nx = 8;
    int x = wg % nx, slot = wg / nx;
    int q = total / nx, rem = total % nx;
    return x < rem ? x * (q + 1) + slot : rem * (q + 1) + (x - rem) * q + slot;
}
#endif

}  // namespace sg
