/*
 * CPU oracle for the sharded GEMM path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct fp64 loops.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library; the GPU
 * path never calls it and shares no code with it (its own bf16/fp16 decoders,
 * its own slicing, its own dequantisation).
 *
 * Sources (page title, then section):
 *  [MLX]   "MLX 张量并行（Tensor Parallelism）实战指南：用 AllToShardedLinear 与
 *          ShardedToAllLinear 实现 Llama 多设备推理"
 *  [HSYM]  "Sharded Matrices and How to Multiply Them 精华笔记" (How To Scale Your
 *          Model, part 3 notes)
 *  [SUMMA] "ColossalAI 2D 张量并行：基于 SUMMA 的二维模型切分原理与实现"
 *  [EAI]   "拆解EnergonAI的张量并行实现：Linear1D与词表并行的2个关键技巧"
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - weights are (out, in) row-major and a linear layer computes y = x W^T
 *    ([MLX] 2.1: local weight shape (output_dims // N, input_dims); 2.2:
 *    x @ weight.T);
 *  - splitting a dimension into N parts gives N equal contiguous parts, part r
 *    to rank r; with segments S the dimension is first cut into S segments
 *    and rank r takes its part of every segment, concatenated in segment
 *    order ([MLX] 3.2); divisibility of dim by S and of dim/S by N is
 *    required ([MLX] 2.1 and 6 state the N case);
 *  - all-to-sharded splits weight rows and the bias; sharded-to-all splits
 *    weight columns and adds the full bias once after the sum ([MLX] 2.2);
 *  - 4-bit affine: w = scale_g * q + bias_g per group of group_size
 *    consecutive input elements of one output row; eight 4-bit codes per
 *    uint32, element k in bits [4 (k mod 8), 4 (k mod 8) + 4) ([MLX] 2.3
 *    gives only group_size 64 / bits 4 / affine; the layout is this
 *    library's own).
 *
 * Status codes: 0 ok, 1 invalid argument, 3 not divisible.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_INVALID 1
#define OR_NOT_DIVISIBLE 3

/* dtype codes of stored inputs */
#define OR_F32 0
#define OR_BF16 1
#define OR_F16 2
#define OR_F64 3

/* ------------------------------------------------------------------ */
/* decoding of stored bit patterns                                     */
/* ------------------------------------------------------------------ */
static double dec_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int or_decode(const void* src, int dtype, int64_t n, double* dst) {
    if (n < 0 || (n > 0 && (!src || !dst))) return OR_INVALID;
    for (int64_t i = 0; i < n; ++i) {
        switch (dtype) {
        case OR_F32: dst[i] = (double)((const float*)src)[i]; break;
        case OR_BF16: dst[i] = dec_bf16(((const uint16_t*)src)[i]); break;
        case OR_F16: dst[i] = dec_f16(((const uint16_t*)src)[i]); break;
        case OR_F64: dst[i] = ((const double*)src)[i]; break;
        default: return OR_INVALID;
        }
    }
    return OR_OK;
}

/* Round an fp64 value to the nearest value of a narrower binary format with
 * `bits` significant bits and minimum normal exponent emin (value
 * 2^(emin-1) * 2 ... ), ties to even.  Used only for the stored activation
 * between the two sharded layers. */
static double round_sig(double x, int bits, int emin) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1 */
    if (e < emin) e = emin; /* subnormal range: fixed spacing */
    double q = nearbyint(ldexp(x, bits - e)); /* default mode: nearest even */
    return ldexp(q, e - bits);
}

double or_round(double x, int dtype) {
    switch (dtype) {
    case OR_F32: return round_sig(x, 24, -125);
    case OR_BF16: return round_sig(x, 8, -125);
    case OR_F16: return round_sig(x, 11, -13);
    default: return x;
    }
}

/* ------------------------------------------------------------------ */
/* O1: shard slicing ([MLX] 3.2)                                       */
/* ------------------------------------------------------------------ */
/* W: rows x cols elements of elem_bytes bytes, row-major.  axis 0 splits
 * rows, axis 1 splits columns.  Rank r's shard is written contiguous
 * (row-major) to out; it is bit-identical to the source bytes. */
int or_slice(const void* W, int64_t elem_bytes, int64_t rows, int64_t cols, int axis, int S,
             int P, int r, void* out) {
    if (!W || !out || elem_bytes <= 0 || rows < 0 || cols < 0 || S < 1 || P < 1 || r < 0 ||
        r >= P || (axis != 0 && axis != 1))
        return OR_INVALID;
    int64_t dim = axis == 0 ? rows : cols;
    if (dim % S) return OR_NOT_DIVISIBLE;
    int64_t seg = dim / S;
    if (seg % P) return OR_NOT_DIVISIBLE;
    int64_t part = seg / P;
    const char* src = (const char*)W;
    char* dst = (char*)out;
    if (axis == 0) {
        /* shard rows, in order: segment s, then rows r*part .. (r+1)*part-1 */
        int64_t o = 0;
        for (int s = 0; s < S; ++s)
            for (int64_t i = 0; i < part; ++i) {
                int64_t row = s * seg + r * part + i;
                memcpy(dst + o * cols * elem_bytes, src + row * cols * elem_bytes,
                       (size_t)(cols * elem_bytes));
                ++o;
            }
    } else {
        int64_t oc = S * part; /* shard column count */
        for (int64_t i = 0; i < rows; ++i) {
            int64_t c = 0;
            for (int s = 0; s < S; ++s)
                for (int64_t j = 0; j < part; ++j) {
                    int64_t col = s * seg + r * part + j;
                    memcpy(dst + (i * oc + c) * elem_bytes, src + (i * cols + col) * elem_bytes,
                           (size_t)elem_bytes);
                    ++c;
                }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O2: all-to-sharded linear ([MLX] 2.1; [HSYM] Case 1)                */
/* ------------------------------------------------------------------ */
/* X (B, in) replicated; W (out, in); bias (out) or NULL.  Shard r holds
 * W_r = slice(W, rows, S, P, r) and b_r likewise; Y_r = X W_r^T + b_r.
 * gather == 0: Y is (P, B, out/P) (the output stays sharded);
 * gather == 1: Y is (B, out) with shard r in columns [r*out/P, (r+1)*out/P)
 *              (what an all-gather of the shards in rank order gives, as
 *              for the vocabulary-parallel head of [EAI]). */
int or_col(const double* X, int64_t B, int64_t in, const double* W, int64_t out,
           const double* bias, int S, int P, int gather, double* Y) {
    if (!X || !W || !Y || B < 0 || in < 1 || out < 1 || S < 1 || P < 1) return OR_INVALID;
    if (out % S || (out / S) % P) return OR_NOT_DIVISIBLE;
    int64_t nloc = out / P;
    double* Wr = (double*)malloc(sizeof(double) * (size_t)(nloc * in));
    double* br = (double*)malloc(sizeof(double) * (size_t)nloc);
    if (!Wr || !br) { free(Wr); free(br); return OR_INVALID; }
    for (int r = 0; r < P; ++r) {
        or_slice(W, sizeof(double), out, in, 0, S, P, r, Wr);
        if (bias) or_slice(bias, sizeof(double), out, 1, 0, S, P, r, br);
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t i = 0; i < B; ++i)
            for (int64_t j = 0; j < nloc; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < in; ++k) acc += X[i * in + k] * Wr[j * in + k];
                if (bias) acc += br[j];
                int64_t dst = gather ? i * out + r * nloc + j : (r * B + i) * nloc + j;
                Y[dst] = acc;
            }
    }
    free(Wr);
    free(br);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O3: SwiGLU on sharded activations ([MLX] 5.2 / 5.3)                 */
/* ------------------------------------------------------------------ */
/* h = round(silu(g) * u), silu(z) = z / (1 + exp(-z)).  The product is an
 * elementwise op, so it keeps the sharding.  round_dtype: the dtype the
 * activation is stored in between the layers (OR_F64 = no rounding). */
int or_swiglu(const double* g, const double* u, int64_t n, int round_dtype, double* h) {
    if (n < 0 || (n > 0 && (!g || !u || !h))) return OR_INVALID;
    for (int64_t i = 0; i < n; ++i) {
        double s = g[i] / (1.0 + exp(-g[i]));
        h[i] = or_round(s * u[i], round_dtype);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O4: sharded-to-all linear ([MLX] 2.2; [HSYM] Case 3 with AllReduce)  */
/* ------------------------------------------------------------------ */
/* Xs (P, B, in/P): slice r is columns [r*in/P, (r+1)*in/P) of the full
 * activation.  W (out, in); shard r holds columns [r*in/P, (r+1)*in/P).
 * Z_r = Xs_r W_r^T (partials, optional output (P, B, out));
 * Y = sum_{r=0}^{P-1} Z_r, then + bias once. */
int or_row(const double* Xs, int64_t B, int64_t in, const double* W, int64_t out,
           const double* bias, int P, double* Y, double* Z) {
    if (!Xs || !W || !Y || B < 0 || in < 1 || out < 1 || P < 1) return OR_INVALID;
    if (in % P) return OR_NOT_DIVISIBLE;
    int64_t kloc = in / P;
    double* Wr = (double*)malloc(sizeof(double) * (size_t)(out * kloc));
    double* Zr = (double*)malloc(sizeof(double) * (size_t)(B * out + 1));
    if (!Wr || !Zr) { free(Wr); free(Zr); return OR_INVALID; }
    for (int64_t i = 0; i < B * out; ++i) Y[i] = 0.0;
    for (int r = 0; r < P; ++r) {
        or_slice(W, sizeof(double), out, in, 1, 1, P, r, Wr);
        const double* Xr = Xs + (int64_t)r * B * kloc;
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t i = 0; i < B; ++i)
            for (int64_t o = 0; o < out; ++o) {
                double acc = 0.0;
                for (int64_t k = 0; k < kloc; ++k) acc += Xr[i * kloc + k] * Wr[o * kloc + k];
                Zr[i * out + o] = acc;
            }
        for (int64_t i = 0; i < B * out; ++i) {
            Y[i] += Zr[i]; /* all_sum, rank order */
            if (Z) Z[(int64_t)r * B * out + i] = Zr[i];
        }
    }
    if (bias)
        for (int64_t i = 0; i < B; ++i)
            for (int64_t o = 0; o < out; ++o) Y[i * out + o] += bias[o];
    free(Wr);
    free(Zr);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O5: 4-bit affine dequantisation ([MLX] 2.3 / 6)                     */
/* ------------------------------------------------------------------ */
/* Wq (out, in/8) uint32; scales, biases (out, in/group_size) fp16 bits.
 * W[o, k] = s[o, k/gs] * q[o, k] + b[o, k/gs], exact in fp64. */
int or_deq4(const uint32_t* Wq, const uint16_t* scales, const uint16_t* biases, int64_t out,
            int64_t in, int group_size, double* W) {
    if (!Wq || !scales || !biases || !W || out < 0 || in < 0 || group_size < 1) return OR_INVALID;
    if (in % 8 || in % group_size) return OR_NOT_DIVISIBLE;
    int64_t ng = in / group_size;
    for (int64_t o = 0; o < out; ++o)
        for (int64_t k = 0; k < in; ++k) {
            uint32_t word = Wq[o * (in / 8) + k / 8];
            unsigned q = (word >> (4 * (k % 8))) & 0xFu;
            double s = dec_f16(scales[o * ng + k / group_size]);
            double b = dec_f16(biases[o * ng + k / group_size]);
            W[o * in + k] = s * (double)q + b;
        }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O5b: MX FP8 dequantisation ([MLX] 2.3: non-affine mode "mxfp8", and 4: */
/* such a layer has no biases).  Read as the OCP Microscaling format:      */
/* FP8 E4M3 elements, one E8M0 power-of-two scale per block of inputs.    */
/* ------------------------------------------------------------------ */
/* E4M3: sign, exponent e (4 bits, bias 7), mantissa m (3 bits); e = 0 is
 * subnormal (m 2^-9); e = 15 with m = 7 is NaN (no infinity). */
double or_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e ? ldexp(8.0 + m, e - 10) : ldexp((double)m, -9);
    return s ? -v : v;
}
/* E8M0: 2^(x - 127); 255 is NaN. */
double or_e8m0(uint8_t x) { return x == 255 ? NAN : ldexp(1.0, (int)x - 127); }

int or_deqmx8(const uint8_t* codes, const uint8_t* scales, int64_t out, int64_t in, int block, double* W) {
    if (!codes || !scales || !W || out < 0 || in < 0 || block < 1) return OR_INVALID;
    if (in % block) return OR_NOT_DIVISIBLE;
    for (int64_t o = 0; o < out; ++o)
        for (int64_t k = 0; k < in; ++k)
            W[o * in + k] = or_e8m0(scales[o * (in / block) + k / block]) * or_e4m3(codes[o * in + k]);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O6: SUMMA ([SUMMA] "SUMMA 算法", equations (1), (2) and their sum)   */
/* ------------------------------------------------------------------ */
/* Y = X A with X (M, K), A (K, N), both cut into q x q blocks.  For every
 * block (i, j): Y_ij = 0, then for t = 0 .. q-1: Y_ij += X_it A_tj. */
int or_summa(const double* X, const double* A, int64_t M, int64_t K, int64_t N, int q,
             double* Y) {
    if (!X || !A || !Y || M < 0 || K < 0 || N < 0 || q < 1) return OR_INVALID;
    if (M % q || K % q || N % q) return OR_NOT_DIVISIBLE;
    int64_t bm = M / q, bk = K / q, bn = N / q;
#pragma omp parallel for collapse(2) schedule(static)
    for (int i = 0; i < q; ++i)
        for (int j = 0; j < q; ++j) {
            for (int64_t a = 0; a < bm; ++a)
                for (int64_t b = 0; b < bn; ++b) Y[(i * bm + a) * N + j * bn + b] = 0.0;
            for (int t = 0; t < q; ++t) /* step t: local product of the broadcast blocks */
                for (int64_t a = 0; a < bm; ++a)
                    for (int64_t b = 0; b < bn; ++b) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < bk; ++c)
                            acc += X[(i * bm + a) * K + t * bk + c] * A[(t * bk + c) * N + j * bn + b];
                        Y[(i * bm + a) * N + j * bn + b] += acc;
                    }
        }
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* O7: the gated MLP chain ([MLX] 4 and 5.2)                           */
/* ------------------------------------------------------------------ */
/* gate and up are all-to-sharded (outputs stay sharded, (P, B, F/P)), the
 * elementwise product runs on the shards, down is sharded-to-all: one
 * reduction for the whole chain.  h is stored in round_dtype. */
int or_mlp(const double* X, int64_t B, int64_t D, int64_t F, const double* Wg,
           const double* Wu, const double* Wd, int P, int round_dtype, double* Y) {
    if (!X || !Wg || !Wu || !Wd || !Y || B < 0 || D < 1 || F < 1 || P < 1) return OR_INVALID;
    if (F % P) return OR_NOT_DIVISIBLE;
    size_t n = (size_t)(B * F);
    double* g = (double*)malloc(sizeof(double) * (n + 1));
    double* u = (double*)malloc(sizeof(double) * (n + 1));
    int rc = OR_INVALID;
    if (g && u) {
        rc = or_col(X, B, D, Wg, F, NULL, 1, P, 0, g);
        if (!rc) rc = or_col(X, B, D, Wu, F, NULL, 1, P, 0, u);
        if (!rc) rc = or_swiglu(g, u, (int64_t)n, round_dtype, g); /* h, (P, B, F/P) */
        if (!rc) rc = or_row(g, B, F, Wd, D, NULL, P, Y, NULL);
    }
    free(g);
    free(u);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Backward of the two sharded layers ([MLX] 2.1 with its sum_gradients */
/* wrapper, and 2.2): the vector-Jacobian products of O2 and O4.        */
/* ------------------------------------------------------------------ */
/* All-to-sharded: Y_r = X W_r^T with X shared by every rank, so the input
 * gradient is the all_sum over ranks of dY_r W_r (each rank's product formed
 * whole, then added in rank order r = 0 .. P-1, as or_row sums partials), and
 * rank r's weight gradient is dY_r^T X, laid out like slice(W, rows, S, P, r).
 *   X (B, in), W (out, in), dY (P, B, out/P); dx (B, in) and dW (P, out/P, in)
 *   may each be NULL. */
int or_col_bwd(const double* X, int64_t B, int64_t in, const double* W, int64_t out, const double* dY, int S,
               int P, double* dx, double* dW) {
    if (!W || !dY || B < 0 || in < 1 || out < 1 || S < 1 || P < 1 || (!dx && !dW) || (dW && !X))
        return OR_INVALID;
    if (out % S || (out / S) % P) return OR_NOT_DIVISIBLE;
    int64_t nloc = out / P;
    double* Wr = (double*)malloc(sizeof(double) * (size_t)(nloc * in));
    double* Zr = (double*)malloc(sizeof(double) * (size_t)(B * in + 1));
    if (!Wr || !Zr) { free(Wr); free(Zr); return OR_INVALID; }
    if (dx)
        for (int64_t i = 0; i < B * in; ++i) dx[i] = 0.0;
    for (int r = 0; r < P; ++r) {
        const double* G = dY + (int64_t)r * B * nloc;
        if (dx) {
            or_slice(W, sizeof(double), out, in, 0, S, P, r, Wr);
#pragma omp parallel for collapse(2) schedule(static)
            for (int64_t i = 0; i < B; ++i)
                for (int64_t k = 0; k < in; ++k) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < nloc; ++j) acc += G[i * nloc + j] * Wr[j * in + k];
                    Zr[i * in + k] = acc;
                }
            for (int64_t i = 0; i < B * in; ++i) dx[i] += Zr[i]; /* all_sum, rank order */
        }
        if (dW) {
            double* D = dW + (int64_t)r * nloc * in;
#pragma omp parallel for collapse(2) schedule(static)
            for (int64_t j = 0; j < nloc; ++j)
                for (int64_t k = 0; k < in; ++k) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < B; ++i) acc += G[i * nloc + j] * X[i * in + k];
                    D[j * in + k] = acc;
                }
        }
    }
    free(Wr);
    free(Zr);
    return OR_OK;
}

/* Sharded-to-all: Y = sum_r Xs_r W_r^T (+ b); the gradient of the summed
 * output reaches every rank whole, so rank r's input gradient dY W_r stays
 * sharded (no reduction) and its weight gradient is dY^T Xs_r, laid out like
 * slice(W, columns, 1, P, r).
 *   Xs (P, B, in/P), W (out, in), dY (B, out); dXs (P, B, in/P) and
 *   dW (P, out, in/P) may each be NULL. */
int or_row_bwd(const double* Xs, int64_t B, int64_t in, const double* W, int64_t out, const double* dY, int P,
               double* dXs, double* dW) {
    if (!W || !dY || B < 0 || in < 1 || out < 1 || P < 1 || (!dXs && !dW) || (dW && !Xs)) return OR_INVALID;
    if (in % P) return OR_NOT_DIVISIBLE;
    int64_t kloc = in / P;
    double* Wr = (double*)malloc(sizeof(double) * (size_t)(out * kloc));
    if (!Wr) return OR_INVALID;
    for (int r = 0; r < P; ++r) {
        if (dXs) {
            or_slice(W, sizeof(double), out, in, 1, 1, P, r, Wr);
            double* D = dXs + (int64_t)r * B * kloc;
#pragma omp parallel for collapse(2) schedule(static)
            for (int64_t i = 0; i < B; ++i)
                for (int64_t k = 0; k < kloc; ++k) {
                    double acc = 0.0;
                    for (int64_t o = 0; o < out; ++o) acc += dY[i * out + o] * Wr[o * kloc + k];
                    D[i * kloc + k] = acc;
                }
        }
        if (dW) {
            const double* Xr = Xs + (int64_t)r * B * kloc;
            double* D = dW + (int64_t)r * out * kloc;
#pragma omp parallel for collapse(2) schedule(static)
            for (int64_t o = 0; o < out; ++o)
                for (int64_t k = 0; k < kloc; ++k) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < B; ++i) acc += dY[i * out + o] * Xr[i * kloc + k];
                    D[o * kloc + k] = acc;
                }
        }
    }
    free(Wr);
    return OR_OK;
}

/* SUMMA backward ([SUMMA] Matmul_ABT_2D): for Y = X A, dX = dY A^T with the
 * shared dimension N cut into the q step blocks; for every output, the
 * block products are added in step order t = 0 .. q-1:
 *   dX[i][k] = sum_t sum_{c in block t} dY[i][c] A[k][c].
 *   dY (M, N), A (K, N), dX (M, K). */
int or_summa_abt(const double* dY, const double* A, int64_t M, int64_t K, int64_t N, int q, double* dX) {
    if (!dY || !A || !dX || M < 0 || K < 0 || N < 0 || q < 1) return OR_INVALID;
    if (N % q) return OR_NOT_DIVISIBLE;
    int64_t bn = N / q;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) {
            double sum = 0.0;
            for (int t = 0; t < q; ++t) {
                double acc = 0.0;
                for (int64_t c = t * bn; c < (t + 1) * bn; ++c) acc += dY[i * N + c] * A[k * N + c];
                sum += acc;
            }
            dX[i * K + k] = sum;
        }
    return OR_OK;
}

/* SUMMA backward ([SUMMA] Matmul_ATB_2D): dA = X^T dY with the token
 * dimension M cut into the q step blocks, added in step order:
 *   dA[k][j] = sum_t sum_{m in block t} X[m][k] dY[m][j].
 *   X (M, K), dY (M, N), dA (K, N). */
int or_summa_atb(const double* X, const double* dY, int64_t M, int64_t K, int64_t N, int q, double* dA) {
    if (!X || !dY || !dA || M < 0 || K < 0 || N < 0 || q < 1) return OR_INVALID;
    if (M % q) return OR_NOT_DIVISIBLE;
    int64_t bm = M / q;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            double sum = 0.0;
            for (int t = 0; t < q; ++t) {
                double acc = 0.0;
                for (int64_t m = t * bm; m < (t + 1) * bm; ++m) acc += X[m * K + k] * dY[m * N + j];
                sum += acc;
            }
            dA[k * N + j] = sum;
        }
    return OR_OK;
}

/* Number of threads the parallel loops use (1 without OpenMP). */
int or_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
