/*
 * shardgemm -- the sharded GEMMs of 1-D tensor parallelism and SUMMA's 2-D
 * block accumulation, with every shard of a layer held on one MI355X GPU.
 *
 * Sources (page title, then the section the entry point follows):
 *  [MLX]   "MLX 张量并行（Tensor Parallelism）实战指南：用 AllToShardedLinear 与
 *          ShardedToAllLinear 实现 Llama 多设备推理"
 *  [HSYM]  "Sharded Matrices and How to Multiply Them 精华笔记"
 *  [SUMMA] "ColossalAI 2D 张量并行：基于 SUMMA 的二维模型切分原理与实现"
 *  [EAI]   "拆解EnergonAI的张量并行实现：Linear1D与词表并行的2个关键技巧"
 *
 * Conventions shared by every entry point
 *  - Weights use the (out, in) row-major layout and a linear layer computes
 *    y = x W^T ([MLX] 2.1 and 2.2).  Activations are row-major (tokens, features).
 *  - P shards are emulated on the current HIP device: the shard copies of a
 *    layer live in one allocation, shard r at offset r.
 *  - Pointers named x, y, X, A, Y, workspace are device pointers owned by the
 *    caller.  Layer weights passed to the constructors may be host or device
 *    memory; they are read, never modified ([MLX] 3.1: the source layer is
 *    only read).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; results are ready after the stream synchronises.
 *  - Validation happens on the host before any device work and returns a
 *    status; sg_last_error() then describes the failure (thread-local).
 *    A device fault surfaces at the next synchronisation of the stream.
 *  - B == 0 tokens is a successful no-op.
 *  - Results are bitwise identical run to run (fixed reduction order).
 *  - Accumulation is fp32; the output dtype is the caller's choice.
 */
#ifndef SHARDGEMM_H
#define SHARDGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SG_OK = 0,
    SG_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad dtype or epilogue */
    SG_ERR_BAD_MODE = 2,      /* sharding is neither all-to-sharded nor sharded-to-all */
    SG_ERR_NOT_DIVISIBLE = 3, /* a dimension does not split evenly */
    SG_ERR_UNSUPPORTED = 4,   /* valid request this library does not implement */
    SG_ERR_WORKSPACE = 5,     /* workspace missing or too small */
    SG_ERR_OOM = 6,           /* device allocation failed */
    SG_ERR_HIP = 7            /* a HIP runtime call failed */
} sg_status;

typedef enum { SG_ALL_TO_SHARDED = 0, SG_SHARDED_TO_ALL = 1 } sg_mode;
typedef enum { SG_F32 = 0, SG_BF16 = 1, SG_F16 = 2 } sg_dtype;
typedef enum { SG_EPI_NONE = 0, SG_EPI_SWIGLU = 1 } sg_epilogue;
/* activation layouts across ranks ([HSYM] Cases 1-3) */
typedef enum { SG_IN_FULL = 0, SG_IN_SHARDED = 1 } sg_in_layout;   /* (B, in) | (P, B, in/P) */
typedef enum { SG_OUT_FULL = 0, SG_OUT_SHARDED = 1 } sg_out_layout; /* (B, n) | (P, B, n/P) */

typedef struct sg_layer sg_layer; /* opaque, owned by the library */

/* Shard a dense linear layer over P ranks ([MLX] 3.1 shard_linear; slicing
 * rule of [MLX] 3.2).
 *   weight   (out_dims, in_dims) of `dtype`, row-major.
 *   bias     (out_dims) of `dtype`, or NULL.
 *   mode     SG_ALL_TO_SHARDED: rank r keeps out_dims/P weight rows and the
 *            matching bias entries ([MLX] 2.1).  SG_SHARDED_TO_ALL: rank r keeps
 *            in_dims/P weight columns; the whole bias is added once after the
 *            cross-rank sum ([MLX] 2.2).  Anything else: SG_ERR_BAD_MODE.
 *   segments the split dimension is first cut into `segments` equal segments
 *            (a fused weight such as [Wq; Wk; Wv]); rank r keeps its part of
 *            every segment, in segment order ([MLX] 3.2).
 *   P        number of ranks (P >= 1; P == 1 is the unsharded layer).
 * Errors: SG_ERR_NOT_DIVISIBLE when the split dimension is not divisible by
 * segments, or dim/segments not by P ([MLX] 2.1 and 6: a layer whose output
 * width does not split evenly over the devices is rejected; the message
 * names the size and the device count).  *out receives the new layer. */
sg_status sg_shard_linear(const void* weight, sg_dtype dtype, int64_t out_dims, int64_t in_dims,
                          const void* bias, int mode, int segments, int P, void* stream,
                          sg_layer** out);

/* Shard a 4-bit affine quantized linear layer ([MLX] 2.3, 6: group_size 64,
 * bits 4, mode affine).  Stored format: w[o,k] = scale[o,g] * q[o,k] + bias[o,g]
 * with g = k / group_size; eight 4-bit codes per uint32 along k, element k in
 * bits [4 (k mod 8), 4 (k mod 8) + 4).
 *   wq       (out_dims, in_dims/8) uint32.
 *   scales   (out_dims, in_dims/group_size) fp16 bit patterns.
 *   qbiases  (out_dims, in_dims/group_size) fp16 bit patterns.
 *   act      activation dtype of the layer (SG_BF16 or SG_F16).
 *   bias     (out_dims) of `act`, or NULL (the layer bias, as for sg_shard_linear).
 * Only group_size 64 and bits 4 are implemented (else SG_ERR_UNSUPPORTED).
 * Up to 32 tokens run on the streaming kernels, more on a matrix-core tile
 * kernel (both when out_dims % 32 == 0 and the rank's in_dims % 256 == 0, the
 * fragment-major code layout); other shapes take the generic kernel.
 * Sharded-to-all needs (in_dims/segments/P) % group_size == 0 so that no
 * quantization group straddles two ranks (SG_ERR_NOT_DIVISIBLE). */
sg_status sg_shard_quantized_linear(const uint32_t* wq, const uint16_t* scales,
                                    const uint16_t* qbiases, int64_t out_dims, int64_t in_dims,
                                    int group_size, int bits, sg_dtype act, const void* bias,
                                    int mode, int segments, int P, void* stream, sg_layer** out);

/* Shard an MX FP8 layer ([MLX] 2.3: the non-affine quantization mode
 * "mxfp8"; [MLX] 4: such a layer has no quantization biases).  Format read as
 * the OCP Microscaling one: w[o,k] = 2^(scales[o, k/32] - 127) * e4m3(codes[o,k]),
 * codes FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, 0x7F /
 * 0xFF NaN), scales E8M0 (255 NaN), one per block of 32 inputs of a row.
 *   codes    (out_dims, in_dims) uint8.   scales (out_dims, in_dims/32) uint8.
 *   act      activation dtype: SG_BF16 only (else SG_ERR_UNSUPPORTED).
 *   bias     (out_dims) bf16, or NULL (the layer bias, as for sg_shard_linear).
 * SG_ERR_NOT_DIVISIBLE when in_dims % 32, or for sharded-to-all when a scale
 * block would straddle two ranks ((in_dims/segments/P) % 32).  Up to 16 tokens
 * run on the streaming kernel (codes converted to bf16 in registers) when the
 * shards tile into 16-row blocks and in/P (sharded-to-all) or in is a multiple
 * of 128; more tokens on the matrix-core tile kernels (codes converted to bf16
 * after the LDS or as they are staged; 17 to 32 tokens stay on the streaming
 * kernel for shards that the few-token tiles do not take); other calls take
 * the generic kernel.  sg_layer_copy_shard returns
 * codes (what 0) and scales (what 2); sg_layer_info reports quantized = 2. */
sg_status sg_shard_mxfp8_linear(const uint8_t* codes, const uint8_t* scales, int64_t out_dims,
                                int64_t in_dims, sg_dtype act, const void* bias, int mode, int segments,
                                int P, void* stream, sg_layer** out);

/* All-to-sharded forward ([MLX] 2.1; [HSYM] Case 1: no communication).
 *   x        (B, in_dims) of the layer's dtype, replicated to every rank.
 *   y        gather == 0: (P, B, n_out/P), rank r's output at offset r
 *            (the output stays sharded); gather == 1: (B, n_out) with rank r
 *            in columns [r n_out/P, (r+1) n_out/P) -- the rank-order all-gather
 *            of the vocabulary-parallel head ([EAI], LM head).
 *   epilogue SG_EPI_NONE: n_out = out_dims, y = x W_r^T (+ b_r).
 *            SG_EPI_SWIGLU: the layer must be all-to-sharded with segments == 2
 *            holding [W_gate; W_up]; n_out = out_dims/2 and
 *            y_r = silu(x Wg_r^T) * (x Wu_r^T), silu(z) = z / (1 + e^-z), computed
 *            in fp32 and rounded once ([MLX] 5.2-5.3: the elementwise product
 *            keeps the sharding).  Bias is not allowed with SWIGLU.
 *   y_dtype  SG_F32, SG_BF16 or SG_F16. */
sg_status sg_all_to_sharded(const sg_layer* layer, const void* x, int64_t B, void* y, int gather,
                            int epilogue, sg_dtype y_dtype, void* stream);

/* All-to-sharded forward with explicit activation layouts ([HSYM] Cases 1 and 2).
 *   in_layout  SG_IN_FULL: x (B, in_dims), replicated to every rank (Case 1).
 *              SG_IN_SHARDED: x (P, B, in_dims/P), slice r holding columns
 *              [r in/P, (r+1) in/P) of the activation; every rank all-gathers it
 *              before its matmul (Case 2), which here is the K loop walking the P
 *              slices in order.  SG_ERR_UNSUPPORTED for fragment-stored dense
 *              weights when (in_dims/P) % 32 != 0, for 4-bit layers when
 *              (in_dims/P) is not a multiple of 256 (fragment-stored codes) or
 *              64 (row-major codes), and for MX FP8 layers when it is not a
 *              multiple of 128 (fragment-stored codes) or 32 (row-major codes);
 *              SG_ERR_NOT_DIVISIBLE when P does not divide in_dims.
 *   out_layout SG_OUT_SHARDED: y (P, B, n_out/P) (gather = 0 of sg_all_to_sharded);
 *              SG_OUT_FULL: y (B, n_out), the rank-order all-gather (gather = 1).
 * Everything else as sg_all_to_sharded. */
sg_status sg_all_to_sharded_ex(const sg_layer* layer, const void* x, int in_layout, int64_t B, void* y,
                               int out_layout, int epilogue, sg_dtype y_dtype, void* stream);

/* Sharded-to-all forward ([MLX] 2.2; [HSYM] Case 3 with AllReduce).
 *   x_partial (P, B, in_dims/P) of the layer's dtype; slice r is rank r's
 *            input (columns r of the full activation under the layer's
 *            segments rule).
 *   y        (B, out_dims) of y_dtype: sum over r = 0..P-1 of
 *            x_partial[r] W_r^T, then + bias once.
 *   workspace device scratch of at least sg_sharded_to_all_workspace(layer, B)
 *            bytes, 16-byte aligned (NULL allowed when that is 0); no
 *            initial contents are needed, and the same workspace serves later
 *            calls of any shape.  Calls that share a workspace must not run
 *            concurrently. */
sg_status sg_sharded_to_all(const sg_layer* layer, const void* x_partial, int64_t B, void* y,
                            sg_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream);

/* Sharded-to-all forward with an explicit output layout ([HSYM] Case 3).
 *   out_layout SG_OUT_FULL: y (B, out_dims), the all-reduce (= sg_sharded_to_all).
 *              SG_OUT_SHARDED: y (P, B, out_dims/P), the reduce-scatter: slice r
 *              holds columns [r out/P, (r+1) out/P) of the same rank-order sum
 *              (+ bias once); SG_ERR_NOT_DIVISIBLE when P does not divide out_dims.
 * Everything else, the workspace included, as sg_sharded_to_all. */
sg_status sg_sharded_to_all_ex(const sg_layer* layer, const void* x_partial, int64_t B, void* y,
                               int out_layout, sg_dtype y_dtype, void* workspace, size_t ws_bytes,
                               void* stream);

/* Gated MLP forward, the chain of [MLX] 5.2-5.3: h_r = silu(x W_gate,r^T) *
 * (x W_up,r^T) on every rank (all-to-sharded with the SwiGLU epilogue), then
 * y = sum over r = 0..P-1 of h_r W_down,r^T (+ the down bias once), with the
 * sharded h kept in the workspace instead of a caller array.  Results are
 * bitwise those of sg_all_to_sharded(gate_up, ..., SG_EPI_SWIGLU, act dtype)
 * followed by sg_sharded_to_all(down, ...).
 *   gate_up  all-to-sharded layer, segments = 2 ([W_gate; W_up]), no bias.
 *   down     sharded-to-all layer over the same P, in_dims = gate_up's
 *            out_dims / 2, the same activation dtype.
 *   x        (B, in_dims) of that dtype; y (B, out_dims of down) of y_dtype.
 *   workspace device memory of at least sg_mlp_workspace(...) bytes, 16-byte
 *            aligned, no initial contents needed: the down layer's
 *            sg_sharded_to_all workspace first, then h (when both layers
 *            run on a streaming kernel and B >= 8, stored fragment-major in
 *            the down kernel's operand order so that it reads each 16-token
 *            operand fragment as one contiguous 1 KB).  The same workspace serves later calls of any B
 *            it is large enough for; calls sharing it must not run concurrently.
 * Errors: SG_ERR_INVALID_ARG for layers that do not form such a pair (the
 * message says which rule fails), SG_ERR_WORKSPACE for a missing, small or
 * misaligned workspace; B = 0 is a no-op. */
sg_status sg_mlp(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, void* y,
                 sg_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace sg_mlp needs for B tokens (0 for layers that do not form
 * a gate|up, down pair or B <= 0). */
size_t sg_mlp_workspace(const sg_layer* gate_up, const sg_layer* down, int64_t B);

/* sg_mlp for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and bitwise the same results as sg_mlp, with the workspace taken
 * from a fixed scratch array of SG_MLP_STATIC_SCRATCH_BYTES (16 MiB) that the
 * library holds on every device it runs on until the process ends.  The
 * caller passes x and y as for sg_mlp; nothing is allocated or freed.
 * Errors: as sg_mlp, and SG_ERR_WORKSPACE when sg_mlp_workspace(gate_up,
 * down, B) exceeds the scratch (on 4096 x 14336 decode-MLP layers over 8
 * ranks the scratch holds every token count up to 64, bf16, MX FP8 and 4-bit
 * layers alike: beyond, the down layer's rank split needs more).
 * All calls on one device share its scratch, so calls that overlap on one
 * GPU (other streams or threads) race: the caller serialises them. */
#define SG_MLP_STATIC_SCRATCH_BYTES (16u << 20)
sg_status sg_mlp_static(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, void* y,
                        sg_dtype y_dtype, void* stream);

/* Backward of an all-to-sharded layer: the vector-Jacobian product of [MLX]
 * 2.1 with its sum_gradients wrapper.  The input x is shared by every rank,
 * so its gradient is the all_sum of the rank gradients, summed here on chip in
 * rank order:
 *   dx (B, in_dims) of dx_dtype = sum over r = 0..P-1 of dy[r] W_r;
 *   dw (P, out_dims/P, in_dims) of dw_dtype, dw[r] = dy[r]^T x, laid out like
 *      rank r's shard (the rows sg_layer_copy_shard returns, segments rule).
 *   x  (B, in_dims) of the layer's dtype (needed for dw only; may be NULL
 *      otherwise); dy (P, B, out_dims/P) of the layer's dtype, the layout of
 *      the forward's sharded output.
 *   workspace device scratch of at least sg_layer_backward_workspace(layer, B)
 *      bytes, 16-byte aligned, or NULL.  dw runs on the matrix cores: up to
 *      128 tokens reading dy and x in place (no workspace), beyond that over
 *      x and dy transposed into the workspace (tokens padded to a multiple of
 *      32), or on the vector units when no workspace is given.  No
 *      initialisation needed; calls that share a workspace must not overlap.
 *      SG_ERR_WORKSPACE when a needed workspace is given too small or
 *      misaligned.
 * dx runs on the forward kernels over a transposed copy of the rank shards
 * that the layer builds on the first backward call that reads it (16-bit
 * layers whose out_dims/P is a multiple of 32 and in_dims of 16; the same
 * bytes as the weights again, held until sg_layer_free; that first call
 * allocates and synchronises the stream).  Backward calls on one layer must not
 * run concurrently with its first one.
 * dx or dw may be NULL (not both).  Dense layers only (SG_ERR_UNSUPPORTED for
 * 4-bit and MX FP8 layers); no bias gradient.  fp32 accumulation; the rank sum
 * is deterministic.  B = 0 is a no-op. */
sg_status sg_all_to_sharded_backward(const sg_layer* layer, const void* x, const void* dy, int64_t B, void* dx,
                                     sg_dtype dx_dtype, void* dw, sg_dtype dw_dtype, void* workspace,
                                     size_t ws_bytes, void* stream);

/* Backward of a sharded-to-all layer ([MLX] 2.2): every rank receives the
 * full gradient dy (B, out_dims) of the summed output, so
 *   dx_partial (P, B, in_dims/P) of dx_dtype, slice r = dy W_r (stays sharded,
 *      no reduction);
 *   dw (P, out_dims, in_dims/P) of dw_dtype, dw[r] = dy^T x_partial[r].
 *   x_partial (P, B, in_dims/P) of the layer's dtype (for dw only).
 * The transposed shard copy needs out_dims % 32 == 0 and (in_dims/P) % 16 == 0.
 * Everything else, the workspace included, as sg_all_to_sharded_backward. */
sg_status sg_sharded_to_all_backward(const sg_layer* layer, const void* x_partial, const void* dy, int64_t B,
                                     void* dx_partial, sg_dtype dx_dtype, void* dw, sg_dtype dw_dtype,
                                     void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace the matrix-core weight gradient of either backward needs
 * for B tokens ((out_dims + in_dims) x B rounded up to 32, 16-bit); 0 when it
 * needs none (at most 128 tokens), when the layer's gradients run on the
 * vector units only (fp32, quantized, or shapes whose transposes do not
 * tile), or on bad input. */
size_t sg_layer_backward_workspace(const sg_layer* layer, int64_t B);

/* SUMMA backward ([SUMMA] Matmul_ABT_2D and Matmul_ATB_2D, the gradients of
 * Y = X A): with the inner dimension of each product cut into the q SUMMA step
 * blocks, summed in step order t = 0..q-1,
 *   dX (M, K) fp32 = dY A^T   (dX_ik = sum_t dY_it A_kt^T),
 *   dA (K, N) fp32 = X^T dY   (dA_kj = sum_t X_tk^T dY_tj).
 *   X (M, K), A (K, N), dY (M, N): row-major, of dtype.  dX or dA may be NULL
 *   (not both); each output is overwritten.
 *   workspace device scratch of at least sg_summa_backward_workspace(...)
 *   bytes, 16-byte aligned, or NULL: with it dA runs on the matrix cores over
 *   X^T and the transposed step blocks of dY written into it; without it on
 *   the vector units.  dX always runs on the matrix cores (16-bit dtypes).
 * Errors as sg_summa_matmul (q must divide M, K and N); SG_ERR_WORKSPACE for a
 * workspace below the size the query gives. */
sg_status sg_summa_backward(const void* X, const void* A, const void* dY, sg_dtype dtype, int64_t M, int64_t K,
                            int64_t N, int q, float* dX, float* dA, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace sg_summa_backward's matrix-core dA needs ((K + N) M
 * 16-bit elements): 0 unless dtype is 16-bit, (M/q) % 32 == 0, N % 16 == 0 and
 * K % 8 == 0. */
size_t sg_summa_backward_workspace(sg_dtype dtype, int64_t M, int64_t K, int64_t N, int q);

/* Bytes of workspace sg_sharded_to_all needs for B tokens (0 on bad input, and
 * when the call runs without one).  Non-zero when the output alone gives too
 * few tiles to fill the chip (dense 16-bit and MX FP8 layers beyond 16 tokens,
 * 4-bit layers beyond 32): groups of ranks are then workgroups of their own, their
 * partial tiles stored in the workspace and summed in rank order by a second
 * kernel. */
size_t sg_sharded_to_all_workspace(const sg_layer* layer, int64_t B);

/* SUMMA on a q x q grid ([SUMMA], SUMMA section, equations (1), (2)).
 *   X (M, K) and A (K, N) row-major of `dtype` (SG_BF16 or SG_F16); Y (M, N)
 *   fp32.  Both operands are cut into q x q blocks; for t = 0 .. q-1 every
 *   block performs Y_ij += X_it A_tj.
 *   accumulate 0: Y = X A; 1: Y += X A.
 *   fused      0: q launches, step t adds its block products into Y in place
 *              (the step structure of the derivation); 1: one launch that keeps
 *              each block's accumulator in registers across the q steps.
 *   workspace  device scratch of at least sg_summa_workspace(dtype, K, N, q)
 *              bytes, or NULL.  With it, each call first writes A_t^T for every
 *              t into the workspace in the fragment-major layout the matrix-core
 *              kernels read (as for a linear layer's weights); without it they
 *              read A in place, more slowly.  Contents need no initialisation;
 *              calls that share a workspace must not run concurrently.
 * Errors: SG_ERR_NOT_DIVISIBLE when q does not divide M, K and N or q < 1
 * (P = q x q processors); SG_ERR_WORKSPACE when workspace is not NULL and
 * ws_bytes is below the required size. */
sg_status sg_summa_matmul(const void* X, const void* A, sg_dtype dtype, int64_t M, int64_t K,
                          int64_t N, int q, float* Y, int accumulate, int fused, void* workspace,
                          size_t ws_bytes, void* stream);

/* Bytes of workspace sg_summa_matmul can use for these sizes: K N element
 * sizes for SG_BF16 / SG_F16 when N % 16 == 0 and (K / q) % 32 == 0, else 0
 * (the call then reads A in place whatever workspace it is given). */
size_t sg_summa_workspace(sg_dtype dtype, int64_t K, int64_t N, int q);

/* Layer description (any output pointer may be NULL); quantized: 0 dense,
 * 1 4-bit affine, 2 MX FP8. */
sg_status sg_layer_info(const sg_layer* layer, int64_t* out_dims, int64_t* in_dims, int* mode,
                        int* segments, int* P, sg_dtype* dtype, int* quantized);

/* Copy rank r's stored shard of one layer tensor into dst (device or host).
 *   what 0: weight (dense: (rows_r, cols_r) of dtype; quantized: packed uint32)
 *        1: bias (all-to-sharded: out_dims/P entries; sharded-to-all: the full bias)
 *        2: quantization scales, 3: quantization biases.
 * Synchronous with respect to `stream`; dst_bytes must be at least the size. */
sg_status sg_layer_copy_shard(const sg_layer* layer, int r, int what, void* dst, size_t dst_bytes,
                              void* stream);

/* Release a layer and its device memory (NULL is ignored). */
void sg_layer_free(sg_layer* layer);

/* Profiling: arm two hipEvent_t (created with timing enabled; either may be
 * NULL) for the next kernel this thread launches through the library, which
 * records start_event when that kernel begins and stop_event when it ends
 * (hipExtLaunchKernel), so hipEventElapsedTime gives its execution time
 * without launch overhead.  One-shot: disarmed by that launch.  For entry
 * points that launch several kernels, the first one is timed. */
sg_status sg_time_next_launch(void* start_event, void* stop_event);

/* Message describing the last failure on this thread ("" if none). */
const char* sg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SHARDGEMM_H */
