// C-ABI entry points: validation, layer objects, shard slicing and kernel
// dispatch.  Every check runs on the host before any HIP call, so argument
// errors never touch the device.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "internal.h"

struct sg_layer {
    int mode, segments, P, quantized;
    sg_dtype dtype;  // weight dtype (dense) or activation dtype (4-bit)
    int64_t out_dims, in_dims;
    int64_t rows_r, cols_r;  // one rank's weight shape in elements
    void* w;                 // dense: P x rows_r x cols_r; 4-bit: P x rows_r x cols_r/8 words
    uint16_t* qs;            // 4-bit scales: P x rows_r x cols_r/64
    uint16_t* qb;            // 4-bit biases
    void* bias;              // all-to-sharded: P x rows_r (rank order); sharded-to-all: out_dims
    int wfrag;               // dense weights stored fragment-major (sg::frag_offset)
    int qfrag;               // 4-bit codes / scales / biases fragment-major (sg::q4_*_offset)
    int mx;                  // MX FP8 layer: w holds E4M3 code bytes (dense layouts, wfrag), ms its scales
    uint8_t* ms;             // MX FP8 E8M0 scales: P x rows_r x cols_r/32 (sg::mx_scale_offset when wfrag)
    int device;
    // dense 16-bit layers: the rank shards transposed, fragment-major (built by
    // the first backward call that reads them): all-to-sharded, P matrices
    // W_r^T (cols_r, rows_r); sharded-to-all, the stack of W_r^T, (in, out)
    void* wt;
    std::mutex wt_mu;
};

namespace sg {
ArmedEvents& armed_events() {
    static thread_local ArmedEvents ev;
    return ev;
}
}  // namespace sg

namespace {

thread_local std::string g_err;

sg_status fail(sg_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

sg_status hip_fail(hipError_t e, const char* what) {
    return fail(e == hipErrorOutOfMemory ? SG_ERR_OOM : SG_ERR_HIP, "%s: %s", what,
                hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                        \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

size_t dtype_size(int dt) { return dt == SG_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == SG_F32 || dt == SG_BF16 || dt == SG_F16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Rank r's part of an axis cut into S segments and P parts per segment:
// offsets s * seg + r * part for s = 0..S-1, each `part` long.
sg_status check_split(int64_t dim, int S, int P, const char* what) {
    if (dim % S)
        return fail(SG_ERR_NOT_DIVISIBLE, "Cannot split the %s of size %lld into %d segments.", what,
                    (long long)dim, S);
    if ((dim / S) % P)
        return fail(SG_ERR_NOT_DIVISIBLE, "Cannot shard the %s of size %lld across %d devices.", what,
                    (long long)dim, P);
    return SG_OK;
}

// Copy rank shards of a row-major (rows, cols) array with element size esz.
// axis 0: shard r = rows of every segment, stacked (P, rows/P, cols).
// axis 1: shard r = columns of every segment, stacked (P, rows, cols/P).
sg_status copy_shards(void* dst, const void* src, int64_t rows, int64_t cols, size_t esz, int axis,
                      int S, int P, hipStream_t st) {
    const char* s8 = (const char*)src;
    char* d8 = (char*)dst;
    if (axis == 0) {
        const int64_t seg = rows / S, part = seg / P;
        for (int r = 0; r < P; ++r)
            for (int s = 0; s < S; ++s) {
                const int64_t srow = s * seg + (int64_t)r * part;
                const int64_t drow = (int64_t)r * S * part + s * part;
                HIP_TRY(hipMemcpyAsync(d8 + drow * cols * esz, s8 + srow * cols * esz,
                                       (size_t)(part * cols) * esz, hipMemcpyDefault, st),
                        "shard copy");
            }
    } else {
        const int64_t seg = cols / S, part = seg / P, cr = S * part;
        for (int r = 0; r < P; ++r)
            for (int s = 0; s < S; ++s) {
                const int64_t scol = s * seg + (int64_t)r * part;
                HIP_TRY(hipMemcpy2DAsync(d8 + ((int64_t)r * rows * cr + s * part) * esz, cr * esz,
                                         s8 + scol * esz, cols * esz, part * esz, rows,
                                         hipMemcpyDefault, st),
                        "shard copy");
            }
    }
    return SG_OK;
}

void free_layer(sg_layer* l) {
    if (!l) return;
    // kernels queued on any stream may still read the shards
    (void)hipDeviceSynchronize();
    if (l->w) (void)hipFree(l->w);
    if (l->qs) (void)hipFree(l->qs);
    if (l->qb) (void)hipFree(l->qb);
    if (l->ms) (void)hipFree(l->ms);
    if (l->bias) (void)hipFree(l->bias);
    if (l->wt) (void)hipFree(l->wt);
    delete l;
}

sg_status common_checks(int mode, int segments, int P, int64_t out_dims, int64_t in_dims, sg_layer** out) {
    if (!out) return fail(SG_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (mode != SG_ALL_TO_SHARDED && mode != SG_SHARDED_TO_ALL)
        return fail(SG_ERR_BAD_MODE,
                    "Sharding type %d not supported, choose one of 'all-to-sharded' or 'sharded-to-all'",
                    mode);
    if (segments < 1 || P < 1) return fail(SG_ERR_INVALID_ARG, "segments and P must be >= 1");
    if (out_dims < 1 || in_dims < 1) return fail(SG_ERR_INVALID_ARG, "layer dimensions must be >= 1");
    if (out_dims > INT32_MAX || in_dims > INT32_MAX)
        return fail(SG_ERR_UNSUPPORTED, "layer dimensions above 2^31 are not supported");
    if (mode == SG_ALL_TO_SHARDED) return check_split(out_dims, segments, P, "output");
    return check_split(in_dims, segments, P, "input");
}

// ---------------------------------------------------------------------------
// kernel choice
// ---------------------------------------------------------------------------
enum Kind { K_GENERIC, K_TILE0, K_TILE1, K_SKINNY, K_Q4, K_Q4TILE, K_NW };

int num_cus() { return sg::device_cus(); }

// dense operands: the MFMA paths need 16-byte rows
bool mfma_ok(const sg_layer* l, const void* x) {
    return l->dtype != SG_F32 && l->cols_r % 8 == 0 && aligned16(x) && aligned16(l->w);
}

// the few-token tile kernel: 17 to 256 tokens (MX FP8 layers: any count above
// 16), 32-wide k tiles, weights and activations addressable through 32-bit
// offsets.  From 17 tokens the streaming kernels need a second token tile,
// and the few-token tiles (64 tokens) win on the decode-MLP layer shapes:
// separate calls at 17-32 tokens, dense gate|up 47-48 -> 45 us, down 28-41 ->
// 27-28 us; MX FP8 gate|up 35-36 -> 32 us, down 24-32 -> 25 us.  The tile
// count (a 32-bit grid dimension) stays far below 2^31.
bool nw_ok(const sg_layer* l, int64_t B) {
    return B > 16 && (B <= 256 || l->mx) && l->cols_r % 32 == 0 &&
           (double)l->P * l->rows_r * l->cols_r * 2 < 2.0e9 && (double)B * l->P * l->cols_r * 2 < 2.0e9 &&
           (double)(B / 64 + 1) * (double)(l->out_dims / 64 + 1) < 1.0e9;
}
// ... and at 17 to 32 tokens only while one wave of workgroups covers the
// layer's tiles: the vocabulary head (393 tiles of 64 tokens on 256 CUs) ran
// 2% slower on them than on the streaming kernel, whose 16-row blocks balance
// across the CUs
bool nw_fills(const sg_layer* l, int64_t B, int swiglu) {
    if (B > 32) return true;
    const int n = (int)(swiglu ? l->out_dims / 2 : l->out_dims);
    return sg::tile_nw_count((int)B, n, swiglu, l->mx) <= num_cus();
}

// the streaming kernels keep one LDS slot per (rank, part): bounded ranks only
// nseg: K segments of the call (ranks of a sharded-to-all layer, or the input
// shards of an all-to-sharded call whose input arrives sharded)
bool skinny_fits(const sg_layer* l, int64_t B, int swiglu, int nseg) {
    const int n = (int)(swiglu ? l->out_dims / 2 : l->out_dims);
    return sg::skinny_shape((int)B, n, nseg, swiglu).lds <= sg::kMaxStreamLds;
}
bool q4_fits(const sg_layer* l, int64_t B, int swiglu) {
    const int n = (int)(swiglu ? l->out_dims / 2 : l->out_dims);
    const int nseg = l->mode == SG_SHARDED_TO_ALL ? l->P : 1;
    return sg::q4_shape((int)B, n, nseg, swiglu).lds <= sg::kMaxStreamLds;
}

// MX FP8 layers: the streaming kernel for few tokens when the codes are
// fragment-major; more tokens on the tile kernels (codes converted to bf16 in
// the loader), inputs with 16-byte rows; else the generic kernel
Kind choose_mx(const sg_layer* l, int64_t B, const void* x, int swiglu, int nseg) {
    // from 17 tokens the few-token tiles with the FP8 conversion after the
    // LDS, at every token count (decode MLP shapes at 64 tokens: gate|up 155 ->
    // 35 us, down 77 -> 26 us against the 128 x 128 tile kernel with the FP8
    // loader; at 512 tokens 329 -> 194 and 160 -> 85 us; at 4096 tokens 2221
    // -> 1305 and 1079 -> 603 us); the tile kernel keeps the layers whose codes
    // do not come in whole 16-row blocks of 128-wide k tiles
    const bool blocks16 = (swiglu ? (l->rows_r / 2) % 16 : l->rows_r % 16) == 0;
    if (l->wfrag && l->cols_r % 128 == 0 && blocks16 && aligned16(x) && nw_ok(l, B) && nw_fills(l, B, swiglu))
        return K_NW;
    const bool ok = B <= 32 && l->wfrag && (l->cols_r / 32) % 4 == 0 && aligned16(x) && aligned16(l->w);
    if (ok && skinny_fits(l, B, swiglu, nseg)) return K_SKINNY;
    if (B > 32 && aligned16(x) && l->cols_r % 8 == 0) return K_TILE1;
    return K_GENERIC;
}

Kind choose(const sg_layer* l, int64_t B, const void* x, int swiglu = 0, int nseg = 1) {
    if (l->mx) return choose_mx(l, B, x, swiglu, nseg);
    if (l->quantized) {
        if (!l->qfrag || !aligned16(x)) return K_GENERIC;
        // few tokens: the streaming kernels; more: the 4-bit tile kernel
        return (B <= 32 && nseg == 1 && q4_fits(l, B, swiglu)) ? K_Q4 : K_Q4TILE;
    }
    if (!mfma_ok(l, x)) return K_GENERIC;
    // up to 256 tokens the few-token tiles (decode-MLP gate|up at 64 tokens:
    // 98 us on the 128 x 128 tiles, 54 on them; at 160, 113 against 95 us);
    // beyond, the ping-pong kernel (at 384 tokens: 187 us on the 128 x 128
    // tiles, 122 on it)
    if (nw_ok(l, B) && nw_fills(l, B, swiglu)) return K_NW;
    if (B <= 32 && skinny_fits(l, B, swiglu, nseg)) return K_SKINNY;
    return B > 256 ? K_TILE0 : K_TILE1;
}

// Split sharded-to-all work by rank when the output alone gives too few
// workgroups to fill the chip.
sg::SplitLayout split_layout(const sg_layer* l, Kind k, int64_t B);

bool want_split(const sg_layer* l, Kind k, int64_t B) {
    if (l->P < 2) return false;
    const int cus = num_cus();
    switch (k) {
    case K_TILE0: return sg::tile_count((int)B, (int)l->out_dims, 0) * 2 <= cus;
    case K_TILE1: return sg::tile_count((int)B, (int)l->out_dims, 1) * 2 <= cus;
    case K_NW: return sg::tile_nw_count((int)B, (int)l->out_dims, 0, l->mx) * 2 <= cus;
    // the 4-bit tile kernel (three workgroups per CU) splits up to one tile
    // per CU (decode-MLP down projection: 126 -> 45 us at 192 tokens, 143 ->
    // 101 us at 512)
    case K_Q4TILE: return sg::q4_tile_count((int)B, (int)l->out_dims) <= cus;
    default: return false;
    }
}

sg::SplitLayout split_layout(const sg_layer* l, Kind k, int64_t B) {
    switch (k) {
    case K_TILE0: return sg::tile_split_layout((int)B, (int)l->out_dims, l->P, 0);
    case K_TILE1: return sg::tile_split_layout((int)B, (int)l->out_dims, l->P, 1);
    case K_NW: {
        const size_t t = (size_t)sg::tile_nw_count((int)B, (int)l->out_dims, 0, l->mx);
        return {t * (size_t)sg::tile_nw_tm((int)B, l->mx) * 128 * (size_t)sg::split_groups((int)t, l->P), t};
    }
    case K_Q4TILE: {
        const size_t t = (size_t)sg::q4_tile_count((int)B, (int)l->out_dims);
        return {t * (size_t)sg::q4_tile_rows((int)B) * 128 * l->P, t};
    }
    default: return {0, 0};
    }
}

// kernel family for a sharded-to-all call (alignment of the caller's pointers
// is checked separately; misaligned pointers fall back to the generic path)
Kind choose_row(const sg_layer* l, int64_t B) {
    if (l->mx) return choose_mx(l, B, l->w, 0, l->P);
    // 4-bit: the streaming kernels up to 32 tokens, as for the gate|up layer, so
    // that the fused MLP (h fragment-major for the 16-row streaming kernel) and
    // the separate calls run the same kernels
    if (l->quantized) return !l->qfrag ? K_GENERIC : (B <= 32 && q4_fits(l, B, 0) ? K_Q4 : K_Q4TILE);
    if (l->dtype == SG_F32 || l->cols_r % 8) return K_GENERIC;
    // up to 256 tokens the few-token tiles, beyond them the ping-pong kernel,
    // either split into groups of ranks whenever the output gives too few
    // tiles (decode-MLP down projection at 64 tokens: 93 us on the split
    // 128 x 128 tiles, 56 on the split ping-pong kernel, 36 on the few-token
    // tiles; at 256 tokens 139, 69 and 58 us)
    if (nw_ok(l, B) && nw_fills(l, B, 0)) return K_NW;
    if (B <= 32 && skinny_fits(l, B, 0, l->P)) return K_SKINNY;
    return K_TILE0;
}

hipError_t run(const sg::Problem& p, Kind k, hipStream_t st) {
    // fragment-major activations (the fused MLP's h) exist for the streaming kernels only
    if ((p.xfrag || p.out_map == sg::OUT_FRAG || p.out_map == sg::OUT_FRAG_Q4) && k != K_SKINNY && k != K_Q4)
        return hipErrorInvalidValue;
    if (k == K_Q4TILE && !sg::q4_tile_fits(p)) k = K_GENERIC;
    switch (k) {
    case K_TILE0: return sg::launch_tile(p, st, 0);
    case K_TILE1: return sg::launch_tile(p, st, 1);
    case K_SKINNY: return sg::launch_skinny(p, st);
    case K_Q4: return sg::launch_q4(p, st);
    case K_Q4TILE: return sg::launch_q4_tile(p, st);
    // (a split call's workspace is laid out for this kernel: no fallback then)
    case K_NW: return sg::tile_nw_fits(p) ? sg::launch_tile_nw(p, st)
                      : p.split ? hipErrorInvalidValue : sg::launch_tile(p, st, 1);
    default: return sg::launch_generic(p, st);
    }
}

void set_weights(sg::Problem& p, const sg_layer* l) {
    if (l->quantized) {
        p.wq = (const uint32_t*)l->w;
        p.qs = l->qs;
        p.qb = l->qb;
        p.ldq = l->cols_r / 8;
        p.ldg = l->cols_r / 64;
        p.q_seg = l->rows_r * p.ldq;
        p.g_seg = l->rows_r * p.ldg;
        p.qfrag = l->qfrag;
    } else {
        p.W = l->w;
        p.ldw = l->cols_r;
        p.w_seg = l->rows_r * l->cols_r;
        p.wfrag = l->wfrag;
        p.wsteps = l->cols_r / 32;
        if (l->mx) {
            p.fp8 = 1;
            p.ms = l->ms;
            p.ms_seg = l->rows_r * (l->cols_r / 32);
        }
    }
}

}  // namespace

extern "C" {

const char* sg_last_error(void) { return g_err.c_str(); }

sg_status sg_shard_linear(const void* weight, sg_dtype dtype, int64_t out_dims, int64_t in_dims,
                          const void* bias, int mode, int segments, int P, void* stream,
                          sg_layer** out) {
    g_err.clear();
    sg_status st = common_checks(mode, segments, P, out_dims, in_dims, out);
    if (st) return st;
    if (!weight) return fail(SG_ERR_INVALID_ARG, "weight is NULL");
    if (!dtype_ok(dtype)) return fail(SG_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    hipStream_t hs = (hipStream_t)stream;
    sg_layer* l = new sg_layer{};
    l->mode = mode;
    l->segments = segments;
    l->P = P;
    l->dtype = dtype;
    l->out_dims = out_dims;
    l->in_dims = in_dims;
    l->rows_r = mode == SG_ALL_TO_SHARDED ? out_dims / P : out_dims;
    l->cols_r = mode == SG_ALL_TO_SHARDED ? in_dims : in_dims / P;
    (void)hipGetDevice(&l->device);
    const size_t esz = dtype_size(dtype);
    const size_t wbytes = (size_t)(out_dims * in_dims) * esz;
    // 16-bit weights that tile into 16 x 32 MFMA fragments are stored
    // fragment-major (one coalesced 1 KB read per fragment).  All-to-sharded
    // ranks are stacked rows of one (out, in) matrix, so the layout covers the
    // whole stack; sharded-to-all ranks are separate (out, in/P) matrices.
    l->wfrag = dtype != SG_F32 && out_dims % 16 == 0 && l->cols_r % 32 == 0;
    const int frag_mats = mode == SG_ALL_TO_SHARDED ? 1 : P;
    const int64_t frag_rows = mode == SG_ALL_TO_SHARDED ? out_dims : l->rows_r;
    void* rowmajor = nullptr;
    hipError_t e = hipMalloc(&rowmajor, wbytes);
    if (e != hipSuccess) {
        free_layer(l);
        return hip_fail(e, "weight allocation");
    }
    st = copy_shards(rowmajor, weight, out_dims, in_dims, esz, mode == SG_ALL_TO_SHARDED ? 0 : 1, segments, P, hs);
    if (!st && l->wfrag) {
        e = hipMalloc(&l->w, wbytes);
        if (e == hipSuccess) e = sg::frag_transform(l->w, rowmajor, frag_mats, frag_rows, l->cols_r, 1, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        (void)hipFree(rowmajor);
        if (e != hipSuccess) st = hip_fail(e, "weight layout");
    } else {
        l->w = rowmajor;
    }
    if (!st && bias) {
        e = hipMalloc(&l->bias, (size_t)out_dims * esz);
        if (e != hipSuccess) st = hip_fail(e, "bias allocation");
        else if (mode == SG_ALL_TO_SHARDED)
            st = copy_shards(l->bias, bias, out_dims, 1, esz, 0, segments, P, hs);
        else {
            e = hipMemcpyAsync(l->bias, bias, (size_t)out_dims * esz, hipMemcpyDefault, hs);
            if (e != hipSuccess) st = hip_fail(e, "bias copy");
        }
    }
    if (!st) {
        e = hipStreamSynchronize(hs);
        if (e != hipSuccess) st = hip_fail(e, "shard copy");
    }
    if (st) {
        free_layer(l);
        return st;
    }
    *out = l;
    return SG_OK;
}

sg_status sg_shard_quantized_linear(const uint32_t* wq, const uint16_t* scales, const uint16_t* qbiases,
                                    int64_t out_dims, int64_t in_dims, int group_size, int bits,
                                    sg_dtype act, const void* bias, int mode, int segments, int P,
                                    void* stream, sg_layer** out) {
    g_err.clear();
    sg_status st = common_checks(mode, segments, P, out_dims, in_dims, out);
    if (st) return st;
    if (!wq || !scales || !qbiases) return fail(SG_ERR_INVALID_ARG, "quantized tensors must not be NULL");
    if (group_size != 64 || bits != 4)
        return fail(SG_ERR_UNSUPPORTED, "only group_size 64 and bits 4 are implemented (got %d, %d)",
                    group_size, bits);
    if (act != SG_BF16 && act != SG_F16) return fail(SG_ERR_INVALID_ARG, "activation dtype must be bf16 or fp16");
    if (in_dims % group_size) return fail(SG_ERR_NOT_DIVISIBLE, "in_dims %lld is not a multiple of group_size %d", (long long)in_dims, group_size);
    if (mode == SG_SHARDED_TO_ALL && (in_dims / segments / P) % group_size)
        return fail(SG_ERR_NOT_DIVISIBLE,
                    "Cannot shard the input of size %lld across %d devices: a quantization group of %d "
                    "would straddle two ranks.", (long long)in_dims, P, group_size);
    hipStream_t hs = (hipStream_t)stream;
    sg_layer* l = new sg_layer{};
    l->mode = mode;
    l->segments = segments;
    l->P = P;
    l->quantized = 1;
    l->dtype = act;
    l->out_dims = out_dims;
    l->in_dims = in_dims;
    l->rows_r = mode == SG_ALL_TO_SHARDED ? out_dims / P : out_dims;
    l->cols_r = mode == SG_ALL_TO_SHARDED ? in_dims : in_dims / P;
    (void)hipGetDevice(&l->device);
    const int axis = mode == SG_ALL_TO_SHARDED ? 0 : 1;
    const int64_t words = in_dims / 8, groups = in_dims / group_size;
    hipError_t e = hipMalloc(&l->w, (size_t)(out_dims * words) * 4);
    if (e == hipSuccess) e = hipMalloc((void**)&l->qs, (size_t)(out_dims * groups) * 2);
    if (e == hipSuccess) e = hipMalloc((void**)&l->qb, (size_t)(out_dims * groups) * 2);
    if (e != hipSuccess) {
        free_layer(l);
        return hip_fail(e, "quantized weight allocation");
    }
    st = copy_shards(l->w, wq, out_dims, words, 4, axis, segments, P, hs);
    if (!st) st = copy_shards(l->qs, scales, out_dims, groups, 2, axis, segments, P, hs);
    if (!st) st = copy_shards(l->qb, qbiases, out_dims, groups, 2, axis, segments, P, hs);
    if (!st) {
        e = sg::q4_repack((uint32_t*)l->w, out_dims * words, 1, hs);
        if (e != hipSuccess) st = hip_fail(e, "code reorder");
    }
    // codes, scales and biases fragment-major when the rank matrices tile into
    // 32-row blocks and runs of 4 groups (the streaming kernel's layout)
    l->qfrag = out_dims % 32 == 0 && l->cols_r % 256 == 0;
    if (!st && l->qfrag) {
        const int mats = mode == SG_ALL_TO_SHARDED ? 1 : P;
        const int64_t rows = mode == SG_ALL_TO_SHARDED ? out_dims : l->rows_r;
        void *w2 = nullptr, *s2 = nullptr, *b2 = nullptr;
        e = hipMalloc(&w2, (size_t)(out_dims * words) * 4);
        if (e == hipSuccess) e = hipMalloc(&s2, (size_t)(out_dims * groups) * 2);
        if (e == hipSuccess) e = hipMalloc(&b2, (size_t)(out_dims * groups) * 2);
        if (e == hipSuccess)
            e = sg::q4_transform((uint32_t*)w2, (const uint32_t*)l->w, (uint16_t*)s2, l->qs, mats, rows, l->cols_r, 1, hs);
        if (e == hipSuccess) e = sg::q4_transform(nullptr, nullptr, (uint16_t*)b2, l->qb, mats, rows, l->cols_r, 1, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e == hipSuccess) {
            (void)hipFree(l->w);
            (void)hipFree(l->qs);
            (void)hipFree(l->qb);
            l->w = w2;
            l->qs = (uint16_t*)s2;
            l->qb = (uint16_t*)b2;
        } else {
            (void)hipFree(w2);
            (void)hipFree(s2);
            (void)hipFree(b2);
            st = hip_fail(e, "4-bit layout");
        }
    }
    if (!st && bias) {
        e = hipMalloc(&l->bias, (size_t)out_dims * 2);
        if (e != hipSuccess) st = hip_fail(e, "bias allocation");
        else if (mode == SG_ALL_TO_SHARDED)
            st = copy_shards(l->bias, bias, out_dims, 1, 2, 0, segments, P, hs);
        else {
            e = hipMemcpyAsync(l->bias, bias, (size_t)out_dims * 2, hipMemcpyDefault, hs);
            if (e != hipSuccess) st = hip_fail(e, "bias copy");
        }
    }
    if (!st) {
        e = hipStreamSynchronize(hs);
        if (e != hipSuccess) st = hip_fail(e, "shard copy");
    }
    if (st) {
        free_layer(l);
        return st;
    }
    *out = l;
    return SG_OK;
}

sg_status sg_shard_mxfp8_linear(const uint8_t* codes, const uint8_t* scales, int64_t out_dims, int64_t in_dims,
                                sg_dtype act, const void* bias, int mode, int segments, int P, void* stream,
                                sg_layer** out) {
    g_err.clear();
    sg_status st = common_checks(mode, segments, P, out_dims, in_dims, out);
    if (st) return st;
    if (!codes || !scales) return fail(SG_ERR_INVALID_ARG, "codes and scales must not be NULL");
    if (act != SG_BF16) return fail(SG_ERR_UNSUPPORTED, "MX FP8 layers take bf16 activations");
    if (in_dims % 32) return fail(SG_ERR_NOT_DIVISIBLE, "in_dims %lld is not a multiple of the block of 32", (long long)in_dims);
    if (mode == SG_SHARDED_TO_ALL && (in_dims / segments / P) % 32)
        return fail(SG_ERR_NOT_DIVISIBLE,
                    "Cannot shard the input of size %lld across %d devices: a scale block of 32 would straddle "
                    "two ranks.", (long long)in_dims, P);
    hipStream_t hs = (hipStream_t)stream;
    sg_layer* l = new sg_layer{};
    l->mode = mode;
    l->segments = segments;
    l->P = P;
    l->mx = 1;
    l->dtype = act;
    l->out_dims = out_dims;
    l->in_dims = in_dims;
    l->rows_r = mode == SG_ALL_TO_SHARDED ? out_dims / P : out_dims;
    l->cols_r = mode == SG_ALL_TO_SHARDED ? in_dims : in_dims / P;
    (void)hipGetDevice(&l->device);
    const int axis = mode == SG_ALL_TO_SHARDED ? 0 : 1;
    const int64_t blocks = in_dims / 32;
    hipError_t e = hipMalloc(&l->w, (size_t)(out_dims * in_dims));
    if (e == hipSuccess) e = hipMalloc((void**)&l->ms, (size_t)(out_dims * blocks));
    if (e != hipSuccess) {
        free_layer(l);
        return hip_fail(e, "MX FP8 allocation");
    }
    st = copy_shards(l->w, codes, out_dims, in_dims, 1, axis, segments, P, hs);
    if (!st) st = copy_shards(l->ms, scales, out_dims, blocks, 1, axis, segments, P, hs);
    // codes and scales fragment-major when the rank matrices tile into 16-row
    // blocks and runs of 4 scale blocks (the streaming kernel's layout)
    l->wfrag = out_dims % 16 == 0 && l->cols_r % 128 == 0 && (mode == SG_ALL_TO_SHARDED || l->rows_r % 16 == 0);
    if (!st && l->wfrag) {
        const int mats = mode == SG_ALL_TO_SHARDED ? 1 : P;
        const int64_t rows = mode == SG_ALL_TO_SHARDED ? out_dims : l->rows_r;
        void *c2 = nullptr, *s2 = nullptr;
        e = hipMalloc(&c2, (size_t)(out_dims * in_dims));
        if (e == hipSuccess) e = hipMalloc(&s2, (size_t)(out_dims * blocks));
        if (e == hipSuccess)
            e = sg::mx_transform((uint8_t*)c2, (const uint8_t*)l->w, (uint8_t*)s2, l->ms, mats, rows, l->cols_r, 1, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e == hipSuccess) {
            (void)hipFree(l->w);
            (void)hipFree(l->ms);
            l->w = c2;
            l->ms = (uint8_t*)s2;
        } else {
            (void)hipFree(c2);
            (void)hipFree(s2);
            st = hip_fail(e, "MX FP8 layout");
        }
    }
    if (!st && bias) {
        e = hipMalloc(&l->bias, (size_t)out_dims * 2);
        if (e != hipSuccess) st = hip_fail(e, "bias allocation");
        else if (mode == SG_ALL_TO_SHARDED)
            st = copy_shards(l->bias, bias, out_dims, 1, 2, 0, segments, P, hs);
        else {
            e = hipMemcpyAsync(l->bias, bias, (size_t)out_dims * 2, hipMemcpyDefault, hs);
            if (e != hipSuccess) st = hip_fail(e, "bias copy");
        }
    }
    if (!st) {
        e = hipStreamSynchronize(hs);
        if (e != hipSuccess) st = hip_fail(e, "shard copy");
    }
    if (st) {
        free_layer(l);
        return st;
    }
    *out = l;
    return SG_OK;
}

sg_status sg_all_to_sharded_ex(const sg_layer* l, const void* x, int in_layout, int64_t B, void* y,
                               int out_layout, int epilogue, sg_dtype y_dtype, void* stream) {
    g_err.clear();
    if (!l) return fail(SG_ERR_INVALID_ARG, "layer is NULL");
    if (l->mode != SG_ALL_TO_SHARDED) return fail(SG_ERR_INVALID_ARG, "layer is sharded-to-all; use sg_sharded_to_all");
    if (B < 0 || B > INT32_MAX) return fail(SG_ERR_INVALID_ARG, "token count %lld out of range", (long long)B);
    if (in_layout != SG_IN_FULL && in_layout != SG_IN_SHARDED)
        return fail(SG_ERR_INVALID_ARG, "unknown input layout %d", in_layout);
    if (out_layout != SG_OUT_FULL && out_layout != SG_OUT_SHARDED)
        return fail(SG_ERR_INVALID_ARG, "unknown output layout %d", out_layout);
    if (epilogue != SG_EPI_NONE && epilogue != SG_EPI_SWIGLU) return fail(SG_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
    if (!dtype_ok(y_dtype)) return fail(SG_ERR_INVALID_ARG, "unknown output dtype %d", (int)y_dtype);
    if (epilogue == SG_EPI_SWIGLU && (l->segments != 2 || l->bias))
        return fail(SG_ERR_INVALID_ARG, "the SwiGLU epilogue needs an all-to-sharded layer with segments == 2 ([gate; up]) and no bias");
    const bool xsh = in_layout == SG_IN_SHARDED;
    if (xsh) {
        if (l->in_dims % l->P)
            return fail(SG_ERR_NOT_DIVISIBLE, "Cannot shard the input of size %lld across %d devices.",
                        (long long)l->in_dims, l->P);
        // MX FP8: no scale block may straddle two input shards, and in the
        // fragment-major layout a row's scales come in runs of four blocks
        if (l->mx && (l->in_dims / l->P) % (l->wfrag ? 128 : 32))
            return fail(SG_ERR_UNSUPPORTED, "a sharded input on an MX FP8 layer needs in_dims / P to be a multiple of %d",
                        l->wfrag ? 128 : 32);
        // 4-bit: no quantization group (in the stored layout, no run of four)
        // may straddle two input shards
        if (l->quantized && (l->in_dims / l->P) % (l->qfrag ? 256 : 64))
            return fail(SG_ERR_UNSUPPORTED, "a sharded input on a 4-bit layer needs in_dims / P to be a multiple of %d",
                        l->qfrag ? 256 : 64);
        if (l->wfrag && (l->in_dims / l->P) % 32)
            return fail(SG_ERR_UNSUPPORTED, "a sharded input needs in_dims / P to be a multiple of 32 (got %lld)",
                        (long long)(l->in_dims / l->P));
    }
    if (B == 0) return SG_OK;
    if (!x || !y) return fail(SG_ERR_INVALID_ARG, "x and y must not be NULL");
    sg::Problem p{};
    p.A = x;
    p.M = (int)B;
    p.dtype = l->dtype;
    set_weights(p, l);
    if (xsh) {
        // [HSYM] Case 2: the all-gather of the input shards is the K loop
        // walking shard r's columns for r = 0 .. P-1
        const int64_t kr = l->in_dims / l->P;
        p.lda = kr;
        p.a_seg = B * kr;
        p.Kseg = (int)kr;
        p.nseg = l->P;
        p.w_seg = l->wfrag ? kr * 16 : kr;  // next k range of every weight row
        if (l->quantized) {  // shard s starts kr / 64 groups further along each row
            p.q_seg = l->qfrag ? 4 * kr : kr / 8;
            p.g_seg = l->qfrag ? kr / 2 : kr / 64;
        }
        if (l->mx) p.ms_seg = l->wfrag ? kr / 2 : kr / 32;  // (codes: w_seg bytes, as above)
    } else {
        p.lda = l->in_dims;
        p.Kseg = (int)l->cols_r;
        p.nseg = 1;
    }
    p.swiglu = epilogue == SG_EPI_SWIGLU;
    p.N = (int)(p.swiglu ? l->out_dims / 2 : l->out_dims);
    p.floc = p.swiglu ? l->rows_r / 2 : 0;
    p.out = y;
    p.out_dtype = y_dtype;
    p.out_map = out_layout == SG_OUT_FULL ? sg::OUT_ROWMAJOR : sg::OUT_SHARDED;
    p.ldo = p.N;
    p.nloc = p.N / l->P;
    p.bias = l->bias;
    Kind k = choose(l, B, x, p.swiglu, p.nseg);
    if (xsh && (p.Kseg % 8)) k = K_GENERIC;  // 16-byte input rows for the vector paths
    if (k != K_GENERIC && k != K_Q4 && !aligned16(y)) k = K_GENERIC;
    hipError_t e = run(p, k, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "all_to_sharded launch");
    return SG_OK;
}

sg_status sg_all_to_sharded(const sg_layer* l, const void* x, int64_t B, void* y, int gather,
                            int epilogue, sg_dtype y_dtype, void* stream) {
    if (gather != 0 && gather != 1) {
        g_err.clear();
        return fail(SG_ERR_INVALID_ARG, "gather must be 0 or 1");
    }
    return sg_all_to_sharded_ex(l, x, SG_IN_FULL, B, y, gather ? SG_OUT_FULL : SG_OUT_SHARDED, epilogue,
                                y_dtype, stream);
}

size_t sg_sharded_to_all_workspace(const sg_layer* l, int64_t B) {
    if (!l || l->mode != SG_SHARDED_TO_ALL || B <= 0 || B > INT32_MAX) return 0;
    const Kind k = choose_row(l, B);
    return want_split(l, k, B) ? sg::split_workspace_bytes(split_layout(l, k, B)) : 0;
}

sg_status sg_sharded_to_all_ex(const sg_layer* l, const void* x_partial, int64_t B, void* y, int out_layout,
                               sg_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!l) return fail(SG_ERR_INVALID_ARG, "layer is NULL");
    if (l->mode != SG_SHARDED_TO_ALL) return fail(SG_ERR_INVALID_ARG, "layer is all-to-sharded; use sg_all_to_sharded");
    if (B < 0 || B > INT32_MAX) return fail(SG_ERR_INVALID_ARG, "token count %lld out of range", (long long)B);
    if (out_layout != SG_OUT_FULL && out_layout != SG_OUT_SHARDED)
        return fail(SG_ERR_INVALID_ARG, "unknown output layout %d", out_layout);
    if (out_layout == SG_OUT_SHARDED && l->out_dims % l->P)
        return fail(SG_ERR_NOT_DIVISIBLE, "Cannot shard the output of size %lld across %d devices.",
                    (long long)l->out_dims, l->P);
    if (!dtype_ok(y_dtype)) return fail(SG_ERR_INVALID_ARG, "unknown output dtype %d", (int)y_dtype);
    if (B == 0) return SG_OK;
    if (!x_partial || !y) return fail(SG_ERR_INVALID_ARG, "x_partial and y must not be NULL");
    sg::Problem p{};
    p.A = x_partial;
    p.lda = l->cols_r;
    p.a_seg = B * l->cols_r;
    p.M = (int)B;
    p.Kseg = (int)l->cols_r;
    p.nseg = l->P;
    p.dtype = l->dtype;
    set_weights(p, l);
    p.N = (int)l->out_dims;
    p.out = y;
    p.out_dtype = y_dtype;
    // SG_OUT_SHARDED: [HSYM]'s reduce-scatter -- rank r receives columns
    // [r out/P, (r+1) out/P) of the summed result
    p.out_map = out_layout == SG_OUT_FULL ? sg::OUT_ROWMAJOR : sg::OUT_SHARDED;
    p.ldo = p.N;
    p.nloc = p.N / l->P;
    p.bias = l->bias;
    Kind k = choose_row(l, B);
    if (k != K_GENERIC && (!aligned16(x_partial) || !aligned16(l->w) || (k != K_Q4 && !aligned16(y))))
        k = K_GENERIC;  // the vector paths need 16-byte aligned rows
    if (want_split(l, k, B)) {
        const sg::SplitLayout lay = split_layout(l, k, B);
        const size_t bytes = sg::split_workspace_bytes(lay);
        if (!workspace || ws_bytes < bytes)
            return fail(SG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, bytes);
        if (!aligned16(workspace)) return fail(SG_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        p.split = 1;
        p.ws = (float*)workspace;
    }
    hipError_t e = run(p, k, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "sharded_to_all launch");
    return SG_OK;
}

sg_status sg_sharded_to_all(const sg_layer* l, const void* x_partial, int64_t B, void* y, sg_dtype y_dtype,
                            void* workspace, size_t ws_bytes, void* stream) {
    return sg_sharded_to_all_ex(l, x_partial, B, y, SG_OUT_FULL, y_dtype, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Fused gated MLP: gate|up all-to-sharded with SwiGLU, then the down
// sharded-to-all, the sharded h kept in the caller's workspace.
// ---------------------------------------------------------------------------
namespace {

const char* mlp_check(const sg_layer* gu, const sg_layer* dn) {
    if (!gu || !dn) return "layer is NULL";
    if (gu->mode != SG_ALL_TO_SHARDED || gu->segments != 2 || gu->bias)
        return "the gate|up layer must be all-to-sharded with segments == 2 ([gate; up]) and no bias";
    if (dn->mode != SG_SHARDED_TO_ALL) return "the down layer must be sharded-to-all";
    if (gu->P != dn->P) return "the two layers must be sharded over the same P";
    if (gu->out_dims / 2 != dn->in_dims) return "the down layer's input width must be half the gate|up output width";
    if (gu->dtype != dn->dtype) return "the two layers must take the same activation dtype";
    return nullptr;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// bytes of h: P rank blocks of act_rows(B) x (F / P) activations
size_t mlp_h_bytes(const sg_layer* gu, int64_t B) {
    return align256((size_t)sg::act_rows(B) * (size_t)(gu->out_dims / 2) * dtype_size(gu->dtype));
}

}  // namespace

// The down layer's workspace (partial tiles when it splits by rank), then h.
static size_t mlp_down_bytes(const sg_layer* dn, int64_t B) { return align256(sg_sharded_to_all_workspace(dn, B)); }

size_t sg_mlp_workspace(const sg_layer* gate_up, const sg_layer* down, int64_t B) {
    if (mlp_check(gate_up, down) || B <= 0 || B > INT32_MAX) return 0;
    return mlp_down_bytes(down, B) + mlp_h_bytes(gate_up, B);
}

// the launches of sg_mlp on a checked workspace of at least sg_mlp_workspace bytes
static sg_status mlp_run(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, void* y,
                         sg_dtype y_dtype, void* workspace, void* stream) {
    const size_t db = mlp_down_bytes(down, B);
    void* h = (char*)workspace + db;
    const sg_layer* gu = gate_up;
    const sg_layer* dn = down;
    // the down layer reading h fragment-major
    sg::Problem q{};
    q.A = h;
    q.xfrag = 1;
    q.a_seg = sg::act_rows(B) * dn->cols_r;
    q.M = (int)B;
    q.Kseg = (int)dn->cols_r;
    q.nseg = dn->P;
    q.dtype = dn->dtype;
    set_weights(q, dn);
    q.N = (int)dn->out_dims;
    q.out = y;
    q.out_dtype = y_dtype;
    q.out_map = sg::OUT_ROWMAJOR;
    q.ldo = q.N;
    q.bias = dn->bias;
    // Both layers on a streaming kernel and at least 8 tokens: h fragment-major
    // in the order the down kernel reads (skinny.hip: act_frag_offset; 4-bit,
    // the 16-row kernel: act_frag_offset_q4), so that its activation loads are
    // contiguous 1 KB reads instead of 16 rows x 64 bytes (measured on the
    // 4-bit down projection: 16.2 -> 13.7 us at 8 tokens, 33.0 -> 18.8 us at
    // 32).  With fewer tokens a row-major load touches fewer cache lines than
    // a 1 KB fragment (13.1 against 13.5 us at one token), so the two separate
    // calls with a row-major h run instead, as for every other pair.
    const Kind kg = choose(gu, B, x, 1, 1), kd = choose_row(dn, B);
    const bool frag_pays = B >= 8;
    int hmap = -1;
    if (frag_pays && kg == K_SKINNY && kd == K_SKINNY && dn->wfrag && aligned16(y) && aligned16(dn->w) &&
        dn->cols_r % 32 == 0)
        hmap = sg::OUT_FRAG;
    else if (frag_pays && kg == K_Q4 && kd == K_Q4 && sg::q4s_takes(q))
        hmap = sg::OUT_FRAG_Q4;
    if (hmap < 0) {
        sg_status st = sg_all_to_sharded_ex(gu, x, SG_IN_FULL, B, h, SG_OUT_SHARDED, SG_EPI_SWIGLU, gu->dtype, stream);
        if (st != SG_OK) return st;
        return sg_sharded_to_all_ex(dn, h, B, y, SG_OUT_FULL, y_dtype, workspace, db, stream);
    }
    sg::Problem p{};
    p.A = x;
    p.M = (int)B;
    p.dtype = gu->dtype;
    set_weights(p, gu);
    p.lda = gu->in_dims;
    p.Kseg = (int)gu->cols_r;
    p.nseg = 1;
    p.swiglu = 1;
    p.N = (int)(gu->out_dims / 2);
    p.floc = gu->rows_r / 2;
    p.out = h;
    p.out_dtype = gu->dtype;
    p.out_map = hmap;
    p.nloc = p.N / gu->P;
    hipError_t e = run(p, kg, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mlp gate|up launch");
    e = run(q, kd, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mlp down launch");
    return SG_OK;
}

// argument checks shared by sg_mlp and sg_mlp_static; *done is set for B == 0
static sg_status mlp_args(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, const void* y,
                          sg_dtype y_dtype, bool* done) {
    *done = false;
    if (const char* why = mlp_check(gate_up, down)) return fail(SG_ERR_INVALID_ARG, "%s", why);
    if (B < 0 || B > INT32_MAX) return fail(SG_ERR_INVALID_ARG, "token count %lld out of range", (long long)B);
    if (!dtype_ok(y_dtype)) return fail(SG_ERR_INVALID_ARG, "unknown output dtype %d", (int)y_dtype);
    if (B == 0) {
        *done = true;
        return SG_OK;
    }
    if (!x || !y) return fail(SG_ERR_INVALID_ARG, "x and y must not be NULL");
    return SG_OK;
}

sg_status sg_mlp(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, void* y, sg_dtype y_dtype,
                 void* workspace, size_t ws_bytes, void* stream) {
    g_err.clear();
    bool done = false;
    sg_status st = mlp_args(gate_up, down, x, B, y, y_dtype, &done);
    if (st != SG_OK || done) return st;
    const size_t need = sg_mlp_workspace(gate_up, down, B);
    if (!workspace || ws_bytes < need)
        return fail(SG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (!aligned16(workspace)) return fail(SG_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    return mlp_run(gate_up, down, x, B, y, y_dtype, workspace, stream);
}

// ---------------------------------------------------------------------------
// sg_mlp without a workspace argument: a fixed scratch array per device.
// In host code `mlp_scratch` names a host-side stand-in, not the device
// array: every use goes through the device address hipGetSymbolAddress
// returns, looked up once per device (with that device current) and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char mlp_scratch[SG_MLP_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// the device address of the current device's scratch (nothing in it needs
// clearing: every call writes what it reads)
sg_status scratch_for_current_device(void** out) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev), "device query");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SG_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(mlp_scratch)), "scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SG_OK;
}
}  // namespace

sg_status sg_mlp_static(const sg_layer* gate_up, const sg_layer* down, const void* x, int64_t B, void* y,
                        sg_dtype y_dtype, void* stream) {
    g_err.clear();
    bool done = false;
    sg_status st = mlp_args(gate_up, down, x, B, y, y_dtype, &done);
    if (st != SG_OK || done) return st;
    const size_t need = sg_mlp_workspace(gate_up, down, B);
    if (need > (size_t)SG_MLP_STATIC_SCRATCH_BYTES)
        return fail(SG_ERR_WORKSPACE,
                    "sg_mlp_static: %lld tokens need %zu bytes of workspace, the static scratch holds %zu; "
                    "use sg_mlp with a caller workspace", (long long)B, need, (size_t)SG_MLP_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != SG_OK) return st;
    return mlp_run(gate_up, down, x, B, y, y_dtype, ws, stream);
}

// ---------------------------------------------------------------------------
// Backward (vector-Jacobian products) of the two sharded layers
//
// Input gradients run on the forward kernels: dx of an all-to-sharded layer,
// sum_r dY_r W_r, is a sharded-to-all product with the rank shards
// transposed (the rank-order sum fused as in the forward), and dX_r = dY W_r
// of a sharded-to-all layer is an all-to-sharded product with the stack of
// W_r^T and a sharded output.  The transposed shards are a second,
// fragment-major copy of the layer's weights, built once by the first
// backward call that needs it.  Weight gradients (a contraction over the
// tokens) and SUMMA's dA = X^T dY run on the matrix-core tile kernels with
// both operands transposed into the caller's workspace (tokens zero-padded to
// a multiple of 32).  Shapes or dtypes those kernels do not take, or a call
// without a workspace, run on the vector-unit kernels of backward.hip.
// ---------------------------------------------------------------------------
namespace {

const char* bwd_check(const sg_layer* l, int mode, int64_t B, sg_dtype dx_dtype, sg_dtype dw_dtype) {
    if (!l) return "layer is NULL";
    if (l->mode != mode)
        return mode == SG_ALL_TO_SHARDED ? "layer is sharded-to-all; use sg_sharded_to_all_backward"
                                         : "layer is all-to-sharded; use sg_all_to_sharded_backward";
    if (B < 0 || B > INT32_MAX) return "token count out of range";
    if (!dtype_ok(dx_dtype) || !dtype_ok(dw_dtype)) return "unknown gradient dtype";
    return nullptr;
}

int64_t pad32(int64_t n) { return (n + 31) / 32 * 32; }

// the transposed-shard copy: 16-bit dense layers whose transposes tile into
// 16-row x 32-k fragments (rows_r is the k of the transposed product)
bool wt_ok(const sg_layer* l) {
    return !l->quantized && !l->mx && l->dtype != SG_F32 && l->rows_r % 32 == 0 && l->cols_r % 16 == 0;
}

sg_status ensure_wt(const sg_layer* lc, hipStream_t st) {
    sg_layer* l = const_cast<sg_layer*>(lc);  // the copy is a cache of the layer's own weights
    std::lock_guard<std::mutex> lock(l->wt_mu);
    if (l->wt) return SG_OK;
    const size_t bytes = (size_t)(l->P * l->rows_r * l->cols_r) * dtype_size(l->dtype);
    void* rowmajor = l->w;
    void* tmp = nullptr;
    void* wt = nullptr;
    hipError_t e = hipSuccess;
    if (l->wfrag) {
        e = hipMalloc(&tmp, bytes);
        const int mats = l->mode == SG_ALL_TO_SHARDED ? 1 : l->P;
        const int64_t rows = l->mode == SG_ALL_TO_SHARDED ? l->out_dims : l->rows_r;
        if (e == hipSuccess) e = sg::frag_transform(tmp, l->w, mats, rows, l->cols_r, 0, st);
        rowmajor = tmp;
    }
    if (e == hipSuccess) e = hipMalloc(&wt, bytes);
    // rank r's (rows_r, cols_r) shard -> rows r cols_r .. of the stack, k = its rows
    if (e == hipSuccess) e = sg::t_frag(wt, rowmajor, l->P, l->rows_r, l->cols_r, l->rows_r, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (tmp) (void)hipFree(tmp);
    if (e != hipSuccess) {
        if (wt) (void)hipFree(wt);
        return hip_fail(e, "transposed shard copy");
    }
    l->wt = wt;
    return SG_OK;
}

// kernel family for a product of M tokens against N stacked output rows,
// nseg K segments of Kseg, on fragment-major 16-bit weights (no split)
Kind choose_bwd(int64_t M, int64_t N, int nseg, int swiglu = 0) {
    if (M <= 32 && sg::skinny_shape((int)M, (int)N, nseg, swiglu).lds <= sg::kMaxStreamLds) return K_SKINNY;
    return M >= 512 ? K_TILE0 : K_TILE1;
}

// weight-gradient workspace: A = the upstream gradient transposed (out, Bp)
// row-major, then W = the input transposed, (in, Bp) fragment-major
size_t dw_ws_bytes(const sg_layer* l, int64_t B) {
    return align256((size_t)(l->out_dims * pad32(B)) * 2) + align256((size_t)(l->in_dims * pad32(B)) * 2);
}
bool dw_mfma_ok(const sg_layer* l) {
    if (l->quantized || l->mx || l->dtype == SG_F32) return false;
    return l->mode == SG_ALL_TO_SHARDED ? (l->in_dims % 16 == 0 && l->rows_r % 8 == 0)
                                        : (l->cols_r % 16 == 0 && l->out_dims % 8 == 0);
}

// dW with few tokens: bound by its output writes, on the small-K kernel that
// reads the caller's row-major dy and x directly (no workspace)
bool dw_small_ok(const sg_layer* l, int64_t B) {
    if (l->quantized || l->mx || l->dtype == SG_F32 || (B + 15) / 16 * 16 > sg::kDwSmallMaxTokens) return false;
    return l->mode == SG_ALL_TO_SHARDED ? (l->rows_r % 8 == 0 && l->in_dims % 8 == 0)
                                        : (l->out_dims % 8 == 0 && l->cols_r % 8 == 0);
}

sg_status dw_small(const sg_layer* l, const void* x, const void* dy, int64_t B, void* dw, sg_dtype dw_dtype,
                   hipStream_t st) {
    sg::BwdDwSmall p{};
    const bool a2s = l->mode == SG_ALL_TO_SHARDED;
    p.G = dy;  // a2s: (P, B, out/P), rank blocks of out/P rows; s2a: (B, out)
    p.gl = a2s ? l->rows_r : l->out_dims;
    p.g_seg = a2s ? B * l->rows_r : 0;
    p.ldg = a2s ? l->rows_r : l->out_dims;
    p.X = x;  // a2s: (B, in); s2a: (P, B, in/P), rank blocks of in/P columns
    p.xl = a2s ? l->in_dims : l->cols_r;
    p.x_seg = a2s ? 0 : B * l->cols_r;
    p.ldx = a2s ? l->in_dims : l->cols_r;
    p.dtype = l->dtype;
    p.O = (int)l->out_dims;
    p.I = (int)l->in_dims;
    p.B = (int)B;
    p.Bp = (int)((B + 15) / 16 * 16);
    p.out = dw;
    p.out_dtype = dw_dtype;
    p.nloc = a2s ? 0 : l->cols_r;  // a2s: (P, out/P, in) is the row-major (out, in)
    hipError_t e = sg::launch_dw_small(p, st);
    if (e != hipSuccess) return hip_fail(e, "weight-gradient launch");
    return SG_OK;
}

// dW by the tile kernels: M = out rows (all ranks), N = in, K = Bp tokens
sg_status dw_mfma(const sg_layer* l, const void* x, const void* dy, int64_t B, void* dw, sg_dtype dw_dtype,
                  void* workspace, hipStream_t st) {
    const int64_t Bp = pad32(B);
    void* wa = workspace;
    void* ww = (char*)workspace + align256((size_t)(l->out_dims * Bp) * 2);
    hipError_t e;
    if (l->mode == SG_ALL_TO_SHARDED) {
        e = sg::transpose16(wa, dy, l->P, B, l->rows_r, Bp, st);            // (P, out/P, Bp) = (out, Bp)
        if (e == hipSuccess) e = sg::t_frag(ww, x, 1, B, l->in_dims, Bp, st);  // X^T, (in, Bp)
    } else {
        e = sg::transpose16(wa, dy, 1, B, l->out_dims, Bp, st);               // dY^T, (out, Bp)
        if (e == hipSuccess) e = sg::t_frag(ww, x, l->P, B, l->cols_r, Bp, st);  // X_r^T stacked, (in, Bp)
    }
    if (e != hipSuccess) return hip_fail(e, "weight-gradient operand transform");
    sg::Problem p{};
    p.A = wa;
    p.lda = Bp;
    p.M = (int)l->out_dims;
    p.Kseg = (int)Bp;
    p.nseg = 1;
    p.dtype = l->dtype;
    p.W = ww;
    p.ldw = Bp;
    p.wfrag = 1;
    p.wsteps = Bp / 32;
    p.N = (int)l->in_dims;
    p.out = dw;
    p.out_dtype = dw_dtype;
    if (l->mode == SG_ALL_TO_SHARDED) {
        p.out_map = sg::OUT_ROWMAJOR;  // (P, out/P, in) is the stacked (out, in)
        p.ldo = l->in_dims;
    } else {
        p.out_map = sg::OUT_SHARDED;  // column n -> rank n / (in/P): (P, out, in/P)
        p.nloc = l->cols_r;
    }
    e = run(p, p.M >= 512 ? K_TILE0 : K_TILE1, st);
    if (e != hipSuccess) return hip_fail(e, "weight-gradient launch");
    return SG_OK;
}

}  // namespace

size_t sg_layer_backward_workspace(const sg_layer* l, int64_t B) {
    if (!l || B <= 0 || B > INT32_MAX || !dw_mfma_ok(l) || dw_small_ok(l, B)) return 0;
    return dw_ws_bytes(l, B);
}

sg_status sg_all_to_sharded_backward(const sg_layer* l, const void* x, const void* dy, int64_t B, void* dx,
                                     sg_dtype dx_dtype, void* dw, sg_dtype dw_dtype, void* workspace, size_t ws_bytes,
                                     void* stream) {
    g_err.clear();
    if (const char* why = bwd_check(l, SG_ALL_TO_SHARDED, B, dx_dtype, dw_dtype)) return fail(SG_ERR_INVALID_ARG, "%s", why);
    if (l->quantized || l->mx) return fail(SG_ERR_UNSUPPORTED, "the backward is implemented for dense layers only");
    if (!dx && !dw) return fail(SG_ERR_INVALID_ARG, "neither dx nor dw requested");
    if (B == 0) return SG_OK;
    if (!dy) return fail(SG_ERR_INVALID_ARG, "dy must not be NULL");
    if (dw && !x) return fail(SG_ERR_INVALID_ARG, "dw needs the forward input x");
    const bool small = dw_small_ok(l, B);
    const bool ws_ok = !small && workspace && aligned16(workspace) && dw_mfma_ok(l) && ws_bytes >= dw_ws_bytes(l, B);
    if (dw && workspace && !small && !ws_ok && dw_mfma_ok(l))
        return fail(SG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (16-byte aligned)", ws_bytes,
                    dw_ws_bytes(l, B));
    hipStream_t st = (hipStream_t)stream;
    if (dx) {
        if (wt_ok(l) && aligned16(dy) && aligned16(dx)) {
            // the sum_gradients all_sum: dx = sum_r dY_r W_r, a sharded-to-all
            // product on the transposed shards, ranks summed in order
            sg_status s2 = ensure_wt(l, st);
            if (s2 != SG_OK) return s2;
            sg::Problem p{};
            p.A = dy;
            p.lda = l->rows_r;
            p.a_seg = B * l->rows_r;
            p.M = (int)B;
            p.Kseg = (int)l->rows_r;
            p.nseg = l->P;
            p.dtype = l->dtype;
            p.W = l->wt;
            p.ldw = l->rows_r;
            p.w_seg = l->cols_r * l->rows_r;
            p.wfrag = 1;
            p.wsteps = l->rows_r / 32;
            p.N = (int)l->cols_r;
            p.out = dx;
            p.out_dtype = dx_dtype;
            p.out_map = sg::OUT_ROWMAJOR;
            p.ldo = l->cols_r;
            hipError_t e = run(p, choose_bwd(B, l->cols_r, l->P), st);
            if (e != hipSuccess) return hip_fail(e, "all_to_sharded backward dx");
        } else {
            sg::BwdDx p{};
            p.A = dy;
            p.lda = l->rows_r;
            p.a_seg = B * l->rows_r;
            p.W = l->w;
            p.ldw = l->cols_r;
            p.w_seg = l->rows_r * l->cols_r;
            p.wsteps = l->cols_r / 32;
            p.wfrag = l->wfrag;
            p.dtype = l->dtype;
            p.M = (int)B;
            p.N = (int)l->cols_r;
            p.K = (int)l->rows_r;
            p.nseg = l->P;
            p.reduce = 1;
            p.stacked = 1;
            p.out = dx;
            p.out_dtype = dx_dtype;
            hipError_t e = sg::launch_bwd_dx(p, st);
            if (e != hipSuccess) return hip_fail(e, "all_to_sharded backward dx");
        }
    }
    if (dw) {
        if (small && aligned16(x) && aligned16(dy)) return dw_small(l, x, dy, B, dw, dw_dtype, st);
        if (ws_ok && aligned16(x) && aligned16(dy) && aligned16(dw)) return dw_mfma(l, x, dy, B, dw, dw_dtype, workspace, st);
        sg::BwdDw q{};
        q.G = dy;
        q.ldg = l->rows_r;
        q.g_seg = B * l->rows_r;
        q.X = x;
        q.ldx = l->cols_r;
        q.x_seg = 0;
        q.dtype = l->dtype;
        q.M = (int)B;
        q.R = (int)l->rows_r;
        q.C = (int)l->cols_r;
        q.nseg = l->P;
        q.out = dw;
        q.out_dtype = dw_dtype;
        hipError_t e = sg::launch_bwd_dw(q, st);
        if (e != hipSuccess) return hip_fail(e, "all_to_sharded backward dw");
    }
    return SG_OK;
}

sg_status sg_sharded_to_all_backward(const sg_layer* l, const void* x_partial, const void* dy, int64_t B,
                                     void* dx_partial, sg_dtype dx_dtype, void* dw, sg_dtype dw_dtype, void* workspace,
                                     size_t ws_bytes, void* stream) {
    g_err.clear();
    if (const char* why = bwd_check(l, SG_SHARDED_TO_ALL, B, dx_dtype, dw_dtype)) return fail(SG_ERR_INVALID_ARG, "%s", why);
    if (l->quantized || l->mx) return fail(SG_ERR_UNSUPPORTED, "the backward is implemented for dense layers only");
    if (!dx_partial && !dw) return fail(SG_ERR_INVALID_ARG, "neither dx nor dw requested");
    if (B == 0) return SG_OK;
    if (!dy) return fail(SG_ERR_INVALID_ARG, "dy must not be NULL");
    if (dw && !x_partial) return fail(SG_ERR_INVALID_ARG, "dw needs the forward input x_partial");
    const bool small = dw_small_ok(l, B);
    const bool ws_ok = !small && workspace && aligned16(workspace) && dw_mfma_ok(l) && ws_bytes >= dw_ws_bytes(l, B);
    if (dw && workspace && !small && !ws_ok && dw_mfma_ok(l))
        return fail(SG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed (16-byte aligned)", ws_bytes,
                    dw_ws_bytes(l, B));
    hipStream_t st = (hipStream_t)stream;
    if (dx_partial) {
        if (wt_ok(l) && aligned16(dy) && aligned16(dx_partial)) {
            // every rank receives the full dY: dX_r = dY W_r, an all-to-sharded
            // product on the stacked W_r^T with a sharded output
            sg_status s2 = ensure_wt(l, st);
            if (s2 != SG_OK) return s2;
            sg::Problem p{};
            p.A = dy;
            p.lda = l->out_dims;
            p.M = (int)B;
            p.Kseg = (int)l->out_dims;
            p.nseg = 1;
            p.dtype = l->dtype;
            p.W = l->wt;
            p.ldw = l->out_dims;
            p.wfrag = 1;
            p.wsteps = l->out_dims / 32;
            p.N = (int)l->in_dims;
            p.out = dx_partial;
            p.out_dtype = dx_dtype;
            p.out_map = sg::OUT_SHARDED;
            p.nloc = l->cols_r;
            hipError_t e = run(p, choose_bwd(B, l->in_dims, 1), st);
            if (e != hipSuccess) return hip_fail(e, "sharded_to_all backward dx");
        } else {
            sg::BwdDx p{};
            p.A = dy;
            p.lda = l->rows_r;
            p.a_seg = 0;
            p.W = l->w;
            p.ldw = l->cols_r;
            p.w_seg = l->rows_r * l->cols_r;
            p.wsteps = l->cols_r / 32;
            p.wfrag = l->wfrag;
            p.dtype = l->dtype;
            p.M = (int)B;
            p.N = (int)l->cols_r;
            p.K = (int)l->rows_r;
            p.nseg = l->P;
            p.reduce = 0;
            p.out = dx_partial;
            p.out_dtype = dx_dtype;
            hipError_t e = sg::launch_bwd_dx(p, st);
            if (e != hipSuccess) return hip_fail(e, "sharded_to_all backward dx");
        }
    }
    if (dw) {
        if (small && aligned16(x_partial) && aligned16(dy)) return dw_small(l, x_partial, dy, B, dw, dw_dtype, st);
        if (ws_ok && aligned16(x_partial) && aligned16(dy) && aligned16(dw))
            return dw_mfma(l, x_partial, dy, B, dw, dw_dtype, workspace, st);
        sg::BwdDw q{};
        q.G = dy;
        q.ldg = l->rows_r;
        q.g_seg = 0;
        q.X = x_partial;
        q.ldx = l->cols_r;
        q.x_seg = B * l->cols_r;
        q.dtype = l->dtype;
        q.M = (int)B;
        q.R = (int)l->rows_r;
        q.C = (int)l->cols_r;
        q.nseg = l->P;
        q.out = dw;
        q.out_dtype = dw_dtype;
        hipError_t e = sg::launch_bwd_dw(q, st);
        if (e != hipSuccess) return hip_fail(e, "sharded_to_all backward dw");
    }
    return SG_OK;
}

// SUMMA backward workspace: X^T (K, M) row-major, then dY's q step blocks
// transposed, dY_t^T (N, M/q), fragment-major
static bool summa_bwd_mfma_ok(sg_dtype dtype, int64_t M, int64_t K, int64_t N, int q) {
    return (dtype == SG_BF16 || dtype == SG_F16) && q >= 1 && M % q == 0 && (M / q) % 32 == 0 && N % 16 == 0 &&
           K % 8 == 0;
}
static size_t summa_bwd_ws(int64_t M, int64_t K, int64_t N) {
    return align256((size_t)(K * M) * 2) + align256((size_t)(N * M) * 2);
}

size_t sg_summa_backward_workspace(sg_dtype dtype, int64_t M, int64_t K, int64_t N, int q) {
    if (M <= 0 || K <= 0 || N <= 0 || M > INT32_MAX || K > INT32_MAX || N > INT32_MAX) return 0;
    return summa_bwd_mfma_ok(dtype, M, K, N, q) ? summa_bwd_ws(M, K, N) : 0;
}

// SUMMA backward ([SUMMA] Matmul_ABT_2D / Matmul_ATB_2D): dX = dY A^T with the
// inner dimension N cut into the q step blocks (the K segments of the matrix-
// core kernels, summed in step order); dA = X^T dY with the tokens M cut into
// the q step blocks, on the same kernels over the workspace's transposed
// copies (else the vector-unit weight-gradient kernel).
sg_status sg_summa_backward(const void* X, const void* A, const void* dY, sg_dtype dtype, int64_t M, int64_t K,
                            int64_t N, int q, float* dX, float* dA, void* workspace, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!dtype_ok(dtype)) return fail(SG_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || K < 0 || N < 0 || M > INT32_MAX || K > INT32_MAX || N > INT32_MAX)
        return fail(SG_ERR_INVALID_ARG, "matrix sizes out of range");
    if (q < 1) return fail(SG_ERR_NOT_DIVISIBLE, "the processor grid must be q x q with q >= 1 (got q = %d)", q);
    if (M % q || K % q || N % q)
        return fail(SG_ERR_NOT_DIVISIBLE, "M, K, N (%lld, %lld, %lld) must be divisible by q = %d",
                    (long long)M, (long long)K, (long long)N, q);
    if (!dX && !dA) return fail(SG_ERR_INVALID_ARG, "neither dX nor dA requested");
    const bool mm = summa_bwd_mfma_ok(dtype, M, K, N, q);
    if (workspace && mm && ws_bytes < summa_bwd_ws(M, K, N))
        return fail(SG_ERR_WORKSPACE, "SUMMA backward workspace of %zu bytes, %zu needed", ws_bytes,
                    summa_bwd_ws(M, K, N));
    if (M == 0 || K == 0 || N == 0) return SG_OK;
    if (!dY || (dX && !A) || (dA && !X)) return fail(SG_ERR_INVALID_ARG, "dY, and A for dX / X for dA, must not be NULL");
    hipStream_t hs = (hipStream_t)stream;
    if (dX) {
        const int64_t bn = N / q;
        sg::Problem p{};
        p.A = dY;
        p.lda = N;
        p.a_seg = bn;  // step t: columns [t bn, (t+1) bn) of dY and of A
        p.W = A;
        p.ldw = N;
        p.w_seg = bn;
        p.M = (int)M;
        p.N = (int)K;
        p.Kseg = (int)bn;
        p.nseg = q;
        p.dtype = dtype;
        p.out = dX;
        p.out_dtype = SG_F32;
        p.out_map = sg::OUT_ROWMAJOR;
        p.ldo = K;
        const bool mfma = dtype != SG_F32 && bn % 8 == 0 && N % 8 == 0 && aligned16(dY) && aligned16(A) && aligned16(dX);
        const Kind k = !mfma ? K_GENERIC : (M >= 512 ? K_TILE0 : K_TILE1);
        hipError_t e = run(p, k, hs);
        if (e != hipSuccess) return hip_fail(e, "summa backward dX");
    }
    if (dA) {
        if (mm && workspace && aligned16(workspace) && aligned16(X) && aligned16(dY) && aligned16(dA)) {
            const int64_t bm = M / q;
            void* xt = workspace;
            void* gt = (char*)workspace + align256((size_t)(K * M) * 2);
            hipError_t e = sg::transpose16(xt, X, 1, M, K, M, hs);     // X^T, (K, M)
            if (e == hipSuccess) e = sg::t_frag(gt, dY, q, bm, N, bm, hs);  // dY_t^T, q x (N, M/q)
            if (e != hipSuccess) return hip_fail(e, "summa backward operand transform");
            sg::Problem p{};
            p.A = xt;
            p.lda = M;
            p.a_seg = bm;  // step t: columns [t bm, (t+1) bm) of X^T
            p.M = (int)K;
            p.Kseg = (int)bm;
            p.nseg = q;
            p.dtype = dtype;
            p.W = gt;
            p.ldw = bm;
            p.w_seg = N * bm;
            p.wfrag = 1;
            p.wsteps = bm / 32;
            p.N = (int)N;
            p.out = dA;
            p.out_dtype = SG_F32;
            p.out_map = sg::OUT_ROWMAJOR;
            p.ldo = N;
            e = run(p, K >= 512 ? K_TILE0 : K_TILE1, hs);
            if (e != hipSuccess) return hip_fail(e, "summa backward dA");
            return SG_OK;
        }
        sg::BwdDw w{};
        w.G = X;  // dA[k][n] = sum_m X[m][k] dY[m][n]
        w.ldg = K;
        w.X = dY;
        w.ldx = N;
        w.dtype = dtype;
        w.M = (int)M;
        w.R = (int)K;
        w.C = (int)N;
        w.nseg = 1;
        w.out = dA;
        w.out_dtype = SG_F32;
        hipError_t e = sg::launch_bwd_dw(w, hs);
        if (e != hipSuccess) return hip_fail(e, "summa backward dA");
    }
    return SG_OK;
}

// bytes of the transposed fragment-major copy of A the MFMA path reads
static size_t summa_ws_bytes(sg_dtype dtype, int64_t K, int64_t N, int q) {
    if (dtype != SG_BF16 && dtype != SG_F16) return 0;
    if (q < 1 || K <= 0 || N <= 0 || K % q || (K / q) % 32 || N % 16) return 0;
    return (size_t)(K * N) * 2;
}

size_t sg_summa_workspace(sg_dtype dtype, int64_t K, int64_t N, int q) {
    if (K > INT32_MAX || N > INT32_MAX) return 0;
    return summa_ws_bytes(dtype, K, N, q);
}

sg_status sg_summa_matmul(const void* X, const void* A, sg_dtype dtype, int64_t M, int64_t K, int64_t N,
                          int q, float* Y, int accumulate, int fused, void* workspace, size_t ws_bytes,
                          void* stream) {
    g_err.clear();
    if (!dtype_ok(dtype)) return fail(SG_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || K < 0 || N < 0 || M > INT32_MAX || K > INT32_MAX || N > INT32_MAX)
        return fail(SG_ERR_INVALID_ARG, "matrix sizes out of range");
    if (q < 1) return fail(SG_ERR_NOT_DIVISIBLE, "the processor grid must be q x q with q >= 1 (got q = %d)", q);
    if (M % q || K % q || N % q)
        return fail(SG_ERR_NOT_DIVISIBLE, "M, K, N (%lld, %lld, %lld) must be divisible by q = %d",
                    (long long)M, (long long)K, (long long)N, q);
    if (accumulate != 0 && accumulate != 1) return fail(SG_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    if (fused != 0 && fused != 1) return fail(SG_ERR_INVALID_ARG, "fused must be 0 or 1");
    const size_t need = summa_ws_bytes(dtype, K, N, q);
    if (workspace && ws_bytes < need)
        return fail(SG_ERR_WORKSPACE, "SUMMA workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (M == 0 || N == 0) return SG_OK;
    if (!X || !A || !Y) return fail(SG_ERR_INVALID_ARG, "X, A and Y must not be NULL");
    hipStream_t hs = (hipStream_t)stream;
    const int64_t bk = K / q;
    const bool mfma = dtype != SG_F32 && N % 8 == 0 && bk % 8 == 0 && aligned16(X) && aligned16(A) && aligned16(Y);
    const Kind k = !mfma ? K_GENERIC : (M >= 512 ? K_TILE0 : K_TILE1);
    // with a workspace the MFMA kernels read A_t^T fragment-major, as they read
    // a linear layer's weights; without one the tile kernels read A in place
    const bool frag = k != K_GENERIC && need > 0 && workspace && aligned16(workspace);
    const size_t esz = dtype_size(dtype);
    sg::Problem p{};
    p.M = (int)M;
    p.N = (int)N;
    p.dtype = dtype;
    p.lda = K;
    p.out = Y;
    p.out_dtype = SG_F32;
    p.out_map = sg::OUT_ROWMAJOR;
    p.ldo = N;
    if (K == 0) {
        if (!accumulate) HIP_TRY(hipMemsetAsync(Y, 0, (size_t)(M * N) * 4, hs), "clear Y");
        return SG_OK;
    }
    if (frag) {
        HIP_TRY(sg::nn_to_frag(workspace, A, K, N, q, hs), "SUMMA operand transform");
        p.wfrag = 1;
        p.wsteps = bk / 32;
        p.ldw = bk;
    } else {
        p.nn = 1;
        p.ldw = N;
    }
    // block t of the right operand: rows [t bk, (t + 1) bk) of A, or its transposed copy
    const int64_t w_block = bk * N;
    if (fused) {
        // one launch: the K loop visits step t's panel X_it, A_tj for t = 0 .. q-1
        p.A = X;
        p.a_seg = bk;
        p.W = frag ? workspace : A;
        p.w_seg = w_block;
        p.Kseg = (int)bk;
        p.nseg = q;
        p.accumulate = accumulate;
        hipError_t e = run(p, k, hs);
        if (e != hipSuccess) return hip_fail(e, "summa launch");
        return SG_OK;
    }
    for (int t = 0; t < q; ++t) {
        // step t: every block (i, j) adds X_it A_tj into Y_ij in place
        p.A = (const char*)X + (size_t)(t * bk) * esz;
        p.W = (const char*)(frag ? workspace : A) + (size_t)(t * w_block) * esz;
        p.Kseg = (int)bk;
        p.nseg = 1;
        p.accumulate = (t > 0) || accumulate;
        hipError_t e = run(p, k, hs);
        if (e != hipSuccess) return hip_fail(e, "summa step launch");
    }
    return SG_OK;
}

sg_status sg_layer_info(const sg_layer* l, int64_t* out_dims, int64_t* in_dims, int* mode, int* segments,
                        int* P, sg_dtype* dtype, int* quantized) {
    g_err.clear();
    if (!l) return fail(SG_ERR_INVALID_ARG, "layer is NULL");
    if (out_dims) *out_dims = l->out_dims;
    if (in_dims) *in_dims = l->in_dims;
    if (mode) *mode = l->mode;
    if (segments) *segments = l->segments;
    if (P) *P = l->P;
    if (dtype) *dtype = l->dtype;
    if (quantized) *quantized = l->mx ? 2 : l->quantized;
    return SG_OK;
}

sg_status sg_layer_copy_shard(const sg_layer* l, int r, int what, void* dst, size_t dst_bytes, void* stream) {
    g_err.clear();
    if (!l || !dst) return fail(SG_ERR_INVALID_ARG, "layer and dst must not be NULL");
    if (r < 0 || r >= l->P) return fail(SG_ERR_INVALID_ARG, "rank %d out of range [0, %d)", r, l->P);
    hipStream_t hs = (hipStream_t)stream;
    const void* src = nullptr;
    size_t bytes = 0;
    const size_t esz = dtype_size(l->dtype);
    switch (what) {
    case 0:
        if (l->quantized) {
            bytes = (size_t)(l->rows_r * (l->cols_r / 8)) * 4;
            src = (const char*)l->w + r * bytes;
        } else if (l->mx) {
            bytes = (size_t)(l->rows_r * l->cols_r);
            src = (const char*)l->w + r * bytes;
        } else {
            bytes = (size_t)(l->rows_r * l->cols_r) * esz;
            src = (const char*)l->w + r * bytes;
        }
        break;
    case 1:
        if (!l->bias) return fail(SG_ERR_INVALID_ARG, "layer has no bias");
        if (l->mode == SG_ALL_TO_SHARDED) {
            bytes = (size_t)l->rows_r * esz;
            src = (const char*)l->bias + r * bytes;
        } else {
            bytes = (size_t)l->out_dims * esz;
            src = l->bias;
        }
        break;
    case 2:
    case 3:
        if (l->mx && what == 2) {
            bytes = (size_t)(l->rows_r * (l->cols_r / 32));
            src = (const char*)l->ms + r * bytes;
            break;
        }
        if (l->mx) return fail(SG_ERR_INVALID_ARG, "an MX FP8 layer has no quantization biases");
        if (!l->quantized) return fail(SG_ERR_INVALID_ARG, "layer is not quantized");
        bytes = (size_t)(l->rows_r * (l->cols_r / 64)) * 2;
        src = (const char*)(what == 2 ? l->qs : l->qb) + r * bytes;
        break;
    default: return fail(SG_ERR_INVALID_ARG, "unknown tensor selector %d", what);
    }
    if (dst_bytes < bytes) return fail(SG_ERR_INVALID_ARG, "dst holds %zu bytes, %zu needed", dst_bytes, bytes);
    if (l->mx && l->wfrag && what != 1) {
        // stored fragment-major: restore the row-major codes or scales of every
        // rank, then copy rank r's
        void* tmp = nullptr;
        const size_t all = bytes * l->P;
        HIP_TRY(hipMalloc(&tmp, all), "staging allocation");
        const int mats = l->mode == SG_ALL_TO_SHARDED ? 1 : l->P;
        const int64_t rows = l->mode == SG_ALL_TO_SHARDED ? l->out_dims : l->rows_r;
        hipError_t e = what == 0
                           ? sg::mx_transform((uint8_t*)tmp, (const uint8_t*)l->w, nullptr, nullptr, mats, rows, l->cols_r, 0, hs)
                           : sg::mx_transform(nullptr, nullptr, (uint8_t*)tmp, l->ms, mats, rows, l->cols_r, 0, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(dst, (const char*)tmp + r * bytes, bytes, hipMemcpyDefault, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        (void)hipFree(tmp);
        if (e != hipSuccess) return hip_fail(e, "shard copy");
        return SG_OK;
    }
    if (what == 0 && l->wfrag) {
        // stored fragment-major: restore the row-major layout of every rank,
        // then copy rank r's rows
        void* tmp = nullptr;
        const size_t all = bytes * l->P;
        HIP_TRY(hipMalloc(&tmp, all), "staging allocation");
        const int mats = l->mode == SG_ALL_TO_SHARDED ? 1 : l->P;
        const int64_t rows = l->mode == SG_ALL_TO_SHARDED ? l->out_dims : l->rows_r;
        hipError_t e = sg::frag_transform(tmp, l->w, mats, rows, l->cols_r, 0, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(dst, (const char*)tmp + r * bytes, bytes, hipMemcpyDefault, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        (void)hipFree(tmp);
        if (e != hipSuccess) return hip_fail(e, "shard copy");
        return SG_OK;
    }
    if (l->quantized && l->qfrag && what != 1) {
        // stored fragment-major: restore the row-major layout of every rank
        // (codes also back to the standard nibble order), then copy rank r
        void* tmp = nullptr;
        const size_t all = bytes * l->P;
        HIP_TRY(hipMalloc(&tmp, all), "staging allocation");
        const int mats = l->mode == SG_ALL_TO_SHARDED ? 1 : l->P;
        const int64_t rows = l->mode == SG_ALL_TO_SHARDED ? l->out_dims : l->rows_r;
        hipError_t e;
        if (what == 0) {
            e = sg::q4_transform((uint32_t*)tmp, (const uint32_t*)l->w, nullptr, nullptr, mats, rows, l->cols_r, 0, hs);
            if (e == hipSuccess) e = sg::q4_repack((uint32_t*)tmp, (int64_t)(all / 4), 0, hs);
        } else {
            e = sg::q4_transform(nullptr, nullptr, (uint16_t*)tmp, what == 2 ? l->qs : l->qb, mats, rows, l->cols_r, 0, hs);
        }
        if (e == hipSuccess) e = hipMemcpyAsync(dst, (const char*)tmp + r * bytes, bytes, hipMemcpyDefault, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        (void)hipFree(tmp);
        if (e != hipSuccess) return hip_fail(e, "shard copy");
        return SG_OK;
    }
    if (what == 0 && l->quantized) {
        // stored codes are in kernel order: restore the standard order
        void* tmp = nullptr;
        HIP_TRY(hipMalloc(&tmp, bytes), "staging allocation");
        hipError_t e = hipMemcpyAsync(tmp, src, bytes, hipMemcpyDeviceToDevice, hs);
        if (e == hipSuccess) e = sg::q4_repack((uint32_t*)tmp, (int64_t)(bytes / 4), 0, hs);
        if (e == hipSuccess) e = hipMemcpyAsync(dst, tmp, bytes, hipMemcpyDefault, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        (void)hipFree(tmp);
        if (e != hipSuccess) return hip_fail(e, "shard copy");
        return SG_OK;
    }
    HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, hs), "shard copy");
    HIP_TRY(hipStreamSynchronize(hs), "shard copy");
    return SG_OK;
}

void sg_layer_free(sg_layer* l) { free_layer(l); }

sg_status sg_time_next_launch(void* start_event, void* stop_event) {
    g_err.clear();
    sg::armed_events() = sg::ArmedEvents{(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return SG_OK;
}

}  // extern "C"
