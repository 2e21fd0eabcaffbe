// MFMA tile GEMMs for gfx950 fed by direct global -> LDS loads.  This file
// holds the ping-pong kernel (tile_pp_kernel: the prefill-shaped sharded GEMMs,
// many tokens against a rank's weight rows) and, further down, the few-token
// kernels for 33 to 256 tokens (tile_nw_kernel, tile_nw64_kernel and, for MX
// FP8 weights at any token count, tile_nw_mx_kernel), which reuse its loads
// and fragment reads.
// Same products and epilogues as tile.hip's NT / SWIGLU modes.
//
// Ping-pong kernel: 256 x 256 output tiles (SwiGLU: 256 tokens x 128 outputs
// from 256 interleaved gate/up rows), BK = 32, 512 threads.
//
// Schedule (ping-pong).  The 8 waves form two groups of four, waves 0-3 and
// 4-7, so every SIMD hosts one wave of each.  Time runs in phases separated by
// workgroup barriers.  In a memory phase a wave reads the 12 MFMA operand
// fragments of one k tile from LDS into registers and then issues its share of
// the global -> LDS loads of the k tile three ahead; in a compute phase it
// runs the 16 MFMAs of the k tile it read (a 128 x 64 block of the tile).
// Group 0 works on k tile t in phases 2t (memory) and 2t + 1 (compute), group 1
// one phase later, so on each SIMD one wave feeds the matrix unit while the
// other waits on memory.  Measured on MI355X, the alternatives lose:
//  * one group with both roles per wave (one barrier per k tile) exposes the
//    LDS latency after every barrier on all waves at once;
//  * issuing the global -> LDS loads from a wave that is running MFMAs, even
//    one at a time between them, stalls that wave for ~150 cycles per load:
//    the loads stay in the memory phase, after the fragment reads.
//
// Loads.  buffer_load_dwordx4 ... lds puts each lane's 16 bytes straight into
// LDS slot (M0 + 16 lane), so the LDS holds 4 stages of 32 KB.  The operands
// are addressed through buffer resources: the per-lane byte offset is computed
// once and stays in one VGPR, the k advance is a scalar offset.  (With 64-bit
// per-lane addresses the compiler reuses those registers for the fragments
// read next, and such a write stalls the wave until the queued load has read
// its address.)  Offsets past a resource's range read zeros.
//
// LDS layout.  A wave-wide load fills 16 tile rows x 64 bytes (with
// fragment-major weights one contiguous 1 KB); the lane that owns LDS chunk c
// of row r fetches global chunk c ^ ((r >> 2) & 3).  A ds_read_b128 is served
// 16 lanes (16 rows) per 256 bytes, four 64-byte rows wide: row & 3 selects the
// quarter and the swizzle gives each row >> 2 its own chunk, so the fragment
// reads are conflict-free (swizzling by (r >> 1) & 3 measured at half rate).
//
// Rank split (sharded-to-all layers whose output gives too few tiles): the
// segments form gridDim.y groups of consecutive ranks; workgroup (tile, y)
// runs group y's k tiles and writes its fp32 partial tile to the caller's
// workspace, and a second kernel (split_reduce_kernel, tile.hip) adds each
// tile's partials in group (rank) order and stores the result.  The kernel boundary
// orders the partials' stores before their loads; an in-kernel handoff (the
// last workgroup of a tile to arrive sums the partials) needs a device-scope
// release per workgroup, and with eight groups of 256 x 256 tiles the
// releases and the one-workgroup sums cost more than the products (512
// tokens x 4096 outputs x 8 ranks of 1792: 230 us in one kernel against
// 90 us for the products alone).
//
// Rows past M or N read a clamped valid row (their outputs are never stored).
// Requirements (tile_dma_fits): NT or SwiGLU weights (no split with SwiGLU), K
// a multiple of 32, operand extents below 2 GiB.
#include "internal.h"

namespace sg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// one wave-wide 16-byte-per-lane load into LDS (dest + 16 lane)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// byte extents of the operands (A: rows x segments; W: the rows the tiles address)
__host__ __device__ inline int64_t a_extent(const Problem& p) {
    return ((int64_t)(p.nseg - 1) * p.a_seg + (int64_t)(p.M - 1) * p.lda + p.Kseg) * 2;
}
__host__ __device__ inline int64_t w_extent(const Problem& p) {
    const int64_t rows = p.swiglu ? 2 * (int64_t)p.N : p.N;
    // fragment-major: the last segment's k steps of the last 16-row block
    const int64_t seg = p.wfrag ? (((rows - 1) >> 4) * p.wsteps + p.Kseg / 32) * 512 : (rows - 1) * p.ldw + p.Kseg;
    return ((int64_t)(p.nseg - 1) * p.w_seg + seg) * 2;
}

// LDS fragment read issued as inline assembly: the compiler's wait insertion
// cannot tell these reads from the direct-to-LDS loads still in flight and
// would otherwise wait for all of them (vmcnt(0)) before each read.  The
// caller waits for the reads with wait_lds, which also ties the registers.
__device__ __forceinline__ u32x4 lds_read16(const uint16_t* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
}

__device__ __forceinline__ u32x2 lds_read8(const uint8_t* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
__device__ __forceinline__ uint32_t lds_read4(const uint8_t* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
    uint32_t r;
    asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
// one wave-wide 4-byte-per-lane load into LDS (dest + 4 lane)
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// wait for every outstanding LDS read; ties the six fragments of one k step so
// that no use of them is scheduled before the wait
__device__ __forceinline__ void wait_lds(u32x4 (&w)[2], u32x4 (&x)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// s_waitcnt vmcnt(n) (n <= 63), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void store4(const Problem& p, int m, int64_t n, float (&v)[4]) {
    if (n >= p.N) return;
    if (p.bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < p.N) v[e] += load_as_f32(p.bias, p.dtype, n + e);
    }
    const bool full = n + 3 < p.N && (p.out_map == OUT_ROWMAJOR ? (p.ldo % 4 == 0) : (p.nloc % 4 == 0));
    const int64_t o = out_index(p, m, n);
    if (full && !p.accumulate && p.out_dtype != SG_F32) {
        u32x2 w;
        if (p.out_dtype == SG_BF16) {
            w[0] = f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            w[1] = f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        } else {
            w[0] = f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
            w[1] = f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
        }
        *(u32x2*)((uint16_t*)p.out + o) = w;
    } else if (full && p.out_dtype == SG_F32) {
        f32x4* dst = (f32x4*)((float*)p.out + o);
        f32x4 r = {v[0], v[1], v[2], v[3]};
        if (p.accumulate) r += *dst;
        *dst = r;
    } else {
        for (int e = 0; e < 4 && n + e < p.N; ++e) {
            const int64_t oe = out_index(p, m, n + e);
            float x = v[e];
            if (p.accumulate && p.out_dtype == SG_F32) x += ((const float*)p.out)[oe];
            store_from_f32(p.out, p.out_dtype, oe, x);
        }
    }
}

}  // namespace

// Buffers and waits of the ping-pong loop:
//  * k tile t lives in LDS stage t mod 4.  Its loads are issued at the end of
//    the memory phases of k tile t - 3 (each group its rows), into the stage
//    of k tile t - 1, whose last reader (group 1, phase 2t - 3) finished its
//    reads before the barrier that ends that phase.
//  * before each barrier that starts an even phase 2t, every wave waits until
//    its own loads of k tile t have landed (those of the two later k tiles may
//    stay in flight); the barrier then publishes k tile t to all waves.
//  * every wave passes the same 2 nkt + 2 barriers.
template <bool F16, bool SWIGLU, bool SPLIT>
__global__ __launch_bounds__(512) void tile_pp_kernel(Problem p, int tiles_m, int tiles_n) {
    constexpr int BM = 256, BN = 256, BK = 32, NW = 8, NS = 4;
    constexpr int WTM = 128, WTN = 64, NBM = WTM / 32, NBN = WTN / 32;
    constexpr int LPT = 2;  // loads per thread per operand and k tile
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    constexpr int TILE = BM * BK;
    __shared__ __attribute__((aligned(1024))) uint16_t sA[NS * TILE], sB[NS * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int group = wave >> 2;
    const int wave_m = wave & 1, wave_n = wave >> 1;

    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int gidx = tile / (GM * tiles_n);
    const int first_m = gidx * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - gidx * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * BM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;

    // load descriptors: load i of wave w fills tile rows (8 i + w) * 16 .. +16;
    // lane -> (row lr, LDS chunk lc); byte offsets from the operand base
    const int lr = lane >> 2, lc = lane & 3;
    uint32_t aoff[LPT], boff[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int row = (NW * i + wave) * 16 + lr;
        const int ch = lc ^ swz4(row);
        const int m = min(m0 + row, p.M - 1);
        aoff[i] = (uint32_t)(((int64_t)m * p.lda + ch * 8) * 2);
        int64_t wrow;
        if constexpr (SWIGLU) {
            const int64_t j = min(n0 + (row >> 6) * 32 + (row & 31), (int64_t)p.N - 1);
            wrow = weight_row(p, j, (row >> 5) & 1);
        } else {
            wrow = min(n0 + row, (int64_t)p.N - 1);
        }
        boff[i] = (uint32_t)((p.wfrag ? frag_offset(wrow, ch * 8, p.wsteps) : wrow * p.ldw + ch * 8) * 2);
    }
    const int bk_step = p.wfrag ? 16 : 1;  // elements of W per element of k
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, 0, (int)a_extent(p), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)p.W, 0, (int)w_extent(p), 0x00020000);
    const int ktiles_seg = p.Kseg / BK;
    const int gsegs = SPLIT ? p.nseg / (int)gridDim.y : p.nseg;  // segments of this workgroup
    const int nkt = ktiles_seg * gsegs;
    const int seg_lo = SPLIT ? (int)blockIdx.y * gsegs : 0;     // its first segment

    auto issue = [&](int kt) {
        const int s = seg_lo + kt / ktiles_seg;
        const int k0 = (kt - (s - seg_lo) * ktiles_seg) * BK;
        const uint32_t sa = (uint32_t)((s * p.a_seg + k0) * 2);
        const uint32_t sw = (uint32_t)((s * p.w_seg + (int64_t)k0 * bk_step) * 2);
        uint16_t* a = sA + (kt % NS) * TILE;
        uint16_t* b = sB + (kt % NS) * TILE;
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            dma16(ra, aoff[i], sa, a + (NW * i + wave) * 16 * BK);
            dma16(rw, boff[i], sw, b + (NW * i + wave) * 16 * BK);
        }
    };
    // wait until this wave's loads of k tile t have landed; it has issued
    // those of every k tile up to min(t + 2, nkt - 1)
    auto wait_tile = [&](int t) {
        const int later = min(t + 2, nkt - 1) - t;
        if (later >= 2) wait_vm<4 * LPT>();
        else if (later == 1) wait_vm<2 * LPT>();
        else wait_vm<0>();
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane & 31, fch = lane >> 5;
    u32x4 w0[NBN], x0[NBM], w1[NBN], x1[NBM];
    auto read = [&](int t, int kk, u32x4 (&wf)[NBN], u32x4 (&xf)[NBM]) {
        const uint16_t* a = sA + (t % NS) * TILE;
        const uint16_t* b = sB + (t % NS) * TILE;
        const int c = kk * 2 + fch;
#pragma unroll
        for (int i = 0; i < NBN; ++i) {
            const int row = wave_n * WTN + i * 32 + frow;
            wf[i] = lds_read16(b + row * BK + ((c ^ swz4(row)) << 3));
        }
#pragma unroll
        for (int j = 0; j < NBM; ++j) {
            const int row = wave_m * WTM + j * 32 + frow;
            xf[j] = lds_read16(a + row * BK + ((c ^ swz4(row)) << 3));
        }
    };
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int t = 0; t < NS - 1 && t < nkt; ++t) issue(t);
    if (nkt > 0) wait_tile(0);
    __builtin_amdgcn_s_barrier();
    // phase 0 of group 1 is idle: one extra barrier puts it one phase behind
    if (group == 1) __builtin_amdgcn_s_barrier();
    for (int t = 0; t < nkt; ++t) {
        // memory phase of k tile t: fragment reads first, then the loads of
        // k tile t + 3 (a load queued ahead of the reads would hold them up)
        read(t, 0, w0, x0);
        read(t, 1, w1, x1);
        if (t + NS - 1 < nkt) issue(t + NS - 1);
        wait_lds(w0, x0);
        wait_lds(w1, x1);
        // for group 1 the next barrier starts phase 2t + 2: k tile t + 1 must land
        if (group == 1 && t + 1 < nkt) wait_tile(t + 1);
        barrier();
        // compute phase of k tile t
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(w0[i], x0[j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(w1[i], x1[j], acc[i][j]);
        if (group == 0 && t + 1 < nkt) wait_tile(t + 1);
        barrier();
    }
    if (group == 0) __builtin_amdgcn_s_barrier();

    // ---- rank split: this group's partial tile to the workspace, thread tid's
    // float4 v (accumulator acc[i][j][4q .. 4q + 3], v = (i NBM + j) 4 + q) at
    // float4 index v * 512 + tid of the tile's slab
    if constexpr (SPLIT) {
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * ntiles + tile) * (BM * BN));
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    mine[((i * NBM + j) * 4 + q) * 512 + tid] = v;
                }
        return;
    }

    // epilogue: lane l of a 32 x 32 block holds column l & 31 (token) and rows
    // 8 blk + 4 (l >> 5) + e (weight rows) of the block
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (SWIGLU) {
                    // 32-row blocks alternate gate / up of the same 32 outputs
                    const int blk32 = wave_n * NBN + i;
                    n = n0 + (blk32 >> 1) * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i | 1][j][4 * blk + e];  // i even: i | 1 = i + 1
                } else {
                    n = n0 + wave_n * WTN + i * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * blk + e];
                }
                store4(p, m, n, v);
            });
        });
    });
}

// Few-token tile kernel (33 to 256 tokens): TM = 64 or 128 tokens x 128
// weight rows (SwiGLU: 64 gate rows and the 64 matching up rows), BK = 32, 4
// waves of TM/2 tokens x 64 rows.  In this range a layer is bound by
// streaming its weights, and the 256 x 256 tiles would waste most of their
// MFMA work on padding rows, so the tile is narrow and the LDS holds a deep
// ring of NS stages: k tile t + NS - 1 is issued while k tile t is read, one
// workgroup barrier per k tile.  The loads, the LDS layout and the fragment
// reads are the ping-pong kernel's (direct-to-LDS 16-byte loads through
// buffer resources, rows XOR-swizzled by (row >> 2) & 3).  Every wave issues
// the same number of loads for every k tile (past the last k tile, a repeat
// of it into a stage never read), so the wait before each barrier is a
// compile-time count.  SPLIT: as the ping-pong kernel (groups of consecutive
// segments, partial tiles summed by split_reduce_kernel).
template <int TM>
struct NarrowShape {
    static constexpr int BN = 128, BK = 32;
    static constexpr int WTM = TM / 2, WTN = 64, NBM = WTM / 32, NBN = WTN / 32;
    static constexpr int LA = TM / 64, LB = BN / 64, L = LA + LB;  // loads per thread per stage
    static constexpr int SA = TM * BK, SB = BN * BK;               // elements per stage
    static constexpr int NS = TM == 64 ? 8 : TM == 128 ? 6 : 4;    // 96 KB of stages
};

template <int NBN, int NBM>
__device__ __forceinline__ void wait_lds_n(u32x4 (&w)[NBN], u32x4 (&x)[NBM]) {
    static_assert(NBN == 2 && (NBM == 1 || NBM == 2 || NBM == 4), "fragment counts of the few-token tiles");
    if constexpr (NBM == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]));
    else if constexpr (NBM == 2)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

template <bool F16, bool SWIGLU, bool SPLIT, int TM>
__global__ __launch_bounds__(256) void tile_nw_kernel(Problem p, int tiles_m, int tiles_n) {
    using S = NarrowShape<TM>;
    constexpr int BN = S::BN, BK = S::BK, NW = 4, NS = S::NS;
    constexpr int WTM = S::WTM, WTN = S::WTN, NBM = S::NBM, NBN = S::NBN;
    constexpr int LA = S::LA, LB = S::LB, L = S::L, SA = S::SA, SB = S::SB;
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sA[NS * SA], sB[NS * SB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave & 1, wave_n = wave >> 1;

    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int gidx = tile / (GM * tiles_n);
    const int first_m = gidx * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - gidx * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * TM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;

    // load i of wave w fills rows (4 i + w) * 16 .. + 16 of its operand
    const int lr = lane >> 2, lc = lane & 3;
    uint32_t aoff[LA], boff[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int row = (NW * i + wave) * 16 + lr;
        const int m = min(m0 + row, p.M - 1);
        aoff[i] = (uint32_t)(((int64_t)m * p.lda + (lc ^ swz4(row)) * 8) * 2);
    }
    // weight fragments that are whole stored 16-row blocks are copied verbatim
    // (lane l at 16 l: the load's lanes walk the 1 KB in address order) and
    // read with the 64-wide form's addressing; others through the swizzled
    // row layout (decode-MLP layers at 256 tokens: gate|up 110 -> 103 us, down
    // 58 -> 53 us, the same results)
    const bool wv = p.wfrag && p.N % 16 == 0 && (!SWIGLU || p.floc % 16 == 0);
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int row = (NW * i + wave) * 16 + lr;
        const int ch = lc ^ swz4(row);
        int64_t wrow;
        if (wv) {
            const int r0 = (NW * i + wave) * 16;
            if constexpr (SWIGLU) {
                const int64_t j = n0 + (r0 >> 6) * 32 + (r0 & 31);
                wrow = weight_row(p, j < p.N ? j : (int64_t)p.N - 16, (r0 >> 5) & 1);
            } else {
                wrow = n0 + r0 < p.N ? n0 + r0 : (int64_t)p.N - 16;
            }
            boff[i] = (uint32_t)(frag_offset(wrow, 0, p.wsteps) * 2 + lane * 16);
            continue;
        }
        if constexpr (SWIGLU) {
            const int64_t j = min(n0 + (row >> 6) * 32 + (row & 31), (int64_t)p.N - 1);
            wrow = weight_row(p, j, (row >> 5) & 1);
        } else {
            wrow = min(n0 + row, (int64_t)p.N - 1);
        }
        boff[i] = (uint32_t)((p.wfrag ? frag_offset(wrow, ch * 8, p.wsteps) : wrow * p.ldw + ch * 8) * 2);
    }
    const int bk_step = p.wfrag ? 16 : 1;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, 0, (int)a_extent(p), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)p.W, 0, (int)w_extent(p), 0x00020000);
    const int ktiles_seg = p.Kseg / BK;
    const int gsegs = SPLIT ? p.nseg / (int)gridDim.y : p.nseg;
    const int nkt = ktiles_seg * gsegs;
    const int seg_lo = SPLIT ? (int)blockIdx.y * gsegs : 0;

    // k tile kt into stage kt mod NS; past the last k tile, the last again
    auto issue = [&](int kt) {
        uint16_t* a = sA + (kt % NS) * SA;
        uint16_t* b = sB + (kt % NS) * SB;
        const int kc = min(kt, nkt - 1);
        const int s = seg_lo + kc / ktiles_seg;
        const int k0 = (kc - (s - seg_lo) * ktiles_seg) * BK;
        const uint32_t sa = (uint32_t)((s * p.a_seg + k0) * 2);
        const uint32_t sw = (uint32_t)((s * p.w_seg + (int64_t)k0 * bk_step) * 2);
#pragma unroll
        for (int i = 0; i < LA; ++i) dma16(ra, aoff[i], sa, a + (NW * i + wave) * 16 * BK);
#pragma unroll
        for (int i = 0; i < LB; ++i) dma16(rw, boff[i], sw, b + (NW * i + wave) * 16 * BK);
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane & 31, fch = lane >> 5;
    u32x4 w0[NBN], x0[NBM], w1[NBN], x1[NBM];
    auto read = [&](int t, int kk, u32x4 (&wf)[NBN], u32x4 (&xf)[NBM]) {
        const uint16_t* a = sA + (t % NS) * SA;
        const uint16_t* b = sB + (t % NS) * SB;
        const int c = kk * 2 + fch;
#pragma unroll
        for (int i = 0; i < NBN; ++i) {
            const int row = wave_n * WTN + i * 32 + frow;
            wf[i] = lds_read16(wv ? b + (row >> 4) * 512 + ((row & 15) + 16 * c) * 8
                                  : b + row * BK + ((c ^ swz4(row)) << 3));
        }
#pragma unroll
        for (int j = 0; j < NBM; ++j) {
            const int row = wave_m * WTM + j * 32 + frow;
            xf[j] = lds_read16(a + row * BK + ((c ^ swz4(row)) << 3));
        }
    };

    if (nkt > 0) {
        for (int t = 0; t < NS - 1; ++t) issue(t);
        for (int t = 0; t < nkt; ++t) {
            // this wave's loads of k tile t have landed (those of the NS - 2
            // later k tiles may be in flight); the barrier publishes k tile t
            // and ends every wave's reads of k tile t - 1, whose stage the
            // loads of k tile t + NS - 1 reuse
            wait_vm<(NS - 2) * L>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read(t, 0, w0, x0);
            read(t, 1, w1, x1);
            issue(t + NS - 1);
            wait_lds_n<NBN, NBM>(w0, x0);
            wait_lds_n<NBN, NBM>(w1, x1);
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(w0[i], x0[j], acc[i][j]);
#pragma unroll
            for (int i = 0; i < NBN; ++i)
#pragma unroll
                for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(w1[i], x1[j], acc[i][j]);
        }
        // no load may still be writing this workgroup's LDS when it ends
        wait_vm<0>();
    }

    if constexpr (SPLIT) {
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * ntiles + tile) * (TM * BN));
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    mine[((i * NBM + j) * 4 + q) * 256 + tid] = v;
                }
        return;
    }

    // epilogue: lane l of a 32 x 32 block holds column l & 31 (token) and rows
    // 8 blk + 4 (l >> 5) + e (weight rows) of the block
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (SWIGLU) {
                    n = n0 + wave_n * 32 + 8 * blk + 4 * hi;  // blocks 2 wave_n (gate), 2 wave_n + 1 (up)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i | 1][j][4 * blk + e];  // i even: i | 1 = i + 1
                } else {
                    n = n0 + wave_n * WTN + i * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * blk + e];
                }
                store4(p, m, n, v);
            });
        });
    });
}

// token tile of the few-token kernel
int tile_nw_tm(int M, bool fp8) { return M <= 64 ? 64 : (M <= 128 || fp8) ? 128 : 256; }


// The few-token tile with 64-wide k tiles, for fragment-major weights whose
// 16-row blocks are whole stored blocks (SwiGLU: rank widths a multiple of
// 16): a wave-wide load then brings one stored 1 KB weight fragment verbatim
// (eight whole 128-byte lines), or eight 128-byte activation rows (XOR-
// swizzled by (row >> 1) & 7), where the 32-wide tiles load 64-byte halves of
// sixteen activation rows.  Fewer cache lines per byte relieve the L1, which
// stalled the address unit for ~44% of the kernel's cycles at 64 tokens
// (decode gate|up at 64 tokens 54 -> 49 us, at 128 tokens 69 -> 58 us, the
// same results bit for bit: the k order is unchanged).  Weight fragment f of
// a stage holds (16-row block f >> 1, 32-wide step f & 1); lane l of a k16
// step kk reads row r's chunk 2 (kk & 1) + (l >> 5) of fragment
// (r >> 4, kk >> 1), which is lane (r & 15) + 16 chunk of it.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// wait for the k tile's fragment reads; ties every fragment register
template <int NBN, int NBM>
__device__ __forceinline__ void wait_lds_k64(u32x4 (&w)[4][NBN], u32x4 (&x)[4][NBM]) {
    static_assert(NBN == 2 && (NBM == 1 || NBM == 2), "fragment counts");
    if constexpr (NBM == 1)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0][0]), "+v"(w[0][1]), "+v"(w[1][0]), "+v"(w[1][1]), "+v"(w[2][0]), "+v"(w[2][1]),
                       "+v"(w[3][0]), "+v"(w[3][1]), "+v"(x[0][0]), "+v"(x[1][0]), "+v"(x[2][0]), "+v"(x[3][0]));
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0][0]), "+v"(w[0][1]), "+v"(w[1][0]), "+v"(w[1][1]), "+v"(w[2][0]), "+v"(w[2][1]),
                       "+v"(w[3][0]), "+v"(w[3][1]), "+v"(x[0][0]), "+v"(x[1][0]), "+v"(x[2][0]), "+v"(x[3][0]),
                       "+v"(x[0][1]), "+v"(x[1][1]), "+v"(x[2][1]), "+v"(x[3][1]));
}

template <int TM>
struct Narrow64 {
    static constexpr int BN = 128, BK = 64;
    static constexpr int WTM = TM / 2, WTN = 64, NBM = WTM / 32, NBN = WTN / 32;
    static constexpr int LA = TM / 32, LB = 4, L = LA + LB;  // loads per thread per stage
    static constexpr int SA = TM * BK, SB = BN * BK;         // elements per stage
    static constexpr int NS = TM == 64 ? 4 : 3;              // 96 KB of stages
};

template <bool F16, bool SWIGLU, bool SPLIT, int TM>
__global__ __launch_bounds__(256) void tile_nw64_kernel(Problem p, int tiles_m, int tiles_n) {
    using S = Narrow64<TM>;
    constexpr int BN = S::BN, BK = S::BK, NW = 4, NS = S::NS;
    constexpr int WTM = S::WTM, WTN = S::WTN, NBM = S::NBM, NBN = S::NBN;
    constexpr int LA = S::LA, LB = S::LB, L = S::L, SA = S::SA, SB = S::SB;
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sA[NS * SA], sB[NS * SB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave & 1, wave_n = wave >> 1;
    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int gidx = tile / (GM * tiles_n);
    const int first_m = gidx * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - gidx * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * TM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;

    // A: load i of wave w fills LDS rows (4 i + w) * 8 .. + 8 (128-byte rows);
    // lane -> row lane >> 3, LDS chunk lane & 7, global chunk (lane & 7) ^ swz8(row).
    // Rows past M read a clamped valid row (never stored).
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int row = (NW * i + wave) * 8 + (lane >> 3);
        const int m = min(m0 + row, p.M - 1);
        aoff[i] = (uint32_t)(((int64_t)m * p.lda + (((lane & 7) ^ swz8(row)) << 3)) * 2);
    }
    // W: load i of wave w = fragment f = 4 i + w: 16-row block f >> 1, k step f & 1,
    // copied verbatim (1 KB, lane at 16 lane)
    uint32_t boff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int f = NW * i + wave, blk = f >> 1, st = f & 1;
        const int row = blk * 16;  // first tile row of the block
        int64_t wrow;
        if constexpr (SWIGLU) {
            const int64_t j = n0 + (row >> 6) * 32 + (row & 31);
            const int64_t jc = j < p.N ? j : (int64_t)p.N - 16;
            wrow = weight_row(p, jc, (row >> 5) & 1);
        } else {
            wrow = n0 + row < p.N ? n0 + row : (int64_t)p.N - 16;
        }
        boff[i] = (uint32_t)(frag_offset(wrow, 32 * st, p.wsteps) * 2 + lane * 16);
    }
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, 0, (int)a_extent(p), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)p.W, 0, (int)w_extent(p), 0x00020000);
    const int ktiles_seg = p.Kseg / BK;
    const int gsegs = SPLIT ? p.nseg / (int)gridDim.y : p.nseg;
    const int nkt = ktiles_seg * gsegs;
    const int seg_lo = SPLIT ? (int)blockIdx.y * gsegs : 0;

    auto issue = [&](int kt) {
        uint16_t* a = sA + (kt % NS) * SA;
        uint16_t* b = sB + (kt % NS) * SB;
        const int kc = min(kt, nkt - 1);
        const int s = seg_lo + kc / ktiles_seg;
        const int k0 = (kc - (s - seg_lo) * ktiles_seg) * BK;
        const uint32_t sa = (uint32_t)((s * p.a_seg + k0) * 2);
        const uint32_t sw = (uint32_t)((s * p.w_seg + (int64_t)k0 * 16) * 2);
#pragma unroll
        for (int i = 0; i < LA; ++i) dma16(ra, aoff[i], sa, a + (NW * i + wave) * 8 * BK);
#pragma unroll
        for (int i = 0; i < LB; ++i) dma16(rw, boff[i], sw, b + (NW * i + wave) * 512);
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane & 31, fch = lane >> 5;
    u32x4 wf[4][NBN], xf[4][NBM];
    auto read = [&](int t, int kk) {
        const uint16_t* a = sA + (t % NS) * SA;
        const uint16_t* b = sB + (t % NS) * SB;
#pragma unroll
        for (int i = 0; i < NBN; ++i) {
            const int r = wave_n * WTN + i * 32 + frow;
            const int chunk = 2 * (kk & 1) + fch;
            wf[kk][i] = lds_read16(b + ((r >> 4) * 2 + (kk >> 1)) * 512 + ((r & 15) + 16 * chunk) * 8);
        }
#pragma unroll
        for (int j = 0; j < NBM; ++j) {
            const int r = wave_m * WTM + j * 32 + frow;
            const int c = 2 * kk + fch;
            xf[kk][j] = lds_read16(a + r * BK + ((c ^ swz8(r)) << 3));
        }
    };

    if (nkt > 0) {
        for (int t = 0; t < NS - 1; ++t) issue(t);
        for (int t = 0; t < nkt; ++t) {
            wait_vm<(NS - 2) * L>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read(t, 0);
            read(t, 1);
            read(t, 2);
            read(t, 3);
            issue(t + NS - 1);
            wait_lds_k64<NBN, NBM>(wf, xf);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < NBN; ++i)
#pragma unroll
                    for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<F16>(wf[kk][i], xf[kk][j], acc[i][j]);
        }
        wait_vm<0>();
    }

    if constexpr (SPLIT) {
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * ntiles + tile) * (TM * BN));
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    mine[((i * NBM + j) * 4 + q) * 256 + tid] = v;
                }
        return;
    }
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (SWIGLU) {
                    n = n0 + wave_n * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i | 1][j][4 * blk + e];
                } else {
                    n = n0 + wave_n * WTN + i * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * blk + e];
                }
                store4(p, m, n, v);
            });
        });
    });
}

// The few-token tile on MX FP8 weights (bf16 activations): 64 or 128 tokens
// x 128 weight rows, 128-wide k tiles (one run of four 32-wide scale steps).
// It serves MX FP8 layers at every token count above 32: a 256-token tile
// would need more LDS than three stages leave, and the 128 x 128 tile kernel
// with a register-staged FP8 loader measured 1.7 to 1.9 times slower from 512
// to 4096 tokens on the decode-MLP layer shapes.
// A stage holds the activations (rows of 256 bytes, 16-byte chunks XOR-
// swizzled by row & 15), the sixteen stored 1 KB code fragments of the tile's
// eight 16-row blocks (two 64-wide pairs each, verbatim) and the blocks' E8M0
// scales of the run (8 x 64 bytes); all three arrive by direct-to-LDS loads,
// three stages in flight.  After the LDS read, each lane's eight codes of a
// k16 step become bf16 operands with v_cvt_scalef32_pk_bf16_fp8 and its row's
// scale of that 32-wide step (exact, as in the streaming kernel), and meet the
// activations in the bf16 MFMA.  Lane l of k16 step kk (pair kk >> 2, step
// parity (kk >> 1) & 1) reads row r's chunk 2 (kk & 1) + (l >> 5) of the
// pair's fragment: lane (r & 15) + 16 chunk of it, bytes 8 parity .. + 8.
template <int TM>
struct NarrowMx {
    static constexpr int BN = 128, BK = 128;
    static constexpr int WTM = TM / 2, WTN = 64, NBM = WTM / 32, NBN = WTN / 32;
    static constexpr int SAB = TM * 256, SWB = BN * BK, SSB = 1024;  // bytes per stage
    static constexpr int ST = SAB + SWB + SSB;
    static constexpr int LA = SAB / 4096, LB = 4, L = LA + LB + 1;  // loads per thread per stage
    static constexpr int NS = 3;
};

template <bool SWIGLU, bool SPLIT, int TM>
__global__ __launch_bounds__(256) void tile_nw_mx_kernel(Problem p, int tiles_m, int tiles_n) {
    using S = NarrowMx<TM>;
    constexpr int BN = S::BN, BK = S::BK, NW = 4, NS = S::NS;
    constexpr int WTM = S::WTM, WTN = S::WTN, NBM = S::NBM, NBN = S::NBN;
    constexpr int SAB = S::SAB, SWB = S::SWB, ST = S::ST, LA = S::LA, LB = S::LB, L = S::L;
    constexpr int NOUT = SWIGLU ? BN / 2 : BN;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * ST];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave & 1, wave_n = wave >> 1;
    const int ntiles = tiles_m * tiles_n;
    const int tile = xcd_remap(blockIdx.x, ntiles);
    constexpr int GM = 4;
    const int gidx = tile / (GM * tiles_n);
    const int first_m = gidx * GM;
    const int gsz = min(GM, tiles_m - first_m);
    const int tin = tile - gidx * GM * tiles_n;
    const int m0 = (first_m + tin % gsz) * TM;
    const int64_t n0 = (int64_t)(tin / gsz) * NOUT;

    // first stored row of the tile's 16-row block b (blocks past N: the last)
    auto block_row = [&](int b) -> int64_t {
        const int row = b * 16;
        if constexpr (SWIGLU) {
            const int64_t j = n0 + (row >> 6) * 32 + (row & 31);
            return weight_row(p, j < p.N ? j : (int64_t)p.N - 16, (row >> 5) & 1);
        } else {
            return n0 + row < p.N ? n0 + row : (int64_t)p.N - 16;
        }
    };
    // activations: load i of wave w fills rows (4 i + w) * 4 .. + 4; lane -> row
    // lane >> 4, LDS chunk lane & 15, global chunk (lane & 15) ^ (row & 15)
    uint32_t aoff[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int row = (NW * i + wave) * 4 + (lane >> 4);
        const int m = min(m0 + row, p.M - 1);
        aoff[i] = (uint32_t)(((int64_t)m * p.lda + (((lane & 15) ^ (row & 15)) << 3)) * 2);
    }
    // codes: load i of wave w = fragment f = 4 i + w (block f >> 1, pair f & 1)
    uint32_t coff[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int f = NW * i + wave;
        coff[i] = (uint32_t)(mx_code_offset(block_row(f >> 1), 64 * (f & 1), p.wsteps) + lane * 16);
    }
    // scales: waves 0 and 1 load blocks 4 w .. 4 w + 3 (16 rows x 4 bytes each);
    // waves 2 and 3 repeat them into the stage's unused half
    const int sb = 4 * (wave & 1) + (lane >> 4);
    const uint32_t soffl = (uint32_t)mx_scale_offset(block_row(sb) + (lane & 15), 0, p.wsteps);

    const int64_t rows = SWIGLU ? 2 * (int64_t)p.N : p.N, nblk = rows / 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, 0, (int)a_extent(p), 0x00020000);
    // extents: the last segment's k range of the last 16-row block
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.W, 0, (int)(((int64_t)p.nseg - 1) * p.w_seg + ((nblk - 1) * (p.wsteps / 2) + p.Kseg / 64) * 1024),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.ms, 0, (int)(((int64_t)p.nseg - 1) * p.ms_seg + ((nblk - 1) * (p.wsteps / 4) + p.Kseg / 128) * 64),
        0x00020000);
    const int ktiles_seg = p.Kseg / BK;
    const int gsegs = SPLIT ? p.nseg / (int)gridDim.y : p.nseg;
    const int nkt = ktiles_seg * gsegs;
    const int seg_lo = SPLIT ? (int)blockIdx.y * gsegs : 0;

    auto issue = [&](int kt) {
        uint8_t* st = smem + (kt % NS) * ST;
        const int kc = min(kt, nkt - 1);
        const int s = seg_lo + kc / ktiles_seg;
        const int k0 = (kc - (s - seg_lo) * ktiles_seg) * BK;
        const uint32_t sa = (uint32_t)((s * p.a_seg + k0) * 2);
        const uint32_t sw = (uint32_t)(s * p.w_seg + (int64_t)(k0 >> 6) * 1024);
        const uint32_t ss = (uint32_t)(s * p.ms_seg + (int64_t)(k0 >> 7) * 64);
#pragma unroll
        for (int i = 0; i < LA; ++i) dma16(ra, aoff[i], sa, (uint16_t*)(st + (NW * i + wave) * 1024));
#pragma unroll
        for (int i = 0; i < LB; ++i) dma16(rw, coff[i], sw, (uint16_t*)(st + SAB + (NW * i + wave) * 1024));
        dma4(rs, soffl, ss, st + SAB + SWB + wave * 256);
    };

    f32x16 acc[NBN][NBM];
#pragma unroll
    for (int i = 0; i < NBN; ++i)
#pragma unroll
        for (int j = 0; j < NBM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int frow = lane & 31, fch = lane >> 5;
    // one half of a stage: k16 steps 4 hf .. 4 hf + 3 (the 64-wide pair hf)
    auto half = [&](const uint8_t* st, int hf, const uint32_t (&sw)[NBN]) {
        u32x2 cw[4][NBN];
        u32x4 xf[4][NBM];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = 4 * hf + q, chunk = 2 * (q & 1) + fch, sp = q >> 1;
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
                const int r = wave_n * WTN + i * 32 + frow;
                cw[q][i] = lds_read8(st + SAB + ((r >> 4) * 2 + hf) * 1024 + ((r & 15) + 16 * chunk) * 16 + 8 * sp);
            }
#pragma unroll
            for (int j = 0; j < NBM; ++j) {
                const int r = wave_m * WTM + j * 32 + frow, c = 2 * kk + fch;
                xf[q][j] = lds_read16((const uint16_t*)(st + r * 256 + ((c ^ (r & 15)) << 4)));
            }
        }
        static_assert(NBN == 2 && (NBM == 1 || NBM == 2), "fragment counts of the few-token tiles");
        if constexpr (NBM == 1)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(cw[0][0]), "+v"(cw[0][1]), "+v"(cw[1][0]), "+v"(cw[1][1]), "+v"(cw[2][0]),
                           "+v"(cw[2][1]), "+v"(cw[3][0]), "+v"(cw[3][1]), "+v"(xf[0][0]), "+v"(xf[1][0]),
                           "+v"(xf[2][0]), "+v"(xf[3][0]));
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(cw[0][0]), "+v"(cw[0][1]), "+v"(cw[1][0]), "+v"(cw[1][1]), "+v"(cw[2][0]),
                           "+v"(cw[2][1]), "+v"(cw[3][0]), "+v"(cw[3][1]), "+v"(xf[0][0]), "+v"(xf[1][0]),
                           "+v"(xf[2][0]), "+v"(xf[3][0]), "+v"(xf[0][1]), "+v"(xf[1][1]), "+v"(xf[2][1]),
                           "+v"(xf[3][1]));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int stp = 2 * hf + (q >> 1);  // 32-wide step of the run
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
                const u32x4 wf = mx8_to_bf16(cw[q][i], (sw[i] >> (8 * stp)) & 0xFFu);
#pragma unroll
                for (int j = 0; j < NBM; ++j) acc[i][j] = mfma32<false>(wf, xf[q][j], acc[i][j]);
            }
        }
    };

    if (nkt > 0) {
        for (int t = 0; t < NS - 1; ++t) issue(t);
        for (int t = 0; t < nkt; ++t) {
            wait_vm<(NS - 2) * L>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t* st = smem + (t % NS) * ST;
            uint32_t sw[NBN];
#pragma unroll
            for (int i = 0; i < NBN; ++i) {
                const int r = wave_n * WTN + i * 32 + frow;
                sw[i] = lds_read4(st + SAB + SWB + (r >> 4) * 64 + (r & 15) * 4);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sw[0]), "+v"(sw[1]));
            half(st, 0, sw);
            // every wave has read k tile t - 1: its stage takes k tile t + NS - 1
            issue(t + NS - 1);
            half(st, 1, sw);
        }
        wait_vm<0>();
    }

    if constexpr (SPLIT) {
        f32x4* mine = (f32x4*)(p.ws + ((int64_t)blockIdx.y * ntiles + tile) * (TM * BN));
#pragma unroll
        for (int i = 0; i < NBN; ++i)
#pragma unroll
            for (int j = 0; j < NBM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    mine[((i * NBM + j) * 4 + q) * 256 + tid] = v;
                }
        return;
    }
    const int hi = lane >> 5;
    static_for<0, NBN>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (SWIGLU && (i & 1)) return;
        static_for<0, NBM>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int m = m0 + wave_m * WTM + j * 32 + (lane & 31);
            if (m >= p.M) return;
            static_for<0, 4>([&](auto bc) {
                constexpr int blk = decltype(bc)::value;
                int64_t n;
                float v[4];
                if constexpr (SWIGLU) {
                    n = n0 + wave_n * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = silu_f32(acc[i][j][4 * blk + e]) * acc[i | 1][j][4 * blk + e];
                } else {
                    n = n0 + wave_n * WTN + i * 32 + 8 * blk + 4 * hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * blk + e];
                }
                store4(p, m, n, v);
            });
        });
    });
}

// tiles of the few-token kernel
int tile_nw_count(int M, int N, int swiglu, bool fp8) {
    const int tm = tile_nw_tm(M, fp8), nout = swiglu ? 64 : 128;
    return ((M + tm - 1) / tm) * ((N + nout - 1) / nout);
}

// MX FP8 weights on the few-token tiles: fragment-major codes in whole stored
// 16-row blocks, 128-wide k tiles, bf16 activations
static bool nw_mx_ok(const Problem& p) {
    return p.wfrag && p.dtype == SG_BF16 && p.Kseg % 128 == 0 && p.N % 16 == 0 &&
           (!p.swiglu || p.floc % 16 == 0);
}

bool tile_nw_fits(const Problem& p) {
    return !p.nn && !(p.split && p.swiglu) && !p.wq && p.Kseg % 32 == 0 && (p.M <= 256 || p.fp8) &&
           (!p.fp8 || nw_mx_ok(p)) && a_extent(p) < (1LL << 31) && w_extent(p) < (1LL << 31);
}

template <int TM, bool SPLIT>
static void launch_nw_mx(const Problem& p, hipStream_t s, dim3 grid, int tm, int tn) {
    if (p.swiglu) {
        if constexpr (!SPLIT) launch(tile_nw_mx_kernel<true, false, TM>, grid, dim3(256), 0, s, p, tm, tn);
    } else {
        launch(tile_nw_mx_kernel<false, SPLIT, TM>, grid, dim3(256), 0, s, p, tm, tn);
    }
}

// the 64-wide k tiles: fragment-major weights whose 16-row blocks are whole
// stored blocks (64- and 128-token tiles; the 256-token tile would need 144 KB)
static bool nw64_ok(const Problem& p) {
    return p.wfrag && p.Kseg % 64 == 0 && p.N % 16 == 0 && (!p.swiglu || p.floc % 16 == 0);
}

template <int TM, bool SPLIT>
static void launch_nw_tm(const Problem& p, hipStream_t s, dim3 grid, int tm, int tn) {
    const bool f16 = p.dtype == SG_F16;
    if constexpr (TM <= 128) {
        if (nw64_ok(p)) {
            if (p.swiglu) {
                if constexpr (!SPLIT) {
                    if (f16) launch(tile_nw64_kernel<true, true, false, TM>, grid, dim3(256), 0, s, p, tm, tn);
                    else launch(tile_nw64_kernel<false, true, false, TM>, grid, dim3(256), 0, s, p, tm, tn);
                }
            } else {
                if (f16) launch(tile_nw64_kernel<true, false, SPLIT, TM>, grid, dim3(256), 0, s, p, tm, tn);
                else launch(tile_nw64_kernel<false, false, SPLIT, TM>, grid, dim3(256), 0, s, p, tm, tn);
            }
            return;
        }
    }
    if (p.swiglu) {
        if constexpr (!SPLIT) {
            if (f16) launch(tile_nw_kernel<true, true, false, TM>, grid, dim3(256), 0, s, p, tm, tn);
            else launch(tile_nw_kernel<false, true, false, TM>, grid, dim3(256), 0, s, p, tm, tn);
        }
    } else {
        if (f16) launch(tile_nw_kernel<true, false, SPLIT, TM>, grid, dim3(256), 0, s, p, tm, tn);
        else launch(tile_nw_kernel<false, false, SPLIT, TM>, grid, dim3(256), 0, s, p, tm, tn);
    }
}

hipError_t launch_tile_nw(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!tile_nw_fits(p)) return hipErrorInvalidValue;
    const int TMv = tile_nw_tm(p.M, p.fp8), nout = p.swiglu ? 64 : 128;
    const int tm = (p.M + TMv - 1) / TMv, tn = (p.N + nout - 1) / nout;
    const int groups = p.split ? split_groups(tm * tn, p.nseg) : 1;
    const dim3 grid(tm * tn, groups);
    if (p.fp8) {  // 64- or 128-token tiles
        if (TMv == 64) {
            if (p.split) launch_nw_mx<64, true>(p, s, grid, tm, tn);
            else launch_nw_mx<64, false>(p, s, grid, tm, tn);
        } else {
            if (p.split) launch_nw_mx<128, true>(p, s, grid, tm, tn);
            else launch_nw_mx<128, false>(p, s, grid, tm, tn);
        }
    } else if (TMv == 64) {
        if (p.split) launch_nw_tm<64, true>(p, s, grid, tm, tn);
        else launch_nw_tm<64, false>(p, s, grid, tm, tn);
    } else if (TMv == 128) {
        if (p.split) launch_nw_tm<128, true>(p, s, grid, tm, tn);
        else launch_nw_tm<128, false>(p, s, grid, tm, tn);
    } else {
        if (p.split) launch_nw_tm<256, true>(p, s, grid, tm, tn);
        else launch_nw_tm<256, false>(p, s, grid, tm, tn);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.split) return e;
    return launch_split_reduce(p, tm, tn, groups, TMv == 64 ? 3 : TMv == 128 ? 4 : 5, s);
}

bool tile_dma_fits(const Problem& p) {
    return !p.nn && !(p.split && p.swiglu) && !p.fp8 && !p.wq && p.Kseg % 32 == 0 && a_extent(p) < (1LL << 31) &&
           w_extent(p) < (1LL << 31);
}

hipError_t launch_tile_dma(const Problem& p, hipStream_t s) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!tile_dma_fits(p)) return hipErrorInvalidValue;
    const int nout = p.swiglu ? 128 : 256;
    const int tm = (p.M + 255) / 256, tn = (p.N + nout - 1) / nout;
    const bool f16 = p.dtype == SG_F16;
    const int groups = p.split ? tile_pp_groups(p.M, p.N, p.nseg) : 1;
    const dim3 grid(tm * tn, groups), block(512);
    if (p.swiglu) {
        if (f16) launch(tile_pp_kernel<true, true, false>, grid, block, 0, s, p, tm, tn);
        else launch(tile_pp_kernel<false, true, false>, grid, block, 0, s, p, tm, tn);
    } else if (p.split) {
        if (f16) launch(tile_pp_kernel<true, false, true>, grid, block, 0, s, p, tm, tn);
        else launch(tile_pp_kernel<false, false, true>, grid, block, 0, s, p, tm, tn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_split_reduce(p, tm, tn, groups, 0, s);
    } else {
        if (f16) launch(tile_pp_kernel<true, false, false>, grid, block, 0, s, p, tm, tn);
        else launch(tile_pp_kernel<false, false, false>, grid, block, 0, s, p, tm, tn);
    }
    return hipGetLastError();
}

}  // namespace sg
