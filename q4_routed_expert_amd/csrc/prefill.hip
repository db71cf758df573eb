// prefill.hip -- the expert part of one MoE layer for a chunk of T tokens:
//   (1) grouped gate/up GEMM over the expert-sorted rows, SiLU(gate)*up fused,
//       plus the shared expert over all tokens            -> h, h_sh (bf16)
//   (2) grouped down GEMM of the routed rows -> part (fp16 scaled by a power
//       of two per 32 columns of a row, one row per assignment)
//   (3) the shared expert's down GEMM with the fixed-order combine in its
//       epilogue:
//       y_t = bf16( sum_s w[t,s] * part[t*k+s] (slot order) + shared_t )
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill: keep routing on the GPU,
// dequantize in flight": the grouped GEMM dequantises one small Q4 tile at a
// time on chip, accumulates in FP32, writes bf16, never materialises the
// expanded weights; 32-row tiles.  Section "Decode: minimize bytes per token":
// the output projection is combined with the routing scores and the shared
// expert.
//
// Kernel design (gfx950).  One work item = up to 128 rows of one expert (the
// 128-row work map written by the routing, or a block of tokens for the shared
// expert) x one block of output columns.  A work group has 8 waves (two per
// SIMD).  Per K chunk of 128 (two quantisation groups):
//   - the activation rows are staged in LDS as bf16, XOR-swizzled by row so
//     that the 32 rows one matrix-core operand read touches fall in distinct
//     banks;
//   - each lane streams 2 x 16 contiguous bytes of one weight row straight
//     from HBM (lane n%32 <-> row n; the two halves of the wave take adjacent
//     16-byte pieces, so one load instruction covers 32 contiguous bytes of
//     each of 32 rows) and dequantises them in registers into the first
//     operand of v_mfma_f32_32x32x16_bf16: eight consecutive k of one row are
//     exactly one packed 32-bit word of codes.  The bf16 weights exist only in
//     VGPRs and each is dequantised once per work item, then reused for all
//     (up to four) 32-row M-subtiles;
//   - the weight stream runs several chunks deep in registers so that enough
//     bytes are outstanding per CU to keep HBM busy.
//
// Routed partial outputs are staged in fp16 for the combine.  fp16 keeps 11
// significant bits but overflows above 65504, so every 32 consecutive
// columns of an assignment's row are stored as fp16(v * 2^-e) with one
// exponent e per block, chosen so that the block's largest magnitude lands in
// [2^14, 2^15): the staging then costs at most 2^-12 of that magnitude for any
// input range (the exponents are one byte per block, [T][d/32][8] with the
// slot last, so the combine reads a token's k exponents in one load).
#include "internal.h"

namespace q4moe {

constexpr int kKC = 128;               // K per chunk
constexpr int kMT = kTileRows;         // rows per work item
constexpr int kSlots = kKC / 8;        // 16-byte slots per staged row
constexpr int kRowBytes = kKC * 2;     // bytes per staged row
constexpr int kTileBytes = kMT * kRowBytes;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 4;             // weight chunks held in registers
constexpr int kALoads = kMT * kSlots / kThreads;
constexpr int kPartCols = 32;          // columns per staging exponent
constexpr int kDnCols = 256;           // output columns of a down work unit: 8 waves x 32
static_assert(kMT * kSlots % kThreads == 0, "A tile split");

template <int N>
struct Int {
    static constexpr int value = N;
};

// s_waitcnt vmcnt(N), leaving the other counters alone (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ int lds_off(int row, int slot) {
    return row * kRowBytes + ((slot ^ (row & 15)) << 4);
}

// The staging exponent of a block of partial outputs whose largest magnitude
// is m: m * 2^-e lies in [2^14, 2^15) (below fp16's largest finite value),
// clamped to [-126, 127] (one signed byte).
__device__ __forceinline__ int part_exp(float m) {
    const int e = __builtin_amdgcn_frexp_expf(m) - 15;
    return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// Largest magnitude over the 32 values a lane pair (l, l + 32) holds of one
// output row in a 32x32 accumulator tile (16 each).
__device__ __forceinline__ float pair_absmax(const f32x16& acc) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(acc[i]));
    return fmaxf(m, __shfl_xor(m, 32, 64));
}

// Byte offset of the staging exponent of assignment a (token a / k, slot
// a % k) for the 32-column block holding column col.
__device__ __forceinline__ size_t part_exp_index(const PrefillArgs& a, int asg, int col) {
    const int t = asg / a.k, s = asg - t * a.k;
    return ((size_t)t * (a.d / kPartCols) + col / kPartCols) * kMaxTopK + s;
}


// ---------------------------------------------------------------------------
// Down projections.  Routed work items are the 128-row work map written by
// the routing (entries at or past *n_tiles are empty).
// ---------------------------------------------------------------------------
struct DownItem {
    int e, row0, M;
};

__device__ __forceinline__ bool routed_item(const PrefillArgs& a, int item, DownItem& it) {
    if (item >= *a.n_tiles) return false;
    it.e = a.tile_map[2 * item];
    it.row0 = a.tile_map[2 * item + 1];
    it.M = min(kMT, a.offsets[it.e + 1] - it.row0);
    return true;
}

// The dequantised weights are the first MFMA operand, so the 32x32 output
// tile is (weight row n) x (activation row): lane l holds activation row
// l % 32 of its subtile and, in elements 4g..4g+3, the four consecutive
// weight rows n = 8g + 4h + 0..3 (h = l / 32).  Lanes l and l + 32 hold the
// same activation row; they trade four-column groups so that each ends with
// two runs of eight consecutive columns, 16m + 8h .. +7 for m = 0, 1.  Both
// lanes of a pair take the same branches (same row).
//
// Routed rows: scaled by the block's staging exponent, stored whole as fp16
// (16 bytes per run) into `part` (row = assignment dst); lane h = 0 of the
// pair stores the exponent.
__device__ __forceinline__ void routed_store(const PrefillArgs& a, int dst, int wc, int half,
                                             const f32x16& acc) {
    const int e = part_exp(pair_absmax(acc));
    if (half == 0) a.pexp[part_exp_index(a, dst, wc)] = (int8_t)e;
    uint16_t* prow = a.part + (size_t)dst * a.d + wc;
    auto h16 = [&](float v0, float v1) {
        return pack_f16x2(__builtin_amdgcn_ldexpf(v0, -e), __builtin_amdgcn_ldexpf(v1, -e));
    };
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        uint2 own_lo, own_hi;
        own_lo.x = h16(acc[8 * m], acc[8 * m + 1]);
        own_lo.y = h16(acc[8 * m + 2], acc[8 * m + 3]);
        own_hi.x = h16(acc[8 * m + 4], acc[8 * m + 5]);
        own_hi.y = h16(acc[8 * m + 6], acc[8 * m + 7]);
        const uint2 send = half ? own_lo : own_hi;
        uint2 recv;
        recv.x = (uint32_t)__shfl_xor((int)send.x, 32, 64);
        recv.y = (uint32_t)__shfl_xor((int)send.y, 32, 64);
        const uint2 lo = half ? recv : own_lo;
        const uint2 hi = half ? own_hi : recv;
        *(u32x4*)(prow + 16 * m + 8 * half) = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
}

// One lane's share of one weight chunk: k in [kc + 32h, +32) (group kc/64)
// and [kc + 64 + 32h, +32) (group kc/64 + 1), h = lane / 32.  Scales and
// biases stay raw bf16 bits until use: converting them right after the load
// would make the wave wait for the load (and, since loads retire in order,
// for every older one), which would collapse the prefetch pipeline.
struct BChunk {
    u32x4 lo, hi;
    uint32_t sp, bp;  // scales / biases of the two groups (low half = the group of lo)
};

// Loads one lane's share of a weight chunk (row wrow, k from kc0 and kc1).
// With an even number of groups per row the two groups' scales (and biases)
// are one aligned 32-bit load; otherwise two 16-bit loads each.
__device__ __forceinline__ void load_bchunk(const Q4& W, size_t wrow, int K, int kc0, int kc1,
                                            int half, bool pair_sb, BChunk& st) {
    const uint32_t* qrow = W.q + wrow * (K / 8) + 4 * half;
    const size_t grow = wrow * (K / kGroup);
    st.lo = *(const u32x4*)(qrow + kc0 / 8);
    st.hi = *(const u32x4*)(qrow + kc1 / 8);
    if (pair_sb) {
        st.sp = *(const uint32_t*)(W.scale + grow + kc0 / kGroup);
        st.bp = *(const uint32_t*)(W.bias + grow + kc0 / kGroup);
    } else {
        st.sp = (uint32_t)W.scale[grow + kc0 / kGroup] | ((uint32_t)W.scale[grow + kc1 / kGroup] << 16);
        st.bp = (uint32_t)W.bias[grow + kc0 / kGroup] | ((uint32_t)W.bias[grow + kc1 / kGroup] << 16);
    }
}

// One work item's down GEMM with the activation tile streamed through LDS one
// K-chunk at a time (any inter, a multiple of 64), double buffered, one
// barrier per chunk; each wave owns 32 output columns (weight rows wrow..) and
// accumulates acc[ms] for the NMS active 32-row subtiles.  The tile has kRowsT
// rows; src_row[p] is the activation row of tile row (tid + kThreads p) / 16
// (-1: none, zeros).  Contains barriers: every thread of the work group calls
// it with the same NMS.  hook(u, c0) runs after the u-th chunk of every group
// of kStages chunks starting at chunk c0 (u a fully unrolled index), so that
// a caller can interleave its own loads and vector work with the GEMM.
struct NoHook {
    __device__ __forceinline__ void operator()(int, int) const {}
};

template <int kRowsT, int NMS, bool kOneGroup = false, class Hook = NoHook>
__device__ __forceinline__ void chunk_gemm(const uint16_t* A, const int (&src_row)[kRowsT * kSlots / kThreads],
                                           int K, const Q4& W, size_t wrow, bool wave_on,
                                           unsigned char* lds, f32x16 (&acc)[4], Hook hook = Hook()) {
    constexpr int kAL = kRowsT * kSlots / kThreads;  // 16-byte activation loads per thread per chunk
    constexpr int kBuf = kRowsT * kRowBytes;
    static_assert(kRowsT * kSlots % kThreads == 0 && 32 * NMS <= kRowsT, "tile split");
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int n_chunks = (K + kKC - 1) / kKC;
    u32x4 ast[kStages][kAL];  // activation chunks in flight (same depth as the weights)
    BChunk bst[kStages];

    // Loads are issued unconditionally from always-valid (clamped) addresses
    // and invalid data is zeroed where it is used: a load under a branch makes
    // the compiler's wait-count analysis fall back to waiting for every
    // outstanding load, which would serialise the pipeline.
    auto load_a = [&](int c, u32x4 (&areg)[kAL]) {
#pragma unroll
        for (int p = 0; p < kAL; ++p) {
            const int slot = (tid + kThreads * p) & 15;
            const int kcol = c * kKC + 8 * slot;
            const int src = src_row[p];
            const size_t off = (size_t)(src >= 0 ? src : 0) * K + (kcol < K ? kcol : 0);
            areg[p] = *(const u32x4*)(A + off);
        }
    };
    auto store_a = [&](int c, int buf, const u32x4 (&areg)[kAL]) {
#pragma unroll
        for (int p = 0; p < kAL; ++p) {
            const int i = tid + kThreads * p, row = i >> 4, slot = i & 15;
            const bool ok = src_row[p] >= 0 && c * kKC + 8 * slot < K;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4*)(lds + buf * kBuf + lds_off(row, slot)) = ok ? areg[p] : z;
        }
    };
    const bool pair_sb = (K / kGroup) % 2 == 0;
    auto load_b = [&](int c, BChunk& st) {
        const int kc0 = c * kKC < K ? c * kKC : 0;  // clamped: always a valid chunk
        const int kc1 = kc0 + kGroup < K ? kc0 + kGroup : kc0;
        load_bchunk(W, wrow, K, kc0, kc1, half, pair_sb, st);
    };

    // One chunk on the matrix cores.  The activation fragments of step j+1 are
    // read from LDS while step j's MFMAs run.
    auto compute = [&](int c, int buf, const BChunk& st) {
        const unsigned char* tile = lds + buf * kBuf;
        // chunks (or second halves) past K contribute zero weights
        const bool ok0 = c * kKC < K, ok1 = c * kKC + kGroup < K;
        const float s0 = ok0 ? dq_scale(st.sp & 0xFFFFu) : 0.0f, b0 = ok0 ? bf16_to_f32(st.bp & 0xFFFFu) : 0.0f;
        const float s1 = ok1 ? dq_scale(st.sp >> 16) : 0.0f, b1 = ok1 ? bf16_to_f32(st.bp >> 16) : 0.0f;
        const int arow = lane & 31;
        bf16x8 Acur[NMS], Anxt[NMS];
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms)
            Acur[ms] = *(const bf16x8*)(tile + lds_off(32 * ms + arow, 4 * half));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < 7) {
                const int slot = (j + 1 < 4 ? 0 : 8) + 4 * half + ((j + 1) & 3);
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    Anxt[ms] = *(const bf16x8*)(tile + lds_off(32 * ms + arow, slot));
            }
            // keep the reads of step j+1 ahead of step j's matrix-core work
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 B = j < 4 ? dequant8(st.lo[j & 3], s0, b0) : dequant8(st.hi[j & 3], s1, b1);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B, Acur[ms], acc[ms], 0, 0, 0);
            if (j < 7) {
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) Acur[ms] = Anxt[ms];
            }
        }
    };

    // Chunks c+1 .. c+kStages-1 are in flight while chunk c is consumed.  The
    // loop runs a multiple of kStages chunks; chunks past K load clamped
    // addresses (recently read lines) and contribute zeros.
    // kOneGroup: the caller guarantees K <= kStages * kKC (one group, a
    // straight-line body)
    const int n_loop = kOneGroup ? kStages : (n_chunks + kStages - 1) / kStages * kStages;
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u) {
        load_a(u, ast[u]);
        load_b(u, bst[u]);
    }
    for (int c0 = 0; c0 < n_loop; c0 += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) {
            const int c = c0 + u;
            store_a(c, u & 1, ast[u]);
            __syncthreads();
            const int nx = (u + kStages - 1) % kStages;
            load_a(c + kStages - 1, ast[nx]);
            load_b(c + kStages - 1, bst[nx]);
            if (wave_on) compute(c, u & 1, bst[u]);
            hook(u, c0);
        }
    }
}

// Routed rows, any inter: one 128-row work item of the routed work map x one
// 256-column block per work group; outputs go to `part` (routed_store).
__global__ __launch_bounds__(kThreads) void down_chunked_kernel(const PrefillArgs a,
                                                                const int n_items, const int n_cb,
                                                                const int n_wg) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kTileBytes];
    __shared__ int s_src[kMT];  // activation row per tile row (-1: none)
    __shared__ int s_dst[kMT];  // output row (assignment) per tile row

    // XCD-aware order: consecutive logical indices (the column blocks of one
    // item, which share the activation rows) stay on one XCD's L2.
    const int b = blockIdx.x;
    const int L = (b & 7) * (n_wg >> 3) + (b >> 3);
    const int item = L / n_cb, cb = L - item * n_cb;
    if (item >= n_items) return;
    DownItem it;
    if (!routed_item(a, item, it)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    if (tid < kMT) {
        int src = -1, dst = -1;
        if (tid < it.M) {
            src = it.row0 + tid;
            dst = a.perm[src];
        }
        s_src[tid] = src;
        s_dst[tid] = dst;
    }
    __syncthreads();

    const int n_ms = (it.M + 31) >> 5;  // active 32-row subtiles
    const int wcol0 = cb * kDnCols + 32 * wave;
    const bool wave_on = wcol0 < a.d;
    const size_t wrow = (size_t)it.e * a.d + (wave_on ? wcol0 + (lane & 31) : 0);
    int src_row[kALoads];
#pragma unroll
    for (int p = 0; p < kALoads; ++p) src_row[p] = s_src[(tid + kThreads * p) >> 4];
    f32x16 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
    switch (n_ms) {
        case 1: chunk_gemm<kMT, 1>(a.h, src_row, a.I, a.down, wrow, wave_on, lds, acc); break;
        case 2: chunk_gemm<kMT, 2>(a.h, src_row, a.I, a.down, wrow, wave_on, lds, acc); break;
        case 3: chunk_gemm<kMT, 3>(a.h, src_row, a.I, a.down, wrow, wave_on, lds, acc); break;
        default: chunk_gemm<kMT, 4>(a.h, src_row, a.I, a.down, wrow, wave_on, lds, acc); break;
    }

    if (!wave_on) return;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        const int row = 32 * ms + (lane & 31);
        if (ms >= n_ms || row >= it.M) continue;
        routed_store(a, s_dst[row], wcol0, half, acc[ms]);
    }
}

// ---------------------------------------------------------------------------
// The shared expert's down projection with the combine.  Work item = a block of
// kRows (32 or 64) tokens x 256 output columns.  Phases:
//   1+2. the shared expert's down GEMM of the block (chunk_gemm), and between
//      its chunks the k staged partial rows of one token row per thread (32
//      threads cover one token's 256 columns with contiguous 16-byte loads,
//      issued a chunk ahead) weighted by the scores times their staging
//      exponents and summed in slot order into an fp32 tile in LDS;
//   3. y = bf16(routed sum + shared output), staged through LDS so that the
//      global stores are contiguous 16-byte pieces.
// ---------------------------------------------------------------------------
constexpr int kShMaxRows = 64;

// 16-byte granule g of row r of the routed-sum tile (1 KB rows), XOR-swizzled
// by row so that a subtile's 32 rows read at one column spread over the banks.
__device__ __forceinline__ int rsum_off(int r, int g) { return r * 1024 + ((g ^ (r & 63)) << 4); }
// 16-byte granule g of row r of the bf16 output tile (512-byte rows).
__device__ __forceinline__ int ytile_off(int r, int g) { return r * 512 + ((g ^ (r & 31)) << 4); }

template <int kRows, bool kInterleave>
__global__ __launch_bounds__(kThreads) void shared_down_combine_kernel(const PrefillArgs a,
                                                                       const int n_items,
                                                                       const int n_cb,
                                                                       const int n_wg) {
    static_assert(kRows == 32 || kRows == 64, "shared rows");
    constexpr int kP = kRows * 32 / kThreads;  // tokens per thread in the routed-sum phase
    constexpr int kAL = kRows * kSlots / kThreads;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kShMaxRows * kRowBytes];
    __shared__ __attribute__((aligned(16))) unsigned char s_rsum[kShMaxRows * 1024];

    const int b = blockIdx.x;
    const int L = (b & 7) * (n_wg >> 3) + (b >> 3);
    const int item = L / n_cb, cb = L - item * n_cb;
    if (item >= n_items) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int T = a.T, d = a.d, k = a.k;
    const int row0 = item * kRows, M = min(kRows, T - row0);
    const int c0 = cb * kDnCols;

    // ---- 1. routed sums: thread (token row tr0 + 16 p, columns c0 + 8 c8 ..) ----
    // kInterleave (inter <= kStages chunks, so the GEMM runs one group of
    // kStages chunks): row p's staged partials, staging exponents and scores
    // are loaded one GEMM chunk ahead and summed after the GEMM's chunk p (the
    // hook below), so that their round trips and vector work run under the
    // shared expert's GEMM; otherwise every row after the GEMM.  Each score is
    // scaled by its slot's staging exponent once (an exact power-of-two
    // scaling), and the fp16 values then enter the fma directly.
    const int c8 = tid & 31, tr0 = tid >> 5;
    const int col = c0 + 8 * c8;
    const bool col_ok = col < d;  // d is a multiple of 64: 8-column pieces are whole
    const int colc = col_ok ? col : c0;
    static_assert(kP <= kStages, "one token row per GEMM chunk");
    u32x4 pv[kP][kMaxTopK];
    uint2 ev[kP];
    float sw[kP][kMaxTopK];
    auto load_rows = [&](int p) {
        const int tr = tr0 + 16 * p;
        const size_t tok = (size_t)row0 + (tr < M ? tr : 0);  // clamped, always valid
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
            pv[p][s] = *(const u32x4*)(a.part + (tok * k + (s < k ? s : 0)) * d + colc);
            sw[p][s] = a.topk_w[tok * k + (s < k ? s : 0)];
        }
        ev[p] = *(const uint2*)(a.pexp + part_exp_index(a, (int)tok * k, colc));
    };
    auto sum_rows = [&](int p) {
        const int tr = tr0 + 16 * p;
        if (tr < M && col_ok) {
            float acc8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < kMaxTopK; ++s) {
                if (s < k) {
                    const int e = (int)(int8_t)(((s < 4 ? ev[p].x : ev[p].y) >> (8 * (s & 3))) & 0xFFu);
                    const float w = __builtin_amdgcn_ldexpf(sw[p][s], e);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc8[2 * i] = __builtin_fmaf(f16_to_f32(pv[p][s][i] & 0xFFFFu), w, acc8[2 * i]);
                        acc8[2 * i + 1] = __builtin_fmaf(f16_to_f32(pv[p][s][i] >> 16), w, acc8[2 * i + 1]);
                    }
                }
            }
            *(f32x4*)(s_rsum + rsum_off(tr, 2 * c8)) = f32x4{acc8[0], acc8[1], acc8[2], acc8[3]};
            *(f32x4*)(s_rsum + rsum_off(tr, 2 * c8 + 1)) = f32x4{acc8[4], acc8[5], acc8[6], acc8[7]};
        }
    };
    if constexpr (kInterleave) load_rows(0);

    // ---- 2. the shared expert's down GEMM of the block, with the routed sums ----
    const int wcol0 = c0 + 32 * wave;
    const bool wave_on = wcol0 < d;
    const size_t wrow = wave_on ? (size_t)(wcol0 + (lane & 31)) : 0;
    int src_row[kAL];
#pragma unroll
    for (int p = 0; p < kAL; ++p) {
        const int r = (tid + kThreads * p) >> 4;
        src_row[p] = r < M ? row0 + r : -1;
    }
    f32x16 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
    const int n_ms = (M + 31) >> 5;
    // with kInterleave the GEMM runs exactly one group of kStages chunks, so the
    // hook sees u = 0 .. kStages - 1 once: token row u is summed after chunk u
    auto hook = [&](int u, int) {
        if constexpr (kInterleave) {
            if (u < kP) {
                if (u + 1 < kP) load_rows(u + 1);
                sum_rows(u);
            }
        }
    };
    if constexpr (kRows == 64) {
        if (n_ms == 2)
            chunk_gemm<kRows, 2, kInterleave>(a.h_sh, src_row, a.I, a.sh_down, wrow, wave_on, lds, acc, hook);
        else
            chunk_gemm<kRows, 1, kInterleave>(a.h_sh, src_row, a.I, a.sh_down, wrow, wave_on, lds, acc, hook);
    } else {
        chunk_gemm<kRows, 1, kInterleave>(a.h_sh, src_row, a.I, a.sh_down, wrow, wave_on, lds, acc, hook);
    }
    if constexpr (!kInterleave) {
#pragma unroll
        for (int p = 0; p < kP; ++p) load_rows(p);
#pragma unroll
        for (int p = 0; p < kP; ++p) sum_rows(p);
    }

    __syncthreads();  // every wave is done with the activation tiles (the y tile reuses them)

    // ---- 3. y = bf16(routed sum + shared output) ----
    // lane: tile row 32 ms + lane % 32, columns 8 g + 4 h .. +3 of its wave's 32
    if (wave_on) {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            const int r = 32 * ms + (lane & 31);
            if (ms < n_ms && r < M) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int cl = 32 * wave + 8 * g + 4 * half;  // column within the block
                    const f32x4 rs = *(const f32x4*)(s_rsum + rsum_off(r, cl >> 2));
                    uint2 v;
                    v.x = pack_bf16x2(rs[0] + acc[ms][4 * g], rs[1] + acc[ms][4 * g + 1]);
                    v.y = pack_bf16x2(rs[2] + acc[ms][4 * g + 2], rs[3] + acc[ms][4 * g + 3]);
                    *(uint2*)(lds + ytile_off(r, cl >> 3) + 8 * half) = v;
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kP; ++p) {
        const int tr = tr0 + 16 * p;
        if (tr < M && col_ok)
            *(u32x4*)(a.y + (size_t)(row0 + tr) * d + col) = *(const u32x4*)(lds + ytile_off(tr, c8));
    }
}

// ---------------------------------------------------------------------------
// Cost-balanced contiguous runs.  The units of a persistent GEMM are ordered
// item by item (n_cb units per item); a unit of an item with M rows is
// estimated to cost 2 + ceil(M / 32) (the dequantisation of its weights being
// worth about two 32-row subtiles of MFMAs).  Every work group computes the
// prefix of these costs in LDS (fixed order, integer) and takes the units
// whose cost midpoints fall in its 1/G share, so the runs tile the unit list
// exactly and carry about the same work.
// ---------------------------------------------------------------------------
// routed 128-row work items at most (the capacity of the 128-row work map)
constexpr int kMaxRoutedItems = MOE_MAX_TOKENS * kMaxTopK / kMT + kMaxExperts;
static_assert((unsigned long long)kMaxRoutedItems * (MOE_MAX_D / 256) * 6 * 2 * 1024 < (1ull << 32),
              "32-bit run starts");

__device__ __forceinline__ int unit_cost(int M) { return 2 + ((M + 31) >> 5); }

// pre[i] = cost of the units of items [0, i) (pre in LDS or global memory);
// rows_of(i) gives item i's row count (and may record per-item data).  Ends
// with a barrier.
template <typename RowsOf>
__device__ __forceinline__ void cost_prefix(int n_items, int n_cb, int* s_pre, int* s_wtot,
                                            RowsOf&& rows_of) {
    constexpr int kPer = (kMaxRoutedItems + kThreads - 1) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = (n_items + kThreads - 1) / kThreads;
    int cost[kPer];
    int loc = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = tid * R + r;
        cost[r] = (r < R && i < n_items) ? unit_cost(rows_of(i)) * n_cb : 0;
        loc += cost[r];
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o, 64);
        if (lane >= o) inc += v;
    }
    if (lane == 63) s_wtot[wave] = inc;
    __syncthreads();
    int run = inc - loc;
    for (int w = 0; w < wave; ++w) run += s_wtot[w];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = tid * R + r;
        if (r < R && i < n_items) s_pre[i] = run;
        run += cost[r];
    }
    if (tid == kThreads - 1) s_pre[n_items] = run;
    __syncthreads();
}

// First unit (item * n_cb + block) of run g of G; n_items * n_cb for g >= G.
__device__ __forceinline__ int run_start(int g, int G, int n_items, int n_cb, const int* s_pre) {
    if (g >= G) return n_items * n_cb;
    // 32-bit arithmetic: 2 x the total cost times G stays below 2^32 (at most
    // kMaxRoutedItems items x 32 column blocks x cost 6 x 2 x 1024 groups)
    const uint32_t C2 = 2u * (uint32_t)__builtin_amdgcn_readfirstlane(s_pre[n_items]);
    auto owner = [&](int i, int b) {
        const int p0 = __builtin_amdgcn_readfirstlane(s_pre[i]);
        const int p1 = __builtin_amdgcn_readfirstlane(s_pre[i + 1]);
        const uint32_t mid = 2u * (uint32_t)p0 + (uint32_t)(2 * b + 1) * (uint32_t)((p1 - p0) / n_cb);
        return (int)(mid * (uint32_t)G / C2);
    };
    int lo = 0, hi = n_items;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (owner(mid, n_cb - 1) >= g) hi = mid;
        else lo = mid + 1;
    }
    if (lo == n_items) return n_items * n_cb;
    int b = 0;
    while (owner(lo, b) < g) ++b;
    return __builtin_amdgcn_readfirstlane(lo * n_cb + b);
}

// ---------------------------------------------------------------------------
// Routed down projection with the activation tile resident in LDS (inter in
// (384, 512], four K-chunks), persistent.  A unit is (routed work item,
// 256-column block); the units are ordered item by item and every work group
// takes one cost-balanced contiguous run of them.  Consecutive units of a run
// mostly share their item, so the M x inter bf16 activation tile is loaded
// into LDS only when the item changes; the weights stream through registers
// as one continuous pipeline over the whole run (three chunks in flight,
// across unit boundaries).  Each 256-column block is written as soon as its
// last chunk is done.
// ---------------------------------------------------------------------------
constexpr int kDnMaxI = 512;

// The down kernel's schedule: the routed items' cost prefix over (n_cb
// 256-column units per item) and their experts, written to the workspace by
// one work group of the gate/up kernel so that the down kernel's work groups
// only load it.
__device__ __forceinline__ void down_schedule(const PrefillArgs& a, int* s_wtot) {
    const int n_items = *a.n_tiles;
    const int n_cb = (a.d + kDnCols - 1) / kDnCols;
    cost_prefix(n_items, n_cb, a.dn_pre, s_wtot, [&](int i) {
        const int e = a.tile_map[2 * i], r0 = a.tile_map[2 * i + 1];
        a.dn_exp[i] = e;
        return min(kMT, a.offsets[e + 1] - r0);
    });
}


// kSB4: inter % 512 == 0 (eight groups per row at most 512, so a unit's whole
// K is one row segment): a unit's scales (and biases) are one 16-byte load
// per lane, issued with the codes of the unit's first chunk.
template <bool kSB4>
__global__ __launch_bounds__(kThreads) void down_resident_kernel(const PrefillArgs a,
                                                                 const int n_cb) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kMT * kDnMaxI * 2];
    __shared__ int s_dst[kMT];
    __shared__ int s_pre[kMaxRoutedItems + 1];  // cost of the units before item i
    __shared__ short s_exp[kMaxRoutedItems];    // expert of item i
    // each wave's 32 x 32 fp16 output tile on its way to `part`: row t,
    // 16-byte slot s at t * 64 + 16 * (s ^ ((t >> 1) & 3))
    __shared__ __attribute__((aligned(16))) uint16_t s_out[kWaves][32 * 32];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int G = gridDim.x, g = blockIdx.x;
    const int K = a.I, Nw = a.d;
    const int n_items = *a.n_tiles;

    // ---- this work group's run of units ----
    // the item cost prefix and the items' experts were computed by the
    // gate/up kernel (down_schedule) into the workspace
    for (int i = tid; i <= n_items; i += kThreads) {
        // both loads in flight before either is used (clamped, always valid)
        const int pv = a.dn_pre[i];
        const int ev = a.dn_exp[i < n_items ? i : 0];
        asm volatile("" ::"v"(pv), "v"(ev));  // keeps the second load out of the branch below
        s_pre[i] = pv;
        if (i < n_items) s_exp[i] = (short)ev;
    }
    __syncthreads();
    const int u_first = run_start(g, G, n_items, n_cb, s_pre);
    const int u_end = run_start(g + 1, G, n_items, n_cb, s_pre);
    if (u_first >= u_end) return;  // uniform: no units for this work group
    const int u_item = u_first / n_cb, u_blk = u_first - u_item * n_cb;
    auto in_run = [&](int i, int b) { return i * n_cb + b < u_end; };

    constexpr int nk = kStages;  // K-chunks per unit
    constexpr int row_bytes = nk * kRowBytes;
    const bool pair_sb = (K / kGroup) % 2 == 0;

    // ---- weight stream: a cursor over (item, block, chunk) of this run ----
    int w_item = u_item, w_blk = u_blk, w_c = 0;
    bool w_end = false;  // past the run: repeat the last chunk (never used)
    u32x4 s4c = {}, b4c = {}, s4n = {}, b4n = {};  // kSB4: this unit's / the next unit's
    // with_sb: the chunk is a unit's first (known where the call sits), so
    // with kSB4 the unit's scales and biases come with it
    auto load_next_b = [&](BChunk& st, u32x4& s4, u32x4& b4, auto with_sb) {
        const int e = __builtin_amdgcn_readfirstlane(s_exp[w_item]);
        const int wc = w_blk * kDnCols + 32 * wave;
        const size_t wrow = (size_t)e * Nw + (wc < Nw ? wc + (lane & 31) : 0);
        const int kc0 = w_c * kKC < K ? w_c * kKC : 0;
        const int kc1 = kc0 + kGroup < K ? kc0 + kGroup : kc0;
        const uint32_t* qrow = a.down.q + wrow * (K / 8) + 4 * half;
        st.lo = *(const u32x4*)(qrow + kc0 / 8);
        st.hi = *(const u32x4*)(qrow + kc1 / 8);
        if (kSB4) {
            if (decltype(with_sb)::value) {
                s4 = *(const u32x4*)(a.down.scale + wrow * (K / kGroup));
                b4 = *(const u32x4*)(a.down.bias + wrow * (K / kGroup));
            }
        } else {
            const size_t grow = wrow * (K / kGroup);
            if (pair_sb) {
                st.sp = *(const uint32_t*)(a.down.scale + grow + kc0 / kGroup);
                st.bp = *(const uint32_t*)(a.down.bias + grow + kc0 / kGroup);
            } else {
                st.sp = (uint32_t)a.down.scale[grow + kc0 / kGroup] |
                        ((uint32_t)a.down.scale[grow + kc1 / kGroup] << 16);
                st.bp = (uint32_t)a.down.bias[grow + kc0 / kGroup] |
                        ((uint32_t)a.down.bias[grow + kc1 / kGroup] << 16);
            }
        }
        if (!w_end && ++w_c == nk) {
            int ni = w_item, nb = w_blk + 1;
            if (nb == n_cb) {
                ++ni;
                nb = 0;
            }
            if (in_run(ni, nb)) {
                w_item = ni;
                w_blk = nb;
                w_c = 0;
            } else {
                w_end = true;
                w_c = nk - 1;
            }
        }
    };
    BChunk bst[kStages];
    load_next_b(bst[0], s4c, b4c, Int<1>{});
    load_next_b(bst[1], s4c, b4c, Int<0>{});
    load_next_b(bst[2], s4c, b4c, Int<0>{});
    static_assert(kStages == 4, "three chunks ahead, four chunks per unit");

    // ---- resident activation tile of item `item` ----
    // row r, 16-byte slot s at r * row_bytes + ((s ^ (r & 15)) << 4).  All of
    // a lane's loads are issued before any store (one round trip).  Rows past
    // M hold copies of row 0 (finite; their products are never stored);
    // columns past K are zero (their weights are zeroed too, and a zero
    // weight times a finite value must stay zero).
    DownItem it;
    auto load_tile = [&](int item) {
        routed_item(a, item, it);
        // tid laundered here, so that the per-lane tile offsets are computed
        // per load instead of being hoisted out of the unit loop (and spilled)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        if (tid < kMT) s_dst[tid] = tid < it.M ? a.perm[it.row0 + tid] : -1;
        constexpr int slots = nk * kSlots;  // 16-byte slots per row (K padded to the chunk)
        constexpr int per = kMT * slots / kThreads;
        static_assert(kMT * slots % kThreads == 0, "resident tile split");
        u32x4 v[per];
#pragma unroll
        for (int p = 0; p < per; ++p) {
            const int i = tid + kThreads * p;
            const int row = i / slots, slot = i - row * slots;
            const int kcol = 8 * slot;
            const size_t off = (size_t)(it.row0 + (row < it.M ? row : 0)) * K + (kcol < K ? kcol : 0);
            v[p] = *(const u32x4*)(a.h + off);
        }
#pragma unroll
        for (int p = 0; p < per; ++p) {
            const int i = tid + kThreads * p;
            const int row = i / slots, slot = i - row * slots;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4*)(lds + row * row_bytes + ((slot ^ (row & 15)) << 4)) = 8 * slot < K ? v[p] : z;
        }
    };

    auto compute = [&](auto nms_tag, int c, const BChunk& st, f32x16 (&acc)[decltype(nms_tag)::value]) {
        constexpr int NMS = decltype(nms_tag)::value;
        const bool ok0 = c * kKC < K, ok1 = c * kKC + kGroup < K;
        const uint32_t spv = kSB4 ? s4c[c & 3] : st.sp, bpv = kSB4 ? b4c[c & 3] : st.bp;
        const float s0 = ok0 ? dq_scale(spv & 0xFFFFu) : 0.0f, b0 = ok0 ? bf16_to_f32(bpv & 0xFFFFu) : 0.0f;
        const float s1 = ok1 ? dq_scale(spv >> 16) : 0.0f, b1 = ok1 ? bf16_to_f32(bpv >> 16) : 0.0f;
        const int arow = lane & 31, sbase = c * kSlots;
        auto aread = [&](int ms, int slot) {
            const int row = 32 * ms + arow;
            return *(const bf16x8*)(lds + row * row_bytes + (((sbase + slot) ^ (row & 15)) << 4));
        };
        bf16x8 Acur[NMS], Anxt[NMS];
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms) Acur[ms] = aread(ms, 4 * half);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < 7) {
                const int slot = (j + 1 < 4 ? 0 : 8) + 4 * half + ((j + 1) & 3);
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) Anxt[ms] = aread(ms, slot);
            }
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 B = j < 4 ? dequant8(st.lo[j & 3], s0, b0) : dequant8(st.hi[j & 3], s1, b1);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B, Acur[ms], acc[ms], 0, 0, 0);
            if (j < 7) {
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) Acur[ms] = Anxt[ms];
            }
        }
    };

    // chunk c of every unit uses stage c, so each unit is one unrolled body
    auto unit_body = [&](auto nms_tag, int blk) {
        constexpr int NMS = decltype(nms_tag)::value;
        const int wc = blk * kDnCols + 32 * wave;
        f32x16 acc[NMS];  // local to the unit: not live across an activation tile load
#pragma unroll
        for (int m = 0; m < NMS; ++m) acc[m] = f32x16{};
        // the loader runs three chunks ahead, so its call at chunk 1 loads
        // the next unit's first chunk (and scales)
        load_next_b(bst[3], s4n, b4n, Int<0>{});
        if (wc < Nw) compute(nms_tag, 0, bst[0], acc);
        load_next_b(bst[0], s4n, b4n, Int<1>{});
        if (wc < Nw) compute(nms_tag, 1, bst[1], acc);
        load_next_b(bst[1], s4n, b4n, Int<0>{});
        if (wc < Nw) compute(nms_tag, 2, bst[2], acc);
        load_next_b(bst[2], s4n, b4n, Int<0>{});
        if (wc < Nw) compute(nms_tag, 3, bst[3], acc);
        if (kSB4) {
            s4c = s4n;
            b4c = b4n;
        }
        if (wc < Nw) {
            // through the wave's LDS tile, so that a store instruction writes
            // 16 rows x 64 contiguous bytes; every row of the tile is scaled by
            // its staging exponent first (a lane pair holds one row)
            unsigned char* so = (unsigned char*)s_out[wave];
            const int t = lane & 31;
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
                const int e = part_exp(pair_absmax(acc[ms]));
                const int row_e = 32 * ms + t;
                if (half == 0 && row_e < it.M) a.pexp[part_exp_index(a, s_dst[row_e], wc)] = (int8_t)e;
                auto h16 = [&](float v0, float v1) {
                    return pack_f16x2(__builtin_amdgcn_ldexpf(v0, -e), __builtin_amdgcn_ldexpf(v1, -e));
                };
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {  // columns 8gq + 4h .. +3: 8-byte unit 2gq + h
                    uint2 v;
                    v.x = h16(acc[ms][4 * gq], acc[ms][4 * gq + 1]);
                    v.y = h16(acc[ms][4 * gq + 2], acc[ms][4 * gq + 3]);
                    const int slot = gq ^ ((t >> 1) & 3);
                    *(uint2*)(so + t * 64 + 16 * slot + 8 * half) = v;
                }
#pragma unroll
                for (int pass = 0; pass < 2; ++pass) {
                    const int r = 16 * pass + (lane >> 2), sg = lane & 3;
                    const u32x4 v = *(const u32x4*)(so + r * 64 + 16 * (sg ^ ((r >> 1) & 3)));
                    const int row = 32 * ms + r;
                    if (row < it.M) *(u32x4*)(a.part + (size_t)s_dst[row] * a.d + wc + 8 * sg) = v;
                }
            }
        }
    };

    int cur_item = -1;
    int ui = u_item, ub = u_blk;
    while (true) {
        if (ui != cur_item) {  // uniform
            if (cur_item >= 0) __syncthreads();  // every wave is done with the old tile
            cur_item = ui;
            load_tile(ui);
            __syncthreads();
        }
        switch ((it.M + 31) >> 5) {
            case 1: unit_body(Int<1>{}, ub); break;
            case 2: unit_body(Int<2>{}, ub); break;
            case 3: unit_body(Int<3>{}, ub); break;
            default: unit_body(Int<4>{}, ub); break;
        }
        if (++ub == n_cb) {
            ++ui;
            ub = 0;
        }
        if (!in_run(ui, ub)) break;
    }
}

// ---------------------------------------------------------------------------
// Persistent gate/up GEMM.  One work group of eight waves per CU walks a
// static list of units (work item, 128-intermediate-column block), numbered
// so that the column blocks of one item run at the same time on one XCD and
// share its L2 for the gathered activation rows (a cost-balanced contiguous
// run per work group, as the down kernel uses, measured slower here: the
// column blocks of an item then run one after another and the rows are
// fetched again).  The descriptors (expert, rows, source and
// destination rows) of up to kBatch units are computed once up front, and
// the K-chunk pipeline then runs continuously from one unit into the next,
// so no per-item start-up (dependent index loads) or pipeline fill/drain is
// paid per item.
//
// Each wave owns 16 intermediate columns j0..j0+15: the 32 weight rows of its
// MFMA operand are gate rows j0..j0+15 (lanes 0-15) and up rows j0..j0+15
// (lanes 16-31).  In the 32x32 output tile a lane then holds gate row r and
// up row r + 16 of the same token in elements i and i + 8, so SiLU(gate)*up
// needs no data exchange.
// Weights stream two chunks ahead and activations one (activations are
// issued before the weights, so waiting for an activation chunk never waits
// for younger weight loads).
// ---------------------------------------------------------------------------
constexpr int kBatch = 8;
constexpr int kGuWaves = 8;
constexpr int kGuThreads = kGuWaves * 64;
constexpr int kGuCols = 16 * kGuWaves;                // intermediate columns per unit
constexpr int kGuALoads = kMT * kSlots / kGuThreads;  // 16-byte activation loads per lane per chunk
constexpr int kGuShRows = 64;                         // rows of a shared-expert item
constexpr bool kGuGrouped = true;
static_assert(kMT * kSlots % kGuThreads == 0, "activation tile split");

struct UnitDesc {
    int e, row0, M, cb, shared;
};

// Vector memory operations of one gate/up wave per chunk position v of a
// four-chunk call (v < 0: the previous call, which for FIRST is the previous
// unit's final call): activation loads (step 0), weight codes (steps 2, 4),
// scales/biases (step 6).
template <bool FIRST, bool LAST, int NMS>
constexpr int gu_n_act(int v) {
    return v < 0 ? (FIRST ? kGuALoads : NMS) : ((LAST && v >= 1) ? kGuALoads : NMS);
}
template <bool SB4>
constexpr int gu_n_sb(int v) {
    return SB4 ? (((v + 4) & 3) == 2 ? 2 : 0) : 2;
}
// Operations a wave issues after its activation loads of the chunk at
// position u (issued at position u - 3) up to the barrier of that chunk.
template <bool SB4, bool FIRST, bool LAST, int NMS>
constexpr int gu_ops_after(int u) {
    return 2 + gu_n_sb<SB4>(u - 3) + gu_n_act<FIRST, LAST, NMS>(u - 2) + 2 + gu_n_sb<SB4>(u - 2) +
           gu_n_act<FIRST, LAST, NMS>(u - 1) + 2 + gu_n_sb<SB4>(u - 1);
}

// A unit descriptor read back from LDS, moved to scalar registers: every
// field is uniform across the work group.
__device__ __forceinline__ UnitDesc uniform_desc(const UnitDesc& d) {
    UnitDesc u;
    u.e = __builtin_amdgcn_readfirstlane(d.e);
    u.row0 = __builtin_amdgcn_readfirstlane(d.row0);
    u.M = __builtin_amdgcn_readfirstlane(d.M);
    u.cb = __builtin_amdgcn_readfirstlane(d.cb);
    u.shared = __builtin_amdgcn_readfirstlane(d.shared);
    return u;
}

// One lane's share of one weight chunk: the codes of k in [kc + 32h, +32)
// and [kc + 64 + 32h, +32) (h = lane / 32), and -- when scales and biases are
// loaded per chunk -- the two groups' scale and bias pairs (low half = the
// group of lo).
struct WChunk {
    u32x4 lo, hi;
    uint32_t sp, bp;
};

// items of the gate/up kernel at most: the routed work map plus the shared
// expert's blocks of kGuShRows tokens
constexpr int kGuMaxItems = kMaxRoutedItems + (MOE_MAX_TOKENS + kGuShRows - 1) / kGuShRows;

// The items of group q of Q (item = routed tile, then the shared expert's row
// blocks), written to s_items[0, n_run) in the order the group runs them.
// The items are ordered by subtile count, largest first (stable inside a
// count), and cut into Q contiguous runs at the cost midpoints: item j of the
// order, of cost c_j = gu_unit_cost(subtiles) and cost prefix P_j, belongs to run
// floor((2 P_j + c_j) Q / (2 P_total)).  Sorting first gives the runs with
// heavy items fewer of them, so the runs carry about the same work even when
// they hold only a few items each.  The order is a counting sort over the
// four subtile counts, so every item's position and cost prefix have a closed
// form in the class totals and its rank inside its class; every work group
// computes only its own run.  Uniform results; contains barriers.
constexpr int kGuPer = (kGuMaxItems + kGuThreads - 1) / kGuThreads;
// estimated cost of a gate/up unit with `ms` 32-row subtiles
__device__ __forceinline__ int gu_unit_cost(int ms) { return 2 + ms; }
constexpr int kGuRunMax = 512;  // items one group may hold (s_items)
static_assert((unsigned long long)kGuPer * 512 * 6 * 2 * 1024 < (1ull << 32), "32-bit run cut");

// Routed item i of the gate/up kernel: part i % S of 128-row tile i / S of the
// tile map (S = 1 << item_sh parts of 128 >> item_sh rows each).  Its rows end
// where the next tile starts: the next tile of the same expert is 128 rows on,
// and the next non-empty expert's rows follow the expert's last row directly
// (the last tile ends at T * k).  So the row count needs only the tile map,
// whose three entries load at once.  n_raw: tiles in the map; M <= 0 for a
// part past the expert's rows.
__device__ __forceinline__ void gu_tile_entries(const PrefillArgs& a, int t, int& e, int& r0,
                                                int& nx) {
    const int tc = min(t, a.tile_bound - 1), tn = min(t + 1, a.tile_bound - 1);  // valid entries
    e = a.tile_map[2 * tc];
    r0 = a.tile_map[2 * tc + 1];
    nx = a.tile_map[2 * tn + 1];
}
__device__ __forceinline__ void gu_item_rows(const PrefillArgs& a, int i, int n_raw, int r0,
                                             int nx, int& row0, int& M) {
    const int rows = kMT >> a.item_sh;
    const int t = i >> a.item_sh, part = i & ((1 << a.item_sh) - 1);
    const int end = t + 1 < n_raw ? nx : a.T * a.k;
    row0 = r0 + part * rows;
    M = min(rows, end - row0);
}

// Items of the gate/up kernel at most, by the host's bound on the tile count.
__device__ __forceinline__ int gu_item_bound(const PrefillArgs& a) {
    return (a.tile_bound << a.item_sh) + (a.T + kGuShRows - 1) / kGuShRows;
}

__device__ __forceinline__ int item_run(const PrefillArgs& a, int n_raw, int n_tiles, int n_items,
                                        int Q, int q, int* s_items) {
    __shared__ int s_cls[2][kGuWaves];  // per-wave class counts, 16 bits per class
    __shared__ int s_cnt[2][kGuWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // items per thread from the host bound, so that the tile-map loads below
    // need not wait for the tile count
    const int R = (gu_item_bound(a) + kGuThreads - 1) / kGuThreads;
    int te[kGuPer], tr0[kGuPer], tnx[kGuPer];
#pragma unroll
    for (int r = 0; r < kGuPer; ++r) gu_tile_entries(a, (tid * R + r) >> a.item_sh, te[r], tr0[r], tnx[r]);
    int cls[kGuPer];  // subtile count - 1 of each of this thread's items (-1: none)
    int lo = 0, hi = 0;  // class counts: lo = classes 0, 1; hi = classes 2, 3
#pragma unroll
    for (int r = 0; r < kGuPer; ++r) {
        const int i = tid * R + r;
        cls[r] = -1;
        if (r < R && i < n_items) {
            int M;
            if (i < n_tiles) {
                int r0;
                gu_item_rows(a, i, n_raw, tr0[r], tnx[r], r0, M);
            } else {
                M = min(kGuShRows, a.T - (i - n_tiles) * kGuShRows);
            }
            if (M <= 0) continue;  // an empty part of a tile: no unit
            const int c = (M + 31) / 32 - 1;
            cls[r] = c;
            const int one = 1 << (16 * (c & 1));
            lo += c < 2 ? one : 0;
            hi += c >= 2 ? one : 0;
        }
    }
    // exclusive scan of the class counts over the threads
    int ilo = lo, ihi = hi;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int vl = __shfl_up(ilo, o, 64), vh = __shfl_up(ihi, o, 64);
        if (lane >= o) {
            ilo += vl;
            ihi += vh;
        }
    }
    if (lane == 63) {
        s_cls[0][wave] = ilo;
        s_cls[1][wave] = ihi;
    }
    __syncthreads();
    int plo = ilo - lo, phi = ihi - hi, tlo = 0, thi = 0;
#pragma unroll
    for (int w = 0; w < kGuWaves; ++w) {
        plo += w < wave ? s_cls[0][w] : 0;
        phi += w < wave ? s_cls[1][w] : 0;
        tlo += s_cls[0][w];
        thi += s_cls[1][w];
    }
    int rank[4] = {plo & 0xFFFF, plo >> 16, phi & 0xFFFF, phi >> 16};
    const int N[4] = {tlo & 0xFFFF, tlo >> 16, thi & 0xFFFF, thi >> 16};
    // classes in order 3, 2, 1, 0: items and cost before each class
    int pos0[4], cost0[4];
    int np = 0, cp = 0;
#pragma unroll
    for (int c = 3; c >= 0; --c) {
        pos0[c] = np;
        cost0[c] = cp;
        np += N[c];
        cp += N[c] * gu_unit_cost(c + 1);
    }
    // 32-bit arithmetic: (2 x cost prefix + cost) x Q stays below 2^32 (at
    // most kGuPer x kGuThreads items of cost 6, Q <= 1024 groups)
    const uint32_t den = 2u * (uint32_t)max(cp, 1);
    int before = 0, mine = 0;
    int pos[kGuPer];
#pragma unroll
    for (int r = 0; r < kGuPer; ++r) {
        pos[r] = -1;
        const int c = cls[r];
        if (c >= 0) {
            const int k = c == 0 ? rank[0]++ : c == 1 ? rank[1]++ : c == 2 ? rank[2]++ : rank[3]++;
            const int cost = gu_unit_cost(c + 1);
            const int pre = (c == 0 ? cost0[0] : c == 1 ? cost0[1] : c == 2 ? cost0[2] : cost0[3]) +
                            k * cost;
            const int run = (int)((uint32_t)(2 * pre + cost) * (uint32_t)Q / den);
            before += run < q;
            if (run == q) {
                ++mine;
                pos[r] = (c == 0 ? pos0[0] : c == 1 ? pos0[1] : c == 2 ? pos0[2] : pos0[3]) + k;
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        before += __shfl_xor(before, o, 64);
        mine += __shfl_xor(mine, o, 64);
    }
    if (lane == 0) {
        s_cnt[0][wave] = before;
        s_cnt[1][wave] = mine;
    }
    __syncthreads();
    int first = 0, n_run = 0;
#pragma unroll
    for (int w = 0; w < kGuWaves; ++w) {
        first += s_cnt[0][w];
        n_run += s_cnt[1][w];
    }
#pragma unroll
    for (int r = 0; r < kGuPer; ++r)
        if (pos[r] >= 0 && pos[r] - first < kGuRunMax) s_items[pos[r] - first] = tid * R + r;
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(min(n_run, kGuRunMax));
}

// kSB4: every row has a multiple of 8 groups (K % 512 == 0), so one 16-byte
// load brings a lane the scales (or biases) of four consecutive chunks; they
// are loaded once per four chunks instead of once per chunk.
template <bool kSB4>
__global__ __launch_bounds__(kGuThreads) void gate_up_kernel(const PrefillArgs a, const int n_cb) {
    // activation ring: chunk c lives in buffer c % 4; four separate objects,
    // so that the compiler tracks the direct-to-LDS loads into each one apart
    __shared__ __attribute__((aligned(16))) unsigned char lds_a0[kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char lds_a1[kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char lds_a2[kTileBytes];
    __shared__ __attribute__((aligned(16))) unsigned char lds_a3[kTileBytes];
    __shared__ UnitDesc s_unit[kBatch];
    __shared__ int s_src[kBatch][kMT];
    __shared__ int s_dst[kBatch][kMT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int G = gridDim.x, g = blockIdx.x;
    const int K = a.d, Nw = a.I;
    const int n_raw = *a.n_tiles;                 // 128-row tiles in the map
    const int n_tiles = n_raw << a.item_sh;       // routed items
    const int sh_items = (a.T + kGuShRows - 1) / kGuShRows;
    const int n_items = n_tiles + sh_items;
    const int NL = ((K + kKC - 1) / kKC + kStages - 1) / kStages * kStages;  // chunks per unit
    const bool pair_sb = (K / kGroup) % 2 == 0;  // scale/bias pairs are 4-byte aligned
    const bool is_up = (lane & 16) != 0;         // weight row lane%32: gate j0+n or up j0+n-16
    const int jrow = lane & 15;
    // x as a raw buffer (T * d * 2 bytes < 2^32 by the size limits): the
    // activation loads go direct to LDS as buffer loads.  The global (flat)
    // form of the same load leaves the compiler unable to order it against
    // the weight loads in the vector memory counter, and it then waits for
    // every outstanding load before the first use of any loaded register;
    // the buffer form keeps those waits exact.
    const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, 0, (int)((uint32_t)a.T * (uint32_t)K * 2u), 0x00020000);

    f32x16 acc[4];
    WChunk bst[kStages];
    u32x4 s4c, b4c, s4n, b4n;                  // kSB4: scales / biases of this and the next 4 chunks
    uint32_t a_row[kGuALoads];                 // activation stream: row offsets of its unit
    // a lane's 16-byte piece of a staged row lands in physical slot lane & 15
    // of tile row 4 * wave + lane / 16 (+ 32 p); it holds logical slot
    // (lane & 15) ^ (row & 15) of the row (the XOR swizzle)
    const int a_lslot = (lane & 15) ^ ((4 * wave + (lane >> 4)) & 15);
    const uint32_t* w_q = nullptr;             // weight stream: this lane's row in its unit
    const uint16_t* w_s = nullptr;
    const uint16_t* w_b = nullptr;
    const uint16_t* v_s = nullptr;             // scale/bias stream (kSB4): its own unit
    const uint16_t* v_b = nullptr;

    // Units u = g, g + G, ... of the list ordered (block of 8 items, column
    // block, item): work groups are dispatched to the 8 XCDs round-robin, so
    // the column blocks of one item have the same u modulo 8 and run at the
    // same time on one XCD, sharing its L2 for the gathered activation rows.
    const int n_units = (n_items + 7) / 8 * 8 * n_cb;
    if (a.dn_pre && g == G - 1) {  // uniform; this work group has the fewest units
        __shared__ int s_wtot[kGuWaves];
        down_schedule(a, s_wtot);
    }
    // Grouped schedule: the work groups on one XCD (g % 8) form groups of
    // n_cb; a group takes a cost-balanced contiguous run of items and its
    // members one column block each, so the column blocks of an item run at
    // the same time on one XCD (sharing its L2 for the gathered activation
    // rows) and every group carries about the same work.  Otherwise (a grid
    // that does not split so): the round-robin list below.
    const int gpx = (G / 8) / n_cb;  // groups per XCD
    // decided from the host's item bound alone, so that the schedule's loads
    // can go out together with the tile count's
    const int n_bound = gu_item_bound(a);
    const bool grouped = kGuGrouped && G % 8 == 0 && gpx > 0 && n_bound <= kGuPer * kGuThreads &&
                         (long long)n_bound <= (long long)kGuRunMax * 8 * gpx / 4;
    __shared__ int s_items[kGuRunMax];
    int i_next = 0, i_end = 0, my_cb = 0;
    if (grouped) {
        const int x = g % 8, j = g / 8;
        if (j >= gpx * n_cb) return;  // uniform: no group for this work group
        my_cb = j % n_cb;
        i_end = item_run(a, n_raw, n_tiles, n_items, 8 * gpx, x * gpx + j / n_cb, s_items);
    }
    int u_next = g;
    while (true) {
        // ---- descriptors of up to kBatch units ----
        __syncthreads();  // the previous batch is done with s_unit / s_src / s_dst
        int nb = 0;
        while (nb < kBatch && (grouped ? i_next < i_end : u_next < n_units)) {
            int cb, item;
            if (grouped) {
                cb = my_cb;
                item = s_items[i_next++];
            } else {
                const int blk = u_next / (8 * n_cb), r = u_next - blk * 8 * n_cb;
                cb = r >> 3;
                item = blk * 8 + (r & 7);
                u_next += G;
                if (item >= n_items) continue;
            }
            int e = 0, row0, M, shared = 0;
            if (item < n_tiles) {
                int r0, nx;
                gu_tile_entries(a, item >> a.item_sh, e, r0, nx);
                gu_item_rows(a, item, n_raw, r0, nx, row0, M);
                if (M <= 0) continue;  // uniform: an empty part of a tile
            } else {
                shared = 1;
                row0 = (item - n_tiles) * kGuShRows;
                M = min(kGuShRows, a.T - row0);
            }
            const int bi = nb++;
            if (tid == 0) s_unit[bi] = UnitDesc{e, row0, M, cb, shared};
            if (tid < kMT) {
                int src = 0, dst = -1;
                if (tid < M) {
                    src = shared ? row0 + tid : a.perm[row0 + tid] / a.k;
                    dst = row0 + tid;
                }
                s_src[bi][tid] = src;
                s_dst[bi][tid] = dst;
            }
        }
        if (nb == 0) break;
        __syncthreads();
        int a_unit = -1, w_unit = -1, v_unit = -1;

        // ---- loaders (clamped to valid addresses, never under a branch) ----
        // Rows past M were given source row 0 in the descriptor (their products
        // are never stored), and columns at or past K read a column of the same
        // row below 64 (their weights are zeroed in compute), so every load
        // stays inside x.  Each stream keeps the per-lane addresses of the unit
        // it is reading in registers and refreshes them from LDS only when it
        // crosses into the next unit, so the per-chunk work is a few adds.
        // Activation load p of a lane covers tile rows 32p..32p+31 (subtile p),
        // so a unit with NMS subtiles needs loads 0..NMS-1 only.
        auto tile_of = [&](auto buf_tag) -> unsigned char* {
            constexpr int b = decltype(buf_tag)::value & 3;
            return b == 0 ? lds_a0 : b == 1 ? lds_a1 : b == 2 ? lds_a2 : lds_a3;
        };
        // Stream positions are (unit bb of the batch, chunk c), uniform; past
        // the batch they are clamped to its last chunk (loads that are never
        // used, at valid addresses).
        auto clamp_pos = [&](int& bb, int& c) {
            if (bb >= nb) {
                bb = nb - 1;
                c = NL - 1;
            }
        };
        // column of this lane's piece of chunk (bb, c) (refreshing the row
        // offsets when the stream enters a new unit)
        auto a_refresh = [&](int bb, int c) {
            clamp_pos(bb, c);
            if (bb != a_unit) {  // uniform: once per unit
                a_unit = bb;
#pragma unroll
                for (int p = 0; p < kGuALoads; ++p)
                    a_row[p] = (uint32_t)s_src[bb][(tid + kGuThreads * p) >> 4] * (uint32_t)K;
            }
            // a piece at or past K (a chunk past K, or the second half of a
            // chunk that ends at K + 64) reads a column of the same row below
            // 64 instead; its weights are zero
            const uint32_t col = (uint32_t)(c * kKC + 8 * a_lslot);
            return col < (uint32_t)K ? col : (uint32_t)((8 * a_lslot) & 63);
        };
        // direct-to-LDS load of rows 32p + 4 * wave .. +3 of an activation chunk
        // (buffer form: see x_rsrc)
        auto dma_a = [&](auto buf_tag, uint32_t col, int p) {
            unsigned char* dst = tile_of(buf_tag) + (32 * p + 4 * wave) * kRowBytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (__attribute__((address_space(3))) void*)dst,
                                                     16, (a_row[p] + col) * 2u, 0, 0, 0);
        };
        auto w_refresh = [&](int bb, int c) {
            clamp_pos(bb, c);
            if (bb != w_unit) {  // uniform: once per unit
                w_unit = bb;
                const UnitDesc ud = uniform_desc(s_unit[bb]);
                // field by field: selecting a whole Q4 by a per-lane condition
                // would read it from the kernel arguments through memory
                const bool sh = ud.shared != 0;
                const uint32_t* gq = sh ? a.sh_gate.q : a.gate.q;
                const uint32_t* uq = sh ? a.sh_up.q : a.up.q;
                const int j0 = ud.cb * kGuCols + 16 * wave;
                const size_t wrow = (size_t)ud.e * Nw + (j0 < Nw ? j0 + jrow : 0);
                w_q = (is_up ? uq : gq) + wrow * (K / 8) + 4 * half;
                if (!kSB4) {
                    const uint16_t* gs = sh ? a.sh_gate.scale : a.gate.scale;
                    const uint16_t* us = sh ? a.sh_up.scale : a.up.scale;
                    const uint16_t* gb = sh ? a.sh_gate.bias : a.gate.bias;
                    const uint16_t* ub = sh ? a.sh_up.bias : a.up.bias;
                    w_s = (is_up ? us : gs) + wrow * (K / kGroup);
                    w_b = (is_up ? ub : gb) + wrow * (K / kGroup);
                }
            }
            return c;
        };
        auto load_w_lo = [&](int c, WChunk& st) {
            const int kc0 = c * kKC < K ? c * kKC : 0;
            st.lo = *(const u32x4*)(w_q + kc0 / 8);
        };
        auto load_w_hi = [&](int c, WChunk& st) {
            const int kc0 = c * kKC < K ? c * kKC : 0;
            const int kc1 = kc0 + kGroup < K ? kc0 + kGroup : kc0;
            st.hi = *(const u32x4*)(w_q + kc1 / 8);
        };
        auto load_w = [&](int c, WChunk& st) {
            load_w_lo(c, st);
            load_w_hi(c, st);
        };
        auto load_sb = [&](int c, WChunk& st) {  // !kSB4: this chunk's pairs
            const int kc0 = c * kKC < K ? c * kKC : 0;
            const int kc1 = kc0 + kGroup < K ? kc0 + kGroup : kc0;
            if (pair_sb) {
                st.sp = *(const uint32_t*)(w_s + kc0 / kGroup);
                st.bp = *(const uint32_t*)(w_b + kc0 / kGroup);
            } else {  // odd group count: two 2-byte loads each
                st.sp = (uint32_t)w_s[kc0 / kGroup] | ((uint32_t)w_s[kc1 / kGroup] << 16);
                st.bp = (uint32_t)w_b[kc0 / kGroup] | ((uint32_t)w_b[kc1 / kGroup] << 16);
            }
        };
        // kSB4: scales and biases of chunks c..c+3 of unit bb (c a multiple of 4)
        auto load_sb4 = [&](int bb, int c, u32x4& s4, u32x4& b4) {
            clamp_pos(bb, c);
            c &= ~3;  // the clamped end is no multiple of 4
            if (bb != v_unit) {  // uniform: once per unit
                v_unit = bb;
                const UnitDesc ud = uniform_desc(s_unit[bb]);
                const bool sh = ud.shared != 0;
                const uint16_t* gs = sh ? a.sh_gate.scale : a.gate.scale;
                const uint16_t* us = sh ? a.sh_up.scale : a.up.scale;
                const uint16_t* gb = sh ? a.sh_gate.bias : a.gate.bias;
                const uint16_t* ub = sh ? a.sh_up.bias : a.up.bias;
                const int j0 = ud.cb * kGuCols + 16 * wave;
                const size_t wrow = (size_t)ud.e * Nw + (j0 < Nw ? j0 + jrow : 0);
                v_s = (is_up ? us : gs) + wrow * (K / kGroup);
                v_b = (is_up ? ub : gb) + wrow * (K / kGroup);
            }
            s4 = *(const u32x4*)(v_s + 2 * c);
            b4 = *(const u32x4*)(v_b + 2 * c);
        };
        // One chunk: 8 steps of (dequantise 8 k of the lane's weight row,
        // NMS MFMAs).  issue(j) puts the next chunks' global loads between the
        // steps, so that the waves of a CU do not all queue their loads at once
        // right after the barrier.
        auto compute = [&](auto nms_tag, int c, const unsigned char* tile, const WChunk& st,
                           uint32_t sp, uint32_t bp, auto&& issue) {
            constexpr int NMS = decltype(nms_tag)::value;
            const bool ok0 = c * kKC < K, ok1 = c * kKC + kGroup < K;
            const float s0 = ok0 ? dq_scale(sp & 0xFFFFu) : 0.0f;
            const float b0 = ok0 ? bf16_to_f32(bp & 0xFFFFu) : 0.0f;
            const float s1 = ok1 ? dq_scale(sp >> 16) : 0.0f;
            const float b1 = ok1 ? bf16_to_f32(bp >> 16) : 0.0f;
            // row 32*ms + lane%32 has (row & 15) == (lane & 15) for every ms, so the
            // swizzled slot offset is shared by the subtiles
            const unsigned char* trow = tile + (lane & 31) * kRowBytes;
            const int sw = lane & 15;
            // each step reads its activation fragments first; the step's
            // dequantisation covers the LDS latency
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int slot = (j < 4 ? 0 : 8) + 4 * half + (j & 3);
                const int so = (slot ^ sw) << 4;
                bf16x8 Af[NMS];
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    Af[ms] = *(const bf16x8*)(trow + 32 * ms * kRowBytes + so);
                __builtin_amdgcn_sched_barrier(0);
                issue(j);
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 B =
                    j < 4 ? dequant8(st.lo[j & 3], s0, b0) : dequant8(st.hi[j & 3], s1, b1);
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B, Af[ms], acc[ms], 0, 0, 0);
            }
        };
        // h = bf16(SiLU(gate) * up): elements i (gate row) and i + 8 (up row)
        auto epilogue = [&](int bb) {
            const UnitDesc ud = uniform_desc(s_unit[bb]);
            const int n_ms = (ud.M + 31) >> 5;
            const int j0 = ud.cb * kGuCols + 16 * wave;
            if (j0 < Nw) {
                uint16_t* out = ud.shared ? a.h_sh : a.h;
#pragma unroll
                for (int ms = 0; ms < 4; ++ms) {
                    const int row = 32 * ms + (lane & 31);
                    if (ms >= n_ms || row >= ud.M) continue;
                    // columns 8gq + 4h .. +3 per lane; lanes l and l + 32 (same
                    // row) trade groups so each stores 8 consecutive columns
                    uint2 own[2];
#pragma unroll
                    for (int gq = 0; gq < 2; ++gq) {
                        float hv[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            hv[r] = silu(acc[ms][4 * gq + r]) * acc[ms][8 + 4 * gq + r];
                        own[gq].x = pack_bf16x2(hv[0], hv[1]);
                        own[gq].y = pack_bf16x2(hv[2], hv[3]);
                    }
                    const uint2 send = half ? own[0] : own[1];
                    uint2 recv;
                    recv.x = (uint32_t)__shfl_xor((int)send.x, 32, 64);
                    recv.y = (uint32_t)__shfl_xor((int)send.y, 32, 64);
                    const uint2 lo = half ? recv : own[0];
                    const uint2 hi = half ? own[1] : recv;
                    *(u32x4*)(out + (size_t)s_dst[bb][row] * a.I + j0 + 8 * half) =
                        u32x4{lo.x, lo.y, hi.x, hi.y};
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
        };
        // Four chunks c0..c0+3 of unit bb.  Activations run three chunks
        // ahead (direct-to-LDS), weights two (registers).  FIRST / LAST: the
        // first / final four chunks of the unit; the activation loads of the
        // final four from the second chunk on belong to the next unit (all
        // four loads: that unit's subtile count is not known here).
        //
        // A wave's reads of chunk c need every wave's loads of it, so each wave
        // waits for its own loads of chunk c explicitly before the barrier
        // that publishes the chunk: vmcnt(N), N = the vector
        // memory operations this wave issued after them, counted from the
        // fixed issue order below (a lower bound where it is not known, which
        // only waits longer).
        auto four_chunks = [&](auto nms_tag, auto first_tag, auto last_tag, int bb, int c0) {
            constexpr int NMS = decltype(nms_tag)::value;
            constexpr bool FIRST = decltype(first_tag)::value != 0;
            constexpr bool LAST = decltype(last_tag)::value != 0;
            auto step = [&](auto u_tag) {
                constexpr int u = decltype(u_tag)::value;
                const int c = c0 + u;
                // stream targets: activations three chunks ahead, weights two
                constexpr bool a_next = LAST && u >= 1, w_next = LAST && u >= 2;
                const int a_bb = a_next ? bb + 1 : bb, a_c = a_next ? u - 1 : c + 3;
                const int w_bb = w_next ? bb + 1 : bb, w_c = w_next ? u - 2 : c + 2;
                constexpr int N = gu_ops_after<kSB4, FIRST, LAST, NMS>(u);
                wait_vmcnt<N>();
                asm volatile("s_barrier" ::: "memory");
                constexpr int nA = (LAST && u >= 1) ? kGuALoads : NMS;
                Int<(u + 3) & 3> nxt;
                int cw = 0;
                // step 0: this wave's activation loads of chunk c+3; steps 2
                // and 4: codes of chunk c+2; step 6: its scales/biases
                auto issue = [&](int j) {
                    if (j == 0) {
                        const uint32_t col = a_refresh(a_bb, a_c);
#pragma unroll
                        for (int p = 0; p < nA; ++p) dma_a(nxt, col, p);
                    } else if (j == 2) {
                        cw = w_refresh(w_bb, w_c);
                        load_w_lo(cw, bst[(u + 2) % kStages]);
                    } else if (j == 4) {
                        load_w_hi(cw, bst[(u + 2) % kStages]);
                    } else if (j == 6) {
                        if (kSB4) {
                            if (u == 2) load_sb4(w_bb, w_c, s4n, b4n);
                        } else {
                            load_sb(cw, bst[(u + 2) % kStages]);
                        }
                    }
                };
                if (kSB4)
                    compute(nms_tag, c, tile_of(u_tag), bst[u], s4c[u], b4c[u], issue);
                else
                    compute(nms_tag, c, tile_of(u_tag), bst[u], bst[u].sp, bst[u].bp, issue);
            };
            step(Int<0>{});
            step(Int<1>{});
            step(Int<2>{});
            step(Int<3>{});
            if (kSB4) {
                s4c = s4n;
                b4c = b4n;
            }
        };
        auto unit_loop = [&](auto nms_tag, int bb) {
            if (NL == kStages) {
                four_chunks(nms_tag, Int<1>{}, Int<1>{}, bb, 0);
                return;
            }
            four_chunks(nms_tag, Int<1>{}, Int<0>{}, bb, 0);
            for (int c0 = kStages; c0 < NL - kStages; c0 += kStages)
                four_chunks(nms_tag, Int<0>{}, Int<0>{}, bb, c0);
            four_chunks(nms_tag, Int<0>{}, Int<1>{}, bb, NL - kStages);
        };

        // ---- the batch: one continuous pipeline over nb units ----
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
        {
            // every wave is done with the ring (the previous batch's last chunks)
            __syncthreads();
            uint32_t col = a_refresh(0, 0);
#pragma unroll
            for (int p = 0; p < kGuALoads; ++p) dma_a(Int<0>{}, col, p);
            col = a_refresh(0, 1);
#pragma unroll
            for (int p = 0; p < kGuALoads; ++p) dma_a(Int<1>{}, col, p);
            col = a_refresh(0, 2);
#pragma unroll
            for (int p = 0; p < kGuALoads; ++p) dma_a(Int<2>{}, col, p);
            load_w(w_refresh(0, 0), bst[0]);
            if (!kSB4) load_sb(0, bst[0]);
            load_w(w_refresh(0, 1), bst[1]);
            if (kSB4)
                load_sb4(0, 0, s4c, b4c);
            else
                load_sb(1, bst[1]);
            // the per-chunk waits count from a steady pipeline; the start of a
            // batch simply waits for everything
            wait_vmcnt<0>();
        }
        for (int bb = 0; bb < nb; ++bb) {
            switch ((__builtin_amdgcn_readfirstlane(s_unit[bb].M) + 31) >> 5) {
                case 1: unit_loop(Int<1>{}, bb); break;
                case 2: unit_loop(Int<2>{}, bb); break;
                case 3: unit_loop(Int<3>{}, bb); break;
                default: unit_loop(Int<4>{}, bb); break;
            }
            epilogue(bb);
        }
    }
}

static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n < 1024 ? n : 1024;  // the schedules' 32-bit run cuts assume <= 1024 groups
    }
    return cus[dev];
}

// Whether the routed down projection runs as down_resident_kernel, whose
// schedule the gate/up kernel writes.
static bool down_is_resident(const PrefillArgs& a) {
    return (a.I + kKC - 1) / kKC == kStages && a.tile_bound <= kMaxRoutedItems;
}

static hipError_t launch_gate_up(const PrefillArgs& a_in, hipStream_t s) {
    PrefillArgs a = a_in;
    if (!down_is_resident(a)) a.dn_pre = nullptr;
    const int n_cb = (a.I + kGuCols - 1) / kGuCols;
    const int sh_items = (a.T + kGuShRows - 1) / kGuShRows;
    const int max_units = (a.tile_bound + sh_items + 7) / 8 * 8 * n_cb;
    int grid = device_cus();
    if (grid > max_units) grid = max_units;
    if (a.d % (8 * kGroup) == 0)
        hipLaunchKernelGGL(gate_up_kernel<true>, dim3(grid), dim3(kGuThreads), 0, s, a, n_cb);
    else
        hipLaunchKernelGGL(gate_up_kernel<false>, dim3(grid), dim3(kGuThreads), 0, s, a, n_cb);
    trace_point(s);
    return hipGetLastError();
}

// The routed rows' down projection into the fp16 staging rows.
static hipError_t launch_down_routed(const PrefillArgs& a, hipStream_t s) {
    const int n_cb = (a.d + kDnCols - 1) / kDnCols;
    if (down_is_resident(a)) {
        if (!a.dn_pre || !a.dn_exp) return hipErrorInvalidValue;
        const int grid = min(device_cus(), a.tile_bound * n_cb);
        if (a.I % (8 * kGroup) == 0)
            hipLaunchKernelGGL(down_resident_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a, n_cb);
        else
            hipLaunchKernelGGL(down_resident_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a, n_cb);
    } else {
        const int n_wg = ((a.tile_bound * n_cb) + 7) & ~7;
        hipLaunchKernelGGL(down_chunked_kernel, dim3(n_wg), dim3(kThreads), 0, s, a, a.tile_bound,
                           n_cb, n_wg);
    }
    trace_point(s);
    return hipGetLastError();
}

// Rows per shared-expert down item: 64, or 32 where 64-token items would leave
// CUs without a work group (the combine's reads of the staged rows are then
// spread over the whole chip).
static int shared_down_rows(int T, int n_cb) {
    return (T + 63) / 64 * n_cb >= device_cus() ? 64 : 32;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    hipError_t err = launch_gate_up(a, s);
    if (err != hipSuccess) return err;
    err = launch_down_routed(a, s);
    if (err != hipSuccess) return err;
    // the shared expert's down projection with the combine
    const int n_cb = (a.d + kDnCols - 1) / kDnCols;
    const int rows = shared_down_rows(a.T, n_cb);
    const int n_items = (a.T + rows - 1) / rows;
    const int n_wg = ((n_items * n_cb) + 7) & ~7;
    const bool il = a.I <= kStages * kKC;  // the shared GEMM is one group of chunks
    if (rows == 64 && il)
        hipLaunchKernelGGL((shared_down_combine_kernel<64, true>), dim3(n_wg), dim3(kThreads), 0, s,
                           a, n_items, n_cb, n_wg);
    else if (rows == 64)
        hipLaunchKernelGGL((shared_down_combine_kernel<64, false>), dim3(n_wg), dim3(kThreads), 0, s,
                           a, n_items, n_cb, n_wg);
    else if (il)
        hipLaunchKernelGGL((shared_down_combine_kernel<32, true>), dim3(n_wg), dim3(kThreads), 0, s,
                           a, n_items, n_cb, n_wg);
    else
        hipLaunchKernelGGL((shared_down_combine_kernel<32, false>), dim3(n_wg), dim3(kThreads), 0, s,
                           a, n_items, n_cb, n_wg);
    trace_point(s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Test hook: the same dequantisation written out as bf16, one word per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(Q4 m, int n_rows, int K,
                                                      uint16_t* __restrict__ w_out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // word index
    const size_t words = (size_t)n_rows * (K / 8);
    if (i >= words) return;
    const size_t n = i / (K / 8), kw = i % (K / 8);
    const size_t g = n * (K / kGroup) + (kw * 8) / kGroup;
    const bf16x8 v = dequant8(m.q[i], dq_scale(m.scale[g]), bf16_to_f32(m.bias[g]));
    *(bf16x8*)(w_out + n * K + kw * 8) = v;
}

hipError_t launch_dequant(Q4 m, int n_rows, int K, uint16_t* w_out, hipStream_t s) {
    const size_t words = (size_t)n_rows * (K / 8);
    if (words == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, m,
                       n_rows, K, w_out);
    return hipGetLastError();
}

}  // namespace q4moe
