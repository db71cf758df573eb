// prefill.hip -- the expert part of one MoE layer for a chunk of T tokens:
//   (1) grouped gate/up GEMM over the expert-sorted rows, SiLU(gate)*up fused,
//       plus the shared expert over all tokens            -> h, h_sh (bf16)
//   (2) grouped down GEMM of the routed rows               -> part (fp16)
//   (3) shared expert's down GEMM fused with the combine:
//       y_t = bf16( sum_s w[t,s] * part[t*k+s] (slot order) + shared )
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill: keep routing on the GPU,
// dequantize in flight": the grouped GEMM dequantises one small Q4 tile at a
// time on chip, accumulates in FP32, writes bf16, never materialises the
// expanded weights; 32-row tiles.  Section "Decode: minimize bytes per token":
// expert input projections fused with the gate activation, the output
// projection with the routing scores and the shared expert.
//
// Kernel design (gfx950).  One work item = up to 128 expert-sorted rows of
// one expert (the 128-row work map written by the routing) x one block of
// output columns.  A work group has 8 waves (two per SIMD); each wave owns 32
// output columns of one weight matrix (for gate/up: waves 0-3 gate, 4-7 up,
// on the same 128 intermediate columns; for the down GEMMs: 256 columns).
// Per K chunk of 128 (two quantisation groups):
//   - the activation rows (gathered through perm for the routed gate/up) are
//     staged in LDS as bf16, XOR-swizzled by row so that the 32 rows one
//     matrix-core operand read touches fall in distinct banks;
//   - each lane streams 2 x 16 contiguous bytes of one weight row straight
//     from HBM (lane n%32 <-> row n; the two halves of the wave take adjacent
//     16-byte pieces, so one load instruction covers 32 contiguous bytes of
//     each of 32 rows) and dequantises them in registers into the B operand
//     of v_mfma_f32_32x32x16_bf16: eight consecutive k of one column are
//     exactly one packed 32-bit word of codes.  The bf16 weights exist only in
//     VGPRs and each is dequantised once per work item, then reused for all
//     (up to four) 32-row M-subtiles;
//   - the weight stream runs kStages chunks deep in registers (three chunks
//     in flight while one is consumed) so that enough bytes are outstanding
//     per CU to keep HBM busy; the activation tile is double buffered in LDS
//     with its next chunk prefetched into registers (one barrier per chunk).
// SiLU(gate)*up pairs gate wave w with up wave w+4 through LDS at the end.
#include "internal.h"

namespace q4moe {

constexpr int kKC = 128;               // K per chunk
constexpr int kMT = kTileRows;         // rows per work item
constexpr int kMT2 = 64;               // token rows per shared-down + combine item
constexpr int kSlots = kKC / 8;        // 16-byte slots per staged row
constexpr int kRowBytes = kKC * 2;     // bytes per staged row
constexpr int kTileBytes = kMT * kRowBytes;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 4;             // weight chunks held in registers
constexpr int kALoads = kMT * kSlots / kThreads;
static_assert(kMT * kSlots % kThreads == 0, "A tile split");

enum { kGateUp = 0, kDownRouted = 1, kDownSharedCombine = 2 };

template <int N>
struct Int {
    static constexpr int value = N;
};

__device__ __forceinline__ int lds_off(int row, int slot) {
    return row * kRowBytes + ((slot ^ (row & 15)) << 4);
}

// One lane's share of one weight chunk: k in [kc + 32h, +32) (group kc/64)
// and [kc + 64 + 32h, +32) (group kc/64 + 1), h = lane / 32.  Scales and
// biases stay raw bf16 bits until use: converting them right after the load
// would make the wave wait for the load (and, since loads retire in order,
// for every older one), which would collapse the prefetch pipeline.
struct BChunk {
    u32x4 lo, hi;
    uint32_t s0, b0, s1, b1;
};

template <int MODE>
__global__ __launch_bounds__(kThreads) void expert_gemm_kernel(const PrefillArgs a, const int n_items,
                                                               const int n_cb, const int n_wg) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kTileBytes];
    __shared__ int s_src[kMT];  // source row of the A operand per tile row (-1: none)
    __shared__ int s_dst[kMT];  // output row per tile row

    // XCD-aware order: consecutive logical indices (the column blocks of one
    // item, which share the activation rows) stay on one XCD's L2.
    const int b = blockIdx.x;
    const int L = (b & 7) * (n_wg >> 3) + (b >> 3);
    const int item = L / n_cb, cb = L - item * n_cb;
    if (item >= n_items) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    int e = 0, row0, M;
    bool shared_item = false;
    const uint16_t* A;
    int K, Nw, lda;
    Q4 W;
    // wave -> (matrix, 32-column block inside the work group)
    const int mat = MODE == kGateUp ? (wave >> 2) : 0;
    const int wcb = MODE == kGateUp ? (wave & 3) : wave;
    const int cols_per_wg = MODE == kGateUp ? 128 : 256;
    if (MODE == kGateUp) {
        K = a.d; Nw = a.I; lda = a.d; A = a.x;
        if (item < a.tile_bound) {
            if (item >= *a.n_tiles) return;
            e = a.tile_map[2 * item];
            row0 = a.tile_map[2 * item + 1];
            M = min(kMT, a.offsets[e + 1] - row0);
            W = mat ? a.up : a.gate;
        } else {
            row0 = (item - a.tile_bound) * kMT;
            M = min(kMT, a.T - row0);
            shared_item = true;
            W = mat ? a.sh_up : a.sh_gate;
        }
    } else if (MODE == kDownRouted) {
        K = a.I; Nw = a.d; lda = a.I; A = a.h;
        if (item >= *a.n_tiles) return;
        e = a.tile_map[2 * item];
        row0 = a.tile_map[2 * item + 1];
        M = min(kMT, a.offsets[e + 1] - row0);
        W = a.down;
    } else {
        K = a.I; Nw = a.d; lda = a.I; A = a.h_sh;
        row0 = item * kMT2;
        M = min(kMT2, a.T - row0);
        W = a.sh_down;
    }
    if (tid < kMT) {
        int src = -1, dst = -1;
        if (tid < M) {
            const int r = row0 + tid;
            if (MODE == kGateUp) {
                src = shared_item ? r : a.perm[r] / a.k;
                dst = r;
            } else if (MODE == kDownRouted) {
                src = r;
                dst = a.perm[r];
            } else {
                src = r;
                dst = r;
            }
        }
        s_src[tid] = src;
        s_dst[tid] = dst;
    }
    __syncthreads();

    const int n_ms = (M + 31) >> 5;  // active 32-row subtiles
    const int wcol0 = cb * cols_per_wg + 32 * wcb;
    const bool wave_on = wcol0 < Nw;
    const int col = wcol0 + (lane & 31);  // this lane's output column
    const int n_chunks = (K + kKC - 1) / kKC;
    const size_t wrow = (size_t)e * Nw + (wave_on ? col : 0);  // weight row (matrix e, row col)

    u32x4 ast[kStages][kALoads];  // activation chunks in flight (same depth as the weights)
    BChunk bst[kStages];
    int src_row[kALoads];
#pragma unroll
    for (int p = 0; p < kALoads; ++p) src_row[p] = s_src[(tid + kThreads * p) >> 4];

    // Loads are issued unconditionally from always-valid (clamped) addresses
    // and invalid data is zeroed where it is used: a load under a branch makes
    // the compiler's wait-count analysis fall back to waiting for every
    // outstanding load, which would serialise the pipeline.
    auto load_a = [&](int c, u32x4 (&areg)[kALoads]) {
#pragma unroll
        for (int p = 0; p < kALoads; ++p) {
            const int slot = (tid + kThreads * p) & 15;
            const int kcol = c * kKC + 8 * slot;
            const int src = src_row[p];
            const size_t off = (size_t)(src >= 0 ? src : 0) * lda + (kcol < K ? kcol : 0);
            areg[p] = *(const u32x4*)(A + off);
        }
    };
    auto store_a = [&](int c, int buf, const u32x4 (&areg)[kALoads]) {
#pragma unroll
        for (int p = 0; p < kALoads; ++p) {
            const int i = tid + kThreads * p, row = i >> 4, slot = i & 15;
            const bool ok = src_row[p] >= 0 && c * kKC + 8 * slot < K;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4*)(lds + buf * kTileBytes + lds_off(row, slot)) = ok ? areg[p] : z;
        }
    };
    auto load_b = [&](int c, BChunk& st) {
        const int kc0 = c * kKC < K ? c * kKC : 0;            // clamped: always a valid chunk
        const int kc1 = kc0 + kGroup < K ? kc0 + kGroup : kc0;
        const uint32_t* qrow = W.q + wrow * (K / 8) + 4 * half;
        const size_t grow = wrow * (K / kGroup);
        st.lo = *(const u32x4*)(qrow + kc0 / 8);
        st.hi = *(const u32x4*)(qrow + kc1 / 8);
        st.s0 = W.scale[grow + kc0 / kGroup];
        st.b0 = W.bias[grow + kc0 / kGroup];
        st.s1 = W.scale[grow + kc1 / kGroup];
        st.b1 = W.bias[grow + kc1 / kGroup];
    };

    f32x16 acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x16{};

    // One chunk on the matrix cores for NMS active 32-row subtiles (a compile-
    // time count, so the inner loop has no branches).  The activation
    // fragments of step j+1 are read from LDS while step j's MFMAs run.
    auto compute = [&](auto nms_tag, int c, int buf, const BChunk& st) {
        constexpr int NMS = decltype(nms_tag)::value;
        const unsigned char* tile = lds + buf * kTileBytes;
        // chunks (or second halves) past K contribute zero weights
        const bool ok0 = c * kKC < K, ok1 = c * kKC + kGroup < K;
        const float s0 = ok0 ? bf16_to_f32(st.s0) : 0.0f, b0 = ok0 ? bf16_to_f32(st.b0) : 0.0f;
        const float s1 = ok1 ? bf16_to_f32(st.s1) : 0.0f, b1 = ok1 ? bf16_to_f32(st.b1) : 0.0f;
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
    const int n_loop = (n_chunks + kStages - 1) / kStages * kStages;
    auto main_loop = [&](auto nms_tag) {
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
                if (wave_on) compute(nms_tag, c, u & 1, bst[u]);
            }
        }
    };
    switch (n_ms) {
        case 1: main_loop(Int<1>{}); break;
        case 2: main_loop(Int<2>{}); break;
        case 3: main_loop(Int<3>{}); break;
        default: main_loop(Int<4>{}); break;
    }

    // The dequantised weights are the first MFMA operand, so the 32x32 output
    // tile is (weight row n) x (activation row): lane l holds activation row
    // l % 32 of its subtile and, in elements 4g..4g+3, the four consecutive
    // weight rows n = 8g + 4*(l/32) + 0..3.  Outputs therefore leave as
    // 8-byte groups of four columns.
    const int n_lane = wcol0 + 4 * half;  // + 8g
    if (MODE == kGateUp) {
        float* xch = (float*)lds;  // gate accumulators: [4 col blocks][4 subtiles][16][64 lanes]
        __syncthreads();
        if (mat == 0 && wave_on) {
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
                if (ms < n_ms)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xch[((wcb * 4 + ms) * 16 + i) * 64 + lane] = acc[ms][i];
        }
        __syncthreads();
        if (mat == 0 || !wave_on) return;
        uint16_t* out = shared_item ? a.h_sh : a.h;
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            const int row = 32 * ms + (lane & 31);
            if (ms >= n_ms || row >= M) continue;
            uint16_t* orow = out + (size_t)s_dst[row] * a.I + n_lane;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float hv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gate = xch[((wcb * 4 + ms) * 16 + 4 * g + r) * 64 + lane];
                    hv[r] = silu(gate) * acc[ms][4 * g + r];
                }
                uint2 v;
                v.x = pack_bf16x2(hv[0], hv[1]);
                v.y = pack_bf16x2(hv[2], hv[3]);
                *(uint2*)(orow + 8 * g) = v;
            }
        }
        return;
    }
    if (!wave_on) return;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        const int row = 32 * ms + (lane & 31);
        if (ms >= n_ms || row >= M) continue;
        const int dst = s_dst[row];
        if (MODE == kDownRouted) {
            uint16_t* prow = a.part + (size_t)dst * a.d + n_lane;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 v;
                v.x = (uint32_t)f32_to_f16(acc[ms][4 * g]) | ((uint32_t)f32_to_f16(acc[ms][4 * g + 1]) << 16);
                v.y = (uint32_t)f32_to_f16(acc[ms][4 * g + 2]) | ((uint32_t)f32_to_f16(acc[ms][4 * g + 3]) << 16);
                *(uint2*)(prow + 8 * g) = v;
            }
        } else {
            // fixed order: routed slots 0..k-1 with their scores, then the shared expert
            const uint16_t* pr = a.part + (size_t)dst * a.k * a.d + n_lane;
            const float* wt = a.topk_w + (size_t)dst * a.k;
            float ws[kMaxTopK];
            uint2 pv[kMaxTopK][4];
#pragma unroll
            for (int s = 0; s < kMaxTopK; ++s) {
                const int ss = s < a.k ? s : 0;  // loads stay unconditional
                ws[s] = wt[ss];
#pragma unroll
                for (int g = 0; g < 4; ++g) pv[s][g] = *(const uint2*)(pr + (size_t)ss * a.d + 8 * g);
            }
            uint16_t* yrow = a.y + (size_t)dst * a.d + n_lane;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < kMaxTopK; ++s) {
                    if (s < a.k) {
                        yv[0] += ws[s] * f16_to_f32(pv[s][g].x & 0xFFFFu);
                        yv[1] += ws[s] * f16_to_f32(pv[s][g].x >> 16);
                        yv[2] += ws[s] * f16_to_f32(pv[s][g].y & 0xFFFFu);
                        yv[3] += ws[s] * f16_to_f32(pv[s][g].y >> 16);
                    }
                }
                uint2 v;
                v.x = pack_bf16x2(yv[0] + acc[ms][4 * g], yv[1] + acc[ms][4 * g + 1]);
                v.y = pack_bf16x2(yv[2] + acc[ms][4 * g + 2], yv[3] + acc[ms][4 * g + 3]);
                *(uint2*)(yrow + 8 * g) = v;
            }
        }
    }
}

template <int MODE>
static hipError_t launch_gemm(const PrefillArgs& a, int n_items, int n_cols, int cols_per_wg,
                              hipStream_t s) {
    const int n_cb = (n_cols + cols_per_wg - 1) / cols_per_wg;
    const int n_wg = ((n_items * n_cb) + 7) & ~7;
    if (n_wg > 0)
        hipLaunchKernelGGL((expert_gemm_kernel<MODE>), dim3(n_wg), dim3(kThreads), 0, s, a,
                           n_items, n_cb, n_wg);
    trace_point(s);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    const int sh_items = (a.T + kMT - 1) / kMT;
    hipError_t err = launch_gemm<kGateUp>(a, a.tile_bound + sh_items, a.I, 128, s);
    if (err != hipSuccess) return err;
    err = launch_gemm<kDownRouted>(a, a.tile_bound, a.d, 256, s);
    if (err != hipSuccess) return err;
    return launch_gemm<kDownSharedCombine>(a, (a.T + kMT2 - 1) / kMT2, a.d, 256, s);
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
    const bf16x8 v = dequant8(m.q[i], bf16_to_f32(m.scale[g]), bf16_to_f32(m.bias[g]));
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
