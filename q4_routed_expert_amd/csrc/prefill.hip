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
// output columns.  A work group of NW waves gives each wave 32 output columns
// (for gate/up: 32 intermediate columns of both gate and up).  Per K chunk of
// 128 (two quantisation groups):
//   - the 128 activation rows (gathered through perm for the routed gate/up)
//     are staged in LDS as bf16, XOR-swizzled by row so that the 32 rows a
//     matrix-core operand read touches fall in distinct banks;
//   - each lane loads 32 contiguous bytes of one weight row (64 codes = one
//     group, one scale, one bias) straight from HBM with two 16-byte loads and
//     dequantises them in registers into the B operand of
//     v_mfma_f32_32x32x16_bf16: lane (n = lane % 32, half = lane / 32) feeds
//     column n with eight consecutive k, which is exactly one packed 32-bit
//     word of codes.  The bf16 weights therefore exist only in VGPRs;
//   - the same dequantised operand is reused for all (up to four) 32-row
//     M-subtiles of the item, so each weight is dequantised once per item.
// Global loads of chunk c+1 are issued before the matrix-core work of chunk
// c; the LDS tile is double buffered (one barrier per chunk).
#include "internal.h"

namespace q4moe {

constexpr int kKC = 128;               // K per chunk
constexpr int kMT = kTileRows;         // rows per work item
constexpr int kSlots = kKC / 8;        // 16-byte slots per staged row
constexpr int kRowBytes = kKC * 2;     // bytes per staged row
constexpr int kTileBytes = kMT * kRowBytes;

enum { kGateUp = 0, kDownRouted = 1, kDownSharedCombine = 2 };

__device__ __forceinline__ int lds_off(int row, int slot) {
    return row * kRowBytes + ((slot ^ (row & 15)) << 4);
}

template <int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void expert_gemm_kernel(const PrefillArgs a, const int n_items,
                                                              const int n_cb, const int n_wg) {
    constexpr int NF = MODE == kGateUp ? 2 : 1;  // weight fragments per wave
    constexpr int NT = NW * 64;
    constexpr int kALoads = kMT * kSlots / NT;
    static_assert(kMT * kSlots % NT == 0, "A tile split");
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
    Q4 W0, W1;
    if (MODE == kGateUp) {
        K = a.d; Nw = a.I; lda = a.d; A = a.x;
        if (item < a.tile_bound) {
            if (item >= *a.n_tiles) return;
            e = a.tile_map[2 * item];
            row0 = a.tile_map[2 * item + 1];
            M = min(kMT, a.offsets[e + 1] - row0);
            W0 = a.gate; W1 = a.up;
        } else {
            row0 = (item - a.tile_bound) * kMT;
            M = min(kMT, a.T - row0);
            shared_item = true;
            W0 = a.sh_gate; W1 = a.sh_up;
        }
    } else if (MODE == kDownRouted) {
        K = a.I; Nw = a.d; lda = a.I; A = a.h;
        if (item >= *a.n_tiles) return;
        e = a.tile_map[2 * item];
        row0 = a.tile_map[2 * item + 1];
        M = min(kMT, a.offsets[e + 1] - row0);
        W0 = a.down; W1 = a.down;
    } else {
        K = a.I; Nw = a.d; lda = a.I; A = a.h_sh;
        row0 = item * kMT;
        M = min(kMT, a.T - row0);
        W0 = a.sh_down; W1 = a.sh_down;
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

    const int n_ms = (M + 31) >> 5;          // active 32-row subtiles
    const int col = cb * 32 * NW + 32 * wave + (lane & 31);  // this lane's output column
    const bool wave_on = cb * 32 * NW + 32 * wave < Nw;
    const int n_chunks = (K + kKC - 1) / kKC;
    const size_t wrow = (size_t)e * Nw + (wave_on ? col : 0);  // weight row (matrix e, row col)

    u32x4 areg[kALoads];
    u32x4 bq[NF][2], bq_next[NF][2];
    float bs[NF], bb[NF], bs_next[NF], bb_next[NF];

    auto load_a = [&](int c) {
#pragma unroll
        for (int p = 0; p < kALoads; ++p) {
            const int i = tid + NT * p, row = i >> 4, slot = i & 15;
            const int kcol = c * kKC + 8 * slot;
            const int src = s_src[row];
            u32x4 v = {0u, 0u, 0u, 0u};
            if (src >= 0 && kcol < K) v = *(const u32x4*)(A + (size_t)src * lda + kcol);
            areg[p] = v;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int p = 0; p < kALoads; ++p) {
            const int i = tid + NT * p, row = i >> 4, slot = i & 15;
            *(u32x4*)(lds + buf * kTileBytes + lds_off(row, slot)) = areg[p];
        }
    };
    auto load_b = [&](int c) {
        const int kk = c * kKC + 64 * half;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const Q4 W = f == 0 ? W0 : W1;
            if (wave_on && kk < K) {
                const uint32_t* qp = W.q + wrow * (K / 8) + kk / 8;
                bq_next[f][0] = *(const u32x4*)qp;
                bq_next[f][1] = *(const u32x4*)(qp + 4);
                const size_t gi = wrow * (K / kGroup) + kk / kGroup;
                bs_next[f] = bf16_to_f32(W.scale[gi]);
                bb_next[f] = bf16_to_f32(W.bias[gi]);
            } else {
                bq_next[f][0] = bq_next[f][1] = u32x4{0u, 0u, 0u, 0u};
                bs_next[f] = bb_next[f] = 0.0f;
            }
        }
    };

    f32x16 acc[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[f][m] = f32x16{};

    load_a(0);
    load_b(0);
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        store_a(buf);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            bq[f][0] = bq_next[f][0];
            bq[f][1] = bq_next[f][1];
            bs[f] = bs_next[f];
            bb[f] = bb_next[f];
        }
        __syncthreads();
        if (c + 1 < n_chunks) {
            load_a(c + 1);
            load_b(c + 1);
        }
        if (wave_on) {
            const unsigned char* tile = lds + buf * kTileBytes;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bf16x8 B[NF];
#pragma unroll
                for (int f = 0; f < NF; ++f) B[f] = dequant8(bq[f][j >> 2][j & 3], bs[f], bb[f]);
#pragma unroll
                for (int ms = 0; ms < 4; ++ms) {
                    if (ms < n_ms) {
                        const int row = 32 * ms + (lane & 31);
                        const bf16x8 Av = *(const bf16x8*)(tile + lds_off(row, 8 * half + j));
#pragma unroll
                        for (int f = 0; f < NF; ++f)
                            acc[f][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Av, B[f],
                                                                                 acc[f][ms], 0, 0, 0);
                    }
                }
            }
        }
    }

    if (!wave_on) return;
    // Accumulator layout of v_mfma_f32_32x32x16_bf16: lane holds column
    // lane % 32 and, in element i, row 8*(i/4) + 4*(lane/32) + i%4.
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
        if (ms >= n_ms) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * ms + 8 * (i >> 2) + 4 * half + (i & 3);
            if (row >= M) continue;
            const int dst = s_dst[row];
            if (MODE == kGateUp) {
                const float v = silu(acc[0][ms][i]) * acc[NF - 1][ms][i];
                uint16_t* out = shared_item ? a.h_sh : a.h;
                out[(size_t)dst * a.I + col] = f32_to_bf16(v);
            } else if (MODE == kDownRouted) {
                a.part[(size_t)dst * a.d + col] = f32_to_f16(acc[0][ms][i]);
            } else {
                const uint16_t* pr = a.part + (size_t)dst * a.k * a.d + col;
                const float* wt = a.topk_w + (size_t)dst * a.k;
                float sum = 0.0f;
                for (int s = 0; s < a.k; ++s) sum += wt[s] * f16_to_f32(pr[(size_t)s * a.d]);
                a.y[(size_t)dst * a.d + col] = f32_to_bf16(sum + acc[0][ms][i]);
            }
        }
    }
}

template <int NW, int MODE>
static hipError_t launch_gemm(const PrefillArgs& a, int n_items, int n_cols, hipStream_t s) {
    const int n_cb = (n_cols + 32 * NW - 1) / (32 * NW);
    const int n_wg = ((n_items * n_cb) + 7) & ~7;
    if (n_wg > 0)
        hipLaunchKernelGGL((expert_gemm_kernel<NW, MODE>), dim3(n_wg), dim3(NW * 64), 0, s, a,
                           n_items, n_cb, n_wg);
    trace_point(s);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    const int sh_items = (a.T + kMT - 1) / kMT;
    hipError_t err = launch_gemm<4, kGateUp>(a, a.tile_bound + sh_items, a.I, s);
    if (err != hipSuccess) return err;
    err = launch_gemm<4, kDownRouted>(a, a.tile_bound, a.d, s);
    if (err != hipSuccess) return err;
    return launch_gemm<4, kDownSharedCombine>(a, sh_items, a.d, s);
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
