// route.hip -- GPU-resident routing of one chunk of T tokens:
//   router logits -> top-k + renormalised scores -> histogram -> exclusive scan
//   -> stable scatter into expert-sorted order -> 32-row block map and the
//   128-row work map of the grouped GEMMs.
// All of it stays on the device in one stream with no host synchronisation
// ([Lily-M5] "Prefill: keep routing on the GPU, dequantize in flight": grouped
// GEMM needs each expert's rows stored together, hence histogram, prefix scan,
// scatter and block map after every top-8 selection, without a CPU round trip).
#include "internal.h"

namespace q4moe {

// ---------------------------------------------------------------------------
// Router logits l[t][e] = sum_j x[t][j] * W_r[j][e] (+ b[e]).
// x is bf16, W_r fp32.  W_r is split on chip into bf16 hi + lo parts
// (hi = bf16(w), lo = bf16(w - hi), residual below 2^-16 |w|) so the
// contraction runs on bf16 MFMA with fp32 accumulation.  Work group: 64
// tokens x 64 experts, four waves of 32x32, K step 32.
// ---------------------------------------------------------------------------
constexpr int kRtM = 64, kRtN = 64, kRtK = 32, kRtPad = 8;

__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, int T, int d, const float* __restrict__ W,
    const float* __restrict__ bias, int E, float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[kRtM][kRtK + kRtPad];
    __shared__ __attribute__((aligned(16))) uint16_t wh[kRtN][kRtK + kRtPad];
    __shared__ __attribute__((aligned(16))) uint16_t wl[kRtN][kRtK + kRtPad];
    const int t0 = blockIdx.x * kRtM, e0 = blockIdx.y * kRtN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc = {};
    for (int k0 = 0; k0 < d; k0 += kRtK) {
        {  // x tile: 64 rows x 32 bf16, one 16-byte piece per thread
            const int row = tid >> 2, c = tid & 3, t = t0 + row;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < T) v = *(const u32x4*)(x + (size_t)t * d + k0 + 8 * c);
            *(u32x4*)&xs[row][8 * c] = v;
        }
        {  // W tile: 32 k x 64 experts fp32, stored transposed as bf16 hi / lo
            const int kk = tid >> 3, c8 = (tid & 7) * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + c8 + i;
                const float f = e < E ? W[(size_t)(k0 + kk) * E + e] : 0.0f;
                const uint16_t hi = f32_to_bf16(f);
                wh[c8 + i][kk] = hi;
                wl[c8 + i][kk] = f32_to_bf16(f - bf16_to_f32(hi));
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRtK / 16; ++j) {
            const int kk = 16 * j + 8 * (lane >> 5);
            const bf16x8 a = *(const bf16x8*)&xs[32 * wm + (lane & 31)][kk];
            const bf16x8 bh = *(const bf16x8*)&wh[32 * wn + (lane & 31)][kk];
            const bf16x8 bl = *(const bf16x8*)&wl[32 * wn + (lane & 31)][kk];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    const int n = e0 + 32 * wn + (lane & 31);
    if (n < E) {
        const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = t0 + 32 * wm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (t < T) logits[(size_t)t * E + n] = acc[i] + bb;
        }
    }
}

hipError_t launch_router_logits(const uint16_t* x, int T, int d, const float* w_router,
                                const float* router_bias, int E, float* logits, hipStream_t s) {
    dim3 grid((T + kRtM - 1) / kRtM, (E + kRtN - 1) / kRtN);
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, x, T, d, w_router,
                       router_bias, E, logits);
    trace_point(s);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;
    int e;
    float ws;
    wave_topk(logits + (size_t)t * E, E, k, lane, &e, &ws);
    if (lane < k) {
        idx[(size_t)t * k + lane] = e;
        w[(size_t)t * k + lane] = ws;
    }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       hipStream_t s) {
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
    trace_point(s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Histogram, exclusive scan, stable scatter and block maps in one work group
// of 16 waves.  Wave w owns a contiguous token range (so ranges are in token
// order across waves).
//   1. per-wave per-expert totals with LDS atomic adds (order independent);
//   2. counts = column sums; each wave's base = exclusive sum over lower waves;
//   3. one wave scans counts, ceil(counts/32) and ceil(counts/128) over the
//      experts: offsets and the starts of each expert's tiles in both maps;
//   4. the maps: (expert, first sorted row) per tile, experts ascending;
//   5. stable scatter: per 64-token chunk each lane ORs its bit into a 64-bit
//      mask per expert; a lane's rank among the chunk's rows of expert e is
//      popcount(mask[e] & lanes-below), so sorted row = offsets[e] +
//      wave base[e] + rows of e in the wave's earlier chunks + rank.
// Every step is deterministic, so perm is the same on every run and equals
// the sequential stable order (token ascending inside each expert).
// ---------------------------------------------------------------------------
constexpr int kSortWaves = 16;

__global__ __launch_bounds__(1024) void route_sort_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ block_map, int32_t* __restrict__ n_blocks,
    int32_t* __restrict__ tile_map, int32_t* __restrict__ n_tiles) {
    __shared__ unsigned long long mask[kSortWaves][kMaxExperts];
    __shared__ int run[kSortWaves][kMaxExperts];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1], s_b32[kMaxExperts + 1], s_b128[kMaxExperts + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_chunks = (T + 63) / 64;
    const int cpw = (n_chunks + kSortWaves - 1) / kSortWaves;  // chunks per wave

    for (int i = tid; i < kSortWaves * kMaxExperts; i += 1024) (&run[0][0])[i] = 0;
    __syncthreads();
    for (int c = 0; c < cpw; ++c) {  // 1
        const int t = (wave * cpw + c) * 64 + lane;
        if (t < T)
            for (int s = 0; s < k; ++s) atomicAdd(&run[wave][idx[(size_t)t * k + s]], 1);
    }
    __syncthreads();
    if (tid < E) {  // 2
        int acc = 0;
        for (int w = 0; w < kSortWaves; ++w) {
            const int v = run[w][tid];
            run[w][tid] = acc;
            acc += v;
        }
        s_cnt[tid] = acc;
    }
    __syncthreads();
    if (wave == 0) {  // 3
        int c[4], b32[4], b128[4], sc = 0, s32 = 0, s128 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            const int v = e < E ? s_cnt[e] : 0;
            c[i] = v;
            b32[i] = (v + kBlockRows - 1) / kBlockRows;
            b128[i] = (v + kTileRows - 1) / kTileRows;
            sc += v;
            s32 += b32[i];
            s128 += b128[i];
        }
        int ic = sc, i32 = s32, i128 = s128;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int a = __shfl_up(ic, o, 64), b = __shfl_up(i32, o, 64),
                      cc = __shfl_up(i128, o, 64);
            if (lane >= o) {
                ic += a;
                i32 += b;
                i128 += cc;
            }
        }
        int ec = ic - sc, e32 = i32 - s32, e128 = i128 - s128;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) {
                s_off[e] = ec;
                s_b32[e] = e32;
                s_b128[e] = e128;
            }
            ec += c[i];
            e32 += b32[i];
            e128 += b128[i];
        }
        if (lane == 63) {
            s_off[E] = ic;
            s_b32[E] = i32;
            s_b128[E] = i128;
        }
    }
    __syncthreads();
    if (tid < E) {  // 4
        const int c = s_cnt[tid], o = s_off[tid];
        counts[tid] = c;
        offsets[tid] = o;
        for (int j = 0; j * kBlockRows < c; ++j) {
            const int b = s_b32[tid] + j;
            block_map[2 * b] = tid;
            block_map[2 * b + 1] = o + kBlockRows * j;
        }
        for (int j = 0; j * kTileRows < c; ++j) {
            const int b = s_b128[tid] + j;
            tile_map[2 * b] = tid;
            tile_map[2 * b + 1] = o + kTileRows * j;
        }
    }
    if (tid == 0) {
        offsets[E] = s_off[E];
        *n_blocks = s_b32[E];
        *n_tiles = s_b128[E];
    }
    for (int c = 0; c < cpw; ++c) {  // 5
        for (int i = lane; i < kMaxExperts; i += 64) mask[wave][i] = 0ull;
        __syncthreads();
        const int t = (wave * cpw + c) * 64 + lane;
        const bool valid = t < T;
        int ex[kMaxTopK];
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
            ex[s] = 0;
            if (valid && s < k) {
                ex[s] = idx[(size_t)t * k + s];
                atomicOr(&mask[wave][ex[s]], 1ull << lane);
            }
        }
        __syncthreads();
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s) {
            if (valid && s < k) {
                const int e = ex[s];
                const int pos = s_off[e] + run[wave][e] + __popcll(mask[wave][e] & below);
                perm[pos] = t * k + s;
                inv_perm[(size_t)t * k + s] = pos;
            }
        }
        __syncthreads();
        for (int i = lane; i < E; i += 64) run[wave][i] += __popcll(mask[wave][i]);
        __syncthreads();
    }
}

hipError_t launch_route_sort(const int32_t* idx, int T, int k, int E, const moe_routing* r,
                             hipStream_t s) {
    hipLaunchKernelGGL(route_sort_kernel, dim3(1), dim3(1024), 0, s, idx, T, k, E, r->counts,
                       r->offsets, r->perm, r->inv_perm, r->block_map, r->n_blocks, r->tile_map,
                       r->n_tiles);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
