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
// x is bf16, W_r fp32.  Each W_r value is split on chip into bf16 hi + lo
// parts (hi = bf16(w), lo = bf16(w - hi); the residual is below 2^-16 |w|) so
// the contraction runs on bf16 MFMA with fp32 accumulation: x*hi + x*lo.
// Work group: 64 tokens x 32 experts, four waves splitting K into quarters;
// each wave loads its operands straight from memory (x: 16 bytes per lane
// per M-fragment; W_r: one fp32 per lane per k, 32 consecutive experts per
// row = one 128-byte line) one K-step ahead of the matrix cores, and the four
// partial tiles are added in a fixed order through LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kRtM = 64, kRtN = 32;

__device__ __forceinline__ void split_hi_lo(const float (&w)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (__bf16)w[i];
        lo[i] = (__bf16)(w[i] - (float)hi[i]);
    }
}

__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, int T, int d, const float* __restrict__ W,
    const float* __restrict__ bias, int E, float* __restrict__ logits) {
    constexpr int S = 4;  // K-steps in flight per wave
    __shared__ float red[3][2][16][64];
    const int t0 = blockIdx.x * kRtM, e0 = blockIdx.y * kRtN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int n = e0 + (lane & 31);
    const bool n_ok = n < E;
    const int kq = d / 4;  // K range of this wave (d % 64 == 0)
    const int kbeg = wave * kq, kend = kbeg + kq;
    const int n_steps = (kq / 16 + S - 1) / S * S;  // padded; steps past kend add zeros
    const int ta = t0 + (lane & 31), tb = ta + 32;
    // clamped, always-valid addresses: loads stay outside branches (see the
    // grouped GEMM) and invalid values are zeroed where they are used
    const uint16_t* xa = x + (size_t)(ta < T ? ta : 0) * d;
    const uint16_t* xb = x + (size_t)(tb < T ? tb : 0) * d;
    const float* wcol = W + (n_ok ? n : 0);
    f32x16 acc0 = {}, acc1 = {};
    float wv[S][8];
    u32x4 av[S], bv[S];
    auto load = [&](int st, int k) {
        const int kk = (k < kend ? k : kbeg) + 8 * half;
        av[st] = *(const u32x4*)(xa + kk);
        bv[st] = *(const u32x4*)(xb + kk);
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[st][i] = wcol[(size_t)(kk + i) * E];
    };
#pragma unroll
    for (int u = 0; u < S - 1; ++u) load(u, kbeg + 16 * u);
    for (int s0 = 0; s0 < n_steps; s0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int k = kbeg + 16 * (s0 + u);
            const bool ok = k < kend && n_ok;
            float w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = ok ? wv[u][i] : 0.0f;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const bf16x8 A0 = __builtin_bit_cast(bf16x8, ta < T ? av[u] : z);
            const bf16x8 A1 = __builtin_bit_cast(bf16x8, tb < T ? bv[u] : z);
            bf16x8 hi, lo;
            split_hi_lo(w, hi, lo);
            load((u + S - 1) % S, k + 16 * (S - 1));
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, hi, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, hi, acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, lo, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, lo, acc1, 0, 0, 0);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            red[wave - 1][0][i][lane] = acc0[i];
            red[wave - 1][1][i][lane] = acc1[i];
        }
    }
    __syncthreads();
    if (wave > 0 || !n_ok) return;
    const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * half + (i & 3);
        const float v0 = ((acc0[i] + red[0][0][i][lane]) + red[1][0][i][lane]) + red[2][0][i][lane];
        const float v1 = ((acc1[i] + red[0][1][i][lane]) + red[1][1][i][lane]) + red[2][1][i][lane];
        if (t0 + r < T) logits[(size_t)(t0 + r) * E + n] = v0 + bb;
        if (t0 + 32 + r < T) logits[(size_t)(t0 + 32 + r) * E + n] = v1 + bb;
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
