// route.hip -- GPU-resident routing of one chunk of T tokens:
//   router logits -> top-k + renormalised scores -> histogram -> exclusive scan
//   -> stable scatter into expert-sorted order -> 32-row block map and the
//   128-row work map of the grouped GEMMs (three kernels: router logits, which
//   also clears the histogram; top-k with the histogram; scan, scatter and
//   maps).
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
// Work group: 64 tokens x 32 experts, eight waves splitting K into eighths;
// each wave loads its operands straight from memory (x: 16 bytes per lane
// per M-fragment; W_r: one fp32 per lane per k, 32 consecutive experts per
// row = one 128-byte line) a few K-steps ahead of the matrix cores, with
// 32-bit element offsets from the uniform base pointers, and the eight
// partial tiles are added in a fixed order through LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kRtM = 64, kRtN = 32, kRtWaves = 8;

__device__ __forceinline__ void split_hi_lo(const float (&w)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (__bf16)w[i];
        lo[i] = (__bf16)(w[i] - (float)hi[i]);
    }
}

__global__ __launch_bounds__(64 * kRtWaves) void router_logits_kernel(
    const uint16_t* __restrict__ x, int T, int d, const float* __restrict__ W,
    const float* __restrict__ bias, int E, float* __restrict__ logits,
    int32_t* __restrict__ blk_counts, int n_counts) {
    constexpr int S = 4;  // K-steps in flight per wave
    __shared__ float red[kRtWaves - 1][2][16][64];
    // the per-block expert counts that the top-k kernel accumulates start at 0
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counts; i += gridDim.x * blockDim.x)
        blk_counts[i] = 0;
    // Work groups go to the 8 XCDs round-robin by linear id.  Work item w =
    // token block * n_eb + expert block, and each XCD takes one contiguous
    // range of work items, so an XCD reads a 1/8 slice of x and all of W_r,
    // which together fit its L2.
    const int n_eb = (E + kRtN - 1) / kRtN;
    const int n_wg = gridDim.x, g = blockIdx.x, xcd = g & 7;
    int base = 0;
    for (int xx = 0; xx < xcd; ++xx) base += (n_wg - xx + 7) >> 3;
    const int wi = base + (g >> 3);
    const int t0 = (wi / n_eb) * kRtM, e0 = (wi - (wi / n_eb) * n_eb) * kRtN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int n = e0 + (lane & 31);
    const bool n_ok = n < E;
    const int kq = d / kRtWaves;  // K range of this wave (d % 64 == 0: a multiple of 8)
    const int kbeg = wave * kq, kend = kbeg + kq;
    const int n_steps = (kq / 16 + (kq % 16 != 0) + S - 1) / S * S;  // padded; extra steps add zeros
    const int ta = t0 + (lane & 31), tb = ta + 32;
    // clamped, always-valid element offsets: loads stay outside branches and
    // invalid values are zeroed where they are used
    const uint32_t xoa = (uint32_t)(ta < T ? ta : 0) * (uint32_t)d;
    const uint32_t xob = (uint32_t)(tb < T ? tb : 0) * (uint32_t)d;
    const uint32_t wo = (uint32_t)(n_ok ? n : 0);
    f32x16 acc0 = {}, acc1 = {};
    float wv[S][8];
    u32x4 av[S], bv[S];
    // a lane reads 8 consecutive k from kk: kk + 8 <= kend always (kq is a
    // multiple of 8, so the first 8 of the range are valid for any step that
    // runs past it)
    auto load = [&](int st, int k) {
        const int kk = k + 8 * half + 8 <= kend ? k + 8 * half : kbeg;
        av[st] = *(const u32x4*)(x + (xoa + (uint32_t)kk));
        bv[st] = *(const u32x4*)(x + (xob + (uint32_t)kk));
        const uint32_t wk = wo + (uint32_t)kk * (uint32_t)E;
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[st][i] = W[wk + (uint32_t)(i * E)];
    };
#pragma unroll
    for (int u = 0; u < S - 1; ++u) load(u, kbeg + 16 * u);
    for (int s0 = 0; s0 < n_steps; s0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int k = kbeg + 16 * (s0 + u);
            const bool ok = k + 8 * half < kend && n_ok;
            float w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = ok ? wv[u][i] : 0.0f;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const bool okx = k + 8 * half < kend;
            const bf16x8 A0 = __builtin_bit_cast(bf16x8, (ta < T && okx) ? av[u] : z);
            const bf16x8 A1 = __builtin_bit_cast(bf16x8, (tb < T && okx) ? bv[u] : z);
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
        float v0 = acc0[i], v1 = acc1[i];
#pragma unroll
        for (int w = 0; w < kRtWaves - 1; ++w) {
            v0 += red[w][0][i][lane];
            v1 += red[w][1][i][lane];
        }
        if (t0 + r < T) logits[(size_t)(t0 + r) * E + n] = v0 + bb;
        if (t0 + 32 + r < T) logits[(size_t)(t0 + 32 + r) * E + n] = v1 + bb;
    }
}

// ---------------------------------------------------------------------------
// The same logits for d a multiple of 1024 (the work group, wave and K split
// as above; the same MFMA operands in the same order, so the same bits), with
// the operands streamed differently: each wave stages its own 64 x rows
// through LDS in chunks of 64 k (8 KB, two buffers per wave), loaded straight
// into LDS 8 rows x 128 bytes per instruction (so a load instruction touches 8
// rows instead of 32) with the 16-byte columns XOR-swizzled by row on the
// source side; W_r comes as 32-bit buffer loads whose row steps are scalar
// offsets, one chunk ahead; hi and lo are formed two values per conversion.
// Rows past T and columns past E read clamped, valid data and are not stored.
// ---------------------------------------------------------------------------
constexpr int kRlChunk = 64;                 // k per staged chunk
constexpr int kRlRowB = kRlChunk * 2;        // bytes per staged row
constexpr int kRlBufB = kRtM * kRlRowB;      // 8 KB per chunk buffer

__device__ __forceinline__ void split_hi_lo_pk(const float (&w)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        h[p] = pack_bf16x2(w[2 * p], w[2 * p + 1]);
        const float h0 = __uint_as_float(h[p] << 16), h1 = __uint_as_float(h[p] & 0xFFFF0000u);
        l[p] = pack_bf16x2(w[2 * p] - h0, w[2 * p + 1] - h1);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// s_waitcnt vmcnt(N), the other counters not waited on
template <int N>
__device__ __forceinline__ void rl_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(64 * kRtWaves) void router_logits_lds_kernel(
    const uint16_t* __restrict__ x, int T, int d, const float* __restrict__ W,
    const float* __restrict__ bias, int E, float* __restrict__ logits,
    int32_t* __restrict__ blk_counts, int n_counts) {
    static_assert((kRtWaves - 1) * 2 * 16 * 64 * 4 <= kRtWaves * 2 * kRlBufB, "reduction fits the staging LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kRtWaves * 2 * kRlBufB];  // 128 KB
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counts; i += gridDim.x * blockDim.x)
        blk_counts[i] = 0;
    const int n_eb = (E + kRtN - 1) / kRtN;
    const int n_wg = gridDim.x, g = blockIdx.x, xcd = g & 7;
    int base = 0;
    for (int xx = 0; xx < xcd; ++xx) base += (n_wg - xx + 7) >> 3;
    const int wi = base + (g >> 3);
    const int t0 = (wi / n_eb) * kRtM, e0 = (wi - (wi / n_eb) * n_eb) * kRtN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int n = e0 + (lane & 31);
    const int kq = d / kRtWaves, kbeg = wave * kq;
    const int n_chunks = kq / kRlChunk;  // even: d % 1024 == 0
    unsigned char* buf = smem + wave * 2 * kRlBufB;
    // direct-to-LDS source offsets: instruction i covers staged rows 8i .. 8i + 7,
    // lane -> row 8i + lane / 8, LDS column lane % 8, source column (lane % 8) ^ (row % 8)
    uint32_t xsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + (lane >> 3);
        const uint32_t t = (uint32_t)(t0 + r < T ? t0 + r : T - 1);  // clamped, always valid
        xsrc[i] = (t * (uint32_t)d + (uint32_t)kbeg) * 2u + (uint32_t)((((lane & 7) ^ (r & 7))) << 4);
    }
    const uint32_t w_b = ((uint32_t)(n < E ? n : E - 1) + (uint32_t)(kbeg + 8 * half) * (uint32_t)E) * 4u;
    f32x16 acc0 = {}, acc1 = {};
    float wv[2][4][8];
    // generic lambdas: the buffer builtins stay out of the host pass
    auto dma = [&](auto, int c, int b) {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            (void*)x, 0, (int)((uint32_t)T * (uint32_t)d * 2u), 0x00020000);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(buf + b * kRlBufB + i * 1024), 16, xsrc[i],
                c * kRlRowB, 0, 0);
    };
    auto wload = [&](auto, int c, int b) {
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)W, 0, (int)((uint32_t)d * (uint32_t)E * 4u), 0x00020000);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wv[b][st][i] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rw, w_b, (c * kRlChunk + 16 * st + i) * E * 4, 0));
    };
    dma(0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    wload(0, 0, 0);
    for (int c0 = 0; c0 < n_chunks; c0 += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int c = c0 + b;
            __builtin_amdgcn_sched_barrier(0);
            // chunk c has landed in LDS: of the loads issued since its direct-to-LDS
            // loads only W's 32 of the same chunk may still be in flight (the
            // compiler does not order these LDS reads after those loads itself)
            rl_wait_vm<32>();
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 A[4][2];
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const int r = 32 * f + (lane & 31), col = 2 * st + half;
                    A[st][f] = *(const bf16x8*)(buf + b * kRlBufB + r * kRlRowB + ((col ^ (r & 7)) << 4));
                }
            // the next chunk into the other buffer (the last one repeats a chunk:
            // the same 40 loads every time keep the counts above exact)
            const int cn = c + 1 < n_chunks ? c + 1 : c;
            dma(0, cn, b ^ 1);
            __builtin_amdgcn_sched_barrier(0);  // the count above needs the LDS loads issued first
            wload(0, cn, b ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                bf16x8 hi, lo;
                split_hi_lo_pk(wv[b][st], hi, lo);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st][0], hi, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st][1], hi, acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st][0], lo, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[st][1], lo, acc1, 0, 0, 0);
            }
        }
    }
    rl_wait_vm<0>();  // the repeated last chunk has landed before the LDS is reused
    __syncthreads();
    float* red = (float*)smem;  // [kRtWaves - 1][2][16][64]
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            red[(((wave - 1) * 2 + 0) * 16 + i) * 64 + lane] = acc0[i];
            red[(((wave - 1) * 2 + 1) * 16 + i) * 64 + lane] = acc1[i];
        }
    }
    __syncthreads();
    if (wave > 0 || n >= E) return;
    const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * half + (i & 3);
        float v0 = acc0[i], v1 = acc1[i];
#pragma unroll
        for (int w = 0; w < kRtWaves - 1; ++w) {
            v0 += red[((w * 2 + 0) * 16 + i) * 64 + lane];
            v1 += red[((w * 2 + 1) * 16 + i) * 64 + lane];
        }
        if (t0 + r < T) logits[(size_t)(t0 + r) * E + n] = v0 + bb;
        if (t0 + 32 + r < T) logits[(size_t)(t0 + 32 + r) * E + n] = v1 + bb;
    }
}

__global__ __launch_bounds__(256) void zero_counts_kernel(int32_t* __restrict__ blk_counts,
                                                          int n_counts) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counts; i += gridDim.x * blockDim.x)
        blk_counts[i] = 0;
}

hipError_t launch_router_logits(const uint16_t* x, int T, int d, const float* w_router,
                                const float* router_bias, int E, float* logits,
                                int32_t* blk_counts, hipStream_t s) {
    const int n_counts = (T + MOE_ROUTE_BLOCK - 1) / MOE_ROUTE_BLOCK * E;
    if (!x) {  // the logits are given: only the counts are cleared
        hipLaunchKernelGGL(zero_counts_kernel, dim3((n_counts + 255) / 256), dim3(256), 0, s,
                           blk_counts, n_counts);
    } else {
        const int grid = ((T + kRtM - 1) / kRtM) * ((E + kRtN - 1) / kRtN);
        if (d % (kRtWaves * 2 * kRlChunk) == 0)
            hipLaunchKernelGGL(router_logits_lds_kernel, dim3(grid), dim3(64 * kRtWaves), 0, s, x, T,
                               d, w_router, router_bias, E, logits, blk_counts, n_counts);
        else
            hipLaunchKernelGGL(router_logits_kernel, dim3(grid), dim3(64 * kRtWaves), 0, s, x, T, d,
                               w_router, router_bias, E, logits, blk_counts, n_counts);
    }
    trace_point(s);
    return hipGetLastError();
}

// One wave per token: top-k selection and scores, and the token's k
// assignments added to its block's expert counts (integer atomics, so the
// counts do not depend on the order of the adds).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w,
                                                   int32_t* __restrict__ blk_counts) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;
    int e;
    float ws;
    wave_topk(logits + (size_t)t * E, E, k, lane, &e, &ws);
    if (lane < k) {
        idx[(size_t)t * k + lane] = e;
        w[(size_t)t * k + lane] = ws;
        atomicAdd(&blk_counts[(size_t)(t / MOE_ROUTE_BLOCK) * E + e], 1);
    }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       int32_t* blk_counts, hipStream_t s) {
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w,
                       blk_counts);
    trace_point(s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Histogram, exclusive scan, stable scatter and block maps over blocks of
// kRouteBlock consecutive tokens.  The histogram is built by the top-k kernel
// (each token's assignments added to blk_counts[block][E], cleared by the
// router kernel); then
//   route_scatter_kernel (one work group per block):
//     1. per expert: the total count and the count of the earlier blocks
//        (a fixed-order sum over the count table);
//     2. one wave scans the totals, ceil(totals/32) and ceil(totals/128) over
//        the experts: offsets and the first entry of each expert's tiles in
//        both maps (block 0 writes counts, offsets and both maps);
//     3. stable scatter: each wave owns 64 consecutive tokens; each lane ORs
//        its bit into a 64-bit mask per expert, and the sorted row of
//        (token, slot) is offsets[e] + rows of e in earlier blocks + rows of e
//        in the block's earlier waves + popcount(mask[e] & lanes below).
// Every step is deterministic and the result equals the sequential stable
// order (token ascending inside each expert).
// ---------------------------------------------------------------------------
constexpr int kRouteBlock = MOE_ROUTE_BLOCK;
constexpr int kRouteWaves = kRouteBlock / 64;
static_assert(kRouteBlock % 64 == 0 && kRouteBlock >= kMaxExperts, "route block");

__global__ __launch_bounds__(kRouteBlock) void route_scatter_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, const int32_t* __restrict__ blk_counts,
    int n_blk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, int32_t* __restrict__ block_map,
    int32_t* __restrict__ n_blocks, int32_t* __restrict__ tile_map, int32_t* __restrict__ n_tiles) {
    __shared__ unsigned long long mask[kRouteWaves][kMaxExperts];
    __shared__ int run[kRouteWaves][kMaxExperts];
    __shared__ int s_cnt[kMaxExperts], s_before[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1], s_b32[kMaxExperts + 1], s_b128[kMaxExperts + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = blockIdx.x;
    // this block's selections, loaded first so that their round trip overlaps
    // the count-table reads below
    const int t = g * kRouteBlock + tid;
    const bool valid = t < T;
    int ex[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) ex[s] = (valid && s < k) ? idx[(size_t)t * k + s] : 0;

    // 1. totals and earlier-block counts
    if (tid < E) {
        // sixteen blocks' counts in flight at a time (one load after another,
        // each waited for, would cost one memory round trip per block)
        int tot = 0, before = 0;
        for (int b0 = 0; b0 < n_blk; b0 += 16) {
            int c[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int b = b0 + u < n_blk ? b0 + u : 0;  // clamped, always valid
                c[u] = blk_counts[(size_t)b * E + tid];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int b = b0 + u;
                const int v = b < n_blk ? c[u] : 0;
                before += b < g ? v : 0;
                tot += v;
            }
        }
        s_cnt[tid] = tot;
        s_before[tid] = before;
    }
    for (int i = tid; i < kRouteWaves * kMaxExperts; i += kRouteBlock) (&mask[0][0])[i] = 0ull;
    __syncthreads();
    // 2. scan over the experts (wave 0, four experts per lane)
    if (wave == 0) {
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
    // 3a. this block's token masks
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
        if (valid && s < k) atomicOr(&mask[wave][ex[s]], 1ull << lane);
    __syncthreads();
    if (g == 0 && tid < E) {  // 2b. counts, offsets and both maps
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
        if (tid == 0) {
            offsets[E] = s_off[E];
            *n_blocks = s_b32[E];
            *n_tiles = s_b128[E];
        }
    }
    if (tid < E) {  // rows of each expert in the block's earlier waves
        int acc = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            run[w][tid] = acc;
            acc += __popcll(mask[w][tid]);
        }
    }
    __syncthreads();
    // 3b. scatter
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (valid && s < k) {
            const int e = ex[s];
            const int pos = s_off[e] + s_before[e] + run[wave][e] + __popcll(mask[wave][e] & below);
            perm[pos] = t * k + s;
            inv_perm[(size_t)t * k + s] = pos;
        }
    }
}

hipError_t launch_route_sort(const int32_t* idx, int T, int k, int E, const moe_routing* r,
                             hipStream_t s) {
    const int n_blk = (T + kRouteBlock - 1) / kRouteBlock;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(n_blk), dim3(kRouteBlock), 0, s, idx, T, k, E,
                       r->blk_counts, n_blk, r->counts, r->offsets, r->perm, r->inv_perm,
                       r->block_map, r->n_blocks, r->tile_map, r->n_tiles);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
