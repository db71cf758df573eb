// lmhead.hip -- greedy decoding's token hand-off on the GPU.
//
// [Lily-M5] "Decode: minimize bytes per token": the greedy token stays on the
// device between decode steps -- the largest output logit picks it and it goes
// straight into the following step's input.  Here that is
// two kernels on the caller's stream:
//   1. lm_head_kernel: logits = head . x, a dequantising GEMV over the V x d Q4
//      output head (the experts' format, used as bf16 weights, fp32 sums),
//      plus each work group's best (logit, row) as a partial result;
//   2. lm_pick_kernel: the best of the partials -- the greedy token -- stored
//      in the caller's token slot, then the token's embedding row dequantised
//      to bf16 into the next step's input.
// With given logits (MOE_LOGITS_IN) lm_scan_kernel forms the partials instead
// of kernel 1.
//
// Order of the pick: larger logit first, equal logits by the lower index, a
// NaN logit counting as minus infinity.  That is a strict total order on
// (logit, index) pairs, so every reduction order gives the same token.
//
// Kernel 1 streams V * (d/2 + d/16) bytes of weights once (286 MB at
// V = 248,320, d = 2048), and its vector-ALU work (the dequantisation and the
// dot products, 23 instructions per 8 weights) takes about as long as that
// stream at full rate, so it is bound by both.  A wave computes four rows; lane l
// covers columns 32l .. 32l + 31 of every row, so one 16-byte load per row
// and lane brings a whole 1 KB row per wave, and all four rows' loads are in
// flight before the first is used.  The lane's slice of x stays in registers.
// Small work groups of four such waves, one per 16 rows, measured faster than
// bigger ones, than more rows per wave, and than persistent waves that
// double-buffer their loads (a work group waits for its slowest wave at its
// final reduction; small, short work groups keep the CUs filled).  The dot
// products stay on the vector ALUs (v_dot2_f32_bf16): a 16-row MFMA form
// was slower, its loads spanning 16 rows at 64 bytes each.
#include "lmhead.h"

namespace q4moe {
namespace {

constexpr int kLmWaves = 4;                    // waves per work group of kernel 1
constexpr int kLmRows = 4;                     // rows per wave
constexpr int kLmWgRows = kLmWaves * kLmRows;  // rows per work group
constexpr int kScanThreads = 256;
constexpr int kScanPer = 8;                    // logits per thread of lm_scan_kernel
constexpr int kPickThreads = 1024;
constexpr int kPickBatch = 16;                 // partials a thread loads before comparing

__device__ __forceinline__ float pick_key(float v) { return v != v ? -INFINITY : v; }

// (v, i) comes before (bv, bi) in the pick order.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Best (key, index) of the wave, returned to every lane.
__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, kWave);
        const int oi = __shfl_xor(i, o, kWave);
        if (beats(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

// Best over the work group's waves (s_v / s_i hold one entry per wave); the
// result goes to partial slot `slot`.  Called by every thread; contains a barrier.
template <int NW>
__device__ __forceinline__ void group_best(float v, int i, float* s_v, int* s_i, int2* part,
                                           int slot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_v[wave] = v;
        s_i[wave] = i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bv = s_v[0];
        int bi = s_i[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            if (beats(s_v[w], s_i[w], bv, bi)) {
                bv = s_v[w];
                bi = s_i[w];
            }
        part[slot] = int2{__float_as_int(bv), bi};  // one 8-byte store
    }
}

__global__ __launch_bounds__(kLmWaves * 64) void lm_head_kernel(const LmArgs a) {
    __shared__ float s_v[kLmWaves];
    __shared__ int s_i[kLmWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = a.d, V = a.V;
    const int row0 = blockIdx.x * kLmWgRows + wave * kLmRows;
    float acc[kLmRows];
#pragma unroll
    for (int r = 0; r < kLmRows; ++r) acc[r] = 0.0f;
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        const int kk = k0 < d ? k0 : 0;  // clamped, always valid; masked below
        u32x4 w[kLmRows];
        uint16_t sr[kLmRows], br[kLmRows];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) {
            const size_t row = (size_t)(row0 + r < V ? row0 + r : V - 1);  // clamped, valid
            w[r] = *(const u32x4*)(a.head.q + row * (size_t)(d / 8) + kk / 8);
            const size_t so = row * (size_t)(d / kGroup) + kk / kGroup;
            sr[r] = a.head.scale[so];
            br[r] = a.head.bias[so];
        }
        // every row's loads are in flight before any of them is used
        __builtin_amdgcn_sched_barrier(0);
        u32x4 xv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) xv[p] = ((const u32x4*)(a.x + kk))[p];
#pragma unroll
        for (int r = 0; r < kLmRows; ++r) {
            const float s9 = dq_scale(sr[r]), b = bf16_to_f32(br[r]);
            float part = 0.0f;
#pragma unroll
            for (int p = 0; p < 4; ++p) part = dot8_bf16(w[r][p], s9, b, xv[p], part);
            acc[r] += k0 < d ? part : 0.0f;
        }
    }
    float best = -INFINITY, mine = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int r = 0; r < kLmRows; ++r) {
        const float l = wave_sum_dpp(acc[r]);  // every lane holds the row's logit
        mine = lane == r ? l : mine;
        if (row0 + r < V && beats(pick_key(l), row0 + r, best, bi)) {
            best = pick_key(l);
            bi = row0 + r;
        }
    }
    if (lane < kLmRows && row0 + lane < V) a.logits[row0 + lane] = mine;
    group_best<kLmWaves>(best, bi, s_v, s_i, a.part, blockIdx.x);
}

// Partials of given logits: work group b covers logits [b * 2048, +2048).
__global__ __launch_bounds__(kScanThreads) void lm_scan_kernel(const LmArgs a) {
    __shared__ float s_v[kScanThreads / 64];
    __shared__ int s_i[kScanThreads / 64];
    const int V = a.V;
    const int i0 = (blockIdx.x * kScanThreads + threadIdx.x) * kScanPer;
    float v[kScanPer];
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) v[j] = a.logits[i0 + j < V ? i0 + j : V - 1];
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < V && beats(pick_key(v[j]), i0 + j, best, bi)) {
            best = pick_key(v[j]);
            bi = i0 + j;
        }
    wave_best(best, bi);
    group_best<kScanThreads / 64>(best, bi, s_v, s_i, a.part, blockIdx.x);
}

// The greedy token from n_part partials, then the next step's input.
__global__ __launch_bounds__(kPickThreads) void lm_pick_kernel(const LmArgs a, int n_part) {
    __shared__ float s_v[kPickThreads / 64];
    __shared__ int s_i[kPickThreads / 64];
    __shared__ int s_tok;
    const int tid = threadIdx.x;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int p0 = 0; p0 < n_part; p0 += kPickThreads * kPickBatch) {
        int2 pp[kPickBatch];
#pragma unroll
        for (int u = 0; u < kPickBatch; ++u) {
            const int p = p0 + u * kPickThreads + tid;
            const int pc = p < n_part ? p : 0;  // clamped, always valid
            pp[u] = a.part[pc];
        }
#pragma unroll
        for (int u = 0; u < kPickBatch; ++u)
            if (p0 + u * kPickThreads + tid < n_part &&
                beats(__int_as_float(pp[u].x), pp[u].y, best, bi)) {
                best = __int_as_float(pp[u].x);
                bi = pp[u].y;
            }
    }
    wave_best(best, bi);
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
        s_v[wave] = best;
        s_i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        float bv = s_v[0];
        int b = s_i[0];
#pragma unroll
        for (int w = 1; w < kPickThreads / 64; ++w)
            if (beats(s_v[w], s_i[w], bv, b)) {
                bv = s_v[w];
                b = s_i[w];
            }
        // every partial names a row below V, so b does too
        s_tok = b;
        *a.token = b;
    }
    if (!a.x_next) return;  // uniform
    __syncthreads();
    const int tok = min(max(s_tok, 0), a.V - 1), d = a.d;  // (already in range)
    const size_t row = (size_t)tok;
    for (int wd = tid; wd < d / 8; wd += kPickThreads) {
        const uint32_t code = a.embed.q[row * (size_t)(d / 8) + wd];
        const size_t g = row * (size_t)(d / kGroup) + wd / 8;
        const bf16x8 wv = dequant8(code, dq_scale(a.embed.scale[g]), bf16_to_f32(a.embed.bias[g]));
        *(bf16x8*)(a.x_next + 8 * (size_t)wd) = wv;
    }
}

}  // namespace

int lm_partials(int V, bool logits_in) {
    return logits_in ? (V + kScanThreads * kScanPer - 1) / (kScanThreads * kScanPer)
                     : (V + kLmWgRows - 1) / kLmWgRows;
}

hipError_t launch_lm_argmax(const LmArgs& a, bool logits_in, hipStream_t s) {
    const int n_part = lm_partials(a.V, logits_in);
    if (logits_in)
        lm_scan_kernel<<<n_part, kScanThreads, 0, s>>>(a);
    else
        lm_head_kernel<<<n_part, kLmWaves * 64, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_point(s);
    lm_pick_kernel<<<1, kPickThreads, 0, s>>>(a, n_part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_point(s);
    return hipSuccess;
}

}  // namespace q4moe
