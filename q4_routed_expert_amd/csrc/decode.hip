// decode.hip -- the whole MoE layer for one token (batch-1 decode).
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill and decode are different
// problems": at batch 1 each token is another full pass over the weights with
// almost no reuse, a memory-bound matrix-vector product that belongs on the
// vector ALUs.  Section "Decode: minimize bytes per token": expert input
// projections fused with the gate activation, the output projection fused
// with the routing scores and the shared expert, intermediates in registers.
//
// Three launches on one stream (every launch boundary costs several
// microseconds at batch 1, so the work is packed into as few as the data
// dependencies allow), each spread over thousands of waves so that the
// weight loads of many waves are in flight at once:
//   1. router partial sums (ceil(d/128) work groups, each sums 128 rows of
//      x . W_r for every expert, a whole row per load instruction; skipped
//      when the logits are given) and, in
//      the same launch, the shared expert's gate/up rows, which need no
//      routing;
//   2. every work group adds the partial sums in a fixed order (+ bias) and
//      runs the top-k itself -- the same arithmetic in every work group, so
//      every one finds the same experts -- then computes gate/up rows of its
//      routed slot: one wave per (slot, intermediate row j), the gate and up
//      rows streamed once with 16-byte loads per lane, h = bf16(SiLU(g) * u);
//   3. down: one wave per output n: each lane takes one code word of each of
//      the k + 1 experts' rows, and the wave combines
//      y = bf16( sum_s w_s * P_s (slot order) + P_shared ).
// Every weight enters as the bf16 value bf16(q * s + b), the same operand the
// grouped GEMM feeds its matrix cores, so prefill and decode compute one
// function of the layer.
#include "internal.h"

namespace q4moe {

constexpr int kRouterRows = 128;  // rows of W_r per router work group (DecodeWs sizes partial by it)
constexpr int kRouterWaves = 16;
constexpr int kRouterWaveRows = kRouterRows / kRouterWaves;
constexpr int kDecRows = 16;  // gate/up rows per 1024-thread work group, one wave each
constexpr int kDownWaves = 8;  // down outputs per work group, one wave each

static_assert(kRouterRows == MOE_DECODE_ROUTER_ROWS, "router partial rows");
static_assert(kRouterWaves * 64 == 1024 && 4 * 64 == kMaxExperts, "router work group shape");

// One wave: h[slot][j] = bf16(SiLU(W_gate[e] x)_j * (W_up[e] x)_j) for expert
// e (or the shared expert); lane covers 32 consecutive k of each 2048-wide
// pass (half a quantisation group).  Weights are the bf16 values
// bf16(q * s + b), as in the grouped GEMM, dotted with bf16 x in fp32.
__device__ __forceinline__ void gate_up_row(const DecodeArgs& a, const uint16_t* s_x, int slot,
                                            bool shared, int e, int j, int lane) {
    const int d = a.d;
    const size_t row = shared ? (size_t)j : (size_t)e * a.I + j;
    const uint32_t* gq = (shared ? a.sh_gate.q : a.gate.q) + row * (d / 8);
    const uint32_t* uq = (shared ? a.sh_up.q : a.up.q) + row * (d / 8);
    const uint16_t* gs = (shared ? a.sh_gate.scale : a.gate.scale) + row * (d / kGroup);
    const uint16_t* gb = (shared ? a.sh_gate.bias : a.gate.bias) + row * (d / kGroup);
    const uint16_t* us = (shared ? a.sh_up.scale : a.up.scale) + row * (d / kGroup);
    const uint16_t* ub = (shared ? a.sh_up.bias : a.up.bias) + row * (d / kGroup);
    float gsum = 0.0f, usum = 0.0f;
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        const int kk = k0 < d ? k0 : 0;  // clamped, always valid; masked below
        const u32x4 gw = *(const u32x4*)(gq + kk / 8);
        const u32x4 uw = *(const u32x4*)(uq + kk / 8);
        const float g_s = dq_scale(gs[kk / kGroup]), g_b = bf16_to_f32(gb[kk / kGroup]);
        const float u_s = dq_scale(us[kk / kGroup]), u_b = bf16_to_f32(ub[kk / kGroup]);
        u32x4 xv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) xv[p] = ((const u32x4*)(s_x + kk))[p];
        float gp = 0.0f, up = 0.0f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            gp = dot8_bf16(gw[p], g_s, g_b, xv[p], gp);
            up = dot8_bf16(uw[p], u_s, u_b, xv[p], up);
        }
        gsum += k0 < d ? gp : 0.0f;
        usum += k0 < d ? up : 0.0f;
    }
    const float g = wave_sum_dpp(gsum), u = wave_sum_dpp(usum);
    if (lane == 0) a.h[(size_t)slot * a.I + j] = f32_to_bf16(silu(g) * u);
}

// Copies x (d bf16, 16-byte pieces) into the work group's LDS: every wave of
// the group then reads its x operand from there instead of from L2.
__device__ __forceinline__ void stage_x(const DecodeArgs& a, uint16_t* s_x, int tid, int n_threads) {
    for (int i = tid; i < a.d / 8; i += n_threads)
        ((u32x4*)s_x)[i] = ((const u32x4*)a.x)[i];
}

// Work groups [0, n_part): partial[g][e] = sum of x[r] W_r[r][e] over the 128
// rows r of group g.  Wave w takes rows 8w .. 8w + 7 of the group, each lane
// four consecutive experts: one 16-byte load per row and lane, so one load
// instruction reads a whole 1 KB row of W_r (E = 256); x[r] is wave-uniform
// and comes through the scalar cache.  The sixteen waves' sums are then added
// in wave order through LDS.  Work groups from n_part on: the shared expert's
// gate/up rows, one per wave.
template <bool VEC>
__global__ __launch_bounds__(1024) void decode_router_shared_kernel(const DecodeArgs a,
                                                                    int n_part) {
    __shared__ float s_q[kRouterWaves][kMaxExperts];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[MOE_MAX_D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if ((int)blockIdx.x >= n_part) {  // uniform per work group
        stage_x(a, s_x, tid, 1024);
        __syncthreads();
        const int j = ((int)blockIdx.x - n_part) * kDecRows + wave;
        if (j < a.I) gate_up_row(a, s_x, a.k, true, 0, j, lane);
        return;
    }
    if (a.logits_in) return;  // uniform
    const int g = blockIdx.x, E = a.E, d = a.d;
    const int e0 = 4 * lane;
    // first row of this wave, made explicitly wave-uniform for the scalar loads of x
    const int r0 = __builtin_amdgcn_readfirstlane(g * kRouterRows + wave * kRouterWaveRows);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 w[kRouterWaveRows];
#pragma unroll
    for (int r = 0; r < kRouterWaveRows; ++r) {
        const uint32_t rr = (uint32_t)(r0 + r < d ? r0 + r : 0);  // clamped, always valid
        if constexpr (VEC) {
            const uint32_t ee = (uint32_t)(e0 < E ? e0 : 0);
            w[r] = *(const u32x4*)(a.w_router + (rr * (uint32_t)E + ee));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ee = (uint32_t)(e0 + i < E ? e0 + i : 0);
                w[r][i] = __float_as_uint(a.w_router[rr * (uint32_t)E + ee]);
            }
        }
    }
    // x[r0 .. r0 + 7]: one uniform 16-byte load (r0 is a multiple of 8 and d of 64)
    const bool r_ok = r0 < d;
    const u32x4 xq = *(const u32x4*)(a.x + (r_ok ? r0 : 0));
#pragma unroll
    for (int r = 0; r < kRouterWaveRows; ++r) {
        const uint32_t xw = xq[r >> 1];
        const float xv = r_ok ? __uint_as_float((r & 1) ? (xw & 0xffff0000u) : (xw << 16)) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(xv, __uint_as_float(w[r][i]), acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (e0 + i < kMaxExperts) s_q[wave][e0 + i] = acc[i];
    __syncthreads();
    if (tid < E) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kRouterWaves; ++q) v += s_q[q][tid];
        a.partial[(size_t)g * E + tid] = v;
    }
}

// Logits (partial sums added in order, + bias; or the given logits), top-k,
// then the gate/up rows of routed slot blockIdx.y.  Work group (0, 0) also
// writes the logits, the selection and the scores for the down kernel and
// the caller.
__global__ __launch_bounds__(1024) void decode_topk_gate_up_kernel(const DecodeArgs a, int n_part) {
    __shared__ float s_logits[kMaxExperts];
    __shared__ int s_sel[kMaxTopK];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[MOE_MAX_D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, E = a.E;
    const int slot = blockIdx.y;
    const bool first = blockIdx.x == 0 && slot == 0;
    stage_x(a, s_x, tid, 1024);  // covered by the barrier after the logits
    if (tid < E) {
        float v;
        if (a.logits_in) {
            v = a.logits[tid];
        } else {
            v = 0.0f;
            for (int g0 = 0; g0 < n_part; g0 += 16) {
                float p[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int gg = g0 + u < n_part ? g0 + u : 0;  // clamped, always valid
                    p[u] = a.partial[(size_t)gg * E + tid];
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) v += g0 + u < n_part ? p[u] : 0.0f;
            }
            if (a.router_bias) v += a.router_bias[tid];
            if (first) a.logits[tid] = v;
        }
        s_logits[tid] = v;
    }
    __syncthreads();
    if (wave == 0) {
        int se;
        float sw;
        wave_topk(s_logits, E, a.k, lane, &se, &sw);
        if (lane < a.k) {
            s_sel[lane] = se;
            if (first) {
                a.sel_idx[lane] = se;
                a.sel_w[lane] = sw;
                if (a.out_idx) a.out_idx[lane] = se;
                if (a.out_w) a.out_w[lane] = sw;
            }
        }
    }
    __syncthreads();
    const int j = blockIdx.x * kDecRows + wave;
    if (j < a.I) gate_up_row(a, s_x, slot, false, s_sel[slot], j, lane);
}

// One wave per output n; lane covers 8 consecutive intermediate k (one code
// word) of each 512-wide pass, for every slot.  All slots' loads are issued
// before the arithmetic; the combine then adds w_s * P_s in slot order and
// the shared expert last.
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_kernel(const DecodeArgs a) {
    // h of all k + 1 experts, staged once per work group
    __shared__ __attribute__((aligned(16))) uint16_t s_h[(kMaxTopK + 1) * MOE_MAX_INTER];
    const int tid = threadIdx.x, lane = tid & 63;
    const int I = a.I, k = a.k, d = a.d;
    for (int i = tid; i < (k + 1) * I / 8; i += 64 * kDownWaves)
        ((u32x4*)s_h)[i] = ((const u32x4*)a.h)[i];
    __syncthreads();
    const int n = blockIdx.x * kDownWaves + (tid >> 6);
    if (n >= d) return;
    float part[kMaxTopK + 1];
#pragma unroll
    for (int s = 0; s <= kMaxTopK; ++s) part[s] = 0.0f;
    for (int jb = 0; jb < I; jb += 64 * 8) {
        const int j0 = jb + 8 * lane;
        const int jj = j0 < I ? j0 : 0;  // clamped, always valid; masked below
        uint32_t q[kMaxTopK + 1];
        uint32_t sc[kMaxTopK + 1], bi[kMaxTopK + 1];
        u32x4 hv[kMaxTopK + 1];
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            const int ss = s <= k ? s : k;  // slots past k repeat the shared expert (discarded)
            const bool shared = ss == k;
            const size_t row = shared ? (size_t)n : (size_t)a.sel_idx[ss] * d + n;
            const Q4 D = shared ? a.sh_down : a.down;
            q[s] = D.q[row * (I / 8) + jj / 8];
            sc[s] = D.scale[row * (I / kGroup) + jj / kGroup];
            bi[s] = D.bias[row * (I / kGroup) + jj / kGroup];
            hv[s] = *(const u32x4*)(s_h + ss * I + jj);
        }
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            const float p = dot8_bf16(q[s], dq_scale(sc[s]), bf16_to_f32(bi[s]), hv[s], 0.0f);
            part[s] += j0 < I ? p : 0.0f;
        }
    }
    float y = 0.0f, sh = 0.0f;
#pragma unroll
    for (int s = 0; s <= kMaxTopK; ++s) {
        if (s <= k) {
            const float p = wave_sum_dpp(part[s]);
            if (s < k) y += a.sel_w[s] * p;
            else sh = p;
        }
    }
    if (lane == 0) a.y[n] = f32_to_bf16(y + sh);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int n_part = (a.d + kRouterRows - 1) / kRouterRows;
    const int n_rows = (a.I + kDecRows - 1) / kDecRows;
    if (a.E % 4 == 0)
        hipLaunchKernelGGL(decode_router_shared_kernel<true>, dim3(n_part + n_rows), dim3(1024), 0,
                           s, a, n_part);
    else
        hipLaunchKernelGGL(decode_router_shared_kernel<false>, dim3(n_part + n_rows), dim3(1024),
                           0, s, a, n_part);
    trace_point(s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(decode_topk_gate_up_kernel, dim3(n_rows, a.k), dim3(1024), 0, s, a, n_part);
    trace_point(s);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(decode_down_kernel, dim3((a.d + kDownWaves - 1) / kDownWaves),
                       dim3(64 * kDownWaves), 0, s, a);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
