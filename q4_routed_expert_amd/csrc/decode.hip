// decode.hip -- the whole MoE layer for one token (batch-1 decode).
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill and decode are different
// problems": at batch 1 each token is another full pass over the weights with
// almost no reuse, a memory-bound matrix-vector product that belongs on the
// vector ALUs.  Section "Decode: minimize bytes per token": expert input
// projections fused with the gate activation, the output projection fused
// with the routing scores and the shared expert, intermediates in registers.
//
// Four launches on one stream:
//   1. router partial sums: d/32 work groups each sum 32 rows of x . W_r for
//      every expert (skipped when the logits are given);
//   2. one work group adds the partial sums in a fixed order, applies the
//      bias and runs the top-k;
//   3. gate/up: one wave per (selected or shared expert, 4 intermediate rows);
//      the gate and up rows are streamed once with 16-byte loads and
//      h = bf16(SiLU(g) * u) is written;
//   4. down: each wave produces 4 outputs; for each it streams the row of all
//      k + 1 experts' down matrices and combines
//      y = bf16( sum_s w_s * P_s (slot order) + P_shared ).
// Every weight enters as the bf16 value bf16(q * s + b), the same operand the
// grouped GEMM feeds its matrix cores, so prefill and decode compute one
// function of the layer.
#include "internal.h"

namespace q4moe {

constexpr int kRouterRows = 32;  // rows of W_r per router work group
constexpr int kGuRows = 4;       // gate/up rows per wave
constexpr int kDnRows = 4;       // down outputs per wave

// Partial router sums over 32 rows of W_r: partial[g][e] = sum_j x[32g+j] W_r[32g+j][e].
__global__ __launch_bounds__(256) void decode_router_partial_kernel(const DecodeArgs a) {
    const int g = blockIdx.x, e = threadIdx.x, E = a.E;
    if (e >= E) return;
    const float* wp = a.w_router + (size_t)kRouterRows * g * E + e;
    const uint16_t* xp = a.x + kRouterRows * g;
    float w[kRouterRows];
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) w[j] = wp[(size_t)j * E];
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kRouterRows; ++j) acc = __builtin_fmaf(bf16_to_f32(xp[j]), w[j], acc);
    a.partial[(size_t)g * E + e] = acc;
}

// Logits = partial sums added in a fixed order (+ bias), then top-k by one wave.
__global__ __launch_bounds__(256) void decode_router_topk_kernel(const DecodeArgs a, int n_part) {
    __shared__ float s_logits[kMaxExperts];
    const int tid = threadIdx.x, E = a.E;
    if (tid < E) {
        float v;
        if (a.logits_in) {
            v = a.logits[tid];
        } else {
            float p[8];
            v = 0.0f;
            for (int g0 = 0; g0 < n_part; g0 += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    p[u] = g0 + u < n_part ? a.partial[(size_t)(g0 + u) * E + tid] : 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) v += p[u];
            }
            if (a.router_bias) v += a.router_bias[tid];
            a.logits[tid] = v;
        }
        s_logits[tid] = v;
    }
    __syncthreads();
    if (tid < 64) {
        int e;
        float w;
        wave_topk(s_logits, E, a.k, tid, &e, &w);
        if (tid < a.k) {
            a.sel_idx[tid] = e;
            a.sel_w[tid] = w;
            if (a.out_idx) a.out_idx[tid] = e;
            if (a.out_w) a.out_w[tid] = w;
        }
    }
}

// One wave per (slot, 4 intermediate rows j); lane covers 32 consecutive k
// of each 2048-wide pass (half a quantisation group).  All of the wave's
// loads are issued before any arithmetic.  Weights are the bf16 values
// bf16(q * s + b), as in the grouped GEMM, dotted with bf16 x in fp32.
__global__ __launch_bounds__(256) void decode_gate_up_kernel(const DecodeArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = blockIdx.y;  // 0..k-1 routed, k = shared
    const int j0 = (blockIdx.x * 4 + wave) * kGuRows;
    if (j0 >= a.I) return;
    const int d = a.d;
    Q4 G, U;
    size_t row0;
    if (slot < a.k) {
        row0 = (size_t)a.sel_idx[slot] * a.I + j0;
        G = a.gate;
        U = a.up;
    } else {
        row0 = j0;
        G = a.sh_gate;
        U = a.sh_up;
    }
    float gsum[kGuRows] = {}, usum[kGuRows] = {};
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        if (k0 < d) {
            u32x4 gq[kGuRows], uq[kGuRows], xv[4];
            float gs[kGuRows], gb[kGuRows], us[kGuRows], ub[kGuRows];
#pragma unroll
            for (int r = 0; r < kGuRows; ++r) {
                const size_t row = row0 + r;
                gq[r] = *(const u32x4*)(G.q + row * (d / 8) + k0 / 8);
                uq[r] = *(const u32x4*)(U.q + row * (d / 8) + k0 / 8);
                const size_t gi = row * (d / kGroup) + k0 / kGroup;
                gs[r] = dq_scale(G.scale[gi]);
                gb[r] = bf16_to_f32(G.bias[gi]);
                us[r] = dq_scale(U.scale[gi]);
                ub[r] = bf16_to_f32(U.bias[gi]);
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) xv[p] = ((const u32x4*)(a.x + k0))[p];
#pragma unroll
            for (int r = 0; r < kGuRows; ++r)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    gsum[r] = dot8_bf16(gq[r][p], gs[r], gb[r], xv[p], gsum[r]);
                    usum[r] = dot8_bf16(uq[r][p], us[r], ub[r], xv[p], usum[r]);
                }
        }
    }
#pragma unroll
    for (int r = 0; r < kGuRows; ++r) {
        const float g = wave_sum(gsum[r]), u = wave_sum(usum[r]);
        if (lane == r) a.h[(size_t)slot * a.I + j0 + r] = f32_to_bf16(silu(g) * u);
    }
}

// Each wave: 4 outputs n, 16 lanes per output, lane covers 32 consecutive k
// of each 512-wide pass over the expert intermediate dimension.  The loads of
// all k + 1 experts' rows are issued before the arithmetic; the combine then
// adds w_s * P_s in slot order and the shared expert last.
__global__ __launch_bounds__(256) void decode_down_kernel(const DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t s_h[];  // [(k+1)][I] bf16
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int I = a.I, k = a.k, d = a.d;
    for (int i = tid; i < (k + 1) * I / 8; i += 256)
        ((u32x4*)s_h)[i] = ((const u32x4*)a.h)[i];
    __syncthreads();
    const int n = (blockIdx.x * 4 + wave) * kDnRows + (lane >> 4);
    const int c = lane & 15;
    if (n >= d) return;
    float part[kMaxTopK + 1] = {};
    for (int kb = 0; kb < I; kb += 16 * 32) {
        const int k0 = kb + 32 * c;
        if (k0 >= I) continue;
        u32x4 q[kMaxTopK + 1];
        float sc[kMaxTopK + 1], bi[kMaxTopK + 1];
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            q[s] = u32x4{0u, 0u, 0u, 0u};
            sc[s] = bi[s] = 0.0f;
            if (s <= k) {
                const bool shared = s == k;
                const Q4 D = shared ? a.sh_down : a.down;
                const size_t row = shared ? (size_t)n : (size_t)a.sel_idx[s] * d + n;
                q[s] = *(const u32x4*)(D.q + row * (I / 8) + k0 / 8);
                const size_t gi = row * (I / kGroup) + k0 / kGroup;
                sc[s] = dq_scale(D.scale[gi]);
                bi[s] = bf16_to_f32(D.bias[gi]);
            }
        }
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            if (s <= k) {
                const u32x4* hv = (const u32x4*)(s_h + (size_t)s * I + k0);
#pragma unroll
                for (int p = 0; p < 4; ++p) part[s] = dot8_bf16(q[s][p], sc[s], bi[s], hv[p], part[s]);
            }
        }
    }
    float y = 0.0f, sh = 0.0f;
#pragma unroll
    for (int s = 0; s <= kMaxTopK; ++s) {
        if (s <= k) {
            const float p = group_sum<16>(part[s]);
            if (s < k) y += a.sel_w[s] * p;
            else sh = p;
        }
    }
    if (c == 0) a.y[n] = f32_to_bf16(y + sh);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int n_part = a.d / kRouterRows;
    if (!a.logits_in)
        hipLaunchKernelGGL(decode_router_partial_kernel, dim3(n_part), dim3(256), 0, s, a);
    trace_point(s);
    hipLaunchKernelGGL(decode_router_topk_kernel, dim3(1), dim3(256), 0, s, a, n_part);
    trace_point(s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int gu_waves = (a.I + kGuRows - 1) / kGuRows;
    hipLaunchKernelGGL(decode_gate_up_kernel, dim3((gu_waves + 3) / 4, a.k + 1), dim3(256), 0, s,
                       a);
    trace_point(s);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds = sizeof(uint16_t) * (size_t)(a.k + 1) * a.I;
    static bool big_lds = false;  // (k+1) * inter bf16 may exceed the 64 KiB default
    if (lds > 65536 && !big_lds) {
        err = hipFuncSetAttribute((const void*)decode_down_kernel,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        big_lds = true;
    }
    const int dn_waves = (a.d + kDnRows - 1) / kDnRows;
    hipLaunchKernelGGL(decode_down_kernel, dim3((dn_waves + 3) / 4), dim3(256), lds, s, a);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
