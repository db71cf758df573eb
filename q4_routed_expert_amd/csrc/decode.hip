// decode.hip -- the whole MoE layer for one token (batch-1 decode).
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill and decode are different
// problems": at batch 1 each token is another full pass over the weights with
// almost no reuse, a memory-bound matrix-vector product that belongs on the
// vector ALUs.  Section "Decode: minimize bytes per token": expert input
// projections fused with the gate activation, the output projection fused
// with the routing scores and the shared expert, intermediates in registers.
//
// Three launches on one stream:
//   1. router: d/32 work groups each sum 32 rows of x . W_r for every expert;
//      the last group to arrive (device-scope counter) adds the partial sums in
//      a fixed order, applies the bias and runs the top-k;
//   2. gate/up: one wave per (selected or shared expert, intermediate row);
//      both the gate and the up row are streamed once with 16-byte loads and
//      h = bf16(SiLU(g) * u) is written;
//   3. down: each wave produces 4 outputs; for each of them it streams the
//      row of all k + 1 experts' down matrices and combines
//      y = bf16( sum_s w_s * P_s (slot order) + P_shared ).
// Every weight enters as the bf16 value bf16(q * s + b), the same operand the
// grouped GEMM feeds its matrix cores, so prefill and decode compute one
// function of the layer.
#include "internal.h"

namespace q4moe {

constexpr int kRouterRows = 32;  // rows of W_r per router work group

__global__ __launch_bounds__(256) void decode_router_kernel(const DecodeArgs a) {
    __shared__ float xs[kRouterRows];
    __shared__ float s_logits[kMaxExperts];
    __shared__ int s_last;
    const int tid = threadIdx.x, E = a.E;
    if (!a.logits_in) {
        const int g = blockIdx.x;
        if (tid < kRouterRows) xs[tid] = bf16_to_f32(a.x[kRouterRows * g + tid]);
        __syncthreads();
        if (tid < E) {
            float acc = 0.0f;
            const float* wp = a.w_router + (size_t)kRouterRows * g * E + tid;
#pragma unroll 8
            for (int j = 0; j < kRouterRows; ++j) acc = __builtin_fmaf(xs[j], wp[(size_t)j * E], acc);
            a.partial[(size_t)g * E + tid] = acc;
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        if (tid < E) {
            float acc = 0.0f;
            for (int gg = 0; gg < (int)gridDim.x; ++gg)
                acc += a.partial[(size_t)gg * E + tid];
            if (a.router_bias) acc += a.router_bias[tid];
            s_logits[tid] = acc;
            if (a.logits) a.logits[tid] = acc;
        }
        if (tid == 0) *a.counter = 0u;
    } else {
        if (tid < E) s_logits[tid] = a.logits[tid];
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

// One wave per (slot, intermediate row j); lane covers 32 consecutive k of
// each 2048-wide pass (half a quantisation group).  Weights are the bf16
// values bf16(q * s + b), as in the grouped GEMM, dotted with bf16 x in fp32.
__global__ __launch_bounds__(256) void decode_gate_up_kernel(const DecodeArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = blockIdx.y;  // 0..k-1 routed, k = shared
    const int j = blockIdx.x * 4 + wave;
    if (j >= a.I) return;
    const int d = a.d;
    Q4 G, U;
    size_t row;
    if (slot < a.k) {
        row = (size_t)a.sel_idx[slot] * a.I + j;
        G = a.gate;
        U = a.up;
    } else {
        row = j;
        G = a.sh_gate;
        U = a.sh_up;
    }
    float gsum = 0.0f, usum = 0.0f;
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        if (k0 < d) {
            const u32x4* xp = (const u32x4*)(a.x + k0);
            const u32x4 gq = *(const u32x4*)(G.q + row * (d / 8) + k0 / 8);
            const u32x4 uq = *(const u32x4*)(U.q + row * (d / 8) + k0 / 8);
            const size_t gi = row * (d / kGroup) + k0 / kGroup;
            const float gs = bf16_to_f32(G.scale[gi]), gb = bf16_to_f32(G.bias[gi]);
            const float us = bf16_to_f32(U.scale[gi]), ub = bf16_to_f32(U.bias[gi]);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const u32x4 xv = xp[p];
                gsum = dot8_bf16(gq[p], gs, gb, xv, gsum);
                usum = dot8_bf16(uq[p], us, ub, xv, usum);
            }
        }
    }
    gsum = wave_sum(gsum);
    usum = wave_sum(usum);
    if (lane == 0) a.h[(size_t)slot * a.I + j] = f32_to_bf16(silu(gsum) * usum);
}

// Each wave: 4 outputs n, 16 lanes per output, lane covers 32 consecutive k
// of each 512-wide pass over the expert intermediate dimension.
__global__ __launch_bounds__(256) void decode_down_kernel(const DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t s_h[];  // [(k+1)][I] bf16
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int I = a.I, k = a.k, d = a.d;
    for (int i = tid; i < (k + 1) * I / 8; i += 256)
        ((u32x4*)s_h)[i] = ((const u32x4*)a.h)[i];
    __syncthreads();
    const int n = blockIdx.x * 16 + wave * 4 + (lane >> 4);
    const int c = lane & 15;
    if (n >= d) return;
    float y = 0.0f;
    for (int s = 0; s <= k; ++s) {
        Q4 D;
        size_t row;
        if (s < k) {
            row = (size_t)a.sel_idx[s] * d + n;
            D = a.down;
        } else {
            row = n;
            D = a.sh_down;
        }
        float part = 0.0f;
        for (int kb = 0; kb < I; kb += 16 * 32) {
            const int k0 = kb + 32 * c;
            if (k0 < I) {
                const u32x4 q = *(const u32x4*)(D.q + row * (I / 8) + k0 / 8);
                const size_t gi = row * (I / kGroup) + k0 / kGroup;
                const float sc = bf16_to_f32(D.scale[gi]), bi = bf16_to_f32(D.bias[gi]);
                const u32x4* hv = (const u32x4*)(s_h + (size_t)s * I + k0);
#pragma unroll
                for (int p = 0; p < 4; ++p) part = dot8_bf16(q[p], sc, bi, hv[p], part);
            }
        }
        part = group_sum<16>(part);
        y = s < k ? y + a.sel_w[s] * part : y + part;
    }
    if (c == 0) a.y[n] = f32_to_bf16(y);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int rgrid = a.logits_in ? 1 : a.d / kRouterRows;
    hipLaunchKernelGGL(decode_router_kernel, dim3(rgrid), dim3(256), 0, s, a);
    trace_point(s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(decode_gate_up_kernel, dim3((a.I + 3) / 4, a.k + 1), dim3(256), 0, s, a);
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
    hipLaunchKernelGGL(decode_down_kernel, dim3((a.d + 15) / 16), dim3(256), lds, s, a);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
