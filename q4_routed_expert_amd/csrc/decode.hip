// decode.hip -- the whole MoE layer for one token (batch-1 decode).
// Sources: [Lily-M5] = "Perplexity's Lily beats MLX-LM on MacBook M5 because
// it only runs one model".  Section "Prefill and decode are different
// problems": at batch 1 each token is another full pass over the weights with
// almost no reuse, a memory-bound matrix-vector product that belongs on the
// vector ALUs.  Section "Decode: minimize bytes per token": expert input
// projections fused with the gate activation, the output projection fused
// with the routing scores and the shared expert, intermediates in registers.
//
// Three launches on one stream (a launch boundary costs about as much as a
// grid-wide wait inside one kernel on this chip, so the two cross-work-group
// dependencies -- the top-k needs every logit, the down projection every h
// value -- are kernel boundaries), each spread over hundreds of work groups so
// that the weight loads of many waves are in flight at once:
//   1. router partial sums over blocks of 128 rows x 64 experts of W_r
//      (skipped when the logits are given) and, in the same launch, the shared
//      expert's gate/up rows, which need no routing;
//   2. every work group adds the partial sums in a fixed order (+ bias) and
//      runs the top-k itself -- the same arithmetic in every work group, so
//      every one finds the same experts -- while its other waves compute rows
//      of the shared expert's down projection (its h is ready, and it needs
//      no routing); then it computes gate/up rows of its routed slot: one
//      wave per (slot, intermediate row j), the gate and up rows streamed
//      once with 16-byte loads per lane, h = bf16(SiLU(g) * u);
//   3. down: 16 lanes per (output row, routed expert) task, 16-byte pieces
//      per lane; the selected experts, h and every weight piece are loaded
//      before any arithmetic, and y = bf16( sum_s w_s * P_s (slot order) +
//      P_shared ).
// Every weight enters as the bf16 value bf16(q * s + b), the same operand the
// grouped GEMM feeds its matrix cores, so prefill and decode compute one
// function of the layer.
#include "internal.h"

namespace q4moe {

constexpr int kRouterRows = 128;  // rows of W_r per router work group (DecodeWs sizes partial by it)
constexpr int kDecRows = 16;  // gate/up rows per 1024-thread work group, one wave each
constexpr int kSharedTokens = 2;  // tokens per shared-expert gate/up work group
constexpr int kSharedRowsPerGroup = 4;  // shared gate/up rows per work group (one per wave)

static_assert(kRouterRows == MOE_DECODE_ROUTER_ROWS, "router partial rows");
static_assert(MOE_MAX_DECODE_TOKENS == 8, "token buckets 1, 2, 4, 8");

// One wave: h[slot][j] = bf16(SiLU(W_gate[e] x)_j * (W_up[e] x)_j) for expert
// e (or the shared expert); lane covers 32 consecutive k of each 2048-wide
// pass (half a quantisation group).  Weights are the bf16 values
// bf16(q * s + b), as in the grouped GEMM, dotted with bf16 x in fp32.
__device__ __forceinline__ void gate_up_row(const DecodeArgs& a, const uint16_t* s_x, int h_row,
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
    if (lane == 0) a.h[(size_t)h_row * a.I + j] = f32_to_bf16(silu(g) * u);
}

// R routed gate/up rows j0, j0 + js, .. of expert e for one token, one wave:
// the loads of all R rows are issued before any arithmetic and x is read from
// LDS once for all of them.  Per row the arithmetic is gate_up_row's.
template <int R>
__device__ __forceinline__ void gate_up_rows(const DecodeArgs& a, const uint16_t* s_x, int h_row,
                                             int e, int j0, int js, int lane) {
    const int d = a.d, I = a.I;
    float gsum[R], usum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) gsum[r] = usum[r] = 0.0f;
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        const int kk = k0 < d ? k0 : 0;  // clamped, always valid; masked below
        u32x4 gw[R], uw[R];
        uint16_t gsr[R], gbr[R], usr[R], ubr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = j0 + r * js;
            const uint32_t row = (uint32_t)(e * I + (j < I ? j : 0));  // clamped, always valid
            const uint32_t qo = row * (uint32_t)(d / 8) + (uint32_t)(kk / 8);
            const uint32_t so = row * (uint32_t)(d / kGroup) + (uint32_t)(kk / kGroup);
            gw[r] = *(const u32x4*)(a.gate.q + qo);
            uw[r] = *(const u32x4*)(a.up.q + qo);
            gsr[r] = a.gate.scale[so];
            gbr[r] = a.gate.bias[so];
            usr[r] = a.up.scale[so];
            ubr[r] = a.up.bias[so];
        }
        // every load of the R rows is in flight before any of them is used
        // (otherwise the compiler waits for each scale load on its own)
        __builtin_amdgcn_sched_barrier(0);
        u32x4 xv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) xv[p] = ((const u32x4*)(s_x + kk))[p];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float g_s = dq_scale(gsr[r]), g_b = bf16_to_f32(gbr[r]);
            const float u_s = dq_scale(usr[r]), u_b = bf16_to_f32(ubr[r]);
            float gp = 0.0f, up = 0.0f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                gp = dot8_bf16(gw[r][p], g_s, g_b, xv[p], gp);
                up = dot8_bf16(uw[r][p], u_s, u_b, xv[p], up);
            }
            gsum[r] += k0 < d ? gp : 0.0f;
            usum[r] += k0 < d ? up : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = j0 + r * js;
        const float g = wave_sum_dpp(gsum[r]), u = wave_sum_dpp(usum[r]);
        if (lane == 0 && j < I) a.h[(size_t)h_row * I + j] = f32_to_bf16(silu(g) * u);
    }
}

// The shared expert's gate/up row j for tokens t0 .. t0 + n_tok - 1 (at most
// NT): each weight is dequantised once and dotted with every token's x (their
// x rows are s_x + t * d).  h row of token t: t * (k + 1) + k.
template <int NT>
__device__ __forceinline__ void shared_gate_up_rows(const DecodeArgs& a, const uint16_t* s_x,
                                                    int t0, int n_tok, int j, int lane) {
    const int d = a.d;
    const size_t row = (size_t)j;
    const uint32_t* gq = a.sh_gate.q + row * (d / 8);
    const uint32_t* uq = a.sh_up.q + row * (d / 8);
    const uint16_t* gs = a.sh_gate.scale + row * (d / kGroup);
    const uint16_t* gb = a.sh_gate.bias + row * (d / kGroup);
    const uint16_t* us = a.sh_up.scale + row * (d / kGroup);
    const uint16_t* ub = a.sh_up.bias + row * (d / kGroup);
    float gsum[NT], usum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) gsum[t] = usum[t] = 0.0f;
    for (int kb = 0; kb < d; kb += 64 * 32) {
        const int k0 = kb + 32 * lane;
        const int kk = k0 < d ? k0 : 0;  // clamped, always valid; masked below
        const u32x4 gw = *(const u32x4*)(gq + kk / 8);
        const u32x4 uw = *(const u32x4*)(uq + kk / 8);
        const float g_s = dq_scale(gs[kk / kGroup]), g_b = bf16_to_f32(gb[kk / kGroup]);
        const float u_s = dq_scale(us[kk / kGroup]), u_b = bf16_to_f32(ub[kk / kGroup]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < n_tok) {  // uniform
                u32x4 xv[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) xv[p] = ((const u32x4*)(s_x + t * d + kk))[p];
                float gp = 0.0f, up = 0.0f;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    gp = dot8_bf16(gw[p], g_s, g_b, xv[p], gp);
                    up = dot8_bf16(uw[p], u_s, u_b, xv[p], up);
                }
                gsum[t] += k0 < d ? gp : 0.0f;
                usum[t] += k0 < d ? up : 0.0f;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n_tok) {
            const float g = wave_sum_dpp(gsum[t]), u = wave_sum_dpp(usum[t]);
            if (lane == 0)
                a.h[(size_t)((t0 + t) * (a.k + 1) + a.k) * a.I + j] = f32_to_bf16(silu(g) * u);
        }
    }
}

// Copies n_tok rows of x from token t0 on (d bf16 each, 16-byte pieces) into
// the work group's LDS: every wave of the group then reads its x operand from
// there instead of from L2.
__device__ __forceinline__ void stage_x(const DecodeArgs& a, uint16_t* s_x, int t0, int n_tok,
                                        int tid, int n_threads) {
    const u32x4* src = (const u32x4*)(a.x + (size_t)t0 * a.d);
    for (int i = tid; i < n_tok * a.d / 8; i += n_threads) ((u32x4*)s_x)[i] = src[i];
}

// Router work groups: g = rb * n_eb + eb, rb < ceil(d / 128), eb < ceil(E / 64):
// partial[rb][t][e] = sum of x[t][r] W_r[r][e] over the 128 rows r of row
// block rb, for the 64 experts e of expert block eb and every token t.  Thread
// (rr = tid / 16, e4 = tid % 16) takes rows rr, rr + 16, .., rr + 112 and experts
// 4 e4 .. 4 e4 + 3: one 16-byte load per row, so one load instruction of a
// wave reads 256 contiguous bytes of each of four rows, and a work group reads
// 32 KB of W_r.  The block's x slice is staged in LDS first.  Sums: over
// the thread's rows in order, then over the four row offsets of a wave
// (shuffles), then over the four waves in order.  Work groups from n_router
// on: the shared expert's gate/up rows, one per wave, for a group of up to
// kSharedTokens tokens (more tokens: more work groups).
constexpr int kRtThreads = 256;
constexpr int kRtExperts = 64;  // experts per router work group
static_assert(kRtThreads / 16 * 8 == kRouterRows, "router rows per work group");

template <int NT, bool VEC>
__global__ __launch_bounds__(kRtThreads) void decode_router_shared_kernel(const DecodeArgs a,
                                                                          int n_router) {
    constexpr int NS = NT < kSharedTokens ? NT : kSharedTokens;
    constexpr int kQBytes = 4 * NT * kRtExperts * 4 + NT * kRouterRows * 2;
    constexpr int kXBytes = NS * MOE_MAX_D * 2;
    // the router's sums and the shared part's x never share a work group
    __shared__ __attribute__((aligned(16))) unsigned char s_mem[kQBytes > kXBytes ? kQBytes : kXBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T;
    if ((int)blockIdx.x >= n_router) {  // uniform per work group
        uint16_t* s_x = (uint16_t*)s_mem;
        const int n_rows = (a.I + kSharedRowsPerGroup - 1) / kSharedRowsPerGroup;
        const int b = (int)blockIdx.x - n_router, rb = b % n_rows, t0 = (b / n_rows) * NS;
        const int n_tok = T - t0 < NS ? T - t0 : NS;
        stage_x(a, s_x, t0, n_tok, tid, kRtThreads);
        __syncthreads();
        const int j = rb * kSharedRowsPerGroup + wave;
        if (j < a.I) shared_gate_up_rows<NS>(a, s_x, t0, n_tok, j, lane);
        return;
    }
    if (a.logits_in) return;  // uniform
    float* s_q = (float*)s_mem;                                     // [4 waves][NT][64]
    uint16_t* s_xr = (uint16_t*)(s_mem + 4 * NT * kRtExperts * 4);  // [NT][128]
    const int E = a.E, d = a.d;
    const int n_eb = (E + kRtExperts - 1) / kRtExperts;
    const int rb = (int)blockIdx.x / n_eb, eb = (int)blockIdx.x - rb * n_eb;
    const int r0 = rb * kRouterRows, rr = tid >> 4, e4 = tid & 15;
    const int e0 = eb * kRtExperts + 4 * e4;
    // W_r rows r0 + rr + 16 j: all loads first (clamped, always valid)
    u32x4 w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = r0 + rr + 16 * j;
        const uint32_t rc = (uint32_t)(r < d ? r : 0);
        if constexpr (VEC) {
            const uint32_t ee = (uint32_t)(e0 < E ? e0 : 0);
            w[j] = *(const u32x4*)(a.w_router + (rc * (uint32_t)E + ee));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ee = (uint32_t)(e0 + i < E ? e0 + i : 0);
                w[j][i] = __float_as_uint(a.w_router[rc * (uint32_t)E + ee]);
            }
        }
    }
    // x[t][r0 .. r0 + 127] (d is a multiple of 64, so a row block is whole or
    // ends at d on a 64-row boundary)
    for (int i = tid; i < NT * kRouterRows / 8; i += kRtThreads) {
        const int t = i / (kRouterRows / 8), c = 8 * (i - t * (kRouterRows / 8));
        const bool ok = t < T && r0 + c < d;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 v = *(const u32x4*)(a.x + ((size_t)(t < T ? t : 0) * d + (ok ? r0 + c : 0)));
        *(u32x4*)(s_xr + t * kRouterRows + c) = ok ? v : z;
    }
    __syncthreads();
    float acc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xv = bf16_to_f32(s_xr[t * kRouterRows + rr + 16 * j]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = __builtin_fmaf(xv, __uint_as_float(w[j][i]), acc[t][i]);
        }
        // the wave's four row offsets (lanes e4, e4 + 16, e4 + 32, e4 + 48)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[t][i] += __shfl_xor(acc[t][i], 16, 64);
            acc[t][i] += __shfl_xor(acc[t][i], 32, 64);
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_q[(wave * NT + t) * kRtExperts + 4 * e4 + i] = acc[t][i];
    }
    __syncthreads();
    for (int i = tid; i < T * kRtExperts; i += kRtThreads) {
        const int t = i / kRtExperts, el = i - t * kRtExperts, e = eb * kRtExperts + el;
        if (e < E) {
            float v = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) v += s_q[(q * NT + t) * kRtExperts + el];
            a.partial[((size_t)rb * T + t) * E + e] = v;
        }
    }
}

// Token t's logits (partial sums added in order, + bias; or the given
// logits), its top-k, then R x 16 gate/up rows of its routed slot s, for the
// assignment blockIdx.y = t * k + s (R grows with T so that the grid stays
// about one work group per CU).  Work group (0, t * k) also writes token t's
// logits, selection and scores for the down kernel and the caller.
template <int R>
__global__ __launch_bounds__(1024) void decode_topk_gate_up_kernel(const DecodeArgs a, int n_part) {
    __shared__ float s_logits[kMaxExperts];
    __shared__ int s_sel[kMaxTopK];
    __shared__ __attribute__((aligned(16))) uint16_t s_x[MOE_MAX_D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, E = a.E, k = a.k;
    const int t = (int)blockIdx.y / k, slot = (int)blockIdx.y - t * k;
    const bool first = blockIdx.x == 0 && slot == 0;
    float* logits = a.logits + (size_t)t * E;
    stage_x(a, s_x, t, 1, tid, 1024);  // covered by the barrier after the logits
    if (tid < E) {
        float v;
        if (a.logits_in) {
            v = logits[tid];
        } else {
            v = 0.0f;
            const size_t stride = (size_t)a.T * E;
            const float* part = a.partial + (size_t)t * E + tid;
            for (int g0 = 0; g0 < n_part; g0 += 16) {
                float p[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int gg = g0 + u < n_part ? g0 + u : 0;  // clamped, always valid
                    p[u] = part[(size_t)gg * stride];
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) v += g0 + u < n_part ? p[u] : 0.0f;
            }
            if (a.router_bias) v += a.router_bias[tid];
            if (first) logits[tid] = v;
        }
        s_logits[tid] = v;
    }
    __syncthreads();
    if (wave > 0) {
        // rows n of the shared expert's down projection for every token (the
        // work groups split the d rows evenly; waves 1..15 take rows in turn):
        // a lane dequantises one code word per 512-wide pass once and dots it
        // with each token's h, then a fixed DPP sum over the wave
        const int n_wg = (int)(gridDim.x * gridDim.y), g = (int)(blockIdx.x + gridDim.x * blockIdx.y);
        const int per = (a.d + n_wg - 1) / n_wg, n_beg = g * per;
        const int n_end = min(a.d, n_beg + per), I = a.I, T = a.T;
        for (int n = n_beg + wave - 1; n < n_end; n += 15) {
            float acc[MOE_MAX_DECODE_TOKENS];
#pragma unroll
            for (int tt = 0; tt < MOE_MAX_DECODE_TOKENS; ++tt) acc[tt] = 0.0f;
            for (int kb = 0; kb < I; kb += 512) {
                const int k0 = kb + 8 * lane;
                const int kk = k0 < I ? k0 : 0;  // clamped, always valid; masked below
                const uint32_t w = a.sh_down.q[(size_t)n * (I / 8) + kk / 8];
                const size_t gi = (size_t)n * (I / kGroup) + kk / kGroup;
                const bf16x8 wv = dequant8(w, dq_scale(a.sh_down.scale[gi]), bf16_to_f32(a.sh_down.bias[gi]));
#pragma unroll
                for (int tt = 0; tt < MOE_MAX_DECODE_TOKENS; ++tt) {
                    if (tt < T) {  // uniform
                        const u32x4 hv = *(const u32x4*)(a.h + ((size_t)(tt * (k + 1) + k) * I + kk));
                        const bf16x8 xv = __builtin_bit_cast(bf16x8, hv);
                        float p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 0, 1),
                                                                  __builtin_shufflevector(xv, xv, 0, 1), 0.0f, false);
                        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 2, 3),
                                                            __builtin_shufflevector(xv, xv, 2, 3), p, false);
                        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 4, 5),
                                                            __builtin_shufflevector(xv, xv, 4, 5), p, false);
                        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(wv, wv, 6, 7),
                                                            __builtin_shufflevector(xv, xv, 6, 7), p, false);
                        acc[tt] += k0 < I ? p : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < MOE_MAX_DECODE_TOKENS; ++tt) {
                if (tt < T) {
                    const float v = wave_sum_dpp(acc[tt]);
                    if (lane == 0) a.y_sh[(size_t)tt * a.d + n] = v;
                }
            }
        }
    }
    if (wave == 0) {
        int se;
        float sw;
        wave_topk(s_logits, E, k, lane, &se, &sw);
        if (lane < k) {
            s_sel[lane] = se;
            if (first) {
                const size_t o = (size_t)t * k + lane;
                a.sel_idx[o] = se;
                a.sel_w[o] = sw;
                if (a.out_idx) a.out_idx[o] = se;
                if (a.out_w) a.out_w[o] = sw;
            }
        }
    }
    __syncthreads();
    const int j0 = blockIdx.x * kDecRows * R + wave;
    if constexpr (R == 1) {
        if (j0 < a.I) gate_up_row(a, s_x, t * (k + 1) + slot, false, s_sel[slot], j0, lane);
    } else {
        gate_up_rows<R>(a, s_x, t * (k + 1) + slot, s_sel[slot], j0, kDecRows, lane);
    }
}

// Down + combine for one token t = blockIdx.y and output rows n0 .. n0 + 7
// (n0 = 8 blockIdx.x): the row tasks (output row, routed slot s < k) go to 32
// groups of 16 lanes (task rt = group + 32 m); lane l of a group takes the
// 16-byte pieces l, l + 16, .. (32 intermediate values each) of its task's
// weight row, so a load instruction reads 64 contiguous bytes of each of four
// rows.  The selected experts are loaded first, then the token's routed h
// (staged in LDS), then every weight piece of the lane, all before any
// arithmetic.  Per task: the lane's pieces in order, then a fixed DPP sum
// over the 16 lanes; the combine adds w_s * P_s in slot order and the shared
// expert's output (computed by the top-k kernel) last.
//   NM: tasks per lane group, ceil(8 k / 32);  JP: pieces per lane per task,
//   ceil(inter / 512).
constexpr int kDnOutRows = 8;
constexpr int kDnThreads = 512;
constexpr int kDnStage = (kMaxTopK * MOE_MAX_INTER / 8 + kDnThreads - 1) / kDnThreads;

// Sum over each row of 16 lanes, left in every lane of the row (fixed order).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm 1,0,3,2
    v += dpp_f32<0x4E>(v);   // quad_perm 2,3,0,1
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return v;
}

template <int NM, int JP>
__global__ __launch_bounds__(kDnThreads) void decode_down_kernel(const DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_h[kMaxTopK * MOE_MAX_INTER];
    __shared__ float s_res[kDnOutRows * kMaxTopK];
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const int I = a.I, k = a.k, d = a.d, t = blockIdx.y, n0 = blockIdx.x * kDnOutRows;
    const int n_rt = kDnOutRows * k, P = I / 32;
    // 1. the experts of this lane's tasks
    int ex[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rt = grp + 32 * m;
        const int s = rt < n_rt ? rt % k : 0;
        ex[m] = a.sel_idx[(size_t)t * k + s];
    }
    // the shared expert's output for the combine (threads 0..7, one row each)
    const float ysh = a.y_sh[(size_t)t * d + n0 + (tid < kDnOutRows ? tid : 0)];
    // the combine's scores (threads 0..7, one output row each)
    float wsc[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) wsc[s] = a.sel_w[(size_t)t * k + (s < k ? s : 0)];
    // 2. the token's routed h: k x inter bf16 (the first k of its k + 1 rows),
    // every load in flight at once
    const int n_h = k * I / 8;
    const u32x4* h_src = (const u32x4*)(a.h + (size_t)t * (k + 1) * I);
    u32x4 hv[kDnStage];
#pragma unroll
    for (int u = 0; u < kDnStage; ++u) {
        const int i = tid + kDnThreads * u;
        hv[u] = h_src[i < n_h ? i : 0];
    }
    // 3. the weight pieces (clamped, always valid; invalid ones zeroed at use)
    u32x4 q[NM][JP];
    uint16_t sc[NM][JP], bi[NM][JP];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rt = grp + 32 * m;
        const int rtc = rt < n_rt ? rt : 0;
        const int nl = rtc / k;
        const uint32_t* Wq = a.down.q;
        const uint16_t* Ws = a.down.scale;
        const uint16_t* Wb = a.down.bias;
        const size_t row = (size_t)ex[m] * d + n0 + nl;
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const int pc = l16 + 16 * j;
            const int pcc = pc < P ? pc : 0;
            q[m][j] = *(const u32x4*)(Wq + row * (I / 8) + 4 * pcc);
            sc[m][j] = Ws[row * (I / kGroup) + pcc / 2];
            bi[m][j] = Wb[row * (I / kGroup) + pcc / 2];
        }
    }
#pragma unroll
    for (int u = 0; u < kDnStage; ++u) {
        const int i = tid + kDnThreads * u;
        if (i < n_h) ((u32x4*)s_h)[i] = hv[u];
    }
    __syncthreads();
    // 4. per task: the lane's pieces, then the 16-lane sum
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int rt = grp + 32 * m;
        const int rtc = rt < n_rt ? rt : 0;
        const int s = rtc % k;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < JP; ++j) {
            const int pc = l16 + 16 * j;
            const int pcc = pc < P ? pc : 0;
            const u32x4* hp = (const u32x4*)(s_h + s * I + 32 * pcc);
            const float s9 = dq_scale(sc[m][j]), b = bf16_to_f32(bi[m][j]);
            float p = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) p = dot8_bf16(q[m][j][w], s9, b, hp[w], p);
            acc += pc < P ? p : 0.0f;
        }
        acc = row16_sum(acc);
        if (l16 == 0 && rt < n_rt) s_res[rt] = acc;
    }
    __syncthreads();
    // 5. the combine, one output row per thread
    if (tid < kDnOutRows) {
        float y = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxTopK; ++s)
            if (s < k) y += wsc[s] * s_res[tid * k + s];
        y += ysh;
        a.y[(size_t)t * d + n0 + tid] = f32_to_bf16(y);
    }
}

template <int NT>
void launch_router_shared(const DecodeArgs& a, int n_router, hipStream_t s) {
    const int n_groups = (a.T + kSharedTokens - 1) / kSharedTokens;
    const int n_rows = (a.I + kSharedRowsPerGroup - 1) / kSharedRowsPerGroup;
    const dim3 g1(n_router + n_rows * n_groups);
    if (a.E % 4 == 0)
        hipLaunchKernelGGL((decode_router_shared_kernel<NT, true>), g1, dim3(kRtThreads), 0, s, a,
                           n_router);
    else
        hipLaunchKernelGGL((decode_router_shared_kernel<NT, false>), g1, dim3(kRtThreads), 0, s, a,
                           n_router);
}

template <int NM>
static void launch_down(const DecodeArgs& a, dim3 g3, hipStream_t s) {
    if (a.I <= 512) hipLaunchKernelGGL((decode_down_kernel<NM, 1>), g3, dim3(kDnThreads), 0, s, a);
    else if (a.I <= 1024) hipLaunchKernelGGL((decode_down_kernel<NM, 2>), g3, dim3(kDnThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_down_kernel<NM, 4>), g3, dim3(kDnThreads), 0, s, a);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int n_part = (a.d + kRouterRows - 1) / kRouterRows;
    const int n_router = n_part * ((a.E + kRtExperts - 1) / kRtExperts);
    const int n_rows = (a.I + kDecRows - 1) / kDecRows;
    if (a.T <= 1) launch_router_shared<1>(a, n_router, s);
    else if (a.T <= 2) launch_router_shared<2>(a, n_router, s);
    else if (a.T <= 4) launch_router_shared<4>(a, n_router, s);
    else launch_router_shared<8>(a, n_router, s);
    trace_point(s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // rows per wave: about one work group per CU in all
    int R = 1;
    while (R < 4 && n_rows * a.T * a.k > 256 * R) R *= 2;
    const dim3 g2((a.I + kDecRows * R - 1) / (kDecRows * R), a.T * a.k);
    if (R == 1) hipLaunchKernelGGL(decode_topk_gate_up_kernel<1>, g2, dim3(1024), 0, s, a, n_part);
    else if (R == 2) hipLaunchKernelGGL(decode_topk_gate_up_kernel<2>, g2, dim3(1024), 0, s, a, n_part);
    else hipLaunchKernelGGL(decode_topk_gate_up_kernel<4>, g2, dim3(1024), 0, s, a, n_part);
    trace_point(s);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 g3(a.d / kDnOutRows, a.T);
    const int n_rt = kDnOutRows * a.k;
    if (n_rt <= 32) launch_down<1>(a, g3, s);
    else if (n_rt <= 64) launch_down<2>(a, g3, s);
    else launch_down<3>(a, g3, s);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
