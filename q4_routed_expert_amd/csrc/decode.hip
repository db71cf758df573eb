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
//   3. down: one wave per output n (several for larger T): each lane takes
//      one code word of each of the k + 1 experts' rows, and the wave combines
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
constexpr int kSharedTokens = 2;  // tokens per shared-expert gate/up work group

static_assert(kRouterRows == MOE_DECODE_ROUTER_ROWS, "router partial rows");
static_assert(MOE_MAX_DECODE_TOKENS == 8, "token buckets 1, 2, 4, 8");
static_assert(kRouterWaves * 64 == 1024 && 4 * 64 == kMaxExperts, "router work group shape");

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

// Work groups [0, n_part): partial[g][t][e] = sum of x[t][r] W_r[r][e] over
// the 128 rows r of group g, for every token t.  Wave w takes rows
// 8w .. 8w + 7 of the group, each lane four consecutive experts: one 16-byte
// load per row and lane, so one load instruction reads a whole 1 KB row of
// W_r (E = 256), and each W_r row is read once for all tokens; x[t][r] is
// wave-uniform and comes through the scalar cache.  The sixteen waves' sums
// are added in wave order through LDS.  Work groups from n_part on: the
// shared expert's gate/up rows, one per wave, for a group of up to
// kSharedTokens tokens (more tokens: more work groups).
template <int NT, bool VEC>
__global__ __launch_bounds__(1024) void decode_router_shared_kernel(const DecodeArgs a,
                                                                    int n_part) {
    constexpr int NS = NT < kSharedTokens ? NT : kSharedTokens;
    constexpr int kQBytes = kRouterWaves * NT * kMaxExperts * 4, kXBytes = NS * MOE_MAX_D * 2;
    // the router's partial sums and the shared part's x never share a work group
    __shared__ __attribute__((aligned(16))) unsigned char s_mem[kQBytes > kXBytes ? kQBytes : kXBytes];
    float* s_q = (float*)s_mem;  // [kRouterWaves][NT][kMaxExperts]
    uint16_t* s_x = (uint16_t*)s_mem;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T;
    if ((int)blockIdx.x >= n_part) {  // uniform per work group
        const int n_rows = (a.I + kDecRows - 1) / kDecRows;
        const int b = (int)blockIdx.x - n_part, rb = b % n_rows, t0 = (b / n_rows) * NS;
        const int n_tok = T - t0 < NS ? T - t0 : NS;
        stage_x(a, s_x, t0, n_tok, tid, 1024);
        __syncthreads();
        const int j = rb * kDecRows + wave;
        if (j < a.I) shared_gate_up_rows<NS>(a, s_x, t0, n_tok, j, lane);
        return;
    }
    if (a.logits_in) return;  // uniform
    const int g = blockIdx.x, E = a.E, d = a.d;
    const int e0 = 4 * lane;
    // first row of this wave, made explicitly wave-uniform for the scalar loads of x
    const int r0 = __builtin_amdgcn_readfirstlane(g * kRouterRows + wave * kRouterWaveRows);
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
    // x[t][r0 .. r0 + 7]: one uniform 16-byte load per token (r0 is a multiple
    // of 8 and d of 64)
    const bool r_ok = r0 < d;
    float acc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int tt = t < T ? t : 0;  // clamped, always valid
        const u32x4 xq = *(const u32x4*)(a.x + ((size_t)tt * d + (r_ok ? r0 : 0)));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = 0.0f;
#pragma unroll
        for (int r = 0; r < kRouterWaveRows; ++r) {
            const uint32_t xw = xq[r >> 1];
            const float xv =
                r_ok ? __uint_as_float((r & 1) ? (xw & 0xffff0000u) : (xw << 16)) : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = __builtin_fmaf(xv, __uint_as_float(w[r][i]), acc[t][i]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_q[(wave * NT + t) * kMaxExperts + e0 + i] = acc[t][i];
    __syncthreads();
    for (int i = tid; i < T * E; i += 1024) {
        const int t = i / E, e = i - t * E;
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < kRouterWaves; ++q) v += s_q[(q * NT + t) * kMaxExperts + e];
        a.partial[((size_t)g * T + t) * E + e] = v;
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

// One wave per NO outputs n (n = first + 8 o); lane covers 8 consecutive
// intermediate k (one code word) of each 512-wide pass, for every slot.  All
// slots' loads are issued before the arithmetic; the combine then adds
// w_s * P_s in slot order and the shared expert last.  NO = 2 for larger T
// (fewer, fuller work groups; at 4 the registers spill).
template <int NO>
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_kernel(const DecodeArgs a) {
    // token t = blockIdx.y: h of its k + 1 experts, staged once per work group
    __shared__ __attribute__((aligned(16))) uint16_t s_h[(kMaxTopK + 1) * MOE_MAX_INTER];
    const int tid = threadIdx.x, lane = tid & 63;
    const int I = a.I, k = a.k, d = a.d, t = blockIdx.y;
    const u32x4* h_src = (const u32x4*)(a.h + (size_t)t * (k + 1) * I);
    for (int i = tid; i < (k + 1) * I / 8; i += 64 * kDownWaves) ((u32x4*)s_h)[i] = h_src[i];
    const int32_t* sel_idx = a.sel_idx + (size_t)t * k;
    const float* sel_w = a.sel_w + (size_t)t * k;
    __syncthreads();
    const int n0 = blockIdx.x * kDownWaves * NO + (tid >> 6);
    if (n0 >= d) return;
    float part[NO][kMaxTopK + 1];
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) part[o][s] = 0.0f;
    for (int jb = 0; jb < I; jb += 64 * 8) {
        const int j0 = jb + 8 * lane;
        const int jj = j0 < I ? j0 : 0;  // clamped, always valid; masked below
        uint32_t q[NO][kMaxTopK + 1];
        uint32_t sc[NO][kMaxTopK + 1], bi[NO][kMaxTopK + 1];
        u32x4 hv[kMaxTopK + 1];
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            const int ss = s <= k ? s : k;  // slots past k repeat the shared expert (discarded)
            const bool shared = ss == k;
            const Q4 D = shared ? a.sh_down : a.down;
            const size_t base = shared ? 0 : (size_t)sel_idx[ss] * d;
#pragma unroll
            for (int o = 0; o < NO; ++o) {
                const int n = n0 + kDownWaves * o;
                const size_t row = base + (n < d ? n : n0);  // clamped, always valid
                q[o][s] = D.q[row * (I / 8) + jj / 8];
                sc[o][s] = D.scale[row * (I / kGroup) + jj / kGroup];
                bi[o][s] = D.bias[row * (I / kGroup) + jj / kGroup];
            }
            hv[s] = *(const u32x4*)(s_h + ss * I + jj);
        }
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
            for (int s = 0; s <= kMaxTopK; ++s) {
                const float p =
                    dot8_bf16(q[o][s], dq_scale(sc[o][s]), bf16_to_f32(bi[o][s]), hv[s], 0.0f);
                part[o][s] += j0 < I ? p : 0.0f;
            }
    }
#pragma unroll
    for (int o = 0; o < NO; ++o) {
        float y = 0.0f, sh = 0.0f;
#pragma unroll
        for (int s = 0; s <= kMaxTopK; ++s) {
            if (s <= k) {
                const float p = wave_sum_dpp(part[o][s]);
                if (s < k) y += sel_w[s] * p;
                else sh = p;
            }
        }
        const int n = n0 + kDownWaves * o;
        if (lane == 0 && n < d) a.y[(size_t)t * d + n] = f32_to_bf16(y + sh);
    }
}

template <int NT>
void launch_router_shared(const DecodeArgs& a, int n_part, int n_rows, hipStream_t s) {
    const int n_groups = (a.T + kSharedTokens - 1) / kSharedTokens;
    const dim3 g1(n_part + n_rows * n_groups);
    if (a.E % 4 == 0)
        hipLaunchKernelGGL((decode_router_shared_kernel<NT, true>), g1, dim3(1024), 0, s, a, n_part);
    else
        hipLaunchKernelGGL((decode_router_shared_kernel<NT, false>), g1, dim3(1024), 0, s, a, n_part);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int n_part = (a.d + kRouterRows - 1) / kRouterRows;
    const int n_rows = (a.I + kDecRows - 1) / kDecRows;
    if (a.T <= 1) launch_router_shared<1>(a, n_part, n_rows, s);
    else if (a.T <= 2) launch_router_shared<2>(a, n_part, n_rows, s);
    else if (a.T <= 4) launch_router_shared<4>(a, n_part, n_rows, s);
    else launch_router_shared<8>(a, n_part, n_rows, s);
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
    // outputs per wave: about two work groups per CU in all
    const int NO = ((a.d + kDownWaves - 1) / kDownWaves) * a.T > 512 ? 2 : 1;
    const dim3 g3((a.d + kDownWaves * NO - 1) / (kDownWaves * NO), a.T);
    if (NO == 1) hipLaunchKernelGGL(decode_down_kernel<1>, g3, dim3(64 * kDownWaves), 0, s, a);
    else hipLaunchKernelGGL(decode_down_kernel<2>, g3, dim3(64 * kDownWaves), 0, s, a);
    trace_point(s);
    return hipGetLastError();
}

}  // namespace q4moe
