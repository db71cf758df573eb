// internal.h -- launchers shared between the translation units of libq4moe.
#pragma once
#include <hip/hip_runtime.h>

#include "q4moe.h"
#include "q4moe_dev.h"

namespace q4moe {

static_assert(kMaxExperts == MOE_MAX_EXPERTS && kMaxTopK == MOE_MAX_TOPK, "limits");
static_assert(kBlockRows == MOE_BLOCK_ROWS && kTileRows == MOE_TILE_ROWS, "map rows");
static_assert(MOE_ROUTE_BLOCK == 256, "the routing kernels use one thread per token of a block");

// Records the next event of the caller's timing hook (moe_trace_events) on s,
// if one is installed on this host thread; called after every kernel launch.
void trace_point(hipStream_t s);

// Routing ([Lily-M5] "Prefill: keep routing on the GPU, dequantize in flight").
// x == NULL: the logits are given; only the histogram is cleared.
hipError_t launch_router_logits(const uint16_t* x, int T, int d, const float* w_router,
                                const float* router_bias, int E, float* logits,
                                int32_t* blk_counts, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                       int32_t* blk_counts, hipStream_t s);
hipError_t launch_route_sort(const int32_t* idx, int T, int k, int E, const moe_routing* r,
                             hipStream_t s);

// Prefill expert GEMMs.
struct PrefillArgs {
    const uint16_t* x;
    int T, d, I, E, k;
    Q4 gate, up, down, sh_gate, sh_up, sh_down;
    const int32_t* perm;
    const int32_t* offsets;
    const int32_t* tile_map;
    const int32_t* n_tiles;
    const float* topk_w;
    int tile_bound;      // host upper bound on *n_tiles
    int item_sh;         // gate/up work items are 128 >> item_sh rows (0 .. 3)
    uint16_t* h;         // bf16 [T*k][I], expert-sorted rows
    uint16_t* h_sh;      // bf16 [T][I]
    uint16_t* part;      // fp16 [T*k][d], routed expert outputs scaled by 2^-pexp, rows in
                         // assignment order
    int8_t* pexp;        // [T][d/32][8] staging exponent per (token, 32 columns, slot)
    int32_t* dn_pre;     // [items + 1] the down kernel's item cost prefix (NULL: not used)
    int32_t* dn_exp;     // [items] the down kernel's item experts (-1: shared)
    uint16_t* y;         // bf16 [T][d]
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// Decode (1 <= T <= MOE_MAX_DECODE_TOKENS tokens).
struct DecodeArgs {
    const uint16_t* x;   // bf16 [T][d]
    int T, d, I, E, k;
    const float* w_router;
    const float* router_bias;
    Q4 gate, up, down, sh_gate, sh_up, sh_down;
    bool logits_in;
    float* logits;       // [T][E]: written, or read when logits_in
    int32_t* out_idx;    // [T][k] or NULL
    float* out_w;        // [T][k] or NULL
    float* partial;      // [ceil(d/MOE_DECODE_ROUTER_ROWS)][T][E] router partial sums
    int32_t* sel_idx;    // [T][k]
    float* sel_w;        // [T][k]
    uint16_t* h;         // bf16 [T][k+1][I], slot k = the shared expert
    float* y_sh;         // [T][d] the shared expert's down projection (fp32)
    uint16_t* y;         // bf16 [T][d]
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

hipError_t launch_dequant(Q4 m, int n_rows, int K, uint16_t* w_out, hipStream_t s);

}  // namespace q4moe
