// lmhead.h -- launcher of the greedy token hand-off, shared by abi.hip and
// lmhead.hip ([Lily-M5] "Decode: minimize bytes per token").
#pragma once
#include "internal.h"

namespace q4moe {

struct LmArgs {
    const uint16_t* x;   // bf16 [d] (unused with given logits)
    int V, d;
    Q4 head, embed;      // [V][d] each
    float* logits;       // [V]: written, or read when the logits are given
    int32_t* token;      // [1] the greedy token
    uint16_t* x_next;    // bf16 [d] the token's embedding row, or NULL
    int2* part;          // [lm_partials(V, .)] per-work-group best (logit bits, row)
};
// Partial results the first kernel writes for V rows (given logits or not).
int lm_partials(int V, bool logits_in);
hipError_t launch_lm_argmax(const LmArgs& a, bool logits_in, hipStream_t s);

}  // namespace q4moe
