/*
 * q4moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN layer
 * with group-64 affine 4-bit expert weights.
 *
 * Sources.  [Lily-M5] is the page "Perplexity's Lily beats MLX-LM on MacBook
 * M5 because it only runs one model"; sections are named in quotes.
 *   - "Why Qwen3.6-35B-A3B is a weird workload": 8 of 256 routed experts per
 *     token plus 1 always-on shared expert.
 *   - "Prefill: keep routing on the GPU, dequantize in flight": 4-bit codes
 *     with an affine map per group of 64 (bf16 scale s and bias b,
 *     w = q * s + b); the prefill GEMM expands one small tile at a time on
 *     chip (FP32 sums, bf16 results, no expanded weight copy in memory); the
 *     histogram, prefix scan, scatter and block map stay on the GPU in the
 *     chunk's stream, with no host round trip; 32-row tiles.
 *   - "Decode: minimize bytes per token": at batch 1 the expert products are
 *     memory-bound matrix-vector products; the gate activation is folded into
 *     the input projections, and the scores and the shared expert into the
 *     output projection.
 *   - "Setup": the engine accepts only the one architecture and quantisation
 *     it was built for.  Every entry point here is likewise fail-closed: an
 *     unsupported shape is refused before anything
 *     is enqueued.
 *
 * What the layer computes, per token t with input x_t (bf16, length d):
 *   l_t    = x_t . W_r (+ b_r)                 fp32 router logits, E experts
 *   idx_t  = the k experts with the largest l_t, larger logit first, equal
 *            logits ordered by lower expert index
 *   w_t    = softmax(l_t) at idx_t, divided by its sum over the k slots
 *   E_e(x) = W_down,e . bf16( SiLU(W_gate,e . x) * (W_up,e . x) )
 *   y_t    = bf16( sum_{s=0..k-1} w_t[s] * E_idx_t[s](x_t)  +  E_shared(x_t) )
 * with the k routed terms added in slot order and the shared expert last,
 * every weight used as the bf16 value bf16(q * scale + bias), and all sums
 * accumulated in fp32.
 *
 * Conventions for every entry point.
 *   - All array arguments are DEVICE pointers owned by the caller, 16-byte
 *     aligned.  bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued on it: no entry point allocates, frees, copies to the host or
 *     synchronises.  A return of MOE_OK means "validated and enqueued"; a
 *     device fault surfaces at the caller's next synchronisation.
 *   - Validation happens on the host before any launch; on any error nothing
 *     is enqueued.  moe_last_error() then returns a one-line reason (kept per
 *     host thread).
 *   - Calls that share a workspace or routing buffers must not overlap
 *     (run them on one stream, or order the streams).
 */
#ifndef Q4MOE_H
#define Q4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* null or misaligned pointer, non-positive size */
    MOE_EUNSUPPORTED = -2, /* shape outside what the kernels support (see limits) */
    MOE_EWORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes() */
    MOE_EHIP = -4          /* a HIP launch reported an error */
};

/* Limits of the kernels.  d and inter must also be multiples of 64 (the
   quantisation group) and 1 <= top_k <= min(MOE_MAX_TOPK, n_experts). */
#define MOE_GROUP 64
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_MAX_TOKENS 32768
#define MOE_MAX_D 8192
#define MOE_MAX_INTER 2048

/* Row heights of the two block maps moe_route writes: the 32-row tile map
   that describes the expert-sorted rows, and the 128-row work map the grouped
   GEMMs walk (one work item = up to four 32-row tiles of one expert, so that a
   dequantised weight tile is reused across them). */
#define MOE_BLOCK_ROWS 32
#define MOE_TILE_ROWS 128

/* moe_route counts assignments per block of this many consecutive tokens
   (see moe_routing.blk_counts). */
#define MOE_ROUTE_BLOCK 256

/* moe_decode sums the router logits in partial sums over this many rows of
   W_r (the workspace holds ceil(d / MOE_DECODE_ROUTER_ROWS) x E of them per
   token). */
#define MOE_DECODE_ROUTER_ROWS 128

/* Most tokens one moe_decode_tokens call takes. */
#define MOE_MAX_DECODE_TOKENS 8

/* moe_route flag: start from the logits already in routing->logits instead of
   computing them (used to route from given fp32 logits). */
#define MOE_LOGITS_IN 1u

/* One stack of group-64 affine 4-bit matrices, each N rows by K columns:
     q     [n_mat][N][K/8]  uint32, eight 4-bit codes per word along K, the
                            lowest nibble holding the lowest k
     scale [n_mat][N][K/64] bf16
     bias  [n_mat][N][K/64] bf16
   Row n of matrix m holds the weights that produce output n from the K
   inputs; w(n, k) = q(n, k) * scale(n, k/64) + bias(n, k/64), used as the
   nearest bf16 value.  That rounding is exact (one rounding of the exact
   affine value) for finite scales below 2^119 in magnitude whose exponent
   lies within 12 of the bias's; the kernels do not check the data. */
typedef struct {
    const uint32_t* q;
    const uint16_t* scale;
    const uint16_t* bias;
} moe_q4mat;

/* One MoE layer.  Routed experts: gate and up are n_experts matrices of
   inter x d, down is n_experts matrices of d x inter.  The shared expert's
   sh_gate, sh_up (inter x d) and sh_down (d x inter) are single matrices. */
typedef struct {
    int32_t d;               /* hidden size */
    int32_t inter;           /* expert intermediate size (shared expert too) */
    int32_t n_experts;       /* E, routed experts */
    int32_t top_k;           /* k */
    const float* w_router;   /* fp32 [d][E], row-major */
    const float* router_bias;/* fp32 [E], added to the logits; may be NULL */
    moe_q4mat gate, up, down;
    moe_q4mat sh_gate, sh_up, sh_down;
} moe_layer;

/* Routing state of one chunk of T tokens, all device arrays owned by the
   caller.  Written by moe_route (logits are read instead when MOE_LOGITS_IN is
   set) and read by moe_prefill.  An "assignment" is a = t*k + s (token t,
   slot s); the "sorted rows" are the assignments grouped by expert (experts
   ascending, tokens ascending inside an expert). */
typedef struct {
    float* logits;      /* [T][E]  fp32 router logits */
    int32_t* topk_idx;  /* [T][k]  selected experts, slot 0 = largest logit */
    float* topk_w;      /* [T][k]  renormalised scores */
    int32_t* counts;    /* [E]     assignments per expert */
    int32_t* offsets;   /* [E+1]   exclusive prefix sum of counts */
    int32_t* perm;      /* [T*k]   sorted row -> assignment */
    int32_t* inv_perm;  /* [T*k]   assignment -> sorted row */
    int32_t* block_map; /* [T*k/32 + E][2]  (expert, first sorted row) per 32-row tile */
    int32_t* n_blocks;  /* [1] */
    int32_t* tile_map;  /* [T*k/128 + E][2] (expert, first sorted row) per 128-row item */
    int32_t* n_tiles;   /* [1] */
    int32_t* blk_counts;/* [ceil(T/MOE_ROUTE_BLOCK)][E] scratch of moe_route: per-block
                           expert counts; contents unspecified afterwards */
} moe_routing;

/* Entries needed in block_map / tile_map for T tokens (pairs of int32). */
int32_t moe_block_map_capacity(int32_t T, int32_t top_k, int32_t n_experts, int32_t rows);

/* Bytes of device workspace moe_prefill (T tokens), moe_decode and
   moe_decode_tokens (up to MOE_MAX_DECODE_TOKENS tokens, whatever T) need for
   this layer shape: the gate/up activations h (bf16), the shared
   expert's activations, the routed experts' outputs staged for the combine
   (fp16 scaled by a power of two per 32 columns, so any finite fp32 value
   keeps 11 significant bits), and the decode path's router partial sums.
   0 on invalid arguments.  The contents need no initialisation and are not
   preserved between calls. */
size_t moe_workspace_bytes(const moe_layer* L, int32_t T);

/* Routing of T tokens, entirely on the device, no host synchronisation:
   router logits (unless MOE_LOGITS_IN), top-k selection and renormalised
   scores, histogram, exclusive scan, stable scatter into expert-sorted order,
   and both block maps (three kernels).  x: bf16 [T][d].  ([Lily-M5] "Prefill: keep routing on
   the GPU, dequantize in flight".) */
int moe_route(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
              const moe_routing* r, void* stream);

/* The expert part of the layer for T tokens routed by moe_route: grouped
   gate/up GEMM with fused SiLU(gate)*up over the expert-sorted rows plus the
   shared expert over all tokens, then the down projection of the routed rows,
   then the shared expert's down projection with the fixed-order combine fused
   into it (slots in order, scores applied, shared expert last; [Lily-M5]
   "Decode: minimize bytes per token": the output projection carries the
   routing scores and the shared expert).  Three kernels.  Dequantisation
   happens on chip, tile by tile; accumulation is fp32; y: bf16 [T][d].
   ws must hold moe_workspace_bytes(L, T) bytes. */
int moe_prefill(const moe_layer* L, const uint16_t* x, int32_t T, const moe_routing* r,
                void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/* moe_prefill with a choice of the gate/up work-item height: the number of
   expert-sorted rows that share one on-chip dequantised weight tile
   ([Lily-M5] "Prefill: keep routing on the GPU, dequantize in flight" compares
   tile heights).  flags = 0: 128 rows (what moe_prefill uses);
   MOE_ITEM_ROWS_64: 64 rows; MOE_ITEM_ROWS_32: 32 rows, one MFMA subtile;
   MOE_ITEM_ROWS_16: 16 rows, the upper half of one MFMA subtile (its other
   16 rows are padding).  Shorter items dequantise an expert's weights once per
   item instead of once per 128 rows and pad less.  The result is the same
   whatever the height: every row's sums are accumulated in the same order.
   More than one of these flags, or any other bit, is MOE_EINVAL. */
#define MOE_ITEM_ROWS_64 2u
#define MOE_ITEM_ROWS_32 4u
#define MOE_ITEM_ROWS_16 8u
int moe_prefill_ex(const moe_layer* L, const uint16_t* x, int32_t T, const moe_routing* r,
                   void* ws, size_t ws_bytes, uint16_t* y, uint32_t flags, void* stream);

/* The whole layer for one token (T = 1): router, top-k, then dequant-GEMVs
   over the k selected experts and the shared expert with SiLU(gate)*up fused,
   then the down GEMVs fused with the scores, the shared expert and the
   combine.  Three kernels: router partial sums with the shared expert's
   gate/up; logits + top-k with the routed gate/up; down + combine.  r may be NULL; when given, r->logits [1][E], r->topk_idx [1][k]
   and r->topk_w [1][k] are written (with MOE_LOGITS_IN, r->logits is read
   and the router is skipped).  x, y: bf16 [1][d].  ([Lily-M5] "Decode:
   minimize bytes per token".) */
int moe_decode(const moe_layer* L, const uint16_t* x, uint32_t flags, const moe_routing* r,
               void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/* The decode layer for a few tokens at once, 1 <= T <= MOE_MAX_DECODE_TOKENS
   (the small-batch decode or draft-verify shape, where the tokens' rows route
   to different experts and the bytes read grow with the experts they select):
   the same three kernels as moe_decode, with every W_r row and every shared
   expert weight read and dequantised once for all T tokens, and every token's
   routed slots as separate work groups.  Per token the arithmetic is exactly
   moe_decode's, so moe_decode_tokens(T) gives each token's moe_decode result
   bit for bit.  x, y: bf16 [T][d]; r may be NULL, else r->logits [T][E],
   r->topk_idx [T][k] and r->topk_w [T][k] are written (MOE_LOGITS_IN: the
   logits are read).  ws must hold moe_workspace_bytes(L, 1) bytes; T outside
   1 .. MOE_MAX_DECODE_TOKENS is MOE_EUNSUPPORTED.  ([Lily-M5] "Decode:
   minimize bytes per token"; "What didn't work": verifying a few draft rows
   at once, whose rows route to different experts and so read more expert
   bytes.) */
int moe_decode_tokens(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                      const moe_routing* r, void* ws, size_t ws_bytes, uint16_t* y,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
   tight serving loops, harnesses that forbid hipMalloc): moe_decode_tokens with
   its workspace taken from a static device array inside the library, of
   MOE_STATIC_SCRATCH_BYTES bytes, one per GPU for the life of the process.
   The call allocates nothing (no hipMalloc, no library routine that does);
   the caller still passes x, y and the optional routing outputs.  Arguments,
   results and errors are moe_decode_tokens's, plus MOE_EUNSUPPORTED when the
   layer's decode scratch (what moe_workspace_bytes(L, 1) gives, less the
   prefill part) exceeds MOE_STATIC_SCRATCH_BYTES.  Every call on a GPU
   shares that GPU's array: calls that overlap in time on one GPU (different
   streams, or different host threads without ordering) race and give
   undefined results.  On the first call on each device the library looks up
   that device's array (hipGetSymbolAddress, with the device current). */
#define MOE_STATIC_SCRATCH_BYTES (1u << 20)
int moe_decode_tokens_static(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                             const moe_routing* r, uint16_t* y, void* stream);

/* Greedy decoding's token hand-off ([Lily-M5] "Decode: minimize bytes per
   token": the chosen token stays on the device between decode steps -- the
   largest output logit selects it and it feeds the following step's input
   directly).  The output head and the input embedding table are
   V x d matrices in the moe_q4mat format above (matrix 0 of each), used as
   bf16 weights like the experts' (the pages give no format of their own). */
#define MOE_MAX_VOCAB 1048576
typedef struct {
    int32_t V;          /* vocabulary rows, 1 <= V <= MOE_MAX_VOCAB */
    int32_t d;          /* hidden size, a multiple of 64, <= MOE_MAX_D */
    moe_q4mat head;     /* [V][d]: logit v = sum_k w(v, k) * x[k] */
    moe_q4mat embed;    /* [V][d]: row v is token v's input; may be all NULL when
                           moe_lm_argmax gets x_next = NULL */
} moe_lm_head;
/* Workspace bytes of moe_lm_argmax for this head (per-work-group partial
   results); 0 on invalid arguments.  Needs no initialisation, not preserved. */
size_t moe_lm_workspace_bytes(const moe_lm_head* lm);
/* One hand-off, two kernels, no host synchronisation:
     logits[v] = fp32 sum over k of bf16(head weight) * x[k]   (unless MOE_LOGITS_IN)
     *token    = the v with the largest logit; equal logits: the lower v; a NaN
                 logit counts as minus infinity (V NaNs give token 0)
     x_next    = bf16 row *token of embed (the next decode step's input), if
                 x_next is not NULL
   x: bf16 [d] (unused, may be NULL, with MOE_LOGITS_IN); logits: fp32 [V],
   written, or read with MOE_LOGITS_IN; token: one int32, only 4-byte aligned
   (so the caller can alternate between two slots of one array, one per step);
   x_next: bf16 [d], may be the same buffer as x.  ws must hold
   moe_lm_workspace_bytes(lm) bytes.  Unknown flags are MOE_EINVAL. */
int moe_lm_argmax(const moe_lm_head* lm, const uint16_t* x, uint32_t flags, float* logits,
                  int32_t* token, uint16_t* x_next, void* ws, size_t ws_bytes, void* stream);
/* The on-chip dequantisation the GEMMs use, exposed for testing: w_out (bf16
   [n_rows][K]) = bf16(q * scale + bias) for matrix 0 of m.  K % 64 == 0. */
int moe_dequant(const moe_q4mat* m, int32_t n_rows, int32_t K, uint16_t* w_out, void* stream);

/* Timing hook.  While `events` is non-NULL, every moe_route, moe_prefill,
   moe_decode, moe_decode_tokens and moe_lm_argmax call made on this host thread records events[0] on its stream
   before its first kernel and events[i] right after its i-th kernel, for
   i < n (moe_route: router logits (with MOE_LOGITS_IN: the clearing of
   the histogram), top-k + histogram, scan + scatter + maps;
   moe_prefill: gate/up, routed down,
   shared down + combine; moe_decode and moe_decode_tokens: router
   partial sums + shared gate/up, logits + top-k + routed gate/up, down +
   combine; moe_lm_argmax: output head (with MOE_LOGITS_IN: the scan of the
   given logits), pick + embedding row).  The
   elapsed time between consecutive events is one kernel's duration.  events
   are hipEvent_t handles created and owned by the caller; pass NULL to stop. */
void moe_trace_events(void* const* events, int32_t n);

/* Text for a status code, and the reason for the last failure on this thread. */
const char* moe_strerror(int code);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* Q4MOE_H */
