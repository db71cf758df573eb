// abi.hip -- the extern "C" entry points declared in include/q4moe.h:
// host-side validation (fail-closed, nothing is enqueued on error), workspace
// layout, and the launches on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "internal.h"
#include "lmhead.h"

namespace {

thread_local char g_err[256] = "";

// Timing hook state (moe_trace_events): caller-owned events, next index.
thread_local hipEvent_t* g_trace = nullptr;
thread_local int g_trace_n = 0, g_trace_next = 0;

void trace_begin(hipStream_t s) {
    g_trace_next = 0;
    q4moe::trace_point(s);
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_ptr(const void* p, const char* what, bool allow_null = false) {
    if (!p) return allow_null ? MOE_OK : fail(MOE_EINVAL, "%s is NULL", what);
    if (!aligned16(p)) return fail(MOE_EINVAL, "%s is not 16-byte aligned", what);
    return MOE_OK;
}

int check_mat(const moe_q4mat& m, const char* name) {
    char buf[64];
    int rc;
    snprintf(buf, sizeof buf, "%s.q", name);
    if ((rc = check_ptr(m.q, buf))) return rc;
    snprintf(buf, sizeof buf, "%s.scale", name);
    if ((rc = check_ptr(m.scale, buf))) return rc;
    snprintf(buf, sizeof buf, "%s.bias", name);
    return check_ptr(m.bias, buf);
}

int check_layer(const moe_layer* L) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (L->d <= 0 || L->inter <= 0 || L->n_experts <= 0 || L->top_k <= 0)
        return fail(MOE_EINVAL, "non-positive layer size (d=%d inter=%d E=%d k=%d)", L->d,
                    L->inter, L->n_experts, L->top_k);
    if (L->d % MOE_GROUP || L->inter % MOE_GROUP)
        return fail(MOE_EUNSUPPORTED, "d=%d and inter=%d must be multiples of %d", L->d,
                    L->inter, MOE_GROUP);
    if (L->d > MOE_MAX_D || L->inter > MOE_MAX_INTER)
        return fail(MOE_EUNSUPPORTED, "d=%d > %d or inter=%d > %d", L->d, MOE_MAX_D, L->inter,
                    MOE_MAX_INTER);
    if (L->n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_EUNSUPPORTED, "n_experts=%d > %d", L->n_experts, MOE_MAX_EXPERTS);
    if (L->top_k > MOE_MAX_TOPK || L->top_k > L->n_experts)
        return fail(MOE_EUNSUPPORTED, "top_k=%d must be <= min(%d, n_experts=%d)", L->top_k,
                    MOE_MAX_TOPK, L->n_experts);
    int rc;
    if ((rc = check_ptr(L->w_router, "w_router"))) return rc;
    if ((rc = check_ptr(L->router_bias, "router_bias", true))) return rc;
    if ((rc = check_mat(L->gate, "gate")) || (rc = check_mat(L->up, "up")) ||
        (rc = check_mat(L->down, "down")) || (rc = check_mat(L->sh_gate, "sh_gate")) ||
        (rc = check_mat(L->sh_up, "sh_up")) || (rc = check_mat(L->sh_down, "sh_down")))
        return rc;
    return MOE_OK;
}

int check_tokens(int32_t T) {
    if (T <= 0) return fail(MOE_EINVAL, "T=%d must be positive", T);
    if (T > MOE_MAX_TOKENS) return fail(MOE_EUNSUPPORTED, "T=%d > %d", T, MOE_MAX_TOKENS);
    return MOE_OK;
}

int check_routing(const moe_routing* r) {
    if (!r) return fail(MOE_EINVAL, "routing is NULL");
    int rc;
    if ((rc = check_ptr(r->logits, "routing.logits")) || (rc = check_ptr(r->topk_idx, "routing.topk_idx")) ||
        (rc = check_ptr(r->topk_w, "routing.topk_w")) || (rc = check_ptr(r->counts, "routing.counts")) ||
        (rc = check_ptr(r->offsets, "routing.offsets")) || (rc = check_ptr(r->perm, "routing.perm")) ||
        (rc = check_ptr(r->inv_perm, "routing.inv_perm")) ||
        (rc = check_ptr(r->block_map, "routing.block_map")) ||
        (rc = check_ptr(r->n_blocks, "routing.n_blocks")) ||
        (rc = check_ptr(r->tile_map, "routing.tile_map")) ||
        (rc = check_ptr(r->n_tiles, "routing.n_tiles")) ||
        (rc = check_ptr(r->blk_counts, "routing.blk_counts")))
        return rc;
    return MOE_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace: [decode region | prefill region], so one workspace sized for T
// tokens serves both entry points.
struct DecodeWs {
    size_t sel_idx, sel_w, logits, partial, h, y_sh, total;
};
DecodeWs decode_ws(const moe_layer* L) {
    DecodeWs w;
    size_t o = 0;
    const size_t nt = MOE_MAX_DECODE_TOKENS;
    w.sel_idx = o; o += align256(sizeof(int32_t) * nt * MOE_MAX_TOPK);
    w.sel_w = o; o += align256(sizeof(float) * nt * MOE_MAX_TOPK);
    w.logits = o; o += align256(sizeof(float) * nt * L->n_experts);
    w.partial = o;
    o += align256(sizeof(float) * (size_t)((L->d + MOE_DECODE_ROUTER_ROWS - 1) / MOE_DECODE_ROUTER_ROWS) *
                  nt * L->n_experts);
    w.h = o; o += align256(sizeof(uint16_t) * nt * (size_t)(L->top_k + 1) * L->inter);
    w.y_sh = o; o += align256(sizeof(float) * nt * (size_t)L->d);
    w.total = o;
    return w;
}
struct PrefillWs {
    size_t h, h_sh, part, pexp, dn_pre, dn_exp, total;
};
PrefillWs prefill_ws(const moe_layer* L, int32_t T, size_t base) {
    PrefillWs w;
    const size_t A = (size_t)T * L->top_k;
    size_t o = base;
    w.h = o; o += align256(sizeof(uint16_t) * A * L->inter);
    w.h_sh = o; o += align256(sizeof(uint16_t) * (size_t)T * L->inter);
    w.part = o; o += align256(sizeof(uint16_t) * A * L->d);
    w.pexp = o; o += align256((size_t)T * (L->d / 32) * MOE_MAX_TOPK);
    const size_t n_items = (size_t)moe_block_map_capacity(T, L->top_k, L->n_experts, MOE_TILE_ROWS);
    w.dn_pre = o; o += align256(sizeof(int32_t) * (n_items + 1));
    w.dn_exp = o; o += align256(sizeof(int32_t) * n_items);
    w.total = o;
    return w;
}

q4moe::Q4 q4(const moe_q4mat& m) { return q4moe::Q4{m.q, m.scale, m.bias}; }

int check_lm(const moe_lm_head* lm) {
    if (!lm) return fail(MOE_EINVAL, "lm head is NULL");
    if (lm->V <= 0 || lm->d <= 0) return fail(MOE_EINVAL, "V=%d and d=%d must be positive", lm->V, lm->d);
    if (lm->d % MOE_GROUP || lm->d > MOE_MAX_D)
        return fail(MOE_EUNSUPPORTED, "d=%d must be a multiple of %d and <= %d", lm->d, MOE_GROUP,
                    MOE_MAX_D);
    if (lm->V > MOE_MAX_VOCAB) return fail(MOE_EUNSUPPORTED, "V=%d > %d", lm->V, MOE_MAX_VOCAB);
    return MOE_OK;
}

// Hand-off workspace: per-work-group best (logit, row) pairs.
size_t lm_part_bytes(int32_t V) { return align256(8 * (size_t)q4moe::lm_partials(V, false)); }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

}  // namespace

namespace q4moe {
void trace_point(hipStream_t s) {
    if (g_trace && g_trace_next < g_trace_n) (void)hipEventRecord(g_trace[g_trace_next++], s);
}
}  // namespace q4moe

extern "C" {

void moe_trace_events(void* const* events, int32_t n) {
    g_trace = (events && n > 0) ? (hipEvent_t*)events : nullptr;
    g_trace_n = g_trace ? n : 0;
    g_trace_next = 0;
}

int32_t moe_block_map_capacity(int32_t T, int32_t top_k, int32_t n_experts, int32_t rows) {
    if (T <= 0 || top_k <= 0 || n_experts <= 0 || rows <= 0) return 0;
    const int64_t A = (int64_t)T * top_k;
    return (int32_t)(A / rows + (n_experts < A ? n_experts : A));
}

size_t moe_workspace_bytes(const moe_layer* L, int32_t T) {
    if (check_layer(L) || check_tokens(T)) return 0;
    const DecodeWs dw = decode_ws(L);
    return prefill_ws(L, T, dw.total).total;
}

int moe_route(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
              const moe_routing* r, void* stream) {
    int rc;
    if ((rc = check_layer(L)) || (rc = check_tokens(T)) || (rc = check_routing(r))) return rc;
    const bool logits_in = flags & MOE_LOGITS_IN;
    if (flags & ~MOE_LOGITS_IN) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
    if (!logits_in && (rc = check_ptr(x, "x"))) return rc;
    hipStream_t s = (hipStream_t)stream;
    trace_begin(s);
    if ((rc = hip_status(q4moe::launch_router_logits(logits_in ? nullptr : x, T, L->d,
                                                     L->w_router, L->router_bias, L->n_experts,
                                                     r->logits, r->blk_counts, s),
                         "router logits")))
        return rc;
    if ((rc = hip_status(q4moe::launch_topk(r->logits, T, L->n_experts, L->top_k, r->topk_idx,
                                            r->topk_w, r->blk_counts, s),
                         "top-k")))
        return rc;
    return hip_status(q4moe::launch_route_sort(r->topk_idx, T, L->top_k, L->n_experts, r, s),
                      "route sort");
}

int moe_prefill(const moe_layer* L, const uint16_t* x, int32_t T, const moe_routing* r, void* ws,
                size_t ws_bytes, uint16_t* y, void* stream) {
    return moe_prefill_ex(L, x, T, r, ws, ws_bytes, y, 0u, stream);
}

int moe_prefill_ex(const moe_layer* L, const uint16_t* x, int32_t T, const moe_routing* r,
                   void* ws, size_t ws_bytes, uint16_t* y, uint32_t flags, void* stream) {
    int rc;
    if ((rc = check_layer(L)) || (rc = check_tokens(T)) || (rc = check_routing(r)) ||
        (rc = check_ptr(x, "x")) || (rc = check_ptr(y, "y")) || (rc = check_ptr(ws, "workspace")))
        return rc;
    const uint32_t rows_flags = MOE_ITEM_ROWS_64 | MOE_ITEM_ROWS_32 | MOE_ITEM_ROWS_16;
    if ((flags & ~rows_flags) || __builtin_popcount(flags & rows_flags) > 1)
        return fail(MOE_EINVAL, "prefill flags 0x%x", flags);
    const size_t need = moe_workspace_bytes(L, T);
    if (ws_bytes < need)
        return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    const PrefillWs pw = prefill_ws(L, T, decode_ws(L).total);
    unsigned char* base = (unsigned char*)ws;
    q4moe::PrefillArgs a;
    a.x = x;
    a.T = T;
    a.d = L->d;
    a.I = L->inter;
    a.E = L->n_experts;
    a.k = L->top_k;
    a.gate = q4(L->gate);
    a.up = q4(L->up);
    a.down = q4(L->down);
    a.sh_gate = q4(L->sh_gate);
    a.sh_up = q4(L->sh_up);
    a.sh_down = q4(L->sh_down);
    a.perm = r->perm;
    a.offsets = r->offsets;
    a.tile_map = r->tile_map;
    a.n_tiles = r->n_tiles;
    a.topk_w = r->topk_w;
    a.tile_bound = moe_block_map_capacity(T, L->top_k, L->n_experts, MOE_TILE_ROWS);
    a.item_sh = (flags & MOE_ITEM_ROWS_16)   ? 3
                : (flags & MOE_ITEM_ROWS_32) ? 2
                : (flags & MOE_ITEM_ROWS_64) ? 1
                                             : 0;
    a.h = (uint16_t*)(base + pw.h);
    a.h_sh = (uint16_t*)(base + pw.h_sh);
    a.part = (uint16_t*)(base + pw.part);
    a.pexp = (int8_t*)(base + pw.pexp);
    a.dn_pre = (int32_t*)(base + pw.dn_pre);
    a.dn_exp = (int32_t*)(base + pw.dn_exp);
    a.y = y;
    trace_begin((hipStream_t)stream);
    return hip_status(q4moe::launch_prefill(a, (hipStream_t)stream), "prefill");
}

int moe_decode(const moe_layer* L, const uint16_t* x, uint32_t flags, const moe_routing* r,
               void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
    return moe_decode_tokens(L, x, 1, flags, r, ws, ws_bytes, y, stream);
}

}  // extern "C"

namespace {

// Validation shared by the decode entry points (everything but the workspace).
int check_decode(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                 const moe_routing* r, const uint16_t* y) {
    int rc;
    if ((rc = check_layer(L)) || (rc = check_ptr(y, "y"))) return rc;
    if (T < 1 || T > MOE_MAX_DECODE_TOKENS)
        return fail(MOE_EUNSUPPORTED, "decode takes 1..%d tokens, not T=%d", MOE_MAX_DECODE_TOKENS,
                    T);
    if (flags & ~MOE_LOGITS_IN) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
    const bool logits_in = flags & MOE_LOGITS_IN;
    if ((rc = check_ptr(x, "x"))) return rc;
    if (logits_in && (!r || !r->logits))
        return fail(MOE_EINVAL, "MOE_LOGITS_IN needs routing->logits");
    if (r) {
        if ((rc = check_ptr(r->logits, "routing.logits", true)) ||
            (rc = check_ptr(r->topk_idx, "routing.topk_idx", true)) ||
            (rc = check_ptr(r->topk_w, "routing.topk_w", true)))
            return rc;
    }
    return MOE_OK;
}

// The decode launches with the decode region of the workspace at `base`.
int decode_launch(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                  const moe_routing* r, unsigned char* base, uint16_t* y, void* stream) {
    const DecodeWs dw = decode_ws(L);
    q4moe::DecodeArgs a;
    a.x = x;
    a.T = T;
    a.d = L->d;
    a.I = L->inter;
    a.E = L->n_experts;
    a.k = L->top_k;
    a.w_router = L->w_router;
    a.router_bias = L->router_bias;
    a.gate = q4(L->gate);
    a.up = q4(L->up);
    a.down = q4(L->down);
    a.sh_gate = q4(L->sh_gate);
    a.sh_up = q4(L->sh_up);
    a.sh_down = q4(L->sh_down);
    a.logits_in = (flags & MOE_LOGITS_IN) != 0;
    a.logits = (r && r->logits) ? r->logits : (float*)(base + dw.logits);
    a.out_idx = r ? r->topk_idx : nullptr;
    a.out_w = r ? r->topk_w : nullptr;
    a.partial = (float*)(base + dw.partial);
    a.sel_idx = (int32_t*)(base + dw.sel_idx);
    a.sel_w = (float*)(base + dw.sel_w);
    a.h = (uint16_t*)(base + dw.h);
    a.y_sh = (float*)(base + dw.y_sh);
    a.y = y;
    trace_begin((hipStream_t)stream);
    return hip_status(q4moe::launch_decode(a, (hipStream_t)stream), "decode");
}

// Scratch of moe_decode_tokens_static: one copy per GPU, for the life of the
// process.  Host code never uses this name as an address (in host code it is
// a stand-in, not device memory); it uses the per-device address that
// hipGetSymbolAddress returns.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's scratch address, looked up once per device with that
// device current.  NULL (and the reason in the error text) on failure.
unsigned char* static_scratch(int* rc) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = fail(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *rc = fail(MOE_EUNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                   kMaxDevices);
        return nullptr;
    }
    unsigned char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !addr) {
            *rc = fail(MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
            return nullptr;
        }
        p = (unsigned char*)addr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int moe_decode_tokens_static(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                             const moe_routing* r, uint16_t* y, void* stream) {
    int rc;
    if ((rc = check_decode(L, x, T, flags, r, y))) return rc;
    const size_t need = decode_ws(L).total;
    if (need > kStaticScratchBytes)
        return fail(MOE_EUNSUPPORTED,
                    "this layer's decode scratch (%zu bytes) exceeds the library's static %zu",
                    need, kStaticScratchBytes);
    unsigned char* base = static_scratch(&rc);
    if (!base) return rc;
    return decode_launch(L, x, T, flags, r, base, y, stream);
}

int moe_decode_tokens(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                      const moe_routing* r, void* ws, size_t ws_bytes, uint16_t* y,
                      void* stream) {
    int rc;
    if ((rc = check_decode(L, x, T, flags, r, y)) || (rc = check_ptr(ws, "workspace")))
        return rc;
    const size_t need = moe_workspace_bytes(L, 1);
    if (ws_bytes < need)
        return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return decode_launch(L, x, T, flags, r, (unsigned char*)ws, y, stream);
}

int moe_dequant(const moe_q4mat* m, int32_t n_rows, int32_t K, uint16_t* w_out, void* stream) {
    int rc;
    if (!m) return fail(MOE_EINVAL, "matrix is NULL");
    if ((rc = check_mat(*m, "m")) || (rc = check_ptr(w_out, "w_out"))) return rc;
    if (n_rows <= 0 || K <= 0) return fail(MOE_EINVAL, "n_rows=%d K=%d", n_rows, K);
    if (K % MOE_GROUP) return fail(MOE_EUNSUPPORTED, "K=%d not a multiple of %d", K, MOE_GROUP);
    return hip_status(q4moe::launch_dequant(q4(*m), n_rows, K, w_out, (hipStream_t)stream),
                      "dequant");
}

size_t moe_lm_workspace_bytes(const moe_lm_head* lm) {
    if (check_lm(lm)) return 0;
    return lm_part_bytes(lm->V);
}

int moe_lm_argmax(const moe_lm_head* lm, const uint16_t* x, uint32_t flags, float* logits,
                  int32_t* token, uint16_t* x_next, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_lm(lm))) return rc;
    if (flags & ~MOE_LOGITS_IN) return fail(MOE_EINVAL, "unknown flags 0x%x", flags);
    const bool logits_in = flags & MOE_LOGITS_IN;
    if (!logits_in && ((rc = check_mat(lm->head, "head")) || (rc = check_ptr(x, "x")))) return rc;
    if ((rc = check_ptr(logits, "logits")) || (rc = check_ptr(ws, "workspace"))) return rc;
    if (!token || ((uintptr_t)token & 3u))
        return fail(MOE_EINVAL, "token is NULL or not 4-byte aligned");
    if (x_next && ((rc = check_ptr(x_next, "x_next")) || (rc = check_mat(lm->embed, "embed"))))
        return rc;
    const size_t need = moe_lm_workspace_bytes(lm);
    if (ws_bytes < need)
        return fail(MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    unsigned char* base = (unsigned char*)ws;
    q4moe::LmArgs a;
    a.x = x;
    a.V = lm->V;
    a.d = lm->d;
    a.head = q4(lm->head);
    a.embed = q4(lm->embed);
    a.logits = logits;
    a.token = token;
    a.x_next = x_next;
    a.part = (int2*)base;
    trace_begin((hipStream_t)stream);
    return hip_status(q4moe::launch_lm_argmax(a, logits_in, (hipStream_t)stream), "lm argmax");
}

const char* moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported shape";
        case MOE_EWORKSPACE: return "workspace too small";
        case MOE_EHIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
