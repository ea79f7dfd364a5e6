// api.hip -- the C ABI of libsiggate (declared in include/siggate.h):
// argument checks, workspace layout and kernel launches (host code), and
// the static device scratch of siggate_forward_noalloc.
#include <string.h>

#include <atomic>
#include <mutex>

// The library is built with hidden visibility: the functions siggate.h
// declares are its only exported symbols.
#pragma GCC visibility push(default)
#include "siggate.h"
#pragma GCC visibility pop
#include "siggate_internal.h"

using namespace siggate;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Validity first (EINVAL), then what this library builds (EUNSUPPORTED).
siggate_status_t check_gate_cfg(const siggate_cfg_t *c)
{
    if (!c) return SIGGATE_EINVAL;
    if (c->T < 0 || c->d <= 0 || c->E <= 0 || c->n_group <= 0 || c->top_k <= 0)
        return SIGGATE_EINVAL;
    if (c->E % c->n_group != 0) return SIGGATE_EINVAL;
    if (c->topk_group < 1 || c->topk_group > c->n_group) return SIGGATE_EINVAL;
    if (c->n_group > 1 && c->E / c->n_group < 2) return SIGGATE_EINVAL;
    if ((long long)c->top_k > (long long)c->topk_group * (c->E / c->n_group)) return SIGGATE_EINVAL;
    if (c->order != 0 && c->order != 1) return SIGGATE_EINVAL;
    if (!(c->route_scale == c->route_scale)) return SIGGATE_EINVAL;   // NaN
    if (c->score_func != 0 && c->score_func != 1) return SIGGATE_EINVAL;
    if (c->renorm < 0 || c->renorm > 2) return SIGGATE_EINVAL;
    if (c->mask_zero != 0 && c->mask_zero != 1) return SIGGATE_EINVAL;
    if (!(c->denom_eps >= 0.0f)) return SIGGATE_EINVAL;               // negative or NaN
    if (c->logits_path != PATH_FP32 && c->logits_path != PATH_BF16X3) return SIGGATE_EINVAL;
    if (c->E % 64 != 0 || c->E > MAX_EXPERTS) return SIGGATE_EUNSUPPORTED;
    if (c->n_group > 64 || (c->n_group & (c->n_group - 1)) != 0) return SIGGATE_EUNSUPPORTED;
    if (c->top_k > MAX_TOPK) return SIGGATE_EUNSUPPORTED;
    if (c->d % 8 != 0) return SIGGATE_EUNSUPPORTED;
    if ((long long)c->T * c->top_k > 0x7fffffffLL) return SIGGATE_EUNSUPPORTED;
    return SIGGATE_OK;
}

siggate_status_t check_dispatch_cfg(const siggate_cfg_t *c)
{
    if (!c) return SIGGATE_EINVAL;
    if (c->T < 0 || c->d <= 0 || c->E <= 0 || c->top_k <= 0) return SIGGATE_EINVAL;
    if (c->top_k > c->E) return SIGGATE_EINVAL;
    if (c->E > MAX_EXPERTS || c->top_k > MAX_TOPK || c->d % 8 != 0) return SIGGATE_EUNSUPPORTED;
    if ((long long)c->T * c->top_k > 0x7fffffffLL) return SIGGATE_EUNSUPPORTED;
    return SIGGATE_OK;
}

size_t forward_bytes(const siggate_cfg_t *c)
{
    return align256(plan_gate(c->T, c->d, c->E, c->logits_path).partial_bytes);
}

// Workspace of siggate_forward_noalloc: a static device array, one copy on
// every device the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never a device address: the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SIGGATE_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mutex;

// The device address of `scratch` on the current device (looked up on the
// first call on that device, with it current).
hipError_t device_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

GateArgs gate_args(const void *x, const float *W, const float *bias, const siggate_cfg_t *c,
                   const GatePlan &p)
{
    GateArgs a;
    memset(&a, 0, sizeof a);
    a.x = (const uint16_t *)x;
    a.W = W;
    a.bias = bias;
    a.T = c->T;
    a.d = c->d;
    a.n_group = c->n_group;
    a.topk_group = c->topk_group;
    a.top_k = c->top_k;
    a.order = c->order;
    a.route_scale = c->route_scale;
    a.score_func = c->score_func;
    a.renorm = c->renorm;
    a.mask_zero = c->mask_zero;
    a.denom_eps = c->denom_eps;
    a.E = c->E;
    a.e_stride = p.e_stride;
    a.chunks_total = (c->d + KC - 1) / KC;
    a.chunks_per_split = p.chunks_per_split;
    a.n_split = p.n_split;
    a.t_tiles = p.t_tiles;
    a.e_tiles = p.e_tiles;
    a.n_tiles = p.t_tiles * p.e_tiles * p.n_split;
    return a;
}

}  // namespace

extern "C" {

size_t siggate_workspace_bytes(const siggate_cfg_t *cfg)
{
    size_t need = 0;
    if (check_gate_cfg(cfg) == SIGGATE_OK) need = forward_bytes(cfg);
    if (check_dispatch_cfg(cfg) == SIGGATE_OK) {
        const size_t db = dispatch_workspace_bytes(cfg->T, cfg->E, cfg->top_k, true);
        if (db > need) need = db;
    }
    return need;
}

siggate_status_t siggate_forward(const void *x, const float *W, const float *bias,
                                 const siggate_cfg_t *cfg, float *weights, int32_t *indices,
                                 void *ws, size_t ws_bytes, void *stream)
{
    siggate_status_t st = check_gate_cfg(cfg);
    if (st != SIGGATE_OK) return st;
    if (!W) return SIGGATE_EINVAL;   // bias may be NULL (no-bias variant)
    if (cfg->T > 0 && (!x || !weights || !indices)) return SIGGATE_EINVAL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(bias) || !aligned16(weights) ||
        !aligned16(indices) || !aligned16(ws))
        return SIGGATE_EINVAL;
    const GatePlan p = plan_gate(cfg->T, cfg->d, cfg->E, cfg->logits_path);
    if (ws_bytes < align256(p.partial_bytes) || (p.partial_bytes && !ws)) return SIGGATE_EWORKSPACE;
    if (cfg->T == 0) return SIGGATE_OK;
    GateArgs a = gate_args(x, W, bias, cfg, p);
    a.weights = weights;
    a.indices = indices;
    a.partial = (float *)ws;
    return launch_gate(a, p, cfg->E, MODE_SELECT, (hipStream_t)stream) == hipSuccess
               ? SIGGATE_OK
               : SIGGATE_EHIP;
}

siggate_status_t siggate_forward_noalloc(const void *x, const float *W, const float *bias,
                                         const siggate_cfg_t *cfg, float *weights,
                                         int32_t *indices, void *stream)
{
    const siggate_status_t st = check_gate_cfg(cfg);
    if (st != SIGGATE_OK) return st;
    if (forward_bytes(cfg) > SIGGATE_SCRATCH_BYTES) return SIGGATE_ESCRATCH;
    void *ws = nullptr;
    if (device_scratch(&ws) != hipSuccess) return SIGGATE_EHIP;
    return siggate_forward(x, W, bias, cfg, weights, indices, ws, SIGGATE_SCRATCH_BYTES, stream);
}

siggate_status_t siggate_logits(const void *x, const float *W, const siggate_cfg_t *cfg,
                                float *logits, void *ws, size_t ws_bytes, void *stream)
{
    siggate_status_t st = check_gate_cfg(cfg);
    if (st != SIGGATE_OK) return st;
    if (!W) return SIGGATE_EINVAL;
    if (cfg->T > 0 && (!x || !logits)) return SIGGATE_EINVAL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(logits) || !aligned16(ws))
        return SIGGATE_EINVAL;
    const GatePlan p = plan_gate(cfg->T, cfg->d, cfg->E, cfg->logits_path);
    if (ws_bytes < align256(p.partial_bytes) || (p.partial_bytes && !ws)) return SIGGATE_EWORKSPACE;
    if (cfg->T == 0) return SIGGATE_OK;
    GateArgs a = gate_args(x, W, nullptr, cfg, p);
    a.logits = logits;
    a.partial = (float *)ws;
    return launch_gate(a, p, cfg->E, MODE_LOGITS, (hipStream_t)stream) == hipSuccess
               ? SIGGATE_OK
               : SIGGATE_EHIP;
}

siggate_status_t siggate_dispatch(const void *x, const int32_t *indices, const siggate_cfg_t *cfg,
                                  int32_t *tokens_per_expert, int32_t *offsets, int32_t *perm,
                                  int32_t *dest, void *permuted_x, void *ws, size_t ws_bytes,
                                  void *stream)
{
    siggate_status_t st = check_dispatch_cfg(cfg);
    if (st != SIGGATE_OK) return st;
    if (!tokens_per_expert) return SIGGATE_EINVAL;
    if (cfg->T > 0 && (!x || !indices || !perm || !permuted_x)) return SIGGATE_EINVAL;
    if (!aligned16(x) || !aligned16(indices) || !aligned16(tokens_per_expert) ||
        !aligned16(offsets) || !aligned16(perm) || !aligned16(dest) || !aligned16(permuted_x) ||
        !aligned16(ws))
        return SIGGATE_EINVAL;
    const int T = cfg->T, E = cfg->E, K = cfg->top_k;
    const size_t need = dispatch_workspace_bytes(T, E, K, dest == nullptr);
    if (ws_bytes < need || (need && !ws)) return SIGGATE_EWORKSPACE;

    DispatchArgs a;
    memset(&a, 0, sizeof a);
    a.x = (const uint16_t *)x;
    a.indices = indices;
    a.T = T;
    a.d = cfg->d;
    a.E = E;
    a.top_k = K;
    a.n_blocks = (T + DISPATCH_BLOCK_TOKENS - 1) / DISPATCH_BLOCK_TOKENS;
    const size_t cnt_bytes = align256((size_t)a.n_blocks * E * sizeof(int32_t));
    char *w = (char *)ws;
    a.block_counts = (int32_t *)w;
    a.block_base = (int32_t *)(w + cnt_bytes);
    a.dest = dest ? dest : (int32_t *)(w + 2 * cnt_bytes);
    a.tokens_per_expert = tokens_per_expert;
    a.offsets = offsets;
    a.perm = perm;
    a.permuted_x = (uint16_t *)permuted_x;
    return launch_dispatch(a, (hipStream_t)stream) == hipSuccess ? SIGGATE_OK : SIGGATE_EHIP;
}

siggate_status_t siggate_combine(const void *expert_out, const float *weights,
                                 const int32_t *dest, const siggate_cfg_t *cfg, void *y,
                                 void *stream)
{
    if (!cfg) return SIGGATE_EINVAL;
    if (cfg->T < 0 || cfg->d <= 0 || cfg->top_k <= 0) return SIGGATE_EINVAL;
    if (cfg->top_k > MAX_TOPK || cfg->d % 8 != 0) return SIGGATE_EUNSUPPORTED;
    if ((long long)cfg->T * cfg->top_k > 0x7fffffffLL) return SIGGATE_EUNSUPPORTED;
    if (cfg->T > 0 && (!expert_out || !weights || !dest || !y)) return SIGGATE_EINVAL;
    if (!aligned16(expert_out) || !aligned16(weights) || !aligned16(dest) || !aligned16(y))
        return SIGGATE_EINVAL;
    if (cfg->T == 0) return SIGGATE_OK;
    CombineArgs a;
    a.expert_out = (const uint16_t *)expert_out;
    a.weights = weights;
    a.dest = dest;
    a.y = (uint16_t *)y;
    a.T = cfg->T;
    a.d = cfg->d;
    a.top_k = cfg->top_k;
    return launch_combine(a, (hipStream_t)stream) == hipSuccess ? SIGGATE_OK : SIGGATE_EHIP;
}

siggate_status_t siggate_ep_send_splits(const int32_t *tokens_per_expert, int32_t E,
                                        int32_t ep_size, int32_t *send_counts,
                                        int32_t *send_offsets, void *stream)
{
    if (E <= 0 || ep_size <= 0 || ep_size > E || E % ep_size != 0) return SIGGATE_EINVAL;
    if (E > 4096) return SIGGATE_EUNSUPPORTED;
    if (!tokens_per_expert || !send_counts || !send_offsets) return SIGGATE_EINVAL;
    return launch_ep_send_splits(tokens_per_expert, E, ep_size, send_counts, send_offsets,
                                 (hipStream_t)stream) == hipSuccess
               ? SIGGATE_OK
               : SIGGATE_EHIP;
}

siggate_status_t siggate_ep_regroup(const int32_t *counts, int32_t ep_size, int32_t per,
                                    int32_t capacity, int32_t *local_counts,
                                    int32_t *regroup, void *stream)
{
    if (ep_size <= 0 || per <= 0 || capacity < 0) return SIGGATE_EINVAL;
    if ((long long)ep_size * per > 4096) return SIGGATE_EUNSUPPORTED;
    if (!counts || !local_counts || (capacity > 0 && !regroup)) return SIGGATE_EINVAL;
    return launch_ep_regroup(counts, ep_size, per, capacity, local_counts, regroup,
                             (hipStream_t)stream) == hipSuccess
               ? SIGGATE_OK
               : SIGGATE_EHIP;
}

static siggate_status_t check_ep_dedup(const siggate_cfg_t *c, int32_t ep_size)
{
    if (!c || c->T < 0 || c->E <= 0 || c->top_k <= 0 || ep_size <= 0) return SIGGATE_EINVAL;
    if (ep_size > c->E || c->E % ep_size != 0) return SIGGATE_EINVAL;
    if (ep_size > MAX_EXPERTS || c->top_k > MAX_TOPK) return SIGGATE_EUNSUPPORTED;
    if ((long long)c->T * c->top_k > 0x7fffffffLL) return SIGGATE_EUNSUPPORTED;
    return SIGGATE_OK;
}

size_t siggate_ep_workspace_bytes(const siggate_cfg_t *cfg, int32_t ep_size)
{
    if (check_ep_dedup(cfg, ep_size) != SIGGATE_OK) return 0;
    const size_t pairs = align256((size_t)cfg->T * cfg->top_k * sizeof(int32_t));
    // rank ids, perm, dest, and the dispatch count tables over ranks
    return 3 * pairs + dispatch_workspace_bytes(cfg->T, ep_size, cfg->top_k, false);
}

siggate_status_t siggate_ep_dedup(const int32_t *indices, const siggate_cfg_t *cfg,
                                  int32_t ep_size, int32_t *rank_counts,
                                  int32_t *rank_offsets, int32_t *send_tokens,
                                  int32_t *pair_slot, void *ws, size_t ws_bytes,
                                  void *stream)
{
    siggate_status_t st = check_ep_dedup(cfg, ep_size);
    if (st != SIGGATE_OK) return st;
    if (!rank_counts || !rank_offsets) return SIGGATE_EINVAL;
    if (cfg->T > 0 && (!indices || !send_tokens || !pair_slot)) return SIGGATE_EINVAL;
    if (!aligned16(indices) || !aligned16(rank_counts) || !aligned16(rank_offsets) ||
        !aligned16(send_tokens) || !aligned16(pair_slot) || !aligned16(ws))
        return SIGGATE_EINVAL;
    const size_t need = siggate_ep_workspace_bytes(cfg, ep_size);
    if (ws_bytes < need || (need && !ws)) return SIGGATE_EWORKSPACE;
    const int T = cfg->T, K = cfg->top_k;
    const size_t pairs = align256((size_t)T * K * sizeof(int32_t));
    char *w = (char *)ws;
    EpDedupArgs e;
    memset(&e, 0, sizeof e);
    e.indices = indices;
    e.rank_ids = (int32_t *)w;
    e.perm = (int32_t *)(w + pairs);
    e.dest = (int32_t *)(w + 2 * pairs);
    e.rank_offsets = rank_offsets;
    e.send_tokens = send_tokens;
    e.pair_slot = pair_slot;
    e.T = T;
    e.top_k = K;
    e.per = cfg->E / ep_size;
    e.ep_size = ep_size;

    DispatchArgs a;
    memset(&a, 0, sizeof a);
    a.indices = e.rank_ids;
    a.T = T;
    a.d = 8;
    a.E = ep_size;
    a.top_k = K;
    a.n_blocks = (T + DISPATCH_BLOCK_TOKENS - 1) / DISPATCH_BLOCK_TOKENS;
    const size_t cnt_bytes = align256((size_t)a.n_blocks * ep_size * sizeof(int32_t));
    a.block_counts = (int32_t *)(w + 3 * pairs);
    a.block_base = (int32_t *)(w + 3 * pairs + cnt_bytes);
    a.tokens_per_expert = rank_counts;
    a.offsets = rank_offsets;
    a.perm = e.perm;
    a.dest = e.dest;

    const hipStream_t s = (hipStream_t)stream;
    if (launch_ep_dedup_map(e, s) != hipSuccess) return SIGGATE_EHIP;
    if (launch_dispatch_meta(a, s) != hipSuccess) return SIGGATE_EHIP;
    return launch_ep_dedup_finish(e, s) == hipSuccess ? SIGGATE_OK : SIGGATE_EHIP;
}

const char *siggate_status_str(siggate_status_t status)
{
    switch (status) {
    case SIGGATE_OK: return "SIGGATE_OK: success";
    case SIGGATE_EINVAL: return "SIGGATE_EINVAL: invalid configuration or null/misaligned pointer";
    case SIGGATE_EUNSUPPORTED: return "SIGGATE_EUNSUPPORTED: configuration not built by this library";
    case SIGGATE_EWORKSPACE: return "SIGGATE_EWORKSPACE: workspace smaller than siggate_workspace_bytes";
    case SIGGATE_EHIP: return "SIGGATE_EHIP: HIP launch error";
    case SIGGATE_ESCRATCH:
        return "SIGGATE_ESCRATCH: the call needs more workspace than the static scratch "
               "(SIGGATE_SCRATCH_BYTES)";
    default: return "unknown siggate status";
    }
}

}  // extern "C"
