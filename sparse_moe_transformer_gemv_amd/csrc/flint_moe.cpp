// flint_moe.cpp -- host side of libflint_moe.so: the C ABI declared in
// include/flint_moe.h.  Argument validation (before any HIP call), device
// check, workspace carving, decode/prefill path choice and kernel enqueueing
// on the caller's stream.  No allocation, host synchronisation or
// device-to-host read happens inside flint_moe_forward.
#include "flint_moe.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "flint_internal.hpp"

using namespace flint;

struct flint_moe {
    flint_moe_config cfg;
    int device;
    void* mem;
    size_t mem_bytes;
    Workspace ws;
    int last_T;
    int decode_max_t;
    int fused_max_t;  // largest batch for the single-launch decode (0: by weight type)
    int n_cu;
    // measurement hook
    int prof_kernel;
    int prof_cap;
    int prof_n;
    std::vector<hipEvent_t> prof_ev;  // 2 per launch
};

namespace {

thread_local char g_err[512] = "";

flint_status fail(flint_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

flint_status ok() {
    g_err[0] = '\0';
    return FLINT_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t act_size(int dt) { return dt == FLINT_F32 ? 4 : 2; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

flint_status check_config(const flint_moe_config* c) {
    if (!c) return fail(FLINT_ERR_INVALID_ARG, "config is NULL");
    if (c->struct_size != sizeof(flint_moe_config))
        return fail(FLINT_ERR_INVALID_ARG, "config.struct_size %u != %zu", c->struct_size,
                    sizeof(flint_moe_config));
    if (c->d_model <= 0 || c->d_model % 64 || c->d_model > 16384)
        return fail(FLINT_ERR_INVALID_ARG, "d_model %d: need a positive multiple of 64, <= 16384",
                    c->d_model);
    if (c->n_experts < 1 || c->n_experts > 256)
        return fail(FLINT_ERR_INVALID_ARG, "n_experts %d: need 1..256", c->n_experts);
    if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
        return fail(FLINT_ERR_INVALID_ARG, "top_k %d: need 1..min(8, n_experts)", c->top_k);
    if (c->d_ff <= 0 || c->d_ff % 32 || c->d_ff > 16384)
        return fail(FLINT_ERR_INVALID_ARG, "d_ff %d: need a positive multiple of 32, <= 16384",
                    c->d_ff);
    if (c->d_ff_shared < 0 || c->d_ff_shared % 32 || c->d_ff_shared > 16384)
        return fail(FLINT_ERR_INVALID_ARG, "d_ff_shared %d: need 0 or a multiple of 32",
                    c->d_ff_shared);
    if (c->act_dtype != FLINT_F32 && c->act_dtype != FLINT_BF16)
        return fail(FLINT_ERR_INVALID_ARG, "act_dtype %d: need FLINT_F32 or FLINT_BF16",
                    c->act_dtype);
    if (c->weight_dtype != FLINT_F32 && c->weight_dtype != FLINT_BF16 &&
        c->weight_dtype != FLINT_NVFP4)
        return fail(FLINT_ERR_INVALID_ARG, "weight_dtype %d unknown", c->weight_dtype);
    if (c->max_tokens < 1 || c->max_tokens > 65536)
        return fail(FLINT_ERR_INVALID_ARG, "max_tokens %d: need 1..65536", c->max_tokens);
    if (c->flags & ~(FLINT_FORCE_DECODE_PATH | FLINT_FORCE_PREFILL_PATH | FLINT_DEBUG_POISON_WORKSPACE |
                     FLINT_UNFUSED_DECODE))
        return fail(FLINT_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
    if ((c->flags & FLINT_FORCE_DECODE_PATH) && (c->flags & FLINT_FORCE_PREFILL_PATH))
        return fail(FLINT_ERR_INVALID_ARG, "both path-forcing flags set");
    if ((c->flags & FLINT_FORCE_PREFILL_PATH) &&
        (c->act_dtype != FLINT_BF16 || (c->weight_dtype != FLINT_BF16 && c->weight_dtype != FLINT_NVFP4)))
        return fail(FLINT_ERR_UNSUPPORTED,
                    "the grouped-MFMA path needs bf16 activations and bf16 or NVFP4 weights");
    return FLINT_OK;
}

flint_status check_device(int* dev_out, int* n_cu) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return fail(FLINT_ERR_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FLINT_ERR_NO_DEVICE, "hipGetDevice failed");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(FLINT_ERR_NO_DEVICE, "hipGetDeviceProperties failed");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(FLINT_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950", dev,
                    prop.gcnArchName);
    *dev_out = dev;
    *n_cu = prop.multiProcessorCount;
    return FLINT_OK;
}

// Per-device result of check_device for the allocation-free entry point, so
// that its calls after the first make no property query.
std::mutex g_dev_mu;
int g_dev_ncu[64];  // 0: not checked yet

flint_status cached_device(int* dev_out, int* n_cu) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(FLINT_ERR_NO_DEVICE, "no usable current HIP device");
    std::lock_guard<std::mutex> lock(g_dev_mu);
    if (!g_dev_ncu[dev]) {
        int d2 = 0, n = 0;
        flint_status st = check_device(&d2, &n);
        if (st != FLINT_OK) return st;
        g_dev_ncu[dev] = n > 0 ? n : 1;
    }
    *dev_out = dev;
    *n_cu = g_dev_ncu[dev];
    return FLINT_OK;
}

int decode_max_t_default() {
    if (const char* s = std::getenv("FLINT_MOE_DECODE_MAX_T")) return std::atoi(s);
    return 64;
}

// Largest batch that runs as the single-launch decode.  Measured on the full
// layer (d = 2048, 256 experts, f = 512) against the separate launches, the
// single launch is faster up to 5 tokens with bf16 weights and up to 4 with
// NVFP4 weights, and slower above (its persistent grid balances the gate/up
// and down work less well).  FLINT_MOE_FUSED_MAX_T overrides both (at most
// the kernel's own limit; 0 turns the single launch off).
int fused_max_t_default() {
    if (const char* s = std::getenv("FLINT_MOE_FUSED_MAX_T")) return std::max(0, std::atoi(s));
    return -1;
}
int fused_max_t_for(int configured, int wdt) {
    if (configured >= 0) return configured;
    return wdt == DT_NVFP4 ? 4 : 5;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Lay the workspace out in `base` (nullptr: just measure).  Three regions, in
// this order: the hand-off tickets (zero between launches), the integer
// routing tables, and the floating-point data (w->float_off onwards: the only
// region the debug poison fills).
size_t carve(const flint_moe_config& c, char* base, Workspace* w) {
    const size_t Tm = (size_t)c.max_tokens, E = (size_t)c.n_experts, k = (size_t)c.top_k;
    const size_t fmax = (size_t)(c.d_ff > c.d_ff_shared ? c.d_ff : c.d_ff_shared);
    const size_t slots = (k + 1) * Tm;
    const size_t max_tiles = slots / kPrefillBM + E + 2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, 256);
        return base ? static_cast<void*>(base + o) : nullptr;
    };
    // tickets
    w->rcount = static_cast<int*>(take((4 * ((E + 15) / 16) + 8) * 4));
    w->counter = static_cast<int*>(take((1 + (Tm + 15) / 16) * 4));
    w->dcount = static_cast<int*>(take((size_t)((c.d_model + 15) / 16) * 4));
    w->kcount = static_cast<int*>(take((E + 1) * (size_t)((c.d_model + 15) / 16) * 4));
    w->fbar = static_cast<int*>(take((size_t)kFusedBarrierInts * 4));
    w->ticket_bytes = off;
    // integer routing tables
    w->sel = static_cast<int*>(take(Tm * k * 4));
    w->counts = static_cast<int*>(take(E * 4));
    w->offsets = static_cast<int*>(take((E + 1) * 4));
    w->sorted_pair = static_cast<int*>(take(Tm * k * 4));
    w->pair_pos = static_cast<int*>(take(Tm * k * 4));
    w->groups = static_cast<int4*>(take((E + 1) * 16));
    w->n_groups = static_cast<int*>(take(4));
    w->tiles = static_cast<int2*>(take(max_tiles * 8));
    w->bhist = static_cast<int*>(take((Tm + 15) / 16 * 256 * 4));
    w->n_tiles = static_cast<int*>(take(4));
    w->float_off = off;
    // floating-point data
    w->logits = static_cast<float*>(take(Tm * E * 4));
    w->wts = static_cast<float*>(take(Tm * k * 4));
    w->sorted_wt = static_cast<float*>(take(Tm * k * 4));
    w->rpart = static_cast<float*>(take((size_t)(c.d_model / 256 > 0 ? c.d_model / 256 : 1) * 64 * E * 4));
    w->w3 = static_cast<uint16_t*>(take(3 * E * (size_t)c.d_model * 2));
    const size_t kchunks = fmax > (size_t)kDownKChunk ? (fmax + kDownKChunk - 1) / kDownKChunk : 0;
    // the down kernel strides its chunks by kSplitRowsMax rows
    w->part = static_cast<float*>(take(kchunks * (size_t)kSplitRowsMax * c.d_model * 4));
    w->h = take(slots * fmax * 8);
    w->y = take(slots * (size_t)c.d_model * 4);
    w->max_tiles = (int)max_tiles;
    return off;
}

flint_status hip_fail(hipError_t e, const char* what) {
    return fail(FLINT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

flint_status check_weights(const flint_moe_config& c, const flint_expert_weights* w,
                           const char* name) {
    if (!w) return fail(FLINT_ERR_INVALID_ARG, "%s weights are NULL", name);
    if (!w->gate_up || !w->down)
        return fail(FLINT_ERR_INVALID_ARG, "%s gate_up/down pointer is NULL", name);
    if (!aligned(w->gate_up, 16) || !aligned(w->down, 16))
        return fail(FLINT_ERR_INVALID_ARG, "%s gate_up/down must be 16-byte aligned", name);
    if (c.weight_dtype == FLINT_NVFP4) {
        if (!w->gate_up_scales || !w->down_scales || !w->tensor_scales)
            return fail(FLINT_ERR_INVALID_ARG, "%s: NVFP4 weights need scale pointers", name);
        if (!aligned(w->tensor_scales, 4))
            return fail(FLINT_ERR_INVALID_ARG, "%s tensor_scales must be 4-byte aligned", name);
    } else if (w->gate_up_scales || w->down_scales || w->tensor_scales) {
        return fail(FLINT_ERR_INVALID_ARG, "%s: scale pointers must be NULL unless NVFP4", name);
    }
    return FLINT_OK;
}

// Debug mode: fill the floating-point region of the workspace with all-ones
// words (NaN as fp32, and as each bf16 / f16 half), so a kernel that reads a
// value no kernel of the same forward wrote makes the output NaN.  The
// tickets and the integer tables keep their contents: a stale index read as
// -1 could address memory outside every buffer.
hipError_t poison(const flint_moe* h, hipStream_t s) {
    const size_t off = h->ws.float_off;
    return launch_fill_u32(reinterpret_cast<uint32_t*>(static_cast<char*>(h->mem) + off),
                           (h->mem_bytes - off) / 4, 0xFFFFFFFFu, s);
}

struct Timer {
    flint_moe* h;
    int id;
    hipStream_t s;
    bool on;
    Timer(flint_moe* h_, int id_, hipStream_t s_) : h(h_), id(id_), s(s_), on(false) {
        if (h->prof_kernel == id && h->prof_n < h->prof_cap) {
            on = true;
            (void)hipEventRecord(h->prof_ev[2 * h->prof_n], s);
        }
    }
    ~Timer() {
        if (on) {
            (void)hipEventRecord(h->prof_ev[2 * h->prof_n + 1], s);
            h->prof_n++;
        }
    }
};

// The forward on handle state h (a created handle, or the stack-built state of
// flint_moe_forward_noalloc over the static scratch).
// The combine launch, or with norm_out the combine and the next layer's
// pre-norm (one launch where the shape allows, else the combine and then the
// RMSNorm kernel).  packed: the y rows come from the prefill down kernels (block format).
hipError_t combine_step(flint_moe* h, const LayerArgs& a, bool packed, hipStream_t stream, float eps, void* norm_out) {
    Timer tm(h, FLINT_KERNEL_COMBINE, stream);
    if (!norm_out) return launch_combine(a, h->ws, packed, stream);
    if (combine_norm_ok(a.dm)) return launch_combine_norm(a, h->ws, packed, eps, norm_out, stream);
    hipError_t e = launch_combine(a, h->ws, packed, stream);
    if (e == hipSuccess) e = launch_rmsnorm(a.dm.T, a.dm.d, static_cast<const float*>(a.out), eps, norm_out, stream);
    return e;
}

flint_status forward_impl(flint_moe* h, int32_t T, const void* hidden, const float* router_w,
                          const float* router_bias, const flint_expert_weights* experts,
                          const flint_expert_weights* shared, const float* residual, void* out,
                          hipStream_t stream, float eps = 0.f, void* norm_out = nullptr) {
    const flint_moe_config& c = h->cfg;
    if (T < 0 || T > c.max_tokens)
        return fail(FLINT_ERR_INVALID_ARG, "T=%d outside 0..max_tokens=%d", T, c.max_tokens);
    if (T == 0) return ok();  // nothing to read or write
    if (!hidden || !router_w || !out)
        return fail(FLINT_ERR_INVALID_ARG, "hidden, router_w and out must be non-NULL");
    if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(router_w, 16) ||
        (residual && !aligned(residual, 16)) || (router_bias && !aligned(router_bias, 4)))
        return fail(FLINT_ERR_INVALID_ARG, "tensors must be 16-byte aligned (bias 4-byte)");
    flint_status st = check_weights(c, experts, "routed");
    if (st != FLINT_OK) return st;
    if (c.d_ff_shared > 0) {
        st = check_weights(c, shared, "shared");
        if (st != FLINT_OK) return st;
    } else if (shared) {
        return fail(FLINT_ERR_INVALID_ARG, "shared weights given but d_ff_shared == 0");
    }
    const size_t xbytes = (size_t)T * c.d_model * act_size(c.act_dtype);
    const size_t obytes = (size_t)T * c.d_model * (residual ? 4 : act_size(c.act_dtype));
    if (overlap(hidden, xbytes, out, obytes))
        return fail(FLINT_ERR_INVALID_ARG, "out overlaps hidden");
    if (residual && residual != out &&
        overlap(residual, (size_t)T * c.d_model * 4, out, obytes))
        return fail(FLINT_ERR_INVALID_ARG, "out partially overlaps residual");
    if (norm_out) {
        const size_t nbytes = (size_t)T * c.d_model * 2;
        if (!residual)
            return fail(FLINT_ERR_INVALID_ARG, "the pre-norm output needs the fp32 residual form");
        if (!aligned(norm_out, 16))
            return fail(FLINT_ERR_INVALID_ARG, "norm_out must be 16-byte aligned");
        if (!(eps >= 0.f) || eps > 1.f)
            return fail(FLINT_ERR_INVALID_ARG, "eps %g outside 0..1", (double)eps);
        if (overlap(norm_out, nbytes, out, obytes) || overlap(norm_out, nbytes, hidden, xbytes) ||
            overlap(norm_out, nbytes, residual, (size_t)T * c.d_model * 4))
            return fail(FLINT_ERR_INVALID_ARG, "norm_out overlaps hidden, residual or out");
    }

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
        return fail(FLINT_ERR_INVALID_ARG, "current device %d is not the handle's device %d", dev,
                    h->device);

    LayerArgs a;
    a.dm = Dims{T, c.d_model, c.n_experts, c.top_k, c.d_ff, c.d_ff_shared, c.act_dtype,
                c.weight_dtype};
    a.x = hidden;
    a.wr = router_w;
    a.bias = router_bias;
    a.routed = WeightPtrs{experts->gate_up, experts->down, experts->gate_up_scales,
                          experts->down_scales, experts->tensor_scales};
    a.shared = shared ? WeightPtrs{shared->gate_up, shared->down, shared->gate_up_scales,
                                   shared->down_scales, shared->tensor_scales}
                      : WeightPtrs{nullptr, nullptr, nullptr, nullptr, nullptr};
    a.residual = residual;
    a.out = out;

    Timer whole(h, FLINT_KERNEL_FORWARD, stream);  // records only when that id is profiled
    const bool mfma_ok = prefill_ok(a.dm);
    bool prefill = false;
    if (c.flags & FLINT_FORCE_PREFILL_PATH) {
        if (!mfma_ok)
            return fail(FLINT_ERR_UNSUPPORTED,
                        "grouped-MFMA path needs d %% 256 == 0 and f, f_s %% 128 == 0");
        prefill = true;
    } else if (!(c.flags & FLINT_FORCE_DECODE_PATH)) {
        prefill = mfma_ok && T > h->decode_max_t;
    }

    hipError_t e;
    if (c.flags & FLINT_DEBUG_POISON_WORKSPACE) {
        e = poison(h, stream);
        if (e != hipSuccess) return hip_fail(e, "workspace poison");
    }
    if (prefill) {
        {
            Timer tm(h, FLINT_KERNEL_ROUTE, stream);
            // logits (matrix cores when the shape allows), then top-k with one
            // wavefront per token
            e = router_gemm_ok(a.dm)  ? launch_router_gemm(a, h->ws, stream)
                : route_mfma_ok(a.dm) ? launch_route_mfma(a, h->ws, false, stream)
                                      : launch_router_logits(a, h->ws, stream);
            if (e == hipSuccess) e = launch_topk(a, h->ws, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "route kernel");
        {
            Timer tm(h, FLINT_KERNEL_SORT, stream);
            e = launch_sort(a, h->ws, kPrefillBM, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "sort kernel");
        {
            Timer tm(h, FLINT_KERNEL_EXPERT_UP, stream);
            e = launch_gateup_prefill(a, h->ws, h->n_cu, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "gate/up kernel");
        {
            Timer tm(h, FLINT_KERNEL_EXPERT_DOWN, stream);
            e = launch_down_prefill(a, h->ws, h->n_cu, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "down kernel");
        e = combine_step(h, a, true, stream, eps, norm_out);
        if (e != hipSuccess) return hip_fail(e, "combine kernel");
        h->last_T = T;
        return ok();
    }
    if (!(c.flags & FLINT_UNFUSED_DECODE) && T <= fused_max_t_for(h->fused_max_t, a.dm.wdt)) {
        const int G = fused_decode_grid(a.dm, h->n_cu);
        if (G > 0) {
            {
                Timer tm(h, FLINT_KERNEL_FUSED, stream);
                e = launch_decode_fused(a, h->ws, G, stream);
            }
            if (e != hipSuccess) return hip_fail(e, "single-launch decode kernel");
            if (norm_out) e = launch_rmsnorm(T, c.d_model, static_cast<const float*>(out), eps, norm_out, stream);
            if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel");
            h->last_T = T;
            return ok();
        }
    }
    {
        Timer tm(h, FLINT_KERNEL_ROUTE, stream);
        if (route_mfma_ok(a.dm))
            e = launch_route_mfma(a, h->ws, true, stream);
        else
            e = launch_route_decode(a, h->ws, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "route kernel");
    {
        Timer tm(h, FLINT_KERNEL_EXPERT_UP, stream);
        e = launch_gateup_decode(a, h->ws, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "gate/up kernel");
    {
        Timer tm(h, FLINT_KERNEL_EXPERT_DOWN, stream);
        e = launch_down_decode(a, h->ws, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "down kernel");
    if (!down_decode_combines(a.dm))
        e = combine_step(h, a, false, stream, eps, norm_out);
    else if (norm_out)
        e = launch_rmsnorm(T, c.d_model, static_cast<const float*>(out), eps, norm_out, stream);
    if (e != hipSuccess) return hip_fail(e, "combine kernel");
    h->last_T = T;
    return ok();
}

}  // namespace

extern "C" {

const char* flint_status_string(flint_status s) {
    // A C caller may pass any int; reading it through the C++ enum type would
    // be undefined for values outside the enumerators' range, so take the bits.
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case FLINT_OK: return "FLINT_OK";
    case FLINT_ERR_INVALID_ARG: return "FLINT_ERR_INVALID_ARG";
    case FLINT_ERR_UNSUPPORTED: return "FLINT_ERR_UNSUPPORTED";
    case FLINT_ERR_OUT_OF_MEMORY: return "FLINT_ERR_OUT_OF_MEMORY";
    case FLINT_ERR_NO_DEVICE: return "FLINT_ERR_NO_DEVICE";
    case FLINT_ERR_HIP: return "FLINT_ERR_HIP";
    }
    return "FLINT_ERR_UNKNOWN";
}

const char* flint_last_error(void) { return g_err; }

flint_status flint_moe_create(const flint_moe_config* cfg, flint_moe_t* out) {
    if (!out) return fail(FLINT_ERR_INVALID_ARG, "out handle pointer is NULL");
    *out = nullptr;
    flint_status st = check_config(cfg);
    if (st != FLINT_OK) return st;
    int dev = 0, n_cu = 0;
    st = check_device(&dev, &n_cu);
    if (st != FLINT_OK) return st;
    flint_moe* h = new (std::nothrow) flint_moe();
    if (!h) return fail(FLINT_ERR_OUT_OF_MEMORY, "host allocation failed");
    h->cfg = *cfg;
    h->device = dev;
    h->n_cu = n_cu;
    h->last_T = 0;
    h->prof_kernel = -1;
    h->prof_cap = 0;
    h->prof_n = 0;
    h->decode_max_t = decode_max_t_default();
    h->fused_max_t = fused_max_t_default();
    Workspace dummy{};
    h->mem_bytes = carve(*cfg, nullptr, &dummy);
    const size_t bytes = h->mem_bytes;
    hipError_t e = hipMalloc(&h->mem, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return fail(FLINT_ERR_OUT_OF_MEMORY, "workspace of %zu bytes: %s", bytes,
                    hipGetErrorString(e));
    }
    carve(*cfg, static_cast<char*>(h->mem), &h->ws);
    // zero everything once: the last-block tickets must start at 0
    e = hipMemset(h->mem, 0, h->mem_bytes);
    if (e == hipSuccess && (cfg->flags & FLINT_DEBUG_POISON_WORKSPACE)) e = poison(h, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipFree(h->mem);
        delete h;
        return hip_fail(e, "workspace init");
    }
    *out = h;
    return ok();
}

flint_status flint_moe_destroy(flint_moe_t h) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    (void)hipDeviceSynchronize();
    for (hipEvent_t ev : h->prof_ev) (void)hipEventDestroy(ev);
    hipError_t e = hipFree(h->mem);
    delete h;
    if (e != hipSuccess) return hip_fail(e, "hipFree");
    return ok();
}

flint_status flint_moe_forward(flint_moe_t h, int32_t T, const void* hidden, const float* router_w,
                               const float* router_bias, const flint_expert_weights* experts,
                               const flint_expert_weights* shared, const float* residual,
                               void* out, hipStream_t stream) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    return forward_impl(h, T, hidden, router_w, router_bias, experts, shared, residual, out, stream);
}

flint_status flint_moe_forward_prenorm(flint_moe_t h, int32_t T, const void* hidden, const float* router_w,
                                       const float* router_bias, const flint_expert_weights* experts,
                                       const flint_expert_weights* shared, const float* residual, float* out,
                                       float eps, void* norm_out, hipStream_t stream) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    if (!residual || !norm_out) return fail(FLINT_ERR_INVALID_ARG, "residual and norm_out must be non-NULL");
    return forward_impl(h, T, hidden, router_w, router_bias, experts, shared, residual, out, stream, eps,
                        norm_out);
}

flint_status flint_moe_forward_noalloc(const flint_moe_config* cfg, int32_t T, const void* hidden,
                                       const float* router_w, const float* router_bias,
                                       const flint_expert_weights* experts,
                                       const flint_expert_weights* shared, const float* residual,
                                       void* out, hipStream_t stream) {
    flint_status st = check_config(cfg);
    if (st != FLINT_OK) return st;
    if (T < 0 || T > 65536) return fail(FLINT_ERR_INVALID_ARG, "T=%d outside 0..65536", T);
    if (T == 0) return ok();
    // the state of a handle sized for exactly T tokens, on the stack
    flint_moe hs;
    hs.cfg = *cfg;
    hs.cfg.max_tokens = T;
    Workspace need{};
    const size_t bytes = carve(hs.cfg, nullptr, &need);
    if (bytes > (size_t)kScratchBytes)
        return fail(FLINT_ERR_INVALID_ARG,
                    "T=%d needs a workspace of %zu bytes, above the %zu-byte static scratch", T, bytes,
                    (size_t)kScratchBytes);
    int dev = 0, n_cu = 0;
    st = cached_device(&dev, &n_cu);
    if (st != FLINT_OK) return st;
    void* base = nullptr;
    hipError_t e = scratch_for_current_device(&base);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    hs.device = dev;
    hs.n_cu = n_cu;
    hs.mem = base;
    hs.mem_bytes = bytes;
    hs.last_T = 0;
    hs.prof_kernel = -1;
    hs.prof_cap = 0;
    hs.prof_n = 0;
    hs.decode_max_t = decode_max_t_default();
    hs.fused_max_t = fused_max_t_default();
    carve(hs.cfg, static_cast<char*>(base), &hs.ws);
    // earlier calls (other layouts) leave their bytes in the scratch: the
    // tickets of this layout start at zero (a fill kernel, not a memset node)
    e = launch_fill_u32(static_cast<uint32_t*>(base), hs.ws.ticket_bytes / 4, 0u, stream);
    if (e != hipSuccess) return hip_fail(e, "ticket clear");
    return forward_impl(&hs, T, hidden, router_w, router_bias, experts, shared, residual, out, stream);
}

flint_status flint_moe_get_routing(flint_moe_t h, int32_t* idx, float* weights,
                                   int32_t* sorted_pair, int32_t* counts, float* logits,
                                   int32_t* T_out, hipStream_t stream) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    const size_t T = (size_t)h->last_T, k = (size_t)h->cfg.top_k, E = (size_t)h->cfg.n_experts;
    if (T_out) *T_out = (int32_t)T;
    if (T == 0) return ok();
    struct Copy {
        void* dst;
        const void* src;
        size_t bytes;
    } copies[] = {{idx, h->ws.sel, T * k * 4},
                  {weights, h->ws.wts, T * k * 4},
                  {sorted_pair, h->ws.sorted_pair, T * k * 4},
                  {counts, h->ws.counts, E * 4},
                  {logits, h->ws.logits, T * E * 4}};
    for (const Copy& cp : copies) {
        if (!cp.dst) continue;
        hipError_t e = hipMemcpyAsync(cp.dst, cp.src, cp.bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "routing copy");
    }
    return ok();
}

flint_status flint_moe_get_fault(flint_moe_t h, int32_t* fault_out, hipStream_t stream) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    if (!fault_out) return fail(FLINT_ERR_INVALID_ARG, "fault_out is NULL");
    hipError_t e = hipMemcpyAsync(fault_out, h->ws.fbar + kFusedFaultInt, sizeof(int32_t),
                                  hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "fault word copy");
    return ok();
}

flint_status flint_moe_profile_begin(flint_moe_t h, int32_t kernel_id, int32_t n_launches) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    if (kernel_id < 0 || kernel_id >= FLINT_KERNEL_COUNT || n_launches < 1 || n_launches > 100000)
        return fail(FLINT_ERR_INVALID_ARG, "kernel_id %d / n_launches %d out of range", kernel_id,
                    n_launches);
    while ((int)h->prof_ev.size() < 2 * n_launches) {
        hipEvent_t ev;
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        h->prof_ev.push_back(ev);
    }
    h->prof_kernel = kernel_id;
    h->prof_cap = n_launches;
    h->prof_n = 0;
    return ok();
}

flint_status flint_moe_profile_end(flint_moe_t h, float* ms_out, int32_t cap, int32_t* n_out) {
    if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
    const int n = h->prof_n;
    h->prof_kernel = -1;
    int w = 0;
    for (int i = 0; i < n; ++i) {
        hipError_t e = hipEventSynchronize(h->prof_ev[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, h->prof_ev[2 * i], h->prof_ev[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        if (ms_out && w < cap) ms_out[w++] = ms;
    }
    if (n_out) *n_out = w;
    h->prof_n = 0;
    return ok();
}

flint_status flint_rmsnorm_forward(int32_t T, int32_t d, const float* in, float eps,
                                   void* out_bf16, hipStream_t stream) {
    if (T < 0 || d <= 0 || d % 64 || !in || !out_bf16 || !(eps >= 0.f))
        return fail(FLINT_ERR_INVALID_ARG, "rmsnorm: bad T=%d d=%d or pointers", T, d);
    if (!aligned(in, 16) || !aligned(out_bf16, 16))
        return fail(FLINT_ERR_INVALID_ARG, "rmsnorm: tensors must be 16-byte aligned");
    if (overlap(in, (size_t)T * d * 4, out_bf16, (size_t)T * d * 2))
        return fail(FLINT_ERR_INVALID_ARG, "rmsnorm: out overlaps in");
    if (T == 0) return ok();
    hipError_t e = launch_rmsnorm(T, d, in, eps, out_bf16, stream);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel");
    return ok();
}

}  // extern "C"
