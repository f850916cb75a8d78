// api.hip -- the C ABI declared in include/ep.h: validation, error codes and
// kernel launches.  No HIP call happens before validation succeeds; nothing
// here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "ep.h"
#include "launch.h"

// Layout scratch of ep_get_layout_static.  In host code `scratch` names a
// host-side stand-in, not the device array: kernels get the array's device
// address, looked up once per device (hipGetSymbolAddress, with that device
// current) and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[EP_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device (nullptr with the
// hipError_t in *err on failure).  Two threads racing on a device's first
// call both look it up and store the same address.
void* static_scratch(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_dev[dev].store(p, std::memory_order_release);
    return p;
}

constexpr int32_t kMaxTokens = 1 << 24;
constexpr int32_t kMaxHidden = 16384;
constexpr int32_t kMaxExperts = 1024;
constexpr int32_t kMaxGroups = 64;
constexpr int32_t kMaxTopk = 32;
constexpr int32_t kMaxTopm = 8;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int effective_topm(const ep_config_t* c) {
    if (c->group_score_topm != 0) return c->group_score_topm;
    const int m = c->topk / c->topk_groups;
    return m > 0 ? m : 1;
}

int validate(const ep_config_t* c) {
    if (!c) return EP_ERR_INVALID_ARG;
    const ep_config_t& v = *c;
    if (v.num_tokens < 0 || v.hidden < 128 || v.hidden % 128 != 0) return EP_ERR_INVALID_ARG;
    if (v.num_experts < 1 || v.num_groups < 1 || v.num_experts % v.num_groups != 0) return EP_ERR_INVALID_ARG;
    if (v.topk_groups < 1 || v.topk_groups > v.num_groups) return EP_ERR_INVALID_ARG;
    const int gs = v.num_experts / v.num_groups;
    if (v.topk < 1 || (long)v.topk > (long)v.topk_groups * gs) return EP_ERR_INVALID_ARG;
    if (v.num_ranks < 1 || v.num_experts % v.num_ranks != 0) return EP_ERR_INVALID_ARG;
    if (v.group_score_topm < 0) return EP_ERR_INVALID_ARG;
    const int m = effective_topm(c);
    if (m > gs) return EP_ERR_INVALID_ARG;
    if ((long)v.num_tokens * v.topk >= (1L << 31)) return EP_ERR_INVALID_ARG;
    if (v.num_tokens > kMaxTokens || v.hidden > kMaxHidden || v.num_experts > kMaxExperts ||
        v.num_groups > kMaxGroups || v.topk > kMaxTopk || m > kMaxTopm)
        return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

// the configuration plus the low-latency receive capacity (rows per expert)
int validate_ll(const ep_config_t* c, int32_t capacity) {
    const int rc = validate(c);
    if (rc) return rc;
    if (capacity < 1 || (long)c->num_experts * capacity >= (1L << 31)) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

ep::Shape shape_of(const ep_config_t* c) {
    return ep::Shape{c->num_tokens, c->hidden,    c->num_experts, c->num_groups,
                     c->topk_groups, c->topk, c->num_ranks,   effective_topm(c)};
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return EP_OK;
    g_last_hip_error = (int)e;
    return EP_ERR_HIP;
}

}  // namespace

extern "C" {

EP_API int ep_abi_version(void) { return EP_ABI_VERSION; }

EP_API const char* ep_strerror(int code) {
    switch (code) {
        case EP_OK: return "success";
        case EP_ERR_INVALID_ARG: return "invalid argument (null pointer or inconsistent sizes)";
        case EP_ERR_ALIGNMENT: return "pointer not aligned as required";
        case EP_ERR_UNSUPPORTED: return "configuration outside the kernels' supported limits";
        case EP_ERR_WORKSPACE: return "workspace missing or too small";
        case EP_ERR_HIP: return "HIP kernel launch failed (see ep_last_hip_error)";
        case EP_ERR_SCRATCH_LIMIT:
            return "layout needs more scratch than the library's static array (EP_STATIC_SCRATCH_BYTES); "
                   "use ep_get_layout with a workspace";
        default: return "unknown error code";
    }
}

EP_API int ep_last_hip_error(void) { return g_last_hip_error; }

EP_API int ep_validate_config(const ep_config_t* cfg) { return validate(cfg); }

EP_API int ep_route(const ep_config_t* cfg, const float* logits, int32_t* topk_idx, float* topk_w,
                    void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!logits || !topk_idx || !topk_w)) return EP_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_route(shape_of(cfg), logits, topk_idx, topk_w,
                                       static_cast<hipStream_t>(stream)));
}

EP_API int ep_scores(const ep_config_t* cfg, const float* logits, float* scores, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!logits || !scores)) return EP_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(scores, 4)) return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_scores(shape_of(cfg), logits, scores, static_cast<hipStream_t>(stream)));
}

EP_API size_t ep_layout_workspace_bytes(const ep_config_t* cfg) {
    if (validate(cfg)) return 0;
    return ep::layout_workspace_bytes(shape_of(cfg));
}

EP_API int ep_get_layout(const ep_config_t* cfg, const int32_t* topk_idx, int32_t* cnt_expert,
                         int32_t* ntok_rank, int32_t* expert_offset, int32_t* slot, int32_t* recv_token,
                         void* workspace, size_t workspace_bytes, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!cnt_expert || !ntok_rank || !expert_offset) return EP_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (!topk_idx || !slot)) return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(cnt_expert, 4) || !aligned(ntok_rank, 4) ||
        !aligned(expert_offset, 4) || !aligned(slot, 4) || !aligned(recv_token, 4))
        return EP_ERR_ALIGNMENT;
    const ep::Shape s = shape_of(cfg);
    const size_t need = ep::layout_workspace_bytes(s);
    if (need > 0 && (!workspace || workspace_bytes < need)) return EP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_layout(s, topk_idx, cnt_expert, ntok_rank, expert_offset, slot, recv_token,
                                        workspace, static_cast<hipStream_t>(stream)));
}

// ep_route_layout takes the two-launch path (routing with column counts,
// then one assign launch) from more than 1024 pairs (below, the
// one-workgroup layout is faster) up to 256 columns of 16 tokens (beyond,
// every assign block would sum too many columns).  Measured per call on
// MI355X, back to back, 256 experts, top-8: 128 tokens 10.9 (separate) vs
// 12.3 us (two launches); 4096 tokens 15.1 vs 14.2 us; 16384 tokens 24.3
// vs 29.4 us.
constexpr long kFusedMinPairs = 1025;
constexpr int kFusedMaxColumns = 256;

// Workspace of ep_route_layout: the routing step's column histograms when
// the two-launch path applies, else the layout workspace.
size_t route_layout_ws(const ep::Shape& s, bool* fused) {
    *fused = (long)s.T * s.k >= kFusedMinPairs && ep::route_hist_columns(s) <= kFusedMaxColumns &&
             ep::route_hist_supported(s) && ep::layout_from_hist_supported(s);
    if (!*fused) return ep::layout_workspace_bytes(s);
    const size_t C = (size_t)ep::route_hist_columns(s);
    return ((C * s.E + 255) & ~(size_t)255) + ((C * s.R + 255) & ~(size_t)255);
}

EP_API size_t ep_route_layout_workspace_bytes(const ep_config_t* cfg) {
    if (validate(cfg)) return 0;
    bool fused;
    return route_layout_ws(shape_of(cfg), &fused);
}

EP_API int ep_route_layout(const ep_config_t* cfg, const float* logits, int32_t* topk_idx, float* topk_w,
                           int32_t* cnt_expert, int32_t* ntok_rank, int32_t* expert_offset, int32_t* slot,
                           int32_t* recv_token, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!cnt_expert || !ntok_rank || !expert_offset) return EP_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (!logits || !topk_idx || !topk_w || !slot)) return EP_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(cnt_expert, 4) ||
        !aligned(ntok_rank, 4) || !aligned(expert_offset, 4) || !aligned(slot, 4) || !aligned(recv_token, 4))
        return EP_ERR_ALIGNMENT;
    const ep::Shape s = shape_of(cfg);
    bool fused = false;
    const size_t need = route_layout_ws(s, &fused);
    if (need > 0 && (!workspace || workspace_bytes < need)) return EP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return EP_ERR_ALIGNMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!fused) {
        rc = hip_status(ep::launch_route(s, logits, topk_idx, topk_w, st));
        if (rc) return rc;
        return hip_status(ep::launch_layout(s, topk_idx, cnt_expert, ntok_rank, expert_offset, slot, recv_token,
                                            workspace, st));
    }
    const int C = ep::route_hist_columns(s);
    uint8_t* hist = static_cast<uint8_t*>(workspace);
    uint8_t* rank_hist = hist + (((size_t)C * s.E + 255) & ~(size_t)255);
    rc = hip_status(ep::launch_route_hist(s, logits, topk_idx, topk_w, hist, rank_hist, st));
    if (rc) return rc;
    return hip_status(ep::launch_layout_from_hist(s, topk_idx, hist, rank_hist, C, ep::route_hist_column_tokens(),
                                                  cnt_expert, ntok_rank, expert_offset, slot, recv_token, st));
}

EP_API int ep_get_layout_static(const ep_config_t* cfg, const int32_t* topk_idx, int32_t* cnt_expert,
                                int32_t* ntok_rank, int32_t* expert_offset, int32_t* slot, int32_t* recv_token,
                                void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!cnt_expert || !ntok_rank || !expert_offset) return EP_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (!topk_idx || !slot)) return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(cnt_expert, 4) || !aligned(ntok_rank, 4) ||
        !aligned(expert_offset, 4) || !aligned(slot, 4) || !aligned(recv_token, 4))
        return EP_ERR_ALIGNMENT;
    const ep::Shape s = shape_of(cfg);
    if (ep::layout_workspace_bytes(s) > EP_STATIC_SCRATCH_BYTES) return EP_ERR_SCRATCH_LIMIT;
    hipError_t e = hipSuccess;
    void* ws = static_scratch(&e);
    if (!ws) {
        (void)hipGetLastError();  // returned here, not left pending for the next call
        return hip_status(e);
    }
    return hip_status(ep::launch_layout(s, topk_idx, cnt_expert, ntok_rank, expert_offset, slot, recv_token, ws,
                                        static_cast<hipStream_t>(stream)));
}

EP_API int ep_dispatch(const ep_config_t* cfg, const void* x, const int32_t* slot, int recv_dtype, void* recv,
                       float* recv_scales, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (recv_dtype != EP_RECV_FP8_E4M3 && recv_dtype != EP_RECV_BF16) return EP_ERR_INVALID_ARG;
    const bool fp8 = recv_dtype == EP_RECV_FP8_E4M3;
    if (cfg->num_tokens > 0 && (!x || !slot || !recv || (fp8 && !recv_scales))) return EP_ERR_INVALID_ARG;
    if (!fp8 && recv_scales) return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16) || !aligned(slot, 4) || !aligned(recv_scales, 4))
        return EP_ERR_ALIGNMENT;
    const ep::Shape s = shape_of(cfg);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fp8)
        return hip_status(ep::launch_dispatch_fp8(s, static_cast<const uint16_t*>(x), slot,
                                                  static_cast<uint8_t*>(recv), recv_scales, st));
    return hip_status(ep::launch_dispatch_bf16(s, static_cast<const uint16_t*>(x), slot,
                                               static_cast<uint16_t*>(recv), st));
}

EP_API int ep_combine(const ep_config_t* cfg, const void* y, const int32_t* slot, const float* topk_w,
                      void* out, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!y || !slot || !topk_w || !out)) return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot, 4) || !aligned(topk_w, 4))
        return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_combine(shape_of(cfg), cfg->num_tokens * cfg->topk, static_cast<const uint16_t*>(y),
                                         slot, topk_w, static_cast<uint16_t*>(out),
                                         static_cast<hipStream_t>(stream)));
}

EP_API int ep_dispatch_ll(const ep_config_t* cfg, const void* x, const int32_t* topk_idx, int32_t capacity,
                          int recv_dtype, void* recv, float* recv_scales, int32_t* recv_count, int32_t* recv_src,
                          int32_t* slot, void* stream) {
    int rc = validate_ll(cfg, capacity);
    if (rc) return rc;
    if ((long)cfg->num_tokens * cfg->topk > ep::kMaxPairsLL) return EP_ERR_UNSUPPORTED;
    if (recv_dtype != EP_RECV_FP8_E4M3 && recv_dtype != EP_RECV_BF16) return EP_ERR_INVALID_ARG;
    const bool fp8 = recv_dtype == EP_RECV_FP8_E4M3;
    if (!recv_count) return EP_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (!x || !topk_idx || !recv || !recv_src || !slot || (fp8 && !recv_scales)))
        return EP_ERR_INVALID_ARG;
    if (!fp8 && recv_scales) return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16) || !aligned(topk_idx, 4) || !aligned(recv_scales, 4) ||
        !aligned(recv_count, 4) || !aligned(recv_src, 4) || !aligned(slot, 4))
        return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_dispatch_ll(shape_of(cfg), capacity, fp8, static_cast<const uint16_t*>(x), topk_idx,
                                             recv, recv_scales, recv_count, recv_src, slot,
                                             static_cast<hipStream_t>(stream)));
}

EP_API int ep_combine_ll(const ep_config_t* cfg, int32_t capacity, const void* y, const int32_t* slot,
                         const float* topk_w, void* out, void* stream) {
    int rc = validate_ll(cfg, capacity);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!y || !slot || !topk_w || !out)) return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot, 4) || !aligned(topk_w, 4))
        return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_combine(shape_of(cfg), cfg->num_experts * capacity,
                                         static_cast<const uint16_t*>(y), slot, topk_w,
                                         static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

EP_API size_t ep_rank_layout_workspace_bytes(const ep_config_t* cfg) {
    if (validate(cfg)) return 0;
    return ep::rank_layout_workspace_bytes(shape_of(cfg));
}

EP_API int ep_get_rank_layout(const ep_config_t* cfg, const int32_t* topk_idx, int32_t* rank_count,
                              int32_t* rank_offset, int32_t* rank_slot, int32_t* rank_token, void* workspace,
                              size_t workspace_bytes, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!rank_count || !rank_offset) return EP_ERR_INVALID_ARG;
    if (cfg->num_tokens > 0 && (!topk_idx || !rank_slot)) return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(rank_count, 4) || !aligned(rank_offset, 4) || !aligned(rank_slot, 4) ||
        !aligned(rank_token, 4))
        return EP_ERR_ALIGNMENT;
    const ep::Shape s = shape_of(cfg);
    const size_t need = ep::rank_layout_workspace_bytes(s);
    if (!workspace || workspace_bytes < need) return EP_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_rank_layout(s, topk_idx, rank_count, rank_offset, rank_slot, rank_token, workspace,
                                             static_cast<hipStream_t>(stream)));
}

EP_API int ep_combine_rank_partial(const ep_config_t* cfg, const void* y, const int32_t* topk_idx,
                                   const int32_t* slot, const float* topk_w, const int32_t* rank_slot,
                                   void* partial, void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!y || !topk_idx || !slot || !topk_w || !rank_slot || !partial))
        return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(partial, 16) || !aligned(topk_idx, 4) || !aligned(slot, 4) ||
        !aligned(topk_w, 4) || !aligned(rank_slot, 4))
        return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_combine_rank_partial(shape_of(cfg), static_cast<const uint16_t*>(y), topk_idx, slot,
                                                      topk_w, rank_slot, static_cast<uint16_t*>(partial),
                                                      static_cast<hipStream_t>(stream)));
}

EP_API int ep_combine_ranks(const ep_config_t* cfg, const void* partial, const int32_t* rank_slot, void* out,
                            void* stream) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (cfg->num_tokens > 0 && (!partial || !rank_slot || !out)) return EP_ERR_INVALID_ARG;
    if (!aligned(partial, 16) || !aligned(out, 16) || !aligned(rank_slot, 4)) return EP_ERR_ALIGNMENT;
    return hip_status(ep::launch_combine_ranks(shape_of(cfg), static_cast<const uint16_t*>(partial), rank_slot,
                                               static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

EP_API int ep_stream_create_cu_range(int first_cu, int num_cus, void** stream) {
    if (!stream || first_cu < 0 || num_cus < 1) return EP_ERR_INVALID_ARG;
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // the error is returned here, not left pending for the next call
        return hip_status(e);
    }
    if ((long)first_cu + num_cus > ncu) return EP_ERR_INVALID_ARG;
    uint32_t mask[64] = {0};  // up to 2048 CUs
    if (ncu > 64 * 32) return EP_ERR_UNSUPPORTED;
    for (int cu = first_cu; cu < first_cu + num_cus; ++cu) mask[cu >> 5] |= 1u << (cu & 31);
    hipStream_t st = nullptr;
    e = hipExtStreamCreateWithCUMask(&st, (uint32_t)((ncu + 31) / 32), mask);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_status(e);
    }
    *stream = st;
    return EP_OK;
}

EP_API int ep_stream_destroy(void* stream) {
    if (!stream) return EP_ERR_INVALID_ARG;
    const hipError_t e = hipStreamDestroy(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) (void)hipGetLastError();
    return hip_status(e);
}

}  // extern "C"
