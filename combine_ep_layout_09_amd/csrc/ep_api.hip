// ep_api.hip -- the exported C ABI: argument checks on the host, then launches.
// Every check happens before anything is enqueued, so an error code other
// than EP_ERR_HIP means the stream was not touched.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ep.h"
#include "ep_internal.h"

// Device scratch of ep_layout_dispatch_noalloc: one copy per GPU (a file-scope
// __device__ array exists once in every device's memory), held until the
// process ends.  Host code never passes `scratch` itself to a kernel -- in
// host code the name stands for a host-side shadow, not a device address --
// but the pointer hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) int32_t scratch[ep::kMaxLayoutWorkspaceBytes / 4];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape checks shared by every entry point.
int check_problem(const ep_problem* p) {
    if (p == nullptr) return EP_ERR_ARG;
    if (p->num_tokens < 0 || p->hidden < 1 || p->num_topk < 1 || p->num_experts < 1 ||
        p->capacity < 0 || p->use_fp8 < 0 || p->use_fp8 > 2)
        return EP_ERR_ARG;
    if (p->num_experts > ep::kMaxExperts || p->num_topk > ep::kMaxTopk ||
        p->hidden > ep::kMaxHidden || p->hidden % 8 != 0 ||
        (p->use_fp8 && p->hidden % 128 != 0))
        return EP_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(p->num_tokens) * p->num_topk >= (int64_t{1} << 31) ||
        static_cast<int64_t>(p->num_experts) * p->capacity >= (int64_t{1} << 31))
        return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

int64_t recv_rows(const ep_problem& p) {
    return p.capacity == 0 ? static_cast<int64_t>(p.num_tokens) * p.num_topk
                           : static_cast<int64_t>(p.num_experts) * p.capacity;
}

int check_layout_ptrs(const ep_problem& p, const ep_layout_t* lay, bool all) {
    if (lay == nullptr) return EP_ERR_ARG;
    const bool need_slots = static_cast<int64_t>(p.num_tokens) * p.num_topk > 0;
    if (need_slots && lay->slot_of == nullptr) return EP_ERR_ARG;
    if (!aligned4(lay->slot_of)) return EP_ERR_ALIGN;
    if (all) {
        if (lay->count == nullptr || lay->offset == nullptr || lay->status == nullptr)
            return EP_ERR_ARG;
        if (recv_rows(p) > 0 && lay->src_of_slot == nullptr) return EP_ERR_ARG;
        if (!aligned4(lay->count) || !aligned4(lay->offset) || !aligned4(lay->status) ||
            !aligned4(lay->src_of_slot))
            return EP_ERR_ALIGN;
    }
    return EP_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

// Arguments of ep_layout_dispatch apart from the workspace.
int check_layout_dispatch_args(const ep_problem* prob, const int32_t* topk_idx,
                               const ep_layout_t* out, const void* x, void* recv_x,
                               void* recv_scales) {
    int rc = check_problem(prob);
    if (rc != EP_OK) return rc;
    rc = check_layout_ptrs(*prob, out, true);
    if (rc != EP_OK) return rc;
    if (static_cast<int64_t>(prob->num_tokens) * prob->num_topk > 0 && topk_idx == nullptr)
        return EP_ERR_ARG;
    if (!aligned16(topk_idx)) return EP_ERR_ALIGN;
    if (prob->num_tokens > 0) {
        if (x == nullptr || recv_x == nullptr) return EP_ERR_ARG;
        if (prob->use_fp8 && recv_scales == nullptr) return EP_ERR_ARG;
    }
    if (!aligned16(x) || !aligned16(recv_x) || (prob->use_fp8 && !aligned16(recv_scales)))
        return EP_ERR_ALIGN;
    return EP_OK;
}

}  // namespace

extern "C" {

int64_t ep_num_recv_rows(const ep_problem* prob) {
    if (check_problem(prob) != EP_OK) return -1;
    return recv_rows(*prob);
}

int64_t ep_layout_workspace_bytes(const ep_problem* prob) {
    if (check_problem(prob) != EP_OK) return -1;
    return ep::layout_workspace_bytes(*prob);
}

int ep_layout(const ep_problem* prob, const int32_t* topk_idx, const ep_layout_t* out,
              void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_problem(prob);
    if (rc != EP_OK) return rc;
    rc = check_layout_ptrs(*prob, out, true);
    if (rc != EP_OK) return rc;
    if (static_cast<int64_t>(prob->num_tokens) * prob->num_topk > 0 && topk_idx == nullptr)
        return EP_ERR_ARG;
    if (!aligned16(topk_idx)) return EP_ERR_ALIGN;
    if (workspace == nullptr ||
        static_cast<int64_t>(workspace_bytes) < ep::layout_workspace_bytes(*prob))
        return EP_ERR_ARG;
    if (!aligned16(workspace)) return EP_ERR_ALIGN;
    return from_hip(ep::launch_layout(*prob, topk_idx, *out, static_cast<int32_t*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

int ep_dispatch(const ep_problem* prob, const void* x, const ep_layout_t* layout, void* recv_x,
                void* recv_scales, void* stream) {
    int rc = check_problem(prob);
    if (rc != EP_OK) return rc;
    rc = check_layout_ptrs(*prob, layout, false);
    if (rc != EP_OK) return rc;
    if (prob->num_tokens > 0) {
        if (x == nullptr || recv_x == nullptr) return EP_ERR_ARG;
        if (prob->use_fp8 && recv_scales == nullptr) return EP_ERR_ARG;
    }
    if (!aligned16(x) || !aligned16(recv_x) || (prob->use_fp8 && !aligned16(recv_scales)))
        return EP_ERR_ALIGN;
    return from_hip(ep::launch_dispatch(*prob, x, layout->slot_of, recv_x,
                                        prob->use_fp8 ? recv_scales : nullptr,
                                        static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch(const ep_problem* prob, const int32_t* topk_idx, const ep_layout_t* out,
                       void* workspace, size_t workspace_bytes, const void* x, void* recv_x,
                       void* recv_scales, void* stream) {
    int rc = check_layout_dispatch_args(prob, topk_idx, out, x, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    if (workspace == nullptr ||
        static_cast<int64_t>(workspace_bytes) < ep::layout_workspace_bytes(*prob))
        return EP_ERR_ARG;
    if (!aligned16(workspace)) return EP_ERR_ALIGN;
    return from_hip(ep::launch_layout_dispatch(*prob, topk_idx, *out, workspace, x, recv_x,
                                               prob->use_fp8 ? recv_scales : nullptr,
                                               static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch_noalloc(const ep_problem* prob, const int32_t* topk_idx,
                               const ep_layout_t* out, const void* x, void* recv_x,
                               void* recv_scales, void* stream) {
    int rc = check_layout_dispatch_args(prob, topk_idx, out, x, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    if (ep::layout_workspace_bytes(*prob) > ep::kMaxLayoutWorkspaceBytes) return EP_ERR_UNSUPPORTED;
    void* ws = nullptr;
    const hipError_t err = scratch_address(&ws);
    if (err != hipSuccess) return EP_ERR_HIP;
    // The workspace needs no initialisation (the histogram kernel writes every
    // word it later reads), so the array's previous contents do not matter.
    return from_hip(ep::launch_layout_dispatch(*prob, topk_idx, *out, ws, x, recv_x,
                                               prob->use_fp8 ? recv_scales : nullptr,
                                               static_cast<hipStream_t>(stream)));
}

static_assert(EP_NOALLOC_SCRATCH_BYTES == ep::kMaxLayoutWorkspaceBytes,
              "ep.h states the size of the allocation-free entry point's device array");

int ep_combine(const ep_problem* prob, const void* expert_out, const ep_layout_t* layout,
               const float* topk_weights, void* y, void* stream) {
    int rc = check_problem(prob);
    if (rc != EP_OK) return rc;
    rc = check_layout_ptrs(*prob, layout, false);
    if (rc != EP_OK) return rc;
    if (prob->num_tokens > 0 && (expert_out == nullptr || topk_weights == nullptr || y == nullptr))
        return EP_ERR_ARG;
    if (!aligned16(expert_out) || !aligned16(y) || !aligned4(topk_weights)) return EP_ERR_ALIGN;
    return from_hip(ep::launch_combine(*prob, expert_out, layout->slot_of, topk_weights, y,
                                       static_cast<hipStream_t>(stream)));
}

int ep_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0) return EP_ERR_ARG;
    if (n > 0 && (in == nullptr || out == nullptr)) return EP_ERR_ARG;
    if (!aligned4(in)) return EP_ERR_ALIGN;
    return from_hip(ep::launch_e4m3_encode(in, out, n, static_cast<hipStream_t>(stream)));
}

const char* ep_strerror(int code) {
    switch (code) {
        case EP_OK: return "ok";
        case EP_ERR_ARG: return "invalid argument (size, null pointer or workspace too small)";
        case EP_ERR_UNSUPPORTED: return "problem size outside the supported envelope";
        case EP_ERR_ALIGN: return "pointer not aligned (data 16 bytes, int32/fp32 arrays 4 bytes)";
        case EP_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status code";
    }
}

}  // extern "C"
