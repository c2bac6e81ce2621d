// mmq_api.hip -- the C ABI declared in include/mmq.h.
//
// Launch protocol ("13 . r7-r8 raw-byte MMQ kernel", sections 3.3 and 6):
// every entry point returns 1 when the kernel was enqueued and 0 when it was
// refused; a refusal is decided before any device work (so no output byte is
// written), printed to stderr and kept in a thread-local string; launch
// errors are read back with hipGetLastError() and reported the same way.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/mmq.h"
#include "mmq_plan.hpp"

static_assert(mmq::kNoAllocMaxRouted == MMQ_MOE_NOALLOC_MAX_ROUTED, "header and library disagree");

namespace mmq {
hipError_t launch_quantize(const float *x, void *y, int64_t M, int64_t K, int cu_count, hipStream_t stream);
hipError_t launch_gemm(const Plan &p, const int *tile_start, int count, const void *x, const void *const *w,
                       void *const *out, const int64_t *N, int64_t M, int64_t K, bool dots, void *workspace,
                       hipStream_t stream);
hipError_t launch_moe(const Plan &p, const void *x, const void *w, const int32_t *ids, int topk, int n_experts,
                      float *out, int64_t T, int64_t N, int64_t K, void *workspace, hipStream_t stream);
const void *plan_kernel(const Plan &p, bool dots, bool moe);
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_pack_q8_0(const void *w, int64_t N, int64_t K, void *packed, int cu_count, hipStream_t stream);
}  // namespace mmq

namespace {

thread_local char g_err[512] = "";
std::atomic<int64_t> g_extra_lds{0};

int refuse(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "mmq: refused: %s\n", g_err);
    return 0;
}

struct DeviceLimits {
    bool valid = false;
    bool is_gfx950 = false;
    int64_t lds_per_block = 0;
    int cu_count = 0;
    char arch[64] = "";
};

constexpr int kMaxDevices = 64;
DeviceLimits g_limits[kMaxDevices];
std::mutex g_limits_mu;

// Current device's limits (cached per device). Returns false and sets the
// error when there is no usable device.
bool current_limits(DeviceLimits *out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        refuse("no HIP device available");
        return false;
    }
    std::lock_guard<std::mutex> lock(g_limits_mu);
    DeviceLimits &L = g_limits[dev];
    if (!L.valid) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            refuse("hipGetDeviceProperties failed for device %d", dev);
            return false;
        }
        int lds = 0, cus = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            refuse("hipDeviceGetAttribute failed for device %d", dev);
            return false;
        }
        std::snprintf(L.arch, sizeof(L.arch), "%s", prop.gcnArchName);
        L.is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        L.lds_per_block = lds;
        L.cu_count = cus;
        L.valid = true;
    }
    *out = L;
    return true;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Registers and scratch of a kernel on the current device
// (hipFuncGetAttributes), cached per (device, kernel).
std::mutex g_fit_mu;
std::map<std::pair<int, const void *>, mmq::KernelFit> g_fit;

bool kernel_fit(const void *fn, mmq::KernelFit *fit) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        refuse("no HIP device available");
        return false;
    }
    const auto key = std::make_pair(dev, fn);
    std::lock_guard<std::mutex> lock(g_fit_mu);
    auto it = g_fit.find(key);
    if (it == g_fit.end()) {
        hipFuncAttributes a;
        if (hipFuncGetAttributes(&a, fn) != hipSuccess) {
            (void)hipGetLastError();
            refuse("hipFuncGetAttributes failed for a kernel on device %d", dev);
            return false;
        }
        mmq::KernelFit f;
        f.vgprs = a.numRegs;
        f.scratch = int64_t(a.localSizeBytes);
        it = g_fit.emplace(key, f).first;
    }
    *fit = it->second;
    return true;
}

// Plan with the nominal kernel, read the attributes of the kernel that plan
// launches, and plan again with them (the kernel choice depends on the
// shape only, so the second plan launches the same kernel).
template <typename MakePlan>
bool plan_with_kernel_fit(MakePlan make, bool dots, bool moe, mmq::Plan *p, char *why, size_t why_len) {
    if (!make(mmq::KernelFit(), p, why, why_len)) return false;
    mmq::KernelFit fit;
    if (!kernel_fit(mmq::plan_kernel(*p, dots, moe), &fit)) {
        std::snprintf(why, why_len, "%s", g_err);
        return false;
    }
    return make(fit, p, why, why_len);
}

// Plan a GEMM set on the current device (with the launched kernel's
// attributes); `workspace`: plan for a split-K workspace; `packed`: Q8_0
// weights in the tile-packed form, which only the tile kernel reads.
bool plan_set(int fmt, int count, const int64_t *N, int64_t M, int64_t K, bool dots, bool workspace,
              const DeviceLimits &L, mmq::Plan *p, int *tile_start, char *why, size_t why_len, bool packed = false) {
    auto make = [&](const mmq::KernelFit &fit, mmq::Plan *q, char *w, size_t wl) {
        if (!mmq::make_plan_multi(fmt, M, count, N, K, L.lds_per_block, L.cu_count, g_extra_lds.load(), q,
                                  tile_start, w, wl, !dots && !packed, fit, workspace))
            return false;
        q->packed = packed;
        return true;
    };
    return plan_with_kernel_fit(make, dots, false, p, why, why_len);
}

// `workspace`: null, or `workspace_bytes` bytes of device memory for a
// split-K plan (mmq_gemm_multi_ws).
int gemm_set(int fmt, const void *x, int count, const void *const *w, void *const *out, const int64_t *N,
             int64_t M, int64_t K, bool dots, void *workspace, int64_t workspace_bytes, void *stream,
             bool packed = false) {
    g_err[0] = '\0';
    if (!mmq::fmt_ok(fmt)) return refuse("unknown weight format %d", fmt);
    if (count < 1 || count > mmq::kMaxGemms) return refuse("count must be 1..%d GEMMs", mmq::kMaxGemms);
    if (!x || !w || !out || !N) return refuse("null pointer argument");
    if (workspace && !aligned(workspace, 16)) return refuse("workspace must be 16-byte aligned");
    if (workspace && workspace_bytes < 0) return refuse("workspace_bytes must be >= 0");
    if (!aligned(x, 16)) return refuse("activation and weight pointers must be 16-byte aligned");
    for (int g = 0; g < count; g++) {
        if (!w[g] || !out[g]) return refuse("null pointer argument");
        if (!aligned(w[g], 16)) return refuse("activation and weight pointers must be 16-byte aligned");
        if (!aligned(out[g], 4)) return refuse("output pointer must be 4-byte aligned");
    }
    DeviceLimits L;
    if (!current_limits(&L)) return 0;
    if (!L.is_gfx950) return refuse("device is %s; this library is built for gfx950 only", L.arch);
    mmq::Plan p;
    int tile_start[mmq::kMaxGemms + 1];
    char why[256];
    // the block-dot output exists for the MMQ kernel only (planned without
    // a workspace: it never splits)
    if (!plan_set(fmt, count, N, M, K, dots, workspace != nullptr && !dots, L, &p, tile_start, why, sizeof(why),
                  packed))
        return refuse("%s%s GEMM M=%lld N=%lld K=%lld%s: %s", mmq::fmt_name(fmt), packed ? " (packed)" : "",
                      (long long)M, (long long)N[0], (long long)K, count > 1 ? " (first of a set)" : "", why);
    const int64_t need = mmq::split_workspace_bytes(p);
    if (need > workspace_bytes)
        return refuse("%s GEMM M=%lld N=%lld K=%lld: the split-K workspace holds %lld bytes, the plan needs %lld",
                      mmq::fmt_name(fmt), (long long)M, (long long)N[0], (long long)K, (long long)workspace_bytes,
                      (long long)need);
    (void)hipGetLastError();   // a stale error must not be blamed on this launch
    const hipError_t e = mmq::launch_gemm(p, tile_start, count, x, w, out, N, M, K, dots, workspace,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return refuse("%s GEMM launch failed: %s", mmq::fmt_name(fmt), hipGetErrorString(e));
    return 1;
}

int gemm_common(int fmt, const void *x, const void *w, void *out, int64_t M, int64_t N, int64_t K,
                bool dots, void *stream) {
    return gemm_set(fmt, x, 1, &w, &out, &N, M, K, dots, nullptr, 0, stream);
}

}  // namespace

extern "C" {

int mmq_quantize_q8_1(const float *x, void *y, int64_t M, int64_t K, void *stream) {
    g_err[0] = '\0';
    if (!x || !y) return refuse("null pointer argument");
    if (!aligned(x, 16) || !aligned(y, 16)) return refuse("x and y must be 16-byte aligned");
    if (const char *bad = mmq::check_quantize_shape(M, K))
        return refuse("quantize M=%lld K=%lld: %s", (long long)M, (long long)K, bad);
    DeviceLimits L;
    if (!current_limits(&L)) return 0;
    if (!L.is_gfx950) return refuse("device is %s; this library is built for gfx950 only", L.arch);
    (void)hipGetLastError();
    const hipError_t e = mmq::launch_quantize(x, y, M, K, L.cu_count, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return refuse("quantize launch failed: %s", hipGetErrorString(e));
    return 1;
}

int mmq_gemm_q8_0(const void *x_q8_1, const void *w_q8_0, float *out, int64_t M, int64_t N, int64_t K,
                  void *stream) {
    return gemm_common(mmq::FMT_Q8_0, x_q8_1, w_q8_0, out, M, N, K, false, stream);
}

int64_t mmq_packed_bytes_q8_0(int64_t N, int64_t K) {
    g_err[0] = '\0';
    const int64_t b = mmq::packed_bytes_q8_0(N, K);
    if (b < 0)
        refuse("packed Q8_0 N=%lld K=%lld: N must be 1..2^31-1 and K a multiple of 32 in 32..8388608", (long long)N,
               (long long)K);
    return b;
}

int mmq_pack_q8_0(const void *w_q8_0, int64_t N, int64_t K, void *packed, int64_t packed_bytes, void *stream) {
    g_err[0] = '\0';
    if (!w_q8_0 || !packed) return refuse("null pointer argument");
    if (!aligned(w_q8_0, 16) || !aligned(packed, 16)) return refuse("weight and packed pointers must be 16-byte aligned");
    const int64_t need = mmq::packed_bytes_q8_0(N, K);
    if (need < 0)
        return refuse("pack Q8_0 N=%lld K=%lld: N must be 1..2^31-1 and K a multiple of 32 in 32..8388608",
                      (long long)N, (long long)K);
    if (packed_bytes < need)
        return refuse("pack Q8_0 N=%lld K=%lld: the packed buffer holds %lld bytes, the packed form needs %lld",
                      (long long)N, (long long)K, (long long)packed_bytes, (long long)need);
    DeviceLimits L;
    if (!current_limits(&L)) return 0;
    if (!L.is_gfx950) return refuse("device is %s; this library is built for gfx950 only", L.arch);
    (void)hipGetLastError();
    const hipError_t e = mmq::launch_pack_q8_0(w_q8_0, N, K, packed, L.cu_count, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return refuse("pack launch failed: %s", hipGetErrorString(e));
    return 1;
}

int mmq_gemm_q8_0_packed(const void *x_q8_1, const void *w_packed, float *out, int64_t M, int64_t N, int64_t K,
                         void *stream) {
    void *o = out;
    return gemm_set(mmq::FMT_Q8_0, x_q8_1, 1, &w_packed, &o, &N, M, K, false, nullptr, 0, stream, true);
}

int mmq_gemm_q4_K(const void *x_q8_1, const void *w_q4_K, float *out, int64_t M, int64_t N, int64_t K,
                  void *stream) {
    return gemm_common(mmq::FMT_Q4_K, x_q8_1, w_q4_K, out, M, N, K, false, stream);
}

int mmq_gemm_q5_K(const void *x_q8_1, const void *w_q5_K, float *out, int64_t M, int64_t N, int64_t K,
                  void *stream) {
    return gemm_common(mmq::FMT_Q5_K, x_q8_1, w_q5_K, out, M, N, K, false, stream);
}

int mmq_gemm_q6_K(const void *x_q8_1, const void *w_q6_K, float *out, int64_t M, int64_t N, int64_t K,
                  void *stream) {
    return gemm_common(mmq::FMT_Q6_K, x_q8_1, w_q6_K, out, M, N, K, false, stream);
}

int mmq_gemm_multi(int fmt, const void *x_q8_1, int count, const void *const *w, float *const *out,
                   const int64_t *N, int64_t M, int64_t K, void *stream) {
    return gemm_set(fmt, x_q8_1, count, w, reinterpret_cast<void *const *>(out), N, M, K, false, nullptr, 0,
                    stream);
}

int64_t mmq_gemm_workspace_bytes(int fmt, int count, const int64_t *N, int64_t M, int64_t K) {
    g_err[0] = '\0';
    if (!mmq::fmt_ok(fmt)) return refuse("unknown weight format %d", fmt), -1;
    if (count < 1 || count > mmq::kMaxGemms) return refuse("count must be 1..%d GEMMs", mmq::kMaxGemms), -1;
    if (!N) return refuse("null pointer argument"), -1;
    DeviceLimits L;
    if (!current_limits(&L)) return -1;
    mmq::Plan p;
    int tile_start[mmq::kMaxGemms + 1];
    char why[256];
    if (!plan_set(fmt, count, N, M, K, false, true, L, &p, tile_start, why, sizeof(why)))
        return refuse("%s GEMM M=%lld N=%lld K=%lld: %s", mmq::fmt_name(fmt), (long long)M, (long long)N[0],
                      (long long)K, why), -1;
    return mmq::split_workspace_bytes(p);
}

int mmq_gemm_multi_ws(int fmt, const void *x_q8_1, int count, const void *const *w, float *const *out,
                      const int64_t *N, int64_t M, int64_t K, void *workspace, int64_t workspace_bytes,
                      void *stream) {
    return gemm_set(fmt, x_q8_1, count, w, reinterpret_cast<void *const *>(out), N, M, K, false, workspace,
                    workspace_bytes, stream);
}

int64_t mmq_moe_workspace_bytes(int64_t T, int topk, int n_experts) {
    if (T < 0 || topk < 1 || topk > mmq::kMoeMaxTopk || n_experts < 1 || n_experts > mmq::kMoeMaxExperts ||
        T > INT32_MAX / topk)
        return -1;
    return mmq::moe_workspace_bytes(T * topk, n_experts);
}

}  // extern "C"

namespace {

// Which routing each MoE workspace holds: (device, workspace) -> (routed
// rows, experts) of the last mmq_moe_gemm enqueued with it.  A routed call
// is refused on the host unless its sizes match, so it never launches over
// tables built for other sizes (or never built).  The GEMM kernel keeps its
// own check of the header the routing kernel writes, for a workspace whose
// contents the caller changed after routing.  At most kMaxRoutes
// workspaces are remembered (the oldest is forgotten first; a routed call
// on a forgotten workspace is refused, never run on stale tables).
constexpr size_t kMaxRoutes = 1024;
std::mutex g_routes_mu;
std::map<std::pair<int, const void *>, std::pair<int64_t, int>> g_routes;
std::deque<std::pair<int, const void *>> g_route_order;

void record_route(const void *workspace, int64_t R, int E) {
    int dev = -1;
    (void)hipGetDevice(&dev);
    const auto key = std::make_pair(dev, workspace);
    std::lock_guard<std::mutex> lock(g_routes_mu);
    if (g_routes.find(key) == g_routes.end()) {
        g_route_order.push_back(key);
        if (g_route_order.size() > kMaxRoutes) {
            g_routes.erase(g_route_order.front());
            g_route_order.pop_front();
        }
    }
    g_routes[key] = std::make_pair(R, E);
}

// Returns nullptr when `workspace` holds a routing of R rows and E experts.
const char *route_mismatch(const void *workspace, int64_t R, int E, char *buf, size_t len) {
    int dev = -1;
    (void)hipGetDevice(&dev);
    std::lock_guard<std::mutex> lock(g_routes_mu);
    const auto it = g_routes.find(std::make_pair(dev, workspace));
    if (it == g_routes.end()) return "the workspace holds no routing from mmq_moe_gemm on this device";
    if (it->second.first != R || it->second.second != E) {
        std::snprintf(buf, len, "the workspace was routed for %lld rows and %d experts, not %lld and %d",
                      (long long)it->second.first, it->second.second, (long long)R, E);
        return buf;
    }
    return nullptr;
}

int moe_common(int fmt, const void *x_q8_1, const void *w, int n_experts, const int32_t *ids, int topk, float *out,
               int64_t T, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream,
               const char *name, bool record = true) {
    g_err[0] = '\0';
    if (!mmq::fmt_ok(fmt)) return refuse("unknown weight format %d", fmt);
    if (!x_q8_1 || !w || !out || !workspace) return refuse("null pointer argument");
    if (!aligned(x_q8_1, 16) || !aligned(w, 16)) return refuse("activation and weight pointers must be 16-byte aligned");
    if (!aligned(ids, 4) || !aligned(out, 4)) return refuse("ids and output pointers must be 4-byte aligned");
    if (!aligned(workspace, 16)) return refuse("workspace must be 16-byte aligned");
    DeviceLimits L;
    if (!current_limits(&L)) return 0;
    if (!L.is_gfx950) return refuse("device is %s; this library is built for gfx950 only", L.arch);
    mmq::Plan p;
    char why[256];
    auto make = [&](const mmq::KernelFit &fit, mmq::Plan *q, char *w, size_t wl) {
        return mmq::make_plan_moe(fmt, T, topk, n_experts, N, K, L.lds_per_block, L.cu_count, g_extra_lds.load(), q,
                                  w, wl, fit);
    };
    if (!plan_with_kernel_fit(make, false, true, &p, why, sizeof(why)))
        return refuse("%s %s T=%lld topk=%d E=%d N=%lld K=%lld: %s", mmq::fmt_name(fmt), name, (long long)T, topk,
                      n_experts, (long long)N, (long long)K, why);
    const int64_t need = mmq::moe_workspace_bytes(T * topk, n_experts);
    if (workspace_bytes < need)
        return refuse("MoE workspace of %lld B given, %lld B needed", (long long)workspace_bytes, (long long)need);
    if (!ids) {
        char buf[160];
        if (const char *bad = route_mismatch(workspace, T * topk, n_experts, buf, sizeof(buf)))
            return refuse("%s %s T=%lld topk=%d E=%d: %s", mmq::fmt_name(fmt), name, (long long)T, topk, n_experts,
                          bad);
    }
    (void)hipGetLastError();
    const hipError_t e = mmq::launch_moe(p, x_q8_1, w, ids, topk, n_experts, out, T, N, K, workspace,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return refuse("%s %s launch failed: %s", mmq::fmt_name(fmt), name, hipGetErrorString(e));
    if (ids && record) record_route(workspace, T * topk, n_experts);
    return 1;
}

}  // namespace

extern "C" {

int mmq_moe_gemm(int fmt, const void *x_q8_1, const void *w, int n_experts, const int32_t *ids, int topk,
                 float *out, int64_t T, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes,
                 void *stream) {
    if (!ids) {
        g_err[0] = '\0';
        return refuse("null pointer argument");
    }
    return moe_common(fmt, x_q8_1, w, n_experts, ids, topk, out, T, N, K, workspace, workspace_bytes, stream,
                      "MoE GEMM");
}

int mmq_moe_gemm_routed(int fmt, const void *x_q8_1, const void *w, int n_experts, int topk, float *out,
                        int64_t T, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream) {
    return moe_common(fmt, x_q8_1, w, n_experts, nullptr, topk, out, T, N, K, workspace, workspace_bytes, stream,
                      "MoE GEMM (reused routing)");
}

int mmq_moe_gemm_noalloc(int fmt, const void *x_q8_1, const void *w, int n_experts, const int32_t *ids, int topk,
                         float *out, int64_t T, int64_t N, int64_t K, void *stream) {
    g_err[0] = '\0';
    if (!ids) return refuse("null pointer argument");
    if (topk >= 1 && T > mmq::kNoAllocMaxRouted / topk)
        return refuse("MoE GEMM (no allocation): T*topk = %lld routed rows exceeds the static scratch's limit of %lld",
                      (long long)T * topk, (long long)mmq::kNoAllocMaxRouted);
    void *scratch = nullptr;
    const hipError_t e = mmq::noalloc_scratch(&scratch);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return refuse("MoE GEMM (no allocation): device address of the static scratch: %s", hipGetErrorString(e));
    }
    // the scratch's tables are never offered to mmq_moe_gemm_routed (its
    // address is not the caller's), so the routing is not recorded
    return moe_common(fmt, x_q8_1, w, n_experts, ids, topk, out, T, N, K, scratch, mmq::kNoAllocScratchBytes, stream,
                      "MoE GEMM (no allocation)", false);
}

int mmq_debug_block_dots(int fmt, const void *x_q8_1, const void *w, int32_t *dots, int64_t M, int64_t N,
                         int64_t K, void *stream) {
    return gemm_common(fmt, x_q8_1, w, dots, M, N, K, true, stream);
}

const char *mmq_last_error(void) { return g_err; }

int mmq_plan_for_limits(int fmt, int64_t M, int64_t N, int64_t K, int64_t lds_limit_bytes, int cu_count,
                        int kernel_vgprs, int64_t kernel_scratch_bytes, char *buf, int64_t len) {
    mmq::Plan p;
    char why[256];
    mmq::KernelFit fit;
    if (kernel_vgprs > 0) fit.vgprs = kernel_vgprs;
    fit.scratch = kernel_scratch_bytes;
    const bool ok = mmq::make_plan(fmt, M, N, K, lds_limit_bytes, cu_count, g_extra_lds.load(), &p, why,
                                   sizeof(why), true, fit);
    mmq::Plan pw;
    const bool okw = ok && mmq::make_plan(fmt, M, N, K, lds_limit_bytes, cu_count, g_extra_lds.load(), &pw,
                                          nullptr, 0, true, fit, true);
    if (buf && len > 0) {
        if (ok)
            mmq::describe(p, okw ? &pw : nullptr, buf, size_t(len));
        else
            std::snprintf(buf, size_t(len), "%s", why);
    }
    return ok ? 1 : 0;
}

int mmq_plan_describe(int fmt, int64_t M, int64_t N, int64_t K, char *buf, int64_t len) {
    DeviceLimits L;
    if (!current_limits(&L)) {
        if (buf && len > 0) std::snprintf(buf, size_t(len), "%s", g_err);
        return 0;
    }
    mmq::Plan p, pw;
    char why[256];
    int tile_start[mmq::kMaxGemms + 1];
    const bool ok = mmq::fmt_ok(fmt) && plan_set(fmt, 1, &N, M, K, false, false, L, &p, tile_start, why, sizeof(why));
    if (!mmq::fmt_ok(fmt)) std::snprintf(why, sizeof(why), "unknown weight format");
    char why2[256];
    const bool okw = ok && plan_set(fmt, 1, &N, M, K, false, true, L, &pw, tile_start, why2, sizeof(why2));
    if (buf && len > 0) {
        if (ok)
            mmq::describe(p, okw ? &pw : nullptr, buf, size_t(len));
        else
            std::snprintf(buf, size_t(len), "%s", why);
    }
    return ok ? 1 : 0;
}

void mmq_debug_set_extra_lds(int64_t extra_bytes) { g_extra_lds.store(extra_bytes < 0 ? 0 : extra_bytes); }

const char *mmq_version(void) { return "mmq-gfx950 0.1"; }

}  // extern "C"
