// xp_static.hip — the two-call decode path (xp_route_gateup, then
// xp_down_combine) as one entry point that allocates nothing and takes no
// workspace: the routing plan lives in a fixed device array of this library.
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation). Each GPU holds its
// own copy of the array from module load until the process ends. The host
// never uses the array's name as a device address: on the first call on a
// device (that device current) hipGetSymbolAddress gives that device's
// address, which is kept per device and passed to the kernels as their
// workspace pointer. The routing kernels write every plan field the later
// kernels read, so nothing in the array has to start at zero.
#include <mutex>

#include "xp_common.h"

namespace xp {

constexpr size_t kStaticScratchBytes = size_t(1) << 20;  // 1 MiB: one plan
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per
// device), or nullptr if the runtime refuses.
static void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace xp

using namespace xp;

XP_API int xp_decode_static(const xp_dims* dims, int32_t rows, const float* logits, const uint16_t* x,
                            const xp_expert* experts, int32_t* topk_id, float* topk_w, float* act, float* out,
                            float* y, void* stream) {
    // every argument is checked before anything is enqueued
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!logits || !x || !experts || !topk_id || !topk_w || !act || !out || !y) return XP_ERR_NULL;
    if (ws_layout(dims, rows).total > kStaticScratchBytes) return XP_ERR_WORKSPACE;
    void* ws = scratch_on_current_device();
    if (!ws) return XP_ERR_HIP;
    st = xp_route_gateup(dims, rows, logits, x, experts, topk_id, topk_w, ws, kStaticScratchBytes, act, stream);
    if (st != XP_OK) return st;
    return xp_down_combine(dims, rows, act, experts, topk_w, ws, kStaticScratchBytes, out, y, stream);
}
