// xp_route.hip — routing (top-k + softmax), stable bucketing and pass plans:
// the kernels behind xp_route_bucket, plus the pass-size setting. Up to 64 rows
// run as one workgroup; larger batches run three kernels (masks per block,
// counts and passes, scatter). The device routines are in xp_route_dev.h.
#include <string.h>

#include "xp_route_dev.h"

namespace xp {

constexpr uint32_t kDefaultGu = (1u << 2) | (1u << 4) | (1u << 6) | (1u << 8);
constexpr uint32_t kDefaultDn = (1u << 2) | (1u << 4);
static Tiers g_tiers = {kDefaultGu, kDefaultDn};

Tiers current_tiers() { return g_tiers; }

// ---- up to 64 rows: one workgroup of 1024 threads does everything
__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ logits, int R, int E, int k,
                                                           int32_t* __restrict__ topk_id,
                                                           float* __restrict__ topk_w, WsPtrs w, Tiers T) {
    __shared__ unsigned long long smask[kMaxExperts];
    __shared__ int32_t sid[kSmallRows][kMaxTopK];
    __shared__ int32_t scnt[kMaxExperts];
    __shared__ int32_t soff[kMaxExperts + 1];
    __shared__ int wsum[48];
    for (int e = threadIdx.x; e < E; e += blockDim.x) smask[e] = 0ull;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int r = wave; r < R; r += 16) topk_row(logits, E, k, r, r, topk_id, topk_w, sid[r], smask);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) scnt[e] = __popcll(smask[e]);
    __syncthreads();
    plan_block(E, scnt, T, soff, w.gu_pass, w.dn_pass, w.count, w.offset, w.hdr, nullptr, wsum);
    __syncthreads();
    const int t = threadIdx.x;
    if (t < R * k) {
        const int r = t / k, j = t - r * k;
        const int e = sid[r][j];
        const unsigned long long below = (r == 0) ? 0ull : (smask[e] & ((1ull << r) - 1ull));
        w.entry[soff[e] + __popcll(below)] = t;
    }
}

// ---- more rows: (1) top-k and masks per 64-row block
__global__ __launch_bounds__(1024) void route_blocks_kernel(const float* __restrict__ logits, int R, int E, int k,
                                                            int32_t* __restrict__ topk_id,
                                                            float* __restrict__ topk_w, WsPtrs w) {
    __shared__ unsigned long long smask[kMaxExperts];
    __shared__ int32_t sid[kSmallRows][kMaxTopK];
    for (int e = threadIdx.x; e < E; e += blockDim.x) smask[e] = 0ull;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.x;
    for (int rl = wave; rl < kSmallRows; rl += 16) {
        const int r = b * kSmallRows + rl;
        if (r < R) topk_row(logits, E, k, r, rl, topk_id, topk_w, sid[rl], smask);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) w.masks[(size_t)b * E + e] = smask[e];
}

// (2) counts per expert, per-block bases, offsets and passes (one workgroup)
__global__ __launch_bounds__(1024) void route_plan_kernel(int E, int nblk, WsPtrs w, Tiers T) {
    __shared__ int32_t scnt[kMaxExperts];
    __shared__ int32_t soff[kMaxExperts + 1];
    __shared__ int wsum[48];
    const int e = threadIdx.x;
    if (e < E) {
        // the blocks' masks sixteen at a time (all loads in flight together),
        // then their running counts
        constexpr int kB = 16;
        const unsigned long long* __restrict__ mk = w.masks + e;
        int32_t* __restrict__ bs = w.base + e;
        int c = 0;
        for (int b0 = 0; b0 < nblk; b0 += kB) {
            int pc[kB];
#pragma unroll
            for (int i = 0; i < kB; ++i) pc[i] = __popcll(mk[(size_t)min(b0 + i, nblk - 1) * E]);
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                if (b0 + i < nblk) {
                    bs[(size_t)(b0 + i) * E] = c;
                    c += pc[i];
                }
            }
        }
        scnt[e] = c;
    }
    __syncthreads();
    plan_block(E, scnt, T, soff, w.gu_pass, w.dn_pass, w.count, w.offset, w.hdr, nullptr, wsum);
}

// (3) scatter entries
__global__ __launch_bounds__(1024) void route_scatter_kernel(int R, int E, int k, const int32_t* __restrict__ topk_id,
                                                             WsPtrs w) {
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    if (t >= kSmallRows * k) return;
    int rl = t / k, j = t - rl * k;
    int r = b * kSmallRows + rl;
    if (r >= R) return;
    int e = topk_id[(size_t)r * k + j];
    unsigned long long m = w.masks[(size_t)b * E + e];
    unsigned long long below = (rl == 0) ? 0ull : (m & ((1ull << rl) - 1ull));
    w.entry[w.offset[e] + w.base[(size_t)b * E + e] + __popcll(below)] = r * k + j;
}


static bool tiers_valid(const int32_t* t, int32_t n) {
    if (n < 1 || n > 7) return false;
    for (int i = 0; i < n; ++i) {
        if (t[i] < 2 || t[i] > kMaxPass) return false;
        if (i > 0 && t[i] <= t[i - 1]) return false;
    }
    return true;
}

}  // namespace xp

using namespace xp;

XP_API size_t xp_workspace_bytes(const xp_dims* dims, int32_t max_rows) {
    if (check_dims(dims) != XP_OK || max_rows < 0) return 0;
    return ws_layout(dims, max_rows).total;
}

XP_API int xp_workspace_layout(const xp_dims* dims, int32_t max_rows, size_t off[6]) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (!off) return XP_ERR_NULL;
    if (max_rows < 0) return XP_ERR_SHAPE;
    WsLayout L = ws_layout(dims, max_rows);
    off[0] = L.hdr; off[1] = L.count; off[2] = L.offset;
    off[3] = L.entry; off[4] = L.gu_pass; off[5] = L.dn_pass;
    return XP_OK;
}

XP_API int xp_route_bucket(const xp_dims* dims, int32_t rows, const float* logits, int32_t* topk_id,
                           float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!logits || !topk_id || !topk_w || !workspace) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int E = dims->n_experts, k = dims->top_k;
    WsPtrs w = ws_ptrs(workspace, dims, rows);
    if (rows <= kSmallRows) {
        hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(1024), 0, s, logits, rows, E, k, topk_id, topk_w, w,
                           g_tiers);
        return launch_status();
    }
    int nblk = (rows + kSmallRows - 1) / kSmallRows;
    hipLaunchKernelGGL(route_blocks_kernel, dim3(nblk), dim3(1024), 0, s, logits, rows, E, k, topk_id, topk_w, w);
    if (launch_status() != XP_OK) return XP_ERR_HIP;
    hipLaunchKernelGGL(route_plan_kernel, dim3(1), dim3(1024), 0, s, E, nblk, w, g_tiers);
    if (launch_status() != XP_OK) return XP_ERR_HIP;
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nblk), dim3(1024), 0, s, rows, E, k, (const int32_t*)topk_id, w);
    return launch_status();
}

static uint32_t tier_mask(const int32_t* t, int32_t n) {
    uint32_t m = 0;
    for (int i = 0; i < n; ++i) m |= 1u << t[i];
    return m;
}

static int tier_list(uint32_t m, int32_t* out) {
    int n = 0;
    for (int p = 2; p <= kMaxPass; ++p)
        if (m & (1u << p)) out[n++] = p;
    for (int i = n; i < 8; ++i) out[i] = 0;
    return n;
}

XP_API int xp_set_tiers(const int32_t* gu, int32_t n_gu, const int32_t* dn, int32_t n_dn) {
    Tiers t = g_tiers;
    if (!gu || n_gu == 0) {
        t.gu = kDefaultGu;
    } else {
        if (!tiers_valid(gu, n_gu)) return XP_ERR_TIERS;
        t.gu = tier_mask(gu, n_gu);
    }
    if (!dn || n_dn == 0) {
        t.dn = kDefaultDn;
    } else {
        if (!tiers_valid(dn, n_dn)) return XP_ERR_TIERS;
        t.dn = tier_mask(dn, n_dn);
    }
    g_tiers = t;
    return XP_OK;
}

XP_API int xp_get_tiers(int32_t* gu, int32_t* n_gu, int32_t* dn, int32_t* n_dn) {
    if (!gu || !n_gu || !dn || !n_dn) return XP_ERR_NULL;
    *n_gu = tier_list(g_tiers.gu, gu);
    *n_dn = tier_list(g_tiers.dn, dn);
    return XP_OK;
}

XP_API const char* xp_status_string(int status) {
    switch (status) {
        case XP_OK: return "XP_OK";
        case XP_ERR_NULL: return "XP_ERR_NULL: a required pointer is NULL";
        case XP_ERR_SHAPE: return "XP_ERR_SHAPE: a dimension or row count is out of range";
        case XP_ERR_TOPK: return "XP_ERR_TOPK: top_k out of range";
        case XP_ERR_WORKSPACE: return "XP_ERR_WORKSPACE: workspace too small";
        case XP_ERR_TIERS: return "XP_ERR_TIERS: malformed pass-size list";
        case XP_ERR_HIP: return "XP_ERR_HIP: the HIP runtime refused a launch";
        default: return "unknown xp status";
    }
}
