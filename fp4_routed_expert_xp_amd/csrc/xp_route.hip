// xp_route.hip — routing (top-k + softmax), stable bucketing and pass plans.
//
// Routing is not described on the #2983 page; it is the plain top-k over the
// router logits (ties to the lower expert id, NaN last) with softmax over the
// chosen logits as combine weights. Bucketing groups each expert's rows in
// ascending row order with no atomics whose order could leak into the plan;
// pass sizes follow the rows left [#2983, "What this changes"].
//
// Rows are handled in blocks of 64 with one 64-bit row mask per (block,
// expert): the rank of a row inside its expert is a popcount, so the plan is a
// pure function of the logits. Up to 64 rows run as one workgroup; larger
// batches run three kernels (masks per block, counts and passes, scatter).
#include <string.h>

#include "xp_common.h"

namespace xp {

static Tiers g_tiers = {{2, 4, 6, 8, 0, 0, 0, 0}, 4, {2, 4, 0, 0, 0, 0, 0, 0}, 2};

// Larger key = ranks earlier: logit order, then lower id. NaN -> order 0 (last).
__device__ __forceinline__ uint64_t cand_key(float v, int id) {
    uint32_t u = __float_as_uint(v);
    uint32_t o;
    if (v != v) {
        o = 0u;
    } else {
        if (u == 0x80000000u) u = 0u;  // -0 ties with +0
        o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// One wave selects row r's top-k; lane 0 writes ids and softmax weights.
// The chosen ids are also returned in sid[0..k) (LDS) and their row bit set
// in the block's expert masks.
__device__ void topk_row(const float* __restrict__ logits, int E, int k, int r, int r_local,
                         int32_t* __restrict__ topk_id, float* __restrict__ topk_w,
                         int32_t* sid, unsigned long long* smask) {
    const int lane = threadIdx.x & 63;
    const float* lr = logits + (size_t)r * E;
    uint64_t cand[kMaxExperts / 64];
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
        int e = lane + 64 * i;
        cand[i] = (e < E) ? cand_key(lr[e], e) : 0ull;
    }
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kMaxExperts / 64; ++i) best = cand[i] > best ? cand[i] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            uint64_t o = __shfl_xor(best, off, 64);
            best = o > best ? o : best;
        }
#pragma unroll
        for (int i = 0; i < kMaxExperts / 64; ++i)
            if (cand[i] == best) cand[i] = 0ull;
        if (lane == 0) sid[j] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    }
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) {
        float ex[kMaxTopK];
        float top = lr[sid[0]];
        float s = 0.0f;
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(lr[sid[j]] - top);
            s = s + ex[j];
        }
        for (int j = 0; j < k; ++j) {
            topk_id[(size_t)r * k + j] = sid[j];
            topk_w[(size_t)r * k + j] = ex[j] / s;
        }
    }
    if (lane < k) atomicOr(&smask[sid[lane]], 1ull << r_local);
}

__device__ __forceinline__ int n_passes(int n, const int32_t* t, int nt) {
    if (n <= 0) return 0;
    if (n == 1) return 1;
    int mx = t[nt - 1];
    return n / mx + (n % mx != 0);
}

__device__ void write_passes(int e, int n, int first, const int32_t* t, int nt, int4* out) {
    if (n <= 0) return;
    if (n == 1) {
        out[0] = make_int4(e, first, 1, 1);
        return;
    }
    int mx = t[nt - 1];
    int left = n, i = 0;
    while (left > 0) {
        int p = mx;
        if (left < mx)
            for (int q = 0; q < nt; ++q)
                if (t[q] >= left) { p = t[q]; break; }
        int real = left < p ? left : p;
        out[i++] = make_int4(e, first, real, p);
        first += real;
        left -= real;
    }
}

// Block-wide exclusive scan of three ints (blockDim.x == 1024). Returns totals in tot[3].
__device__ void block_scan3(int v0, int v1, int v2, int* x0, int* x1, int* x2, int* wsum, int* tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int a = v0, b = v1, c = v2;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int ta = __shfl_up(a, off, 64), tb = __shfl_up(b, off, 64), tc = __shfl_up(c, off, 64);
        if (lane >= off) { a += ta; b += tb; c += tc; }
    }
    if (lane == 63) { wsum[3 * w] = a; wsum[3 * w + 1] = b; wsum[3 * w + 2] = c; }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s0 = 0, s1 = 0, s2 = 0;
        for (int i = 0; i < 16; ++i) {
            int t0 = wsum[3 * i], t1 = wsum[3 * i + 1], t2 = wsum[3 * i + 2];
            wsum[3 * i] = s0; wsum[3 * i + 1] = s1; wsum[3 * i + 2] = s2;
            s0 += t0; s1 += t1; s2 += t2;
        }
        tot[0] = s0; tot[1] = s1; tot[2] = s2;
    }
    __syncthreads();
    *x0 = a - v0 + wsum[3 * w];
    *x1 = b - v1 + wsum[3 * w + 1];
    *x2 = c - v2 + wsum[3 * w + 2];
}

struct WsPtrs {
    int32_t* hdr;
    int32_t* count;
    int32_t* offset;
    int32_t* entry;
    int4* gu_pass;
    int4* dn_pass;
    unsigned long long* masks;
    int32_t* base;
};

// Counts, offsets and both pass lists from per-expert row counts held by
// thread e. soff receives each expert's first entry (LDS, E entries).
__device__ void plan_from_counts(int E, int c, const Tiers& T, WsPtrs w, int* soff, int* wsum, int* tot) {
    const int e = threadIdx.x;
    int pg = (e < E) ? n_passes(c, T.gu, T.n_gu) : 0;
    int pd = (e < E) ? n_passes(c, T.dn, T.n_dn) : 0;
    int xo, xg, xd;
    block_scan3(e < E ? c : 0, pg, pd, &xo, &xg, &xd, wsum, tot);
    if (e < E) {
        soff[e] = xo;
        w.count[e] = c;
        w.offset[e] = xo;
        write_passes(e, c, xo, T.gu, T.n_gu, w.gu_pass + xg);
        write_passes(e, c, xo, T.dn, T.n_dn, w.dn_pass + xd);
    }
    if (e == 0) {
        w.offset[E] = tot[0];
        w.hdr[0] = tot[1];
        w.hdr[1] = tot[2];
    }
}

// ---- up to 64 rows: one workgroup of 1024 threads does everything
__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ logits, int R, int E, int k,
                                                           int32_t* __restrict__ topk_id,
                                                           float* __restrict__ topk_w, WsPtrs w, Tiers T) {
    __shared__ unsigned long long smask[kMaxExperts];
    __shared__ int32_t sid[kSmallRows][kMaxTopK];
    __shared__ int soff[kMaxExperts];
    __shared__ int wsum[48];
    __shared__ int tot[3];
    for (int e = threadIdx.x; e < E; e += blockDim.x) smask[e] = 0ull;
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    for (int r = wave; r < R; r += 16) topk_row(logits, E, k, r, r, topk_id, topk_w, sid[r], smask);
    __syncthreads();
    int c = (threadIdx.x < E) ? __popcll(smask[threadIdx.x]) : 0;
    plan_from_counts(E, c, T, w, soff, wsum, tot);
    __syncthreads();
    const int t = threadIdx.x;
    if (t < R * k) {
        int r = t / k, j = t - r * k;
        int e = sid[r][j];
        unsigned long long below = (r == 0) ? 0ull : (smask[e] & ((1ull << r) - 1ull));
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
        int r = b * kSmallRows + rl;
        if (r < R) topk_row(logits, E, k, r, rl, topk_id, topk_w, sid[rl], smask);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) w.masks[(size_t)b * E + e] = smask[e];
}

// (2) counts per expert, per-block bases, offsets and passes (one workgroup)
__global__ __launch_bounds__(1024) void route_plan_kernel(int E, int nblk, WsPtrs w, Tiers T) {
    __shared__ int soff[kMaxExperts];
    __shared__ int wsum[48];
    __shared__ int tot[3];
    const int e = threadIdx.x;
    int c = 0;
    if (e < E) {
        for (int b = 0; b < nblk; ++b) {
            w.base[(size_t)b * E + e] = c;
            c += __popcll(w.masks[(size_t)b * E + e]);
        }
    }
    plan_from_counts(E, c, T, w, soff, wsum, tot);
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

static WsPtrs ws_ptrs(void* ws, const xp_dims* d, int32_t rows) {
    WsLayout L = ws_layout(d, rows);
    char* b = (char*)ws;
    return WsPtrs{(int32_t*)(b + L.hdr),   (int32_t*)(b + L.count), (int32_t*)(b + L.offset),
                  (int32_t*)(b + L.entry), (int4*)(b + L.gu_pass),  (int4*)(b + L.dn_pass),
                  (unsigned long long*)(b + L.masks), (int32_t*)(b + L.base)};
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

XP_API int xp_set_tiers(const int32_t* gu, int32_t n_gu, const int32_t* dn, int32_t n_dn) {
    Tiers t = g_tiers;
    if (!gu || n_gu == 0) {
        const int32_t d[4] = {2, 4, 6, 8};
        memset(t.gu, 0, sizeof t.gu);
        memcpy(t.gu, d, sizeof d);
        t.n_gu = 4;
    } else {
        if (!tiers_valid(gu, n_gu)) return XP_ERR_TIERS;
        memset(t.gu, 0, sizeof t.gu);
        memcpy(t.gu, gu, sizeof(int32_t) * n_gu);
        t.n_gu = n_gu;
    }
    if (!dn || n_dn == 0) {
        const int32_t d[2] = {2, 4};
        memset(t.dn, 0, sizeof t.dn);
        memcpy(t.dn, d, sizeof d);
        t.n_dn = 2;
    } else {
        if (!tiers_valid(dn, n_dn)) return XP_ERR_TIERS;
        memset(t.dn, 0, sizeof t.dn);
        memcpy(t.dn, dn, sizeof(int32_t) * n_dn);
        t.n_dn = n_dn;
    }
    g_tiers = t;
    return XP_OK;
}

XP_API int xp_get_tiers(int32_t* gu, int32_t* n_gu, int32_t* dn, int32_t* n_dn) {
    if (!gu || !n_gu || !dn || !n_dn) return XP_ERR_NULL;
    memcpy(gu, g_tiers.gu, sizeof g_tiers.gu);
    memcpy(dn, g_tiers.dn, sizeof g_tiers.dn);
    *n_gu = g_tiers.n_gu;
    *n_dn = g_tiers.n_dn;
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
