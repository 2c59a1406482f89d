// xp_route_dev.h — device routines of routing, bucketing and pass planning,
// shared by the routing kernels and the fused route + gate/up kernel.
//
// Routing is not described on the #2983 page; it is the plain top-k over the
// router logits (ties to the lower expert id, NaN last) with softmax over the
// chosen logits as combine weights. Bucketing groups each expert's rows in
// ascending row order; pass sizes follow the rows left [#2983, "What this
// changes"]. Rows are handled in blocks of 64 with one 64-bit row mask per
// (block, expert), so a row's rank inside its expert is a popcount and the plan
// is a pure function of the logits.
#pragma once

#include "xp_common.h"

namespace xp {

// Rank order of a logit as an unsigned key: larger logit = larger key, -0
// equal to +0, NaN = 0 (after every number, -Inf included).
__device__ __forceinline__ uint32_t logit_order(float v) {
    uint32_t u = __float_as_uint(v);
    if (v != v) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit an order key was made from (-0 comes back as +0, NaN as a NaN).
__device__ __forceinline__ float order_logit(uint32_t o) {
    if (o == 0u) return __builtin_nanf("");
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// One wave selects the first kk picks of a logit row: kk rounds, each taking
// the largest order over the wave and, among the lanes holding it, the smallest
// expert id (so equal logits go to the lower id and NaN comes last). Lane j
// (j < kk) gets round j's order key and id. CPL = candidates per lane
// (E <= 64 * CPL).
template <int CPL>
__device__ __forceinline__ void topk_picks(const float* __restrict__ lr, int E, int kk, uint32_t& mine_ord,
                                           uint32_t& mine_id) {
    const int lane = threadIdx.x & 63;
    float v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = lr[e < E ? e : E - 1];
    }
    uint32_t ord[CPL];   // order keys of this lane's candidates
    bool live[CPL];      // present and not yet taken
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        live[i] = lane + 64 * i < E;
        ord[i] = logit_order(v[i]);
    }
    mine_ord = 0u;
    mine_id = 0u;
    for (int j = 0; j < kk; ++j) {
        // this lane's best live candidate: larger order, then smaller id
        uint32_t bo = 0u, bi = 0xFFFFFFFFu;
        bool any = false;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t id = (uint32_t)(lane + 64 * i);
            if (live[i] && (!any || ord[i] > bo)) { bo = ord[i]; bi = id; any = true; }
        }
        const uint32_t wo = wave_max_u32(any ? bo : 0u);
        const uint32_t wi = wave_min_u32((any && bo == wo) ? bi : 0xFFFFFFFFu);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            if ((uint32_t)(lane + 64 * i) == wi) live[i] = false;
        if (lane == j) { mine_ord = wo; mine_id = wi; }
    }
}

// topk_picks for E <= 1024.
__device__ __forceinline__ void topk_picks_any(const float* __restrict__ lr, int E, int kk, uint32_t& mo,
                                               uint32_t& mi) {
    if (E <= 64) topk_picks<1>(lr, E, kk, mo, mi);
    else if (E <= 128) topk_picks<2>(lr, E, kk, mo, mi);
    else if (E <= 256) topk_picks<4>(lr, E, kk, mo, mi);
    else if (E <= 512) topk_picks<8>(lr, E, kk, mo, mi);
    else topk_picks<16>(lr, E, kk, mo, mi);
}

// Softmax weight of lane j's pick over the k picks (fp32): exp of its logit
// minus the largest (lane 0's), divided by the sum of those terms taken in
// slot order. Every lane of the wave must call this.
__device__ __forceinline__ float topk_weight(uint32_t mine_ord, int k) {
    const float top = order_logit((uint32_t)__builtin_amdgcn_readfirstlane((int)mine_ord));
    const float ex = expf(order_logit(mine_ord) - top);
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = s + __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(ex), j));
    return ex / s;
}

// One wave routes row r: ids and softmax weights to global memory when topk_id
// is given, ids to sid[0..k) in LDS, and bit r_local of each chosen expert's mask.
template <int CPL>
__device__ void topk_row_n(const float* __restrict__ logits, int E, int k, int r, int r_local,
                           int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* sid,
                           unsigned long long* smask) {
    const int lane = threadIdx.x & 63;
    uint32_t mine_ord, mine_id;
    topk_picks<CPL>(logits + (size_t)r * E, E, k, mine_ord, mine_id);
    const float w = topk_weight(mine_ord, k);
    if (lane < k) {
        const int id = (int)mine_id;
        sid[lane] = id;
        if (topk_id) {
            topk_id[(size_t)r * k + lane] = id;
            topk_w[(size_t)r * k + lane] = w;
        }
        atomicOr(&smask[id], 1ull << r_local);
    }
}

__device__ __forceinline__ void topk_row(const float* __restrict__ logits, int E, int k, int r, int r_local,
                                         int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* sid,
                                         unsigned long long* smask) {
    if (E <= 64) topk_row_n<1>(logits, E, k, r, r_local, topk_id, topk_w, sid, smask);
    else if (E <= 128) topk_row_n<2>(logits, E, k, r, r_local, topk_id, topk_w, sid, smask);
    else if (E <= 256) topk_row_n<4>(logits, E, k, r, r_local, topk_id, topk_w, sid, smask);
    else if (E <= 512) topk_row_n<8>(logits, E, k, r, r_local, topk_id, topk_w, sid, smask);
    else topk_row_n<16>(logits, E, k, r, r_local, topk_id, topk_w, sid, smask);
}

__device__ __forceinline__ int largest_tier(uint32_t t) { return 31 - __clz(t); }

// Smallest allowed size holding `left` rows (left below the largest size).
__device__ __forceinline__ int tier_at_least(uint32_t t, int left) { return __ffs(t & ~((1u << left) - 1u)) - 1; }

__device__ __forceinline__ int n_passes(int n, uint32_t t) {
    if (n <= 0) return 0;
    if (n == 1) return 1;
    const int mx = largest_tier(t);
    return (n + mx - 1) / mx;
}

__device__ void write_passes(int e, int n, int first, uint32_t t, int4* out) {
    if (n <= 0) return;
    if (n == 1) {
        out[0] = make_int4(e, first, 1, 1);
        return;
    }
    const int mx = largest_tier(t);
    int left = n, i = 0;
    while (left > 0) {
        const int p = left >= mx ? mx : tier_at_least(t, left);
        const int real = left < p ? left : p;
        out[i++] = make_int4(e, first, real, p);
        first += real;
        left -= real;
    }
}

// Offsets and both pass lists from per-expert row counts cnt[e] (LDS). Thread
// e (of a 1024-thread workgroup) takes expert e; the three exclusive scans are
// wave prefix sums joined through LDS. Writes soff[0..E] (LDS), gu (LDS or
// global), and, when given, dn, count, offset and the header in global memory;
// *n_gu_out (LDS) gets the gate/up pass count. Every thread must call this.
__device__ void plan_block(int E, const int32_t* cnt, const Tiers& T, int32_t* soff, int4* gu, int4* dn,
                           int32_t* count, int32_t* offset, int32_t* hdr, int32_t* n_gu_out, int* wsum /*[48]*/) {
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    const int c = e < E ? cnt[e] : 0;
    const int pg = n_passes(c, T.gu), pd = n_passes(c, T.dn);
    const int ic = wave_incl_sum(c), ig = wave_incl_sum(pg), id = wave_incl_sum(pd);
    if (lane == 63) { wsum[3 * wave] = ic; wsum[3 * wave + 1] = ig; wsum[3 * wave + 2] = id; }
    __syncthreads();
    int bc = 0, bg = 0, bd = 0, tc = 0, tg = 0, td = 0;
    const int nw = (blockDim.x + 63) >> 6;
    for (int w = 0; w < nw; ++w) {
        const int a0 = wsum[3 * w], a1 = wsum[3 * w + 1], a2 = wsum[3 * w + 2];
        if (w < wave) { bc += a0; bg += a1; bd += a2; }
        tc += a0; tg += a1; td += a2;
    }
    const int oc = bc + ic - c, og = bg + ig - pg, od = bd + id - pd;
    if (e < E) {
        soff[e] = oc;
        if (count) count[e] = c;
        if (offset) offset[e] = oc;
        write_passes(e, c, oc, T.gu, gu + og);
        if (dn) write_passes(e, c, oc, T.dn, dn + od);
    }
    if (e == 0) {
        soff[E] = tc;
        if (offset) offset[E] = tc;
        if (hdr) { hdr[0] = tg; hdr[1] = td; }
        if (n_gu_out) *n_gu_out = tg;
    }
}

// Routing inputs of the one-row route + gate/up launch.
struct RouteIn {
    const float* logits;
    int E;
    int32_t* topk_id;
    float* topk_w;
    WsPtrs w;
};

// Publish what xp_route_bucket writes for a batch of one row, from the wave
// that ran topk_picks for all k rounds (lane j holds pick j's order key mo and
// id mi): top-k ids and weights, counts, offsets, entries and both pass lists
// (one one-row pass per chosen expert, experts ascending). Every lane of the
// wave must call this.
__device__ __forceinline__ void publish_one_row(const RouteIn& ri, int k, uint32_t mo, uint32_t mi) {
    const int lane = threadIdx.x & 63;
    const float w = topk_weight(mo, k);
    int rank = 0;  // position of this lane's pick among the picks by expert id
    for (int i = 0; i < k; ++i) rank += ((uint32_t)__builtin_amdgcn_readlane((int)mi, i) < mi) ? 1 : 0;
    if (lane < k) {
        ri.topk_id[lane] = (int32_t)mi;
        ri.topk_w[lane] = w;
        ri.w.gu_pass[rank] = make_int4((int)mi, rank, 1, 1);
        ri.w.dn_pass[rank] = make_int4((int)mi, rank, 1, 1);
        ri.w.entry[rank] = lane;  // row 0, slot lane
    }
    for (int e0 = 0; e0 <= ri.E; e0 += 64) {
        const int e = e0 + lane;
        int below = 0, hit = 0;
        for (int i = 0; i < k; ++i) {
            const int o = __builtin_amdgcn_readlane((int)mi, i);
            below += o < e ? 1 : 0;
            hit |= o == e ? 1 : 0;
        }
        if (e <= ri.E) ri.w.offset[e] = below;
        if (e < ri.E) ri.w.count[e] = hit;
    }
    if (lane == 0) {
        ri.w.hdr[0] = k;
        ri.w.hdr[1] = k;
    }
}

}  // namespace xp
