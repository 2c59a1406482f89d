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

__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// The logit a key was made from (-0 comes back as +0, any NaN as a NaN).
__device__ __forceinline__ float key_logit(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    if (o == 0u) return __builtin_nanf("");
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// One wave selects row r's top-k by k rounds of a wave-wide maximum. Writes the
// ids and the softmax weights (fp32: exp of each chosen logit minus the largest,
// summed in slot order, one division) to global memory when topk_id is given,
// the ids to sid[0..k) in LDS, and sets bit r_local of each chosen expert's mask.
__device__ void topk_row(const float* __restrict__ logits, int E, int k, int r, int r_local,
                         int32_t* __restrict__ topk_id, float* __restrict__ topk_w, int32_t* sid,
                         unsigned long long* smask) {
    const int lane = threadIdx.x & 63;
    const float* lr = logits + (size_t)r * E;
    const int cpl = (E + 63) >> 6;  // candidates per lane
    uint64_t cand[kMaxExperts / 64];
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
        const int e = lane + 64 * i;
        cand[i] = (i < cpl && e < E) ? cand_key(lr[e], e) : 0ull;
    }
    uint64_t mine = 0ull;  // lane j keeps the key chosen in round j
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kMaxExperts / 64; ++i)
            if (i < cpl) best = cand[i] > best ? cand[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < kMaxExperts / 64; ++i)
            if (i < cpl && cand[i] == best) cand[i] = 0ull;
        if (lane == j) mine = best;
    }
    // lane 0 holds the largest chosen logit; every lane j < k its own exp term
    const float top = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(key_logit(mine))));
    const float ex = expf(key_logit(mine) - top);
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = s + __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(ex), j));
    if (lane < k) {
        const int id = key_id(mine);
        sid[lane] = id;
        if (topk_id) {
            topk_id[(size_t)r * k + lane] = id;
            topk_w[(size_t)r * k + lane] = ex / s;
        }
        atomicOr(&smask[id], 1ull << r_local);
    }
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


// Offsets and both pass lists from per-expert row counts cnt[e] (LDS), by one
// wave: lane l takes a contiguous run of experts, so the scans are one wave
// prefix sum each. Writes soff[0..E] (LDS), gu (LDS or global), and, when
// given, dn, count, offset and the header in global memory.
__device__ void plan_wave(int E, const int32_t* cnt, const Tiers& T, int32_t* soff, int4* gu, int4* dn,
                          int32_t* count, int32_t* offset, int32_t* hdr, int32_t* n_gu_out) {
    const int lane = threadIdx.x & 63;
    const int epl = (E + 63) >> 6;
    const int e0 = lane * epl;
    const int e1 = min(E, e0 + epl);
    int sc = 0, sg = 0, sd = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        sc += c;
        sg += n_passes(c, T.gu, T.n_gu);
        sd += n_passes(c, T.dn, T.n_dn);
    }
    const int ic = wave_incl_sum(sc), ig = wave_incl_sum(sg), id = wave_incl_sum(sd);
    int oc = ic - sc, og = ig - sg, od = id - sd;
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        soff[e] = oc;
        if (count) count[e] = c;
        if (offset) offset[e] = oc;
        write_passes(e, c, oc, T.gu, T.n_gu, gu + og);
        if (dn) write_passes(e, c, oc, T.dn, T.n_dn, dn + od);
        oc += c;
        og += n_passes(c, T.gu, T.n_gu);
        od += n_passes(c, T.dn, T.n_dn);
    }
    if (lane == 63) {
        soff[E] = ic;
        if (offset) offset[E] = ic;
        if (hdr) { hdr[0] = ig; hdr[1] = id; }
        if (n_gu_out) *n_gu_out = ig;
    }
}

}  // namespace xp
