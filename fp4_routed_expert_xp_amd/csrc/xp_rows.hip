// xp_rows.hip — the multi-row gate/up and down passes.
//
// A work item is (pass, tile of 64 output columns). Lane c of a wave owns column
// tile*64 + c; each wave owns one leaf j of the eight-leaf tree, i.e. the
// 32-weight groups g = j, j+8, j+16, ... of the K axis, which it walks in
// ascending order. Gate/up items run 8 waves, each walking its leaf of both
// matrices (or, for batches with no more items than CUs, 16 waves: 0-7 the gate
// leaves, 8-15 the up leaves); down items run 8 waves. For each of its groups a lane loads
// 16 bytes of codes (one coalesced 1 KiB read per wave in the packed layout) and
// one scale byte, decodes the 32 weights once (v_cvt_scalef32_pk_f32_fp4 with
// scale 1, exact; eight at a time, each dword just before its quarter of the
// chain) and runs every row of the pass through them: per row a fused
// multiply-add chain from +0 over the 32 products in k order (Chain<P>), then
// the group's scale applied by one fused multiply-add into the row's leaf. The
// leaves meet in LDS and one thread per (row, column) adds them by the fixed
// tree ((l0+l1)+(l2+l3))+((l4+l5)+(l6+l7)) and applies the epilogue.
// [#2983, "What this changes" and the rows commit: a pass decodes each 32-group
// once for all of its rows; each row's chain, scaled fma, tree and epilogue are
// the one-row kernel's]
//
// The code for a pass of P rows is the one-row code repeated per row with no
// value crossing between rows, so a row's bits do not depend on P. Padding rows
// (P > real rows) re-read the last real row and are not stored.
#include "xp_pass_dev.h"
#include "xp_route_dev.h"

#include <algorithm>

namespace xp {

// Gate/up passes over the plan in the workspace: work item = (pass, tile).
// WAVES = 8: each wave walks one leaf of both matrices and two workgroups share
// a CU, so that one streams weights while the other reduces and stores; the
// host takes it when the batch can hold more items than there are CUs.
// WAVES = 16: gate and up leaves in separate waves, one workgroup per CU (a
// batch of at most as many items as CUs, e.g. one row).
template <int OUT, bool CODED, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 16 / WAVES) void gateup_kernel(const xp_expert* __restrict__ experts,
                                                      const void* __restrict__ x, const uint8_t* __restrict__ xs,
                                                      const int32_t* __restrict__ hdr,
                                                      const int32_t* __restrict__ entry,
                                                      const int4* __restrict__ passes, int E, int H, int I,
                                                      int k, float* __restrict__ out0, float* __restrict__ out1) {
    __shared__ float red[2 * kLeaves * kMaxPass * kTile];
    const xp_expert* tab = experts;
    const int n_tiles = I / kTile;
    const int n_items = hdr[0] * n_tiles;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pass = item / n_tiles;
        const int tile = item - pass * n_tiles;
        const int4 ps = passes[pass];
        switch (ps.w) {
            case 1: gu_item<1, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 2: gu_item<2, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 3: gu_item<3, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 4: gu_item<4, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 5: gu_item<5, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 6: gu_item<6, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 7: gu_item<7, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 8: gu_item<8, OUT, CODED, WAVES>(tab, x, xs, entry, ps, tile, H, I, k, out0, out1, red); break;
            default: break;
        }
    }
}

// ---------------------------------------------------------- one-row decode
// Routing, plan and gate/up for a batch of one row in one launch. With one row
// every chosen expert has a one-row pass, so item (slot j, tile) needs only the
// row's j-th pick: the workgroup's first wave runs top-k rounds 0..j and the
// workgroup starts its weight stream without the full plan. The workgroup of
// (slot k-1, tile 0) runs all k rounds and publishes what xp_route_bucket
// writes for this row: top-k ids and weights, counts, offsets, entries and both
// pass lists (one P=1 pass per chosen expert, experts ascending).
__global__ __launch_bounds__(1024) void gateup_one_row_kernel(const xp_expert* __restrict__ experts,
                                                              const uint16_t* __restrict__ x, RouteIn ri, int H,
                                                              int I, int k, float* __restrict__ act) {
    __shared__ float red[2 * kLeaves * kTile];
    __shared__ int32_t s_entry[1];
    __shared__ int s_pick;
    const int n_tiles = I / kTile;
    // Workgroups start in blockIdx order over a few microseconds; the slots that
    // need the most top-k rounds go first, so late starters route quickly.
    const int jb = blockIdx.x / n_tiles, tile = blockIdx.x - jb * n_tiles;
    const int j = k - 1 - jb;
    const bool publish = (j == k - 1) && (tile == 0);
    if (threadIdx.x < 64) {
        uint32_t mo, mi;
        topk_picks_any(ri.logits, ri.E, publish ? k : j + 1, mo, mi);
        if ((int)threadIdx.x == j) {
            s_pick = (int)mi;
            s_entry[0] = j;
        }
        if (publish) publish_one_row(ri, k, mo, mi);
    }
    __syncthreads();
    gu_item<1, kActF32>(experts, x, nullptr, s_entry, make_int4(s_pick, 0, 1, 1), tile, H, I, k, act, nullptr, red);
}

// ------------------------------------------------- few-row route + gate/up
// Routing, plan and gate/up for 2..64 rows in one launch. Every workgroup
// routes the whole batch itself (topk_row per row, then plan_block, the
// routing kernel's routines) into LDS and runs its (pass, tile) items from
// that plan, so no workgroup waits on another; workgroup 0 also publishes what
// xp_route_bucket writes: top-k ids and weights, counts, offsets, entries, both
// pass lists and the header. The plan is a pure function of the logits, so
// every workgroup's copy is the same. The routing scratch (masks, picks,
// counts, offsets) lives in the leaf buffer, which is free until the items
// start. Needs E <= 64 * WAVES (one thread per expert in plan_block).
constexpr int kRouteFusedEntries = kSmallRows * kMaxTopK;   // rows * k
// Every workgroup routes the batch before its first item, which delays every
// item when all workgroups have one: sixteen release-width rows (4096
// workgroups) took 200 us this way against 157 us with the routing launch; four
// (1024) gained 1.4 us. So the launch is kept to batches whose grid (one
// workgroup per possible item) stays this small.
#ifndef XP_ROUTE_FUSED_GRID
#define XP_ROUTE_FUSED_GRID 1024
#endif

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 16 / WAVES) void route_gateup_rows_kernel(
    const xp_expert* __restrict__ experts, const uint16_t* __restrict__ x, RouteIn ri, int R, int H, int I, int k,
    Tiers T, float* __restrict__ act) {
    __shared__ __align__(16) float red[2 * kLeaves * kMaxPass * kTile];
    __shared__ int4 sgu[kRouteFusedEntries];
    __shared__ int32_t sentry[kRouteFusedEntries];
    __shared__ int wsum[48];
    __shared__ int s_ngu;
    // routing scratch inside red: masks, picks, counts, offsets (20 KiB of 32)
    unsigned long long* smask = (unsigned long long*)red;                 // [kMaxExperts]
    int32_t* sid = (int32_t*)(smask + kMaxExperts);                       // [kSmallRows][kMaxTopK]
    int32_t* scnt = sid + kSmallRows * kMaxTopK;                          // [kMaxExperts]
    int32_t* soff = scnt + kMaxExperts;                                   // [kMaxExperts + 1]
    const int E = ri.E;
    const bool pub = blockIdx.x == 0;
    const int t = threadIdx.x;
    for (int e = t; e < E; e += blockDim.x) smask[e] = 0ull;
    __syncthreads();
    const int wave = t >> 6;
    for (int r = wave; r < R; r += WAVES)
        topk_row(ri.logits, E, k, r, r, pub ? ri.topk_id : nullptr, ri.topk_w, sid + r * kMaxTopK, smask);
    __syncthreads();
    for (int e = t; e < E; e += blockDim.x) scnt[e] = __popcll(smask[e]);
    __syncthreads();
    plan_block(E, scnt, T, soff, sgu, pub ? ri.w.dn_pass : nullptr, pub ? ri.w.count : nullptr,
               pub ? ri.w.offset : nullptr, pub ? ri.w.hdr : nullptr, &s_ngu, wsum);
    __syncthreads();
    for (int i = t; i < R * k; i += blockDim.x) {
        const int r = i / k, j = i - r * k;
        const int e = sid[r * kMaxTopK + j];
        const unsigned long long below = (r == 0) ? 0ull : (smask[e] & ((1ull << r) - 1ull));
        const int at = soff[e] + __popcll(below);
        sentry[at] = i;
        if (pub) ri.w.entry[at] = i;
    }
    const int n_gu = s_ngu;
    if (pub)
        for (int i = t; i < n_gu; i += blockDim.x) ri.w.gu_pass[i] = sgu[i];
    __syncthreads();   // the plan is complete; red is the leaf buffer from here on
    const int n_tiles = I / kTile;
    const int n_items = n_gu * n_tiles;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pass = item / n_tiles;
        const int tile = item - pass * n_tiles;
        const int4 ps = sgu[pass];
        switch (ps.w) {
            case 1: gu_item<1, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 2: gu_item<2, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 3: gu_item<3, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 4: gu_item<4, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 5: gu_item<5, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 6: gu_item<6, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 7: gu_item<7, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            case 8: gu_item<8, kActF32, false, WAVES>(experts, x, nullptr, sentry, ps, tile, H, I, k, act, nullptr, red); break;
            default: break;
        }
    }
}

// A16: act is bf16 (the bf16-storage variant); its pairs reach the chain as
// gate/up's x does (one dword of two bf16 per lane of each row of 16).
// T: output tiles per item (1, or 2: tiles 2*tile and 2*tile+1). With two, each
// wave walks its leaf of both tiles over one load of the rows' act values, so
// twice the weight bytes are in flight per wave; per tile the chain, scaled
// fma, leaf order and tree are the one-tile item's. EXACT: every leaf's walk
// ends on its last group, so no product is discarded (see gu_leaf).
template <int P, bool A16, int T, bool EXACT>
__device__ __forceinline__ void dn_item(const xp_expert* __restrict__ experts, const void* __restrict__ act,
                        const int32_t* __restrict__ entry, int4 ps, int tile, int H, int I,
                        float* __restrict__ out, float* red) {
    constexpr int D = DnDepth<P>::value;
    const int leaf = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int e = ps.x, first = ps.y, real = ps.z;
    const int G = I >> 5;
    const int xl = 2 * (lane & 15);
    const int tile0 = tile * T;

    const xp_expert ex = experts[e];
    const size_t tile_chunks = (size_t)tile0 * G * kTile;
    const size_t tile_step = (size_t)G * kTile;     // chunks from one tile to the next
    const gcodes_t cc = (gcodes_t)ex.down_codes + tile_chunks + lane;
    const gbytes_t ss = (gbytes_t)ex.down_scales + tile_chunks + lane;

    const float* ar[P];
    const uint32_t* ar16[P];
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const size_t row = (size_t)entry[first + (r < real ? r : real - 1)] * I;
        ar[r] = (const float*)act + row;
        ar16[r] = (const uint32_t*)((const uint16_t*)act + row);
    }

    // Branch-free ring over ceil(G/8) groups per leaf, as in gu_leaf.
    const int ng = (G + 7) >> 3;
    float acc[T][P];
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
        for (int r = 0; r < P; ++r) acc[q][r] = 0.0f;
    // Two register sets of D groups (see gu_leaf2).
    u32x4 bc[2][D][T];
    uint32_t bs[2][D][T];
    float2 bx[2][D][P];
    uint32_t bx16[2][D][P];
    auto load = [&](int set, int s, int i) {
        const int g = min(leaf + 8 * i, G - 1);
#pragma unroll
        for (int q = 0; q < T; ++q) {
            bc[set][s][q] = load_codes(cc + q * tile_step + (size_t)g * kTile);
            bs[set][s][q] = ss[q * tile_step + (size_t)g * kTile];
        }
#pragma unroll
        for (int r = 0; r < P; ++r) {
            if constexpr (A16)
                bx16[set][s][r] = ar16[r][16 * g + (lane & 15)];
            else
                bx[set][s][r] = *(const float2*)(ar[r] + 32 * g + xl);
        }
    };
    auto half = [&](int set, int i0) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            float sc[T];
            u32x4 cw[T];
#pragma unroll
            for (int q = 0; q < T; ++q) { sc[q] = e4m3(bs[set][s][q]); cw[q] = bc[set][s][q]; }
            float p[P], xa[P], xb[P];
            if constexpr (A16) {
                uint32_t xc[P];
#pragma unroll
                for (int r = 0; r < P; ++r) xc[r] = bx16[set][s][r];
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cw[0][0], w); Chain<P>::head_bf16(w, xc, xa, xb, p); }
            } else {
#pragma unroll
                for (int r = 0; r < P; ++r) { xa[r] = bx[set][s][r].x; xb[r] = bx[set][s][r].y; }
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cw[0][0], w); Chain<P>::head_f32(w, xa, xb, p); }
            }
            const bool valid = EXACT || leaf + 8 * i < G;
#pragma unroll
            for (int q = 0; q < T; ++q) {
                if (q > 0) { float w[8]; decode8(cw[q][0], w); Chain<P>::head_f32(w, xa, xb, p); }
                { float w[8]; decode8(cw[q][1], w); Chain<P>::tail1(w, xa, xb, p); }
                { float w[8]; decode8(cw[q][2], w); Chain<P>::tail2(w, xa, xb, p); }
                { float w[8]; decode8(cw[q][3], w); Chain<P>::tail3(w, xa, xb, p); }
#pragma unroll
                for (int r = 0; r < P; ++r) {
                    const float v = __builtin_fmaf(p[r], sc[q], acc[q][r]);
                    acc[q][r] = valid ? v : acc[q][r];
                }
            }
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(0, s, s);
    for (int i0 = 0; i0 < ng; i0 += 2 * D) {
        half(0, i0);
        half(1, i0 + D);
    }

    // red[tile q][leaf][row][lane]
#pragma unroll
    for (int q = 0; q < T; ++q)
#pragma unroll
        for (int r = 0; r < P; ++r) red[((q * kLeaves + leaf) * P + r) * kTile + lane] = acc[q][r];
    __syncthreads();
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < T; ++q) {
        if (t < P * kTile) {
            const int r = t >> 6, c = t & 63;
            if (r < real) {
                const float v = tree8(red + (q * kLeaves * P + r) * kTile + c, P * kTile);
                out[(size_t)entry[first + r] * H + (size_t)(tile0 + q) * kTile + c] = v;
            }
        }
    }
    __syncthreads();
}

// Down passes: work item = (pass, T consecutive output tiles).
// True when every leaf's walk over G groups (rounded up to trips of 2*D)
// ends exactly on its last group, so no product needs discarding.
template <int P>
__device__ __forceinline__ bool exact_dn_walk(int G) {
    constexpr int D = DnDepth<P>::value;
    return (G & 7) == 0 && ((G >> 3) % (2 * D)) == 0;
}

template <int P, bool A16, int T>
__device__ __forceinline__ void dn_item_any(const xp_expert* __restrict__ experts, const void* __restrict__ act,
                                            const int32_t* __restrict__ entry, int4 ps, int tile, int H, int I,
                                            float* __restrict__ out, float* red) {
    if (exact_dn_walk<P>(I >> 5))
        dn_item<P, A16, T, true>(experts, act, entry, ps, tile, H, I, out, red);
    else
        dn_item<P, A16, T, false>(experts, act, entry, ps, tile, H, I, out, red);
}

template <bool A16, int T>
__global__ __launch_bounds__(512, 4) void down_kernel(const xp_expert* __restrict__ experts,
                                                      const void* __restrict__ act,
                                                      const int32_t* __restrict__ hdr,
                                                      const int32_t* __restrict__ entry,
                                                      const int4* __restrict__ passes, int E, int H, int I,
                                                      float* __restrict__ out) {
    __shared__ float red[T * kLeaves * kMaxPass * kTile];
    const xp_expert* tab = experts;
    const int n_items_pass = H / (kTile * T);
    const int n_items = hdr[1] * n_items_pass;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pass = item / n_items_pass;
        const int tile = item - pass * n_items_pass;
        const int4 ps = passes[pass];
        switch (ps.w) {
            case 1: dn_item_any<1, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 2: dn_item_any<2, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 3: dn_item_any<3, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 4: dn_item_any<4, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 5: dn_item_any<5, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 6: dn_item_any<6, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 7: dn_item_any<7, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            case 8: dn_item_any<8, A16, T>(tab, act, entry, ps, tile, H, I, out, red); break;
            default: break;
        }
    }
}

// ------------------------------------------------- one-row down + combine
// With one row every down pass is a one-slot pass, and a set of columns needs
// only the k passes' outputs for those columns to be combined. A workgroup
// owns 16 columns (narrow_col0) for every pass: wave w walks leaf w % 8
// for passes 4*(w/8) .. 4*(w/8)+3, one pass per row of 16 lanes, so the DPP
// row broadcast hands each row its own pass's act values (lane m of a row
// holds the act pair (2m, 2m+1) of its pass's group). Per (pass, column) the
// arithmetic is dn_item's: the same chain, scaled fma, leaf order and tree.
// The leaves meet in LDS, out is stored, and the combine's fma chain over
// slots runs in the same workgroup, so no combine launch follows.
// Workgroups: hidden / 16; waves: 8 * ceil(k / 4), so k <= 8.
#ifndef XP_DC_DEPTH
#define XP_DC_DEPTH 2  // groups in flight per wave (4 and 8 measured slower: 10.1 -> 11.4 / 13.4 us)
#endif

__global__ __launch_bounds__(1024) void down_combine_one_row_kernel(
    const xp_expert* __restrict__ experts, const float* __restrict__ act, const int32_t* __restrict__ entry,
    const int4* __restrict__ passes, const float* __restrict__ topk_w, int H, int I, int k,
    float* __restrict__ out, float* __restrict__ y) {
    __shared__ float red[16][kTile];          // [wave][lane] leaf values
    __shared__ float sout[8][kNarrow];        // [slot][column] outputs
    constexpr int D = XP_DC_DEPTH;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int leaf = wave & 7, grp = wave >> 3;
    const int c = lane & 15;
    const int pass = min(4 * grp + (lane >> 4), k - 1);  // rows past the k-th pass repeat the last
    const int4 ps = passes[pass];
    const int slot = entry[ps.y];                        // one row: entry = slot
    const int col0 = narrow_col0(blockIdx.x, gridDim.x);
    const int n = col0 + c;
    const int G = I >> 5;
    const xp_expert ex = experts[ps.x];
    const size_t ch = (size_t)(n / kTile) * G * kTile + (n % kTile);
    const gcodes_t cc = (gcodes_t)ex.down_codes + ch;
    const gbytes_t ss = (gbytes_t)ex.down_scales + ch;
    const float* ar = act + (size_t)slot * I + 2 * c;

    const int ng = (G + 7) >> 3;
    float acc = 0.0f;
    // Two register sets of D groups (see gu_leaf2).
    u32x4 bc[2][D];
    uint32_t bs[2][D];
    float2 bx[2][D];
    auto load = [&](int set, int s, int i) {
        const int g = min(leaf + 8 * i, G - 1);
        bc[set][s] = load_codes(cc + (size_t)g * kTile);
        bs[set][s] = ss[(size_t)g * kTile];
        bx[set][s] = *(const float2*)(ar + 32 * g);
    };
    auto half = [&](int set, int i0) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            const float sc = e4m3(bs[set][s]);
            const u32x4 cw = bc[set][s];
            float p[1], xa[1] = {bx[set][s].x}, xb[1] = {bx[set][s].y};
            load(set ^ 1, s, i + D);
            { float w[8]; decode8(cw[0], w); Chain<1>::head_f32(w, xa, xb, p); }
            { float w[8]; decode8(cw[1], w); Chain<1>::tail1(w, xa, xb, p); }
            { float w[8]; decode8(cw[2], w); Chain<1>::tail2(w, xa, xb, p); }
            { float w[8]; decode8(cw[3], w); Chain<1>::tail3(w, xa, xb, p); }
            const float v = __builtin_fmaf(p[0], sc, acc);
            acc = (leaf + 8 * i < G) ? v : acc;
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(0, s, s);
    for (int i0 = 0; i0 < ng; i0 += 2 * D) {
        half(0, i0);
        half(1, i0 + D);
    }
    red[wave][lane] = acc;
    __syncthreads();
    const int t = threadIdx.x;
    const int n_grp = (k + 3) >> 2;
    if (t < n_grp * kTile) {
        const int g2 = t >> 6, l2 = t & 63;
        const int p2 = 4 * g2 + (l2 >> 4);
        if (p2 < k) {
            const float v = tree8(&red[8 * g2][l2], kTile);
            const int s2 = entry[passes[p2].y];
            out[(size_t)s2 * H + col0 + (l2 & 15)] = v;
            sout[s2][l2 & 15] = v;
        }
    }
    __syncthreads();
    if (t < kNarrow) {
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum = __builtin_fmaf(topk_w[j], sout[j][t], sum);
        y[col0 + t] = sum;
    }
}

// ------------------------------------------ down + combine, few entries
// The one-row layout for any plan with rows * top_k <= kFusedEntries: a
// workgroup owns 16 columns of every down pass and walks the passes eight at
// a time (waves 0-7 the leaves of four passes, one per row of 16 lanes; waves
// 8-15 the next four). A wave runs the largest pass size among its four rows
// of lanes; a shorter pass pads with its last real row, as every pass does.
// Per (row, slot, column) the chain, leaf order and tree are dn_item's; each
// (row, slot)'s 16 outputs wait in LDS until the combine, which runs the same
// slot-order fma chain as combine_kernel once every pass is done.
constexpr int kFusedEntries = 64;


template <int P, bool EXACT>
__device__ __forceinline__ void dc_pass_leaf(const xp_expert* __restrict__ experts, const float* __restrict__ act,
                                             const int32_t* __restrict__ entry, int4 ps, int n, int I, int leaf,
                                             int lane, float* red_wave /* [kMaxPass][kTile] */) {
    constexpr int D = DnDepth<P>::value;
    const int G = I >> 5;
    const int c = lane & 15;
    const xp_expert ex = experts[ps.x];
    const size_t ch = (size_t)(n / kTile) * G * kTile + (n % kTile);
    const gcodes_t cc = (gcodes_t)ex.down_codes + ch;
    const gbytes_t ss = (gbytes_t)ex.down_scales + ch;
    const float* ar[P];
#pragma unroll
    for (int r = 0; r < P; ++r) ar[r] = act + (size_t)entry[ps.y + min(r, ps.z - 1)] * I + 2 * c;

    const int ng = (G + 7) >> 3;
    float acc[P];
#pragma unroll
    for (int r = 0; r < P; ++r) acc[r] = 0.0f;
    // Two register sets of D groups (see gu_leaf2).
    u32x4 bc[2][D];
    uint32_t bs[2][D];
    float2 bx[2][D][P];
    auto load = [&](int set, int s, int i) {
        const int g = min(leaf + 8 * i, G - 1);
        bc[set][s] = load_codes(cc + (size_t)g * kTile);
        bs[set][s] = ss[(size_t)g * kTile];
#pragma unroll
        for (int r = 0; r < P; ++r) bx[set][s][r] = *(const float2*)(ar[r] + 32 * g);
    };
    auto half = [&](int set, int i0) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            const float sc = e4m3(bs[set][s]);
            const u32x4 cw = bc[set][s];
            float p[P], xa[P], xb[P];
#pragma unroll
            for (int r = 0; r < P; ++r) { xa[r] = bx[set][s][r].x; xb[r] = bx[set][s][r].y; }
            load(set ^ 1, s, i + D);
            { float w[8]; decode8(cw[0], w); Chain<P>::head_f32(w, xa, xb, p); }
            { float w[8]; decode8(cw[1], w); Chain<P>::tail1(w, xa, xb, p); }
            { float w[8]; decode8(cw[2], w); Chain<P>::tail2(w, xa, xb, p); }
            { float w[8]; decode8(cw[3], w); Chain<P>::tail3(w, xa, xb, p); }
            const bool valid = EXACT || leaf + 8 * i < G;
#pragma unroll
            for (int r = 0; r < P; ++r) {
                const float v = __builtin_fmaf(p[r], sc, acc[r]);
                acc[r] = valid ? v : acc[r];
            }
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(0, s, s);
    for (int i0 = 0; i0 < ng; i0 += 2 * D) {
        half(0, i0);
        half(1, i0 + D);
    }
#pragma unroll
    for (int r = 0; r < P; ++r) red_wave[r * kTile + lane] = acc[r];
}

__global__ __launch_bounds__(1024) void down_combine_rows_kernel(
    const xp_expert* __restrict__ experts, const float* __restrict__ act, const int32_t* __restrict__ hdr,
    const int32_t* __restrict__ entry, const int4* __restrict__ passes, const float* __restrict__ topk_w, int R,
    int H, int I, int k, float* __restrict__ out, float* __restrict__ y) {
    __shared__ float red[16][kMaxPass * kTile];        // [wave][row][lane] leaf values
    __shared__ float sout[kFusedEntries][kNarrow];     // [row * k + slot][column] outputs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int leaf = wave & 7, half = wave >> 3;
    const int col0 = narrow_col0(blockIdx.x, gridDim.x);
    const int n = col0 + (lane & 15);
    const int t = threadIdx.x;
    const int n_passes = hdr[1];
    for (int pg = 0; pg < n_passes; pg += 8) {
        const int pidx = min(pg + 4 * half + (lane >> 4), n_passes - 1);  // rows past the last pass repeat it
        const int4 ps = passes[pidx];
        // the wave's pass size: the largest of its four rows of lanes
        int pw = max(__builtin_amdgcn_readlane(ps.w, 0), __builtin_amdgcn_readlane(ps.w, 16));
        pw = max(pw, max(__builtin_amdgcn_readlane(ps.w, 32), __builtin_amdgcn_readlane(ps.w, 48)));
        float* rw = &red[wave][0];
        switch (pw) {
            case 1:
                if (exact_dn_walk<1>(I >> 5))
                    dc_pass_leaf<1, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<1, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 2:
                if (exact_dn_walk<2>(I >> 5))
                    dc_pass_leaf<2, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<2, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 3:
                if (exact_dn_walk<3>(I >> 5))
                    dc_pass_leaf<3, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<3, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 4:
                if (exact_dn_walk<4>(I >> 5))
                    dc_pass_leaf<4, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<4, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 5:
                if (exact_dn_walk<5>(I >> 5))
                    dc_pass_leaf<5, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<5, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 6:
                if (exact_dn_walk<6>(I >> 5))
                    dc_pass_leaf<6, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<6, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 7:
                if (exact_dn_walk<7>(I >> 5))
                    dc_pass_leaf<7, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<7, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            case 8:
                if (exact_dn_walk<8>(I >> 5))
                    dc_pass_leaf<8, true>(experts, act, entry, ps, n, I, leaf, lane, rw);
                else
                    dc_pass_leaf<8, false>(experts, act, entry, ps, n, I, leaf, lane, rw);
                break;
            default: break;
        }
        __syncthreads();
        // thread t: half t>>9, row of lanes (t>>7)&3, pass row (t>>4)&7, column t&15
        {
            const int h2 = t >> 9, q2 = (t >> 7) & 3, r2 = (t >> 4) & 7, c2 = t & 15;
            const int p2 = pg + 4 * h2 + q2;
            if (p2 < n_passes) {
                const int4 ps2 = passes[p2];
                if (r2 < ps2.z) {
                    const float v = tree8(&red[8 * h2][r2 * kTile + 16 * q2 + c2], kMaxPass * kTile);
                    const int e2 = entry[ps2.y + r2];
                    out[(size_t)e2 * H + col0 + c2] = v;
                    sout[e2][c2] = v;
                }
            }
        }
        __syncthreads();
    }
    if (t < R * kNarrow) {
        const int r = t >> 4, c2 = t & 15;
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum = __builtin_fmaf(topk_w[r * k + j], sout[r * k + j][c2], sum);
        y[(size_t)r * H + col0 + c2] = sum;
    }
}

#ifndef XP_DN_TILES
#define XP_DN_TILES 2
#endif
// Down batches pair tiles when they can hold more than this many two-tile items (two per CU).
constexpr long kPairItems = 512;

// Gate/up batches of at most this many (pass, tile) items (one per CU) run 16-wave workgroups.
constexpr long kWideItems = 256;

static int grid_for(int rows, int k, int n_tiles) {
    long items = (long)rows * k * n_tiles;  // passes <= rows*k
    return (int)(items < kMaxItemsGrid ? items : kMaxItemsGrid);
}

// mode: a GuOut, or kCoded (act in fp32 from E4M3FN-coded activations with E8M0 scales xs).
constexpr int kCoded = 16;

static int gateup_common(const xp_dims* dims, int32_t rows, const void* x, const uint8_t* xs,
                         const xp_expert* experts, const void* ws, size_t ws_bytes, float* o0, float* o1, int mode,
                         void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!x || !experts || !ws || !o0 || (mode == kSplit && !o1) || (mode == kCoded && !xs)) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    Plan pl = plan_view(ws, dims, rows);
    const int n_tiles = dims->inter / kTile;
    const int grid = grid_for(rows, dims->top_k, n_tiles);
    const bool wide = (long)rows * dims->top_k * n_tiles <= kWideItems;
    hipStream_t s = (hipStream_t)stream;
    const xp_expert* ex = experts;
    const int32_t* hdr = pl.hdr;
    const int32_t* ent = pl.entry;
    const int4* gp = pl.gu_pass;
    const int E = dims->n_experts, H = dims->hidden, I = dims->inter, k = dims->top_k;
    const uint8_t* no_xs = nullptr;
    float* no_o1 = nullptr;
#define XP_GU_LAUNCH(OUT_, CODED_, XS_, O1_)                                                                   \
    if (wide)                                                                                               \
        hipLaunchKernelGGL((gateup_kernel<OUT_, CODED_, 16>), dim3(grid), dim3(1024), 0, s, ex, x, XS_, hdr, ent, \
                           gp, E, H, I, k, o0, O1_);                                                         \
    else                                                                                                    \
        hipLaunchKernelGGL((gateup_kernel<OUT_, CODED_, 8>), dim3(grid), dim3(512), 0, s, ex, x, XS_, hdr, ent,   \
                           gp, E, H, I, k, o0, O1_);
    if (mode == kSplit) {
        XP_GU_LAUNCH(kSplit, false, no_xs, o1)
    } else if (mode == kActBf16) {
        XP_GU_LAUNCH(kActBf16, false, no_xs, no_o1)
    } else if (mode == kCoded) {
        XP_GU_LAUNCH(kActF32, true, xs, no_o1)
    } else {
        XP_GU_LAUNCH(kActF32, false, no_xs, no_o1)
    }
#undef XP_GU_LAUNCH
    return launch_status();
}

}  // namespace xp

using namespace xp;

XP_API int xp_gateup_rows(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                          const void* workspace, size_t ws_bytes, float* act, void* stream) {
    return gateup_common(dims, rows, x, nullptr, experts, workspace, ws_bytes, act, nullptr, kActF32, stream);
}

XP_API int xp_gateup_rows_split(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                                const void* workspace, size_t ws_bytes, float* g, float* u, void* stream) {
    return gateup_common(dims, rows, x, nullptr, experts, workspace, ws_bytes, g, u, kSplit, stream);
}

XP_API int xp_gateup_rows_act16(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                                const void* workspace, size_t ws_bytes, uint16_t* act16, void* stream) {
    return gateup_common(dims, rows, x, nullptr, experts, workspace, ws_bytes, (float*)act16, nullptr, kActBf16,
                         stream);
}

XP_API int xp_gateup_rows_coded(const xp_dims* dims, int32_t rows, const uint8_t* x_codes, const uint8_t* x_scales,
                                const xp_expert* experts, const void* workspace, size_t ws_bytes, float* act,
                                void* stream) {
    return gateup_common(dims, rows, x_codes, x_scales, experts, workspace, ws_bytes, act, nullptr, kCoded, stream);
}

static int down_common(const xp_dims* dims, int32_t rows, const void* act, const xp_expert* experts,
                       const void* workspace, size_t ws_bytes, float* out, bool a16, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    Plan pl = plan_view(workspace, dims, rows);
    const int n_tiles = dims->hidden / kTile;
    const int grid = grid_for(rows, dims->top_k, n_tiles);
    // two tiles per item where the tiles pair up and the pairs can still give
    // every CU two workgroups (XP_DN_TILES=1 forces one tile)
    const bool pair = XP_DN_TILES == 2 && n_tiles % 2 == 0 && (long)rows * dims->top_k * (n_tiles / 2) > kPairItems;
    hipStream_t s = (hipStream_t)stream;
    const int E = dims->n_experts, H = dims->hidden, I = dims->inter;
    if (a16 && pair)
        hipLaunchKernelGGL((down_kernel<true, 2>), dim3(grid), dim3(512), 0, s, experts, act, pl.hdr, pl.entry,
                           pl.dn_pass, E, H, I, out);
    else if (a16)
        hipLaunchKernelGGL((down_kernel<true, 1>), dim3(grid), dim3(512), 0, s, experts, act, pl.hdr, pl.entry,
                           pl.dn_pass, E, H, I, out);
    else if (pair)
        hipLaunchKernelGGL((down_kernel<false, 2>), dim3(grid), dim3(512), 0, s, experts, act, pl.hdr, pl.entry,
                           pl.dn_pass, E, H, I, out);
    else
        hipLaunchKernelGGL((down_kernel<false, 1>), dim3(grid), dim3(512), 0, s, experts, act, pl.hdr, pl.entry,
                           pl.dn_pass, E, H, I, out);
    return launch_status();
}

XP_API int xp_down_rows(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                        const void* workspace, size_t ws_bytes, float* out, void* stream) {
    return down_common(dims, rows, act, experts, workspace, ws_bytes, out, false, stream);
}

XP_API int xp_down_rows_act16(const xp_dims* dims, int32_t rows, const uint16_t* act16, const xp_expert* experts,
                              const void* workspace, size_t ws_bytes, float* out, void* stream) {
    return down_common(dims, rows, act16, experts, workspace, ws_bytes, out, true, stream);
}

XP_API int xp_route_gateup(const xp_dims* dims, int32_t rows, const float* logits, const uint16_t* x,
                           const xp_expert* experts, int32_t* topk_id, float* topk_w, void* workspace,
                           size_t ws_bytes, float* act, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!logits || !x || !experts || !topk_id || !topk_w || !workspace || !act) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    WsPtrs w = ws_ptrs(workspace, dims, rows);
    RouteIn ri{logits, dims->n_experts, topk_id, topk_w, w};
    if (rows > 1) {
        const int n_tiles = dims->inter / kTile;
        const bool wide = (long)rows * dims->top_k * n_tiles <= kWideItems;
        const int threads = wide ? 1024 : 512;
        const int grid = grid_for(rows, dims->top_k, n_tiles);
        if (rows <= kSmallRows && dims->n_experts <= threads && grid <= XP_ROUTE_FUSED_GRID) {
            // routing inside the gate/up launch
            const Tiers T = current_tiers();
            if (wide)
                hipLaunchKernelGGL(route_gateup_rows_kernel<16>, dim3(grid), dim3(1024), 0, (hipStream_t)stream,
                                   experts, x, ri, rows, dims->hidden, dims->inter, dims->top_k, T, act);
            else
                hipLaunchKernelGGL(route_gateup_rows_kernel<8>, dim3(grid), dim3(512), 0, (hipStream_t)stream,
                                   experts, x, ri, rows, dims->hidden, dims->inter, dims->top_k, T, act);
            return launch_status();
        }
        // the routing launch, then gate/up over the published plan
        st = xp_route_bucket(dims, rows, logits, topk_id, topk_w, workspace, ws_bytes, stream);
        if (st != XP_OK) return st;
        return xp_gateup_rows(dims, rows, x, experts, workspace, ws_bytes, act, stream);
    }
    const int grid = dims->top_k * (dims->inter / kTile);
    hipLaunchKernelGGL(gateup_one_row_kernel, dim3(grid), dim3(1024), 0, (hipStream_t)stream, experts, x, ri,
                       dims->hidden, dims->inter, dims->top_k, act);
    return launch_status();
}

XP_API int xp_down_combine(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                           const float* topk_w, void* workspace, size_t ws_bytes, float* out, float* y,
                           void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!topk_w || !y) return XP_ERR_NULL;
    if (rows == 1 && dims->top_k <= 8) {
        // one row: down and combine in one launch (down_combine_one_row_kernel)
        if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
        if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
        Plan pl = plan_view(workspace, dims, rows);
        const int waves = 8 * ((dims->top_k + 3) / 4);
        hipLaunchKernelGGL(down_combine_one_row_kernel, dim3(dims->hidden / kNarrow), dim3(64 * waves), 0,
                           (hipStream_t)stream, experts, act, pl.entry, pl.dn_pass, topk_w, dims->hidden,
                           dims->inter, dims->top_k, out, y);
        return launch_status();
    }
    if ((long)rows * dims->top_k <= kFusedEntries) {
        // few (row, slot) entries: down and combine in one launch (down_combine_rows_kernel)
        if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
        if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
        Plan pl = plan_view(workspace, dims, rows);
        hipLaunchKernelGGL(down_combine_rows_kernel, dim3(dims->hidden / kNarrow), dim3(1024), 0,
                           (hipStream_t)stream, experts, act, pl.hdr, pl.entry, pl.dn_pass, topk_w, rows,
                           dims->hidden, dims->inter, dims->top_k, out, y);
        return launch_status();
    }
    st = xp_down_rows(dims, rows, act, experts, workspace, ws_bytes, out, stream);
    if (st != XP_OK) return st;
    return xp_combine(dims, rows, out, topk_w, y, stream);
}
