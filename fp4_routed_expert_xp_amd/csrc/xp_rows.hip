// xp_rows.hip — the multi-row gate/up and down passes.
//
// A work item is (pass, tile of 64 output columns). Its workgroup has eight
// waves; wave j owns the 32-weight groups g = j, j+8, j+16, ... of the K axis,
// and lane c owns output column tile*64 + c. For each of its groups a lane
// loads the column's 16 bytes of codes (one coalesced 1 KiB read per wave in
// the packed layout) and one scale byte, decodes the 32 weights once, and runs
// every row of the pass through them: per row a fused multiply-add chain from
// +0 over the group's 32 products in k order, then the group's scale applied
// by one fused multiply-add into the row's partial for leaf j. The eight
// leaves meet in LDS and are added by a fixed tree. Activations are
// wave-uniform, so they are read with scalar loads into SGPRs.
// [#2983, "What this changes" and the rows commit: a pass decodes each
// 32-group once for all of its rows; each row's chain is the one-row chain]
//
// The code for a pass of P rows is the code for one row repeated P times, with
// no value crossing between rows: a row's bits are the same at every P.
// Padding rows (P > real rows) re-read the last real row and are not stored.
#include "xp_common.h"

namespace xp {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Two fp4 codes of byte `B` of `v` -> exact fp32 (low nibble first).
template <int B>
__device__ __forceinline__ f32x2 fp4x2(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, B);
}

__device__ __forceinline__ float e4m3(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

__device__ __forceinline__ float tree8(const float* a, int stride) {
    float s01 = a[0] + a[stride];
    float s23 = a[2 * stride] + a[3 * stride];
    float s45 = a[4 * stride] + a[5 * stride];
    float s67 = a[6 * stride] + a[7 * stride];
    float lo = s01 + s23;
    float hi = s45 + s67;
    return lo + hi;
}

typedef const u32x4 __attribute__((address_space(1)))* gcodes_t;
typedef const uint8_t __attribute__((address_space(1)))* gbytes_t;

// Weight codes are read once: non-temporal loads keep them out of the caches' way.
__device__ __forceinline__ u32x4 load_codes(gcodes_t p) { return __builtin_nontemporal_load(p); }

// ------------------------------------------------------------------ gate/up

// One group for P rows. The group's 32 gate and 32 up weights are decoded
// once into registers; then each row runs its two 32-product chains from +0
// in k order and folds them into its leaf with the group's scales.
template <int P>
__device__ __forceinline__ void gu_group(u32x4 cg, u32x4 cu, uint32_t sg, uint32_t su,
                                         const uint32_t* const (&xr)[P], int g, float (&ag)[P],
                                         float (&au)[P]) {
    float wg[32], wu[32];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f32x2 a;
        a = fp4x2<0>(cg[d]); wg[8 * d + 0] = a.x; wg[8 * d + 1] = a.y;
        a = fp4x2<1>(cg[d]); wg[8 * d + 2] = a.x; wg[8 * d + 3] = a.y;
        a = fp4x2<2>(cg[d]); wg[8 * d + 4] = a.x; wg[8 * d + 5] = a.y;
        a = fp4x2<3>(cg[d]); wg[8 * d + 6] = a.x; wg[8 * d + 7] = a.y;
        a = fp4x2<0>(cu[d]); wu[8 * d + 0] = a.x; wu[8 * d + 1] = a.y;
        a = fp4x2<1>(cu[d]); wu[8 * d + 2] = a.x; wu[8 * d + 3] = a.y;
        a = fp4x2<2>(cu[d]); wu[8 * d + 4] = a.x; wu[8 * d + 5] = a.y;
        a = fp4x2<3>(cu[d]); wu[8 * d + 6] = a.x; wu[8 * d + 7] = a.y;
    }
    const float s_g = e4m3(sg), s_u = e4m3(su);
#pragma unroll
    for (int r = 0; r < P; ++r) {
        // keep one row's activations live at a time (16 SGPRs of bf16 pairs)
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t* xp = xr[r] + 16 * g;
        float pg = 0.0f, pu = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint32_t v = xp[q];
            const float x0 = bf16_lo(v), x1 = bf16_hi(v);
            pg = __builtin_fmaf(wg[2 * q], x0, pg);
            pu = __builtin_fmaf(wu[2 * q], x0, pu);
            pg = __builtin_fmaf(wg[2 * q + 1], x1, pg);
            pu = __builtin_fmaf(wu[2 * q + 1], x1, pu);
        }
        ag[r] = __builtin_fmaf(pg, s_g, ag[r]);
        au[r] = __builtin_fmaf(pu, s_u, au[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int P, bool SPLIT>
__device__ void gu_item(const xp_expert* __restrict__ experts, const uint16_t* __restrict__ x,
                        const int32_t* __restrict__ entry, int4 ps, int tile, int H, int I, int k,
                        float* __restrict__ out0, float* __restrict__ out1, float* red) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int e = ps.x, first = ps.y, real = ps.z;
    const int G = H >> 5;
    const int ng = (G > wave) ? (G - wave + 7) >> 3 : 0;

    const xp_expert ex = experts[e];
    const size_t tile_chunks = (size_t)tile * G * kTile;
    const gcodes_t gc = (gcodes_t)ex.gate_codes + tile_chunks + lane;
    const gcodes_t uc = (gcodes_t)ex.up_codes + tile_chunks + lane;
    const gbytes_t gs = (gbytes_t)ex.gate_scales + tile_chunks + lane;
    const gbytes_t us = (gbytes_t)ex.up_scales + tile_chunks + lane;

    const uint32_t* xr[P];
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const int ent = entry[first + (r < real ? r : real - 1)];
        xr[r] = (const uint32_t*)(x + (size_t)(ent / k) * H);
    }

    float ag[P], au[P];
#pragma unroll
    for (int r = 0; r < P; ++r) { ag[r] = 0.0f; au[r] = 0.0f; }

    constexpr int D = 4;  // groups in flight per wave
    u32x4 bg[D], bu[D];
    uint32_t bsg[D], bsu[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        if (s < ng) {
            const size_t o = (size_t)(wave + 8 * s) * kTile;
            bg[s] = load_codes(gc + o);
            bu[s] = load_codes(uc + o);
            bsg[s] = gs[o];
            bsu[s] = us[o];
        }
    }
    for (int i0 = 0; i0 < ng; i0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            if (i < ng) {
                gu_group<P>(bg[s], bu[s], bsg[s], bsu[s], xr, wave + 8 * i, ag, au);
                if (i + D < ng) {
                    const size_t o = (size_t)(wave + 8 * (i + D)) * kTile;
                    bg[s] = load_codes(gc + o);
                    bu[s] = load_codes(uc + o);
                    bsg[s] = gs[o];
                    bsu[s] = us[o];
                }
            }
        }
    }

    // leaves -> LDS: red[wave][row][gate|up][lane]
#pragma unroll
    for (int r = 0; r < P; ++r) {
        red[((wave * P + r) * 2 + 0) * kTile + lane] = ag[r];
        red[((wave * P + r) * 2 + 1) * kTile + lane] = au[r];
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < P * kTile) {
        const int r = t >> 6, c = t & 63;
        if (r < real) {
            const int stride = P * 2 * kTile;
            const float g = tree8(red + (r * 2 + 0) * kTile + c, stride);
            const float u = tree8(red + (r * 2 + 1) * kTile + c, stride);
            const size_t o = (size_t)entry[first + r] * I + (size_t)tile * kTile + c;
            if (SPLIT) {
                out0[o] = g;
                out1[o] = u;
            } else {
                out0[o] = (g / (1.0f + expf(-g))) * u;
            }
        }
    }
    __syncthreads();
}

template <bool SPLIT>
__global__ __launch_bounds__(512) void gateup_kernel(const xp_expert* __restrict__ experts,
                                                     const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ hdr,
                                                     const int32_t* __restrict__ entry,
                                                     const int4* __restrict__ passes, int H, int I, int k,
                                                     float* __restrict__ out0, float* __restrict__ out1) {
    __shared__ float red[kLeaves * kMaxPass * 2 * kTile];
    const int n_tiles = I / kTile;
    const int n_items = hdr[0] * n_tiles;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pass = item / n_tiles;
        const int tile = item - pass * n_tiles;
        const int4 ps = passes[pass];
        switch (ps.w) {
            case 1: gu_item<1, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 2: gu_item<2, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 3: gu_item<3, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 4: gu_item<4, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 5: gu_item<5, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 6: gu_item<6, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 7: gu_item<7, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            case 8: gu_item<8, SPLIT>(experts, x, entry, ps, tile, H, I, k, out0, out1, red); break;
            default: break;
        }
    }
}

// --------------------------------------------------------------------- down

template <int P>
__device__ __forceinline__ void dn_group(u32x4 c, uint32_t sb, const float* const (&ar)[P], int g,
                                         float (&acc)[P]) {
    float w[32];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f32x2 a;
        a = fp4x2<0>(c[d]); w[8 * d + 0] = a.x; w[8 * d + 1] = a.y;
        a = fp4x2<1>(c[d]); w[8 * d + 2] = a.x; w[8 * d + 3] = a.y;
        a = fp4x2<2>(c[d]); w[8 * d + 4] = a.x; w[8 * d + 5] = a.y;
        a = fp4x2<3>(c[d]); w[8 * d + 6] = a.x; w[8 * d + 7] = a.y;
    }
    const float s = e4m3(sb);
#pragma unroll
    for (int r = 0; r < P; ++r) {
        __builtin_amdgcn_sched_barrier(0);
        const float* xp = ar[r] + 32 * g;
        float p = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) p = __builtin_fmaf(w[t], xp[t], p);
        acc[r] = __builtin_fmaf(p, s, acc[r]);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int P>
__device__ void dn_item(const xp_expert* __restrict__ experts, const float* __restrict__ act,
                        const int32_t* __restrict__ entry, int4 ps, int tile, int H, int I,
                        float* __restrict__ out, float* red) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int e = ps.x, first = ps.y, real = ps.z;
    const int G = I >> 5;
    const int ng = (G > wave) ? (G - wave + 7) >> 3 : 0;

    const xp_expert ex = experts[e];
    const size_t tile_chunks = (size_t)tile * G * kTile;
    const gcodes_t dc = (gcodes_t)ex.down_codes + tile_chunks + lane;
    const gbytes_t ds = (gbytes_t)ex.down_scales + tile_chunks + lane;

    const float* ar[P];
#pragma unroll
    for (int r = 0; r < P; ++r) ar[r] = act + (size_t)entry[first + (r < real ? r : real - 1)] * I;

    float acc[P];
#pragma unroll
    for (int r = 0; r < P; ++r) acc[r] = 0.0f;

    constexpr int D = 4;
    u32x4 bc[D];
    uint32_t bs[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        if (s < ng) {
            const size_t o = (size_t)(wave + 8 * s) * kTile;
            bc[s] = load_codes(dc + o);
            bs[s] = ds[o];
        }
    }
    for (int i0 = 0; i0 < ng; i0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            if (i < ng) {
                dn_group<P>(bc[s], bs[s], ar, wave + 8 * i, acc);
                if (i + D < ng) {
                    const size_t o = (size_t)(wave + 8 * (i + D)) * kTile;
                    bc[s] = load_codes(dc + o);
                    bs[s] = ds[o];
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < P; ++r) red[(wave * P + r) * kTile + lane] = acc[r];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < P * kTile) {
        const int r = t >> 6, c = t & 63;
        if (r < real) {
            const float v = tree8(red + r * kTile + c, P * kTile);
            out[(size_t)entry[first + r] * H + (size_t)tile * kTile + c] = v;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(512) void down_kernel(const xp_expert* __restrict__ experts,
                                                   const float* __restrict__ act,
                                                   const int32_t* __restrict__ hdr,
                                                   const int32_t* __restrict__ entry,
                                                   const int4* __restrict__ passes, int H, int I,
                                                   float* __restrict__ out) {
    __shared__ float red[kLeaves * kMaxPass * kTile];
    const int n_tiles = H / kTile;
    const int n_items = hdr[1] * n_tiles;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int pass = item / n_tiles;
        const int tile = item - pass * n_tiles;
        const int4 ps = passes[pass];
        switch (ps.w) {
            case 1: dn_item<1>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 2: dn_item<2>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 3: dn_item<3>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 4: dn_item<4>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 5: dn_item<5>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 6: dn_item<6>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 7: dn_item<7>(experts, act, entry, ps, tile, H, I, out, red); break;
            case 8: dn_item<8>(experts, act, entry, ps, tile, H, I, out, red); break;
            default: break;
        }
    }
}

static int grid_for(int rows, int k, int n_tiles) {
    long items = (long)rows * k * n_tiles;  // passes <= rows*k
    return (int)(items < kMaxItemsGrid ? items : kMaxItemsGrid);
}

static int gateup_common(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                         const void* ws, size_t ws_bytes, float* o0, float* o1, bool split, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!x || !experts || !ws || !o0 || (split && !o1)) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    Plan pl = plan_view(ws, dims, rows);
    const int grid = grid_for(rows, dims->top_k, dims->inter / kTile);
    hipStream_t s = (hipStream_t)stream;
    if (split)
        hipLaunchKernelGGL(gateup_kernel<true>, dim3(grid), dim3(512), 0, s, experts, x, pl.hdr, pl.entry,
                           pl.gu_pass, dims->hidden, dims->inter, dims->top_k, o0, o1);
    else
        hipLaunchKernelGGL(gateup_kernel<false>, dim3(grid), dim3(512), 0, s, experts, x, pl.hdr, pl.entry,
                           pl.gu_pass, dims->hidden, dims->inter, dims->top_k, o0, (float*)nullptr);
    return launch_status();
}

}  // namespace xp

using namespace xp;

XP_API int xp_gateup_rows(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                          const void* workspace, size_t ws_bytes, float* act, void* stream) {
    return gateup_common(dims, rows, x, experts, workspace, ws_bytes, act, nullptr, false, stream);
}

XP_API int xp_gateup_rows_split(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                                const void* workspace, size_t ws_bytes, float* g, float* u, void* stream) {
    return gateup_common(dims, rows, x, experts, workspace, ws_bytes, g, u, true, stream);
}

XP_API int xp_down_rows(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                        const void* workspace, size_t ws_bytes, float* out, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    Plan pl = plan_view(workspace, dims, rows);
    const int grid = grid_for(rows, dims->top_k, dims->hidden / kTile);
    hipLaunchKernelGGL(down_kernel, dim3(grid), dim3(512), 0, (hipStream_t)stream, experts, act, pl.hdr, pl.entry,
                       pl.dn_pass, dims->hidden, dims->inter, out);
    return launch_status();
}
