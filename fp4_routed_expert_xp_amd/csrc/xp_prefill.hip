// xp_prefill.hip — the prefill-chunk contraction: the same layer math as the
// decode passes for thousands of rows, as a grouped bf16 MFMA contraction.
//
// With about a hundred rows per expert the gate/up and down products are dense
// enough for the matrix cores. Every fp4 weight times its E4M3 scale is exact in
// bf16 (two significant bits times four, exponents well inside bf16's range), so
// the weights are decoded exactly to bf16; x is bf16 already; products are exact
// and accumulate in fp32 inside v_mfma_f32_16x16x32_bf16. act (fp32) enters the
// down contraction as two bf16 halves, hi = its top 16 bits and lo = the top 16
// bits of act - hi, which carry about 16 significant bits (relative error below
// 2^-15 per element). The summation order differs from the decode chain's, so
// results are not bit-equal to the decode path; they meet the same per-row
// tolerance against the float64 definition. [#2983, "What this changes" for the
// layer math; the prefill chunk of 4,096 rows is the prompt step's default size
// on the same site's serving page]
//
// Work items are (expert, block of 128 of its rows, block of 128 output
// columns). A workgroup of four waves takes one item: wave w owns 32 columns
// (two 16-column MFMA tiles) for all 128 rows (eight 16-row slabs), so each wave
// decodes only its own columns' weights, and the rows' activations are staged
// once per workgroup in LDS (double-buffered along K, one 32-wide group per
// step). The grid is persistent; items are laid out expert-major and dealt to
// the eight XCDs in contiguous ranges so the workgroups sharing an expert's rows
// and weights share one L2.
#include "xp_common.h"

#include <algorithm>

namespace xp {

constexpr int kPM = 128;        // rows per item
constexpr int kPN = 128;        // output columns per item (two packed 64-column tiles)
constexpr int kPThreads = 256;  // four waves
constexpr int kAStride = 40;    // bf16 per LDS activation row: 32 + 8 padding (conflict-free 16-byte reads)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;

typedef const uint32_t __attribute__((address_space(1)))* gwords_t;
typedef const uint8_t __attribute__((address_space(1)))* gbytes1_t;

// Item bookkeeping shared by both kernels: per-expert blocks of 128 rows and
// their prefix, rebuilt by each workgroup from the plan's counts.
// sP[e] = row blocks of experts before e (sP[E] = all); all threads call.
__device__ __forceinline__ int block_prefix(const int32_t* __restrict__ count, int E, int* sP, int* swave) {
    const int t = threadIdx.x;
    const int per = (E + kPThreads - 1) / kPThreads;  // experts per thread (E <= 1024 -> <= 4)
    int loc[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = t * per + j;
        loc[j] = (j < per && e < E) ? (count[e] + kPM - 1) / kPM : 0;
        sum += loc[j];
    }
    const int incl = wave_incl_sum(sum);
    const int lane = t & 63, wave = t >> 6;
    if (lane == 63) swave[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += swave[w];
    int run = base + incl - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = t * per + j;
        if (j < per && e < E) sP[e] = run;
        run += loc[j];
    }
    if (t == kPThreads - 1) sP[E] = run;
    __syncthreads();
    return sP[E];
}

// Expert whose row blocks hold block q: the last e with sP[e] <= q (and q < sP[e+1]).
__device__ __forceinline__ int find_expert(const int* sP, int E, int q) {
    int lo = 0, hi = E;  // sP[lo] <= q < sP[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sP[mid] <= q) lo = mid; else hi = mid;
    }
    return lo;
}

// Eight fp4 codes (one dword, k ascending from the low nibble) times scale s -> eight bf16.
// Each product is exact in fp32 and in bf16, so keeping the top 16 bits is exact.
__device__ __forceinline__ bf16x8 decode8(uint32_t v, float s) {
    u32x4v r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x2 p;
        switch (b) {
            case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0); break;
            case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1); break;
            case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2); break;
            default: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3); break;
        }
        const float lo = p.x * s, hi = p.y * s;
        r[b] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float e4m3f(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// Item i -> (expert, first row of the block, rows in the block, column block).
struct Item {
    int e, m0, rows, nt;
};

__device__ __forceinline__ Item item_at(int i, int n_tiles, const int* sP, int E, const int32_t* __restrict__ count) {
    Item it;
    const int q = i / n_tiles;
    it.nt = i - q * n_tiles;
    it.e = find_expert(sP, E, q);
    it.m0 = (q - sP[it.e]) * kPM;
    it.rows = min(kPM, count[it.e] - it.m0);
    return it;
}

// The workgroup's range of items: the eight XCDs take contiguous eighths of
// the item list (workgroup b runs on XCD b % 8), each spread over its workgroups.
struct Deal {
    int first, end, step;
};

__device__ __forceinline__ Deal deal(int total) {
    const int g8 = gridDim.x >> 3;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    Deal d;
    d.first = (int)(((long long)total * x) >> 3) + j;
    d.end = (int)(((long long)total * (x + 1)) >> 3);
    d.step = g8;
    return d;
}

// ------------------------------------------------------------------ gate/up
// act[entry][n] = silu(g) * u for the item's rows and columns, where g and u
// are the rows' products with gate and up (K = hidden).
__global__ __launch_bounds__(kPThreads, 2) void prefill_gateup_kernel(
    const xp_expert* __restrict__ experts, const uint16_t* __restrict__ x, const int32_t* __restrict__ count,
    const int32_t* __restrict__ offset, const int32_t* __restrict__ entry, int E, int k, int H, int I,
    float* __restrict__ act) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kPM * kAStride];
    __shared__ int sEntry[kPM];
    __shared__ int sP[kMaxExperts + 1];
    __shared__ int swave[4];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n_tiles = (I + kPN - 1) / kPN;
    const int total = block_prefix(count, E, sP, swave) * n_tiles;
    const int G = H / 32;
    const Deal dl = deal(total);

    for (int i = dl.first; i < dl.end; i += dl.step) {
        const Item it = item_at(i, n_tiles, sP, E, count);
        if (t < kPM) sEntry[t] = entry[offset[it.e] + it.m0 + min(t, it.rows - 1)];
        __syncthreads();

        // Activation rows staged by all threads: row t/2, 16 bf16 at k offset (t&1)*16.
        const int arow = t >> 1, acol = (t & 1) * 16;
        const uint16_t* xrow = x + (size_t)(sEntry[arow] / k) * H + acol;
        u32x4v ra0, ra1;
        auto load_a = [&](int g) {
            const u32x4v* p = (const u32x4v*)(xrow + 32 * g);
            ra0 = p[0];
            ra1 = p[1];
        };
        auto store_a = [&](int buf) {
            u32x4v* q = (u32x4v*)(&sA[buf][arow * kAStride + acol]);
            q[0] = ra0;
            q[1] = ra1;
        };

        // This wave's columns: packed tile pt, columns c0 .. c0+31 of it.
        const int pt = it.nt * 2 + (wave >> 1);
        const int c0 = (wave & 1) * 32;
        const bool live = pt * 64 < I;
        const xp_expert ex = experts[it.e];
        const int col = c0 + (lane & 15);  // column in the packed tile for the first 16-column MFMA tile
        const int word = lane >> 4;        // which 8 k of the 32-group this lane decodes
        gwords_t gc = (gwords_t)(ex.gate_codes) + (size_t)pt * G * 256 + col * 4 + word;
        gwords_t uc = (gwords_t)(ex.up_codes) + (size_t)pt * G * 256 + col * 4 + word;
        gbytes1_t gs = (gbytes1_t)(ex.gate_scales) + (size_t)pt * G * 64 + col;
        gbytes1_t us = (gbytes1_t)(ex.up_scales) + (size_t)pt * G * 64 + col;

        f32x4 acc[8][2][2];
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                acc[s][c][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc[s][c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        const int slabs = (it.rows + 15) >> 4;

        load_a(0);
        store_a(0);
        __syncthreads();
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) load_a(g + 1);
            if (live) {
                // 16 columns apart: +64 words of codes, +16 scale bytes.
                const uint32_t cg0 = gc[g * 256], cg1 = gc[g * 256 + 64];
                const uint32_t cu0 = uc[g * 256], cu1 = uc[g * 256 + 64];
                const float sg0 = e4m3f(gs[g * 64]), sg1 = e4m3f(gs[g * 64 + 16]);
                const float su0 = e4m3f(us[g * 64]), su1 = e4m3f(us[g * 64 + 16]);
                const bf16x8 bg0 = decode8(cg0, sg0), bg1 = decode8(cg1, sg1);
                const bf16x8 bu0 = decode8(cu0, su0), bu1 = decode8(cu1, su1);
                const uint16_t* a_lds = &sA[g & 1][(lane & 15) * kAStride + word * 8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    if (s < slabs) {
                        const bf16x8 a = *(const bf16x8*)(a_lds + s * 16 * kAStride);
                        acc[s][0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bg0, acc[s][0][0], 0, 0, 0);
                        acc[s][1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bg1, acc[s][1][0], 0, 0, 0);
                        acc[s][0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bu0, acc[s][0][1], 0, 0, 0);
                        acc[s][1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bu1, acc[s][1][1], 0, 0, 0);
                    }
                }
            }
            if (g + 1 < G) store_a((g + 1) & 1);
            __syncthreads();
        }

        if (live) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = s * 16 + (lane >> 4) * 4 + r;
                        if (row < it.rows) {
                            const float gv = acc[s][c][0][r], uv = acc[s][c][1][r];
                            act[(size_t)sEntry[row] * I + pt * 64 + c0 + c * 16 + (lane & 15)] =
                                (gv / (1.0f + expf(-gv))) * uv;
                        }
                    }
                }
            }
        }
        __syncthreads();  // sEntry and sA are rewritten by the next item
    }
}

// --------------------------------------------------------------------- down
// out[entry][n] = the rows' act (fp32, as bf16 hi + lo) times down (K = inter).
__global__ __launch_bounds__(kPThreads, 2) void prefill_down_kernel(
    const xp_expert* __restrict__ experts, const float* __restrict__ act, const int32_t* __restrict__ count,
    const int32_t* __restrict__ offset, const int32_t* __restrict__ entry, int E, int H, int I,
    float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t sHi[2][kPM * kAStride];
    __shared__ __attribute__((aligned(16))) uint16_t sLo[2][kPM * kAStride];
    __shared__ int sEntry[kPM];
    __shared__ int sP[kMaxExperts + 1];
    __shared__ int swave[4];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int n_tiles = (H + kPN - 1) / kPN;
    const int total = block_prefix(count, E, sP, swave) * n_tiles;
    const int G = I / 32;
    const Deal dl = deal(total);

    for (int i = dl.first; i < dl.end; i += dl.step) {
        const Item it = item_at(i, n_tiles, sP, E, count);
        if (t < kPM) sEntry[t] = entry[offset[it.e] + it.m0 + min(t, it.rows - 1)];
        __syncthreads();

        // act rows staged by all threads: row t/2, 16 floats at k offset (t&1)*16,
        // split into bf16 hi (top half) and lo (top half of the remainder).
        const int arow = t >> 1, acol = (t & 1) * 16;
        const float* arow_p = act + (size_t)sEntry[arow] * I + acol;
        u32x4v ra[4];
        auto load_a = [&](int g) {
            const u32x4v* p = (const u32x4v*)(arow_p + 32 * g);
#pragma unroll
            for (int q = 0; q < 4; ++q) ra[q] = p[q];
        };
        auto store_a = [&](int buf) {
            uint32_t hi[8], lo[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t a0 = ra[q >> 1][(q & 1) * 2], a1 = ra[q >> 1][(q & 1) * 2 + 1];
                const float r0 = __uint_as_float(a0) - __uint_as_float(a0 & 0xFFFF0000u);
                const float r1 = __uint_as_float(a1) - __uint_as_float(a1 & 0xFFFF0000u);
                hi[q] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
                lo[q] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
            }
            u32x4v* qh = (u32x4v*)(&sHi[buf][arow * kAStride + acol]);
            u32x4v* ql = (u32x4v*)(&sLo[buf][arow * kAStride + acol]);
            qh[0] = u32x4v{hi[0], hi[1], hi[2], hi[3]};
            qh[1] = u32x4v{hi[4], hi[5], hi[6], hi[7]};
            ql[0] = u32x4v{lo[0], lo[1], lo[2], lo[3]};
            ql[1] = u32x4v{lo[4], lo[5], lo[6], lo[7]};
        };

        const int pt = it.nt * 2 + (wave >> 1);
        const int c0 = (wave & 1) * 32;
        const bool live = pt * 64 < H;
        const xp_expert ex = experts[it.e];
        const int col = c0 + (lane & 15);
        const int word = lane >> 4;
        gwords_t dc = (gwords_t)(ex.down_codes) + (size_t)pt * G * 256 + col * 4 + word;
        gbytes1_t ds = (gbytes1_t)(ex.down_scales) + (size_t)pt * G * 64 + col;

        f32x4 acc[8][2];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            acc[s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int slabs = (it.rows + 15) >> 4;

        load_a(0);
        store_a(0);
        __syncthreads();
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) load_a(g + 1);
            if (live) {
                const uint32_t c0w = dc[g * 256], c1w = dc[g * 256 + 64];
                const float s0 = e4m3f(ds[g * 64]), s1 = e4m3f(ds[g * 64 + 16]);
                const bf16x8 b0 = decode8(c0w, s0), b1 = decode8(c1w, s1);
                const int off = (lane & 15) * kAStride + word * 8;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    if (s < slabs) {
                        const bf16x8 ah = *(const bf16x8*)(&sHi[g & 1][off + s * 16 * kAStride]);
                        const bf16x8 al = *(const bf16x8*)(&sLo[g & 1][off + s * 16 * kAStride]);
                        acc[s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b0, acc[s][0], 0, 0, 0);
                        acc[s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b1, acc[s][1], 0, 0, 0);
                        acc[s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b0, acc[s][0], 0, 0, 0);
                        acc[s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b1, acc[s][1], 0, 0, 0);
                    }
                }
            }
            if (g + 1 < G) store_a((g + 1) & 1);
            __syncthreads();
        }

        if (live) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = s * 16 + (lane >> 4) * 4 + r;
                        if (row < it.rows)
                            out[(size_t)sEntry[row] * H + pt * 64 + c0 + c * 16 + (lane & 15)] = acc[s][c][r];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Persistent grid: two workgroups per CU, a multiple of 8 (one share per XCD),
// never more than an upper bound on the items.
static int prefill_grid(int rows, int k, int E, int n_tiles) {
    static int cap = 0;
    if (cap == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cap = ((2 * cus + 7) / 8) * 8;
    }
    const long long nk = (long long)rows * k;
    const long long blocks = (nk + kPM - 1) / kPM + std::min<long long>(E, nk);  // >= sum of ceil(n_e / 128)
    const long long items = blocks * n_tiles;
    const long long g = ((items + 7) / 8) * 8;
    return (int)std::min<long long>(g, cap);
}

}  // namespace xp

using namespace xp;

XP_API int xp_prefill_gateup(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                             const void* workspace, size_t ws_bytes, float* act, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!x || !experts || !workspace || !act) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    WsPtrs w = ws_ptrs(const_cast<void*>(workspace), dims, rows);
    const int n_tiles = (dims->inter + kPN - 1) / kPN;
    const int grid = prefill_grid(rows, dims->top_k, dims->n_experts, n_tiles);
    hipLaunchKernelGGL(prefill_gateup_kernel, dim3(grid), dim3(kPThreads), 0, (hipStream_t)stream, experts, x,
                       w.count, w.offset, w.entry, dims->n_experts, dims->top_k, dims->hidden, dims->inter, act);
    return launch_status();
}

XP_API int xp_prefill_down(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                           const void* workspace, size_t ws_bytes, float* out, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    WsPtrs w = ws_ptrs(const_cast<void*>(workspace), dims, rows);
    const int n_tiles = (dims->hidden + kPN - 1) / kPN;
    const int grid = prefill_grid(rows, dims->top_k, dims->n_experts, n_tiles);
    hipLaunchKernelGGL(prefill_down_kernel, dim3(grid), dim3(kPThreads), 0, (hipStream_t)stream, experts, act,
                       w.count, w.offset, w.entry, dims->n_experts, dims->hidden, dims->inter, out);
    return launch_status();
}
