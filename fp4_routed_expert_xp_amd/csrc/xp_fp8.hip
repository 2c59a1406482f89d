// xp_fp8.hip — dense FP8 projections for decode rows: y = x W^T with W stored
// as E4M3FN bytes and one fp32 scale per 128 x 128 block, x bf16, y fp32.
//
// Source: the matrix-tile commit for the FP8 projections (#2973) listed on the
// TensorFold page "dsv41 metal: decode experts decode an expert's weights once
// for all of its rows" (#2983), commit list: a row's bits do not depend on how
// many rows share the launch or on how K is split across the workgroup, because
// every K-piece's partial result starts from zero and the pieces meet in one
// fixed, zero-padded pair tree.
//
// Arithmetic of one output y[r][n] (every launch form computes exactly this):
//   block root  q_j = four v_mfma_f32_16x16x32_bf16 steps from +0 over the 128 k
//                     of block j, in k order (32 k per step);
//   leaf        c_j = q_j * s[n / 128][j]          (one fp32 multiply);
//   y          = pair tree over j = 0 .. P-1, P the power of two >= K/128, with
//                c_j = +0 for j >= K/128; level by level, node = left + right.
// A row's matrix-core result depends only on its own row of x and the weights,
// so rows never interact; padding rows of a 16-row tile are zero and unstored.
//
// Launch: one workgroup per 16 output columns; its S waves ("slices") each own
// an aligned run of P/S blocks, hold that run's weights in registers for all
// row tiles, reduce their leaves by the low levels of the tree, and meet in LDS
// for the top log2(S) levels. S is a free choice (1..16): the bits are the same.
// Each wave stages its rows of x for two blocks at a time in its own LDS chunk
// with whole-row loads (reading the matrix-core fragments straight from global
// memory touches sixteen rows per instruction and cost about 2.5 us at 16 rows).
#include "xp_common.h"

namespace xp {
namespace fp8 {

constexpr int kCols = 16;        // output columns per workgroup (one MFMA tile)
constexpr int kBlock = 128;      // k per scale block
constexpr int kBlockBytes = 2048;  // packed bytes of one (16-column tile, block)
constexpr int kMaxSlices = 16;
constexpr int kMaxRun = 4;       // blocks per slice held in registers
constexpr int kMaxBlocks = kMaxSlices * kMaxRun;  // K <= 8192

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;

// Eight E4M3FN bytes (two dwords, k order from the low byte) to eight bf16:
// exact, every E4M3FN value is a bf16 value.
__device__ __forceinline__ bf16x8 group_bf16(uint32_t d0, uint32_t d1) {
    const u32x4v r = u32x4v{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true))};
    return __builtin_bit_cast(bf16x8, r);
}

// The operands one slice works on: its weights (32 bytes per lane per block:
// groups 0..3, 8 k each) and scales, and its LDS chunk of x for the current
// 16-row tile: two blocks of bf16 rows at a time, or one block of fp32 rows.
constexpr int kXBlocks = 2;
constexpr int kXRow = 33;   // LDS row of a wave's x chunk: 512 B + 16 B pad, in 16-B units

template <int RUN, bool F32>
struct Slice {
    static constexpr int XB = F32 ? 1 : (RUN < kXBlocks ? RUN : kXBlocks);  // blocks per chunk
    u32x4v w[RUN][2];
    float sc[RUN];
    u32x4v* xs;          // this wave's LDS x chunk: 16 rows x kXRow
    const void* x;
    int R, K, m0;
    bool row_ok;         // row m0 + (lane % 16) exists
    int lane;
    int j0, KB;
};

// Stage x of the chunk starting at block b0 for rows m0 .. m0+15 in this wave's
// LDS chunk, with whole-row coalesced loads (16 B per lane, 512 B per row).
template <int RUN, bool F32>
__device__ __forceinline__ void load_x(Slice<RUN, F32>& sl, int b0) {
    constexpr int n = Slice<RUN, F32>::XB;
    constexpr int lpr = F32 ? 32 : 16 * n, rpi = 64 / lpr;
    const int sub = sl.lane % lpr, rr = sl.lane / lpr;
    const int jb = sl.j0 + b0;
    for (int i = 0; i < 16 / rpi; ++i) {
        const int rl = i * rpi + rr;
        const int r = sl.m0 + rl;
        if (F32) {
            if (r < sl.R && jb < sl.KB)
                sl.xs[rl * kXRow + sub] =
                    *(const u32x4v*)((const float*)sl.x + (size_t)r * sl.K + (size_t)jb * kBlock + 4 * sub);
        } else {
            if (r < sl.R && jb + (sub >> 4) < sl.KB)
                sl.xs[rl * kXRow + sub] =
                    *(const u32x4v*)((const uint16_t*)sl.x + (size_t)r * sl.K + (size_t)jb * kBlock + 8 * sub);
        }
    }
}

// Eight fp32 values as three bf16 parts whose sum is each value exactly (for
// |v| >= 2^-110; non-finite values keep only their first part): v = a + b + c
// with a = v cut to bf16, b = (v - a) cut to bf16, c = v - a - b (both
// differences exact). Pairs pack element 2i in the low half.
__device__ __forceinline__ void split3(const u32x4v& lo, const u32x4v& hi, bf16x8& pa, bf16x8& pb, bf16x8& pc) {
    const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t a[8], b[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = __uint_as_float(u[i]);
        a[i] = u[i] & 0xffff0000u;
        const float r1 = v - __uint_as_float(a[i]);
        b[i] = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(b[i]);
        c[i] = __float_as_uint(r2) & 0xffff0000u;
        if ((u[i] & 0x7f800000u) == 0x7f800000u) b[i] = c[i] = 0u;
    }
    u32x4v A, B, C;
    A.x = (a[0] >> 16) | a[1]; A.y = (a[2] >> 16) | a[3]; A.z = (a[4] >> 16) | a[5]; A.w = (a[6] >> 16) | a[7];
    B.x = (b[0] >> 16) | b[1]; B.y = (b[2] >> 16) | b[3]; B.z = (b[4] >> 16) | b[5]; B.w = (b[6] >> 16) | b[7];
    C.x = (c[0] >> 16) | c[1]; C.y = (c[2] >> 16) | c[3]; C.z = (c[4] >> 16) | c[5]; C.w = (c[6] >> 16) | c[7];
    pa = __builtin_bit_cast(bf16x8, A);
    pb = __builtin_bit_cast(bf16x8, B);
    pc = __builtin_bit_cast(bf16x8, C);
}

// Leaf j0 + b: matrix-core steps from +0 over the block's 128 k in k order,
// then the block scale; +0 for a padding block. bf16 rows: four steps, one per
// 32-k group; fp32 rows: twelve, the group's three bf16 parts in turn. ai: the
// block's place in the LDS chunk. A fragment: lane (c, q) holds row c at
// k = 32g + 8q .. +7.
template <int RUN, bool F32>
__device__ __forceinline__ f32x4 leaf(Slice<RUN, F32>& sl, int b, int ai) {
    if (sl.j0 + b >= sl.KB) return f32x4{0.f, 0.f, 0.f, 0.f};
    // decode here, per row tile, so the x loads are not held behind the weights
    asm volatile("" : "+v"(sl.w[b][0]), "+v"(sl.w[b][1]));
    const int c = sl.lane & 15, q = sl.lane >> 4;
    const u32x4v z = u32x4v{0, 0, 0, 0};
    const bf16x8 wg[4] = {group_bf16(sl.w[b][0].x, sl.w[b][0].y), group_bf16(sl.w[b][0].z, sl.w[b][0].w),
                          group_bf16(sl.w[b][1].x, sl.w[b][1].y), group_bf16(sl.w[b][1].z, sl.w[b][1].w)};
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if constexpr (F32) {
            const u32x4v* p = sl.xs + c * kXRow + 8 * g + 2 * q;
            bf16x8 pa, pb, pc;
            split3(sl.row_ok ? p[0] : z, sl.row_ok ? p[1] : z, pa, pb, pc);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, wg[g], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, wg[g], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pc, wg[g], acc, 0, 0, 0);
        } else {
            const u32x4v v = sl.xs[c * kXRow + 16 * ai + 4 * g + q];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sl.row_ok ? v : z), wg[g],
                                                          acc, 0, 0, 0);
        }
    }
    return acc * sl.sc[b];
}

// Root of the aligned run of LEN leaves starting at b0: (left subtree) + (right
// subtree). A chunk's x is staged on entering the subtree it covers.
template <int RUN, bool F32, int LEN>
struct Run {
    static __device__ __forceinline__ f32x4 root(Slice<RUN, F32>& sl, int b0) {
        if constexpr (LEN == Slice<RUN, F32>::XB) load_x(sl, b0);
        const f32x4 l = Run<RUN, F32, LEN / 2>::root(sl, b0);
        const f32x4 r = Run<RUN, F32, LEN / 2>::root(sl, b0 + LEN / 2);
        return l + r;
    }
};
template <int RUN, bool F32>
struct Run<RUN, F32, 1> {
    static __device__ __forceinline__ f32x4 root(Slice<RUN, F32>& sl, int b0) {
        if constexpr (Slice<RUN, F32>::XB == 1) load_x(sl, b0);
        return leaf(sl, b0, b0 % Slice<RUN, F32>::XB);
    }
};

// Matrices that share x and K, run by one launch: matrix i owns the
// workgroups [tile0[i], tile0[i+1]), one per 16 of its n[i] columns.
constexpr int kMaxMats = 8;
struct MatSet {
    int count;
    int tile0[kMaxMats + 1];
    int n[kMaxMats];
    const uint8_t* pw[kMaxMats];
    const float* scale[kMaxMats];
    float* y[kMaxMats];
};

// One workgroup: 16 columns [16t, 16t + 16), all rows, of one matrix of the
// set. RUN = blocks per slice; F32: rows of x are fp32 (else bf16).
template <int RUN, bool F32>
__global__ __launch_bounds__(1024) void fp8_rows_kernel(int R, int KB, const void* __restrict__ x, MatSet ms) {
    __shared__ float red[kMaxSlices * 4 * 64];
    __shared__ u32x4v xsh[kMaxSlices * 16 * kXRow];
    const int S = blockDim.x >> 6;
    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, q = lane >> 4;
    // this workgroup's matrix (selects with constant indices keep the set in scalar registers)
    int m = 0;
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
        if (i < ms.count && (int)blockIdx.x >= ms.tile0[i]) m = i;
    int N = ms.n[0], t0 = ms.tile0[0];
    const uint8_t* __restrict__ pw = ms.pw[0];
    const float* __restrict__ scale = ms.scale[0];
    float* __restrict__ y = ms.y[0];
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
        if (i == m) { N = ms.n[i]; t0 = ms.tile0[i]; pw = ms.pw[i]; scale = ms.scale[i]; y = ms.y[i]; }
    const int t = (int)blockIdx.x - t0;
    const int K = KB * kBlock;

    Slice<RUN, F32> sl;
    sl.xs = xsh + slice * 16 * kXRow;
    sl.x = x;
    sl.R = R;
    sl.K = K;
    sl.lane = lane;
    sl.j0 = slice * RUN;
    sl.KB = KB;
    const float* srow = scale + (size_t)(t >> 3) * KB;
#pragma unroll
    for (int b = 0; b < RUN; ++b) {
        const int j = sl.j0 + b;
        if (j < KB) {
            const u32x4v* p = (const u32x4v*)(pw + ((size_t)t * KB + j) * kBlockBytes + lane * 32);
            sl.w[b][0] = __builtin_nontemporal_load(p);
            sl.w[b][1] = __builtin_nontemporal_load(p + 1);
            sl.sc[b] = srow[j];
        } else {
            sl.w[b][0] = u32x4v{0, 0, 0, 0};
            sl.w[b][1] = u32x4v{0, 0, 0, 0};
            sl.sc[b] = 0.0f;
        }
    }

    for (int m0 = 0; m0 < R; m0 += 16) {
        sl.m0 = m0;
        sl.row_ok = m0 + c < R;
        // low levels of the pair tree: the slice's run
        const f32x4 v = Run<RUN, F32, RUN>::root(sl, 0);
        if (S == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + 4 * q + i;  // C row 4q + i, column c
                if (r < R) y[(size_t)r * N + (size_t)t * kCols + c] = v[i];
            }
            continue;
        }
        // top levels across slices, through LDS; wave i finishes C rows 4q + i
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(slice * 4 + i) * 64 + lane] = v[i];
        __syncthreads();
        for (int i = slice; i < 4; i += S) {
            float u[kMaxSlices];
#pragma unroll
            for (int s = 0; s < kMaxSlices; ++s) u[s] = s < S ? red[(s * 4 + i) * 64 + lane] : 0.0f;
#pragma unroll
            for (int st = 1; st < kMaxSlices; st *= 2)
#pragma unroll
                for (int s = 0; s < kMaxSlices; s += 2 * st)
                    if (s + st < S) u[s] = u[s] + u[s + st];
            const int r = m0 + 4 * q + i;
            if (r < R) y[(size_t)r * N + (size_t)t * kCols + c] = u[0];
        }
        __syncthreads();
    }
}

// Plain [N][K] bytes -> the kernel's tiles: per (16-column tile t, block j)
// 2,048 bytes, lane l's 32 at l * 32: for groups g = 0..3, the 8 bytes of
// column 16t + l % 16 at k = 128j + 32g + 8(l / 16) .. +7.
__global__ __launch_bounds__(256) void fp8_pack_kernel(int N, int K, const uint8_t* __restrict__ w,
                                                       uint8_t* __restrict__ pw) {
    const int KB = K / kBlock;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)(N / kCols) * KB * 64) return;
    const int lane = (int)(idx & 63);
    const size_t tj = idx >> 6;
    const int t = (int)(tj / KB), j = (int)(tj - (size_t)t * KB);
    const int n = t * kCols + (lane & 15);
    const uint8_t* src = w + (size_t)n * K + (size_t)j * kBlock + 8 * (lane >> 4);
    uint2* dst = (uint2*)(pw + tj * kBlockBytes + lane * 32);
#pragma unroll
    for (int g = 0; g < 4; ++g) dst[g] = *(const uint2*)(src + 32 * g);
}

static int next_pow2(int v) {
    int p = 1;
    while (p < v) p *= 2;
    return p;
}

}  // namespace fp8
}  // namespace xp

using namespace xp;
using namespace xp::fp8;

static bool fp8_shape_ok(int32_t n, int32_t k) {
    return n > 0 && k > 0 && n % kCols == 0 && k % kBlock == 0 && k / kBlock <= kMaxBlocks;
}

XP_API size_t xp_fp8_packed_bytes(int32_t n, int32_t k) {
    return fp8_shape_ok(n, k) ? (size_t)n * (size_t)k : 0;
}

static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

XP_API int xp_fp8_pack(int32_t n, int32_t k, const uint8_t* w, uint8_t* packed, void* stream) {
    if (!fp8_shape_ok(n, k)) return XP_ERR_SHAPE;
    if (!w || !packed) return XP_ERR_NULL;
    if (!aligned(w, 8) || !aligned(packed, 16)) return XP_ERR_SHAPE;
    const size_t threads = (size_t)(n / kCols) * (k / kBlock) * 64;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(fp8_pack_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, n, k, w, packed);
    return launch_status();
}

static int fp8_rows_set(int32_t rows, int32_t k, const void* x, const xp_fp8_matrix* mats, int32_t count,
                        int32_t slices, bool f32, void* stream) {
    if (rows < 0 || k <= 0 || count < 1 || count > kMaxMats) return XP_ERR_SHAPE;
    if (!mats) return XP_ERR_NULL;
    MatSet ms{};
    ms.count = count;
    long long tiles = 0;
    for (int i = 0; i < count; ++i) {
        if (!fp8_shape_ok(mats[i].n, k)) return XP_ERR_SHAPE;
        if (rows > 0 && (!mats[i].packed || !mats[i].scales || !mats[i].y)) return XP_ERR_NULL;
        if (rows > 0 && (!aligned(mats[i].packed, 16) || !aligned(mats[i].scales, 4) || !aligned(mats[i].y, 4)))
            return XP_ERR_SHAPE;
        ms.tile0[i] = (int)tiles;
        ms.n[i] = mats[i].n;
        ms.pw[i] = mats[i].packed;
        ms.scale[i] = mats[i].scales;
        ms.y[i] = mats[i].y;
        tiles += mats[i].n / kCols;
    }
    if (tiles > 0x7fffffffLL) return XP_ERR_SHAPE;
    ms.tile0[count] = (int)tiles;
    if (rows == 0) return XP_OK;
    if (!x) return XP_ERR_NULL;
    if (!aligned(x, 16)) return XP_ERR_SHAPE;
    const int KB = k / kBlock;
    const int P = next_pow2(KB);
    int S = slices;
    if (S == 0) S = P < kMaxSlices ? P : kMaxSlices;
    if (S < 1 || S > kMaxSlices || (S & (S - 1)) != 0 || S > P) return XP_ERR_SHAPE;
    const int run = P / S;
    if (run > kMaxRun) return XP_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)tiles), block(64 * S);
#define XP_FP8_LAUNCH(RUN_, F32_)                                                                            \
    hipLaunchKernelGGL((fp8_rows_kernel<RUN_, F32_>), grid, block, 0, s, rows, KB, x, ms)
    if (f32) {
        switch (run) {
            case 1: XP_FP8_LAUNCH(1, true); break;
            case 2: XP_FP8_LAUNCH(2, true); break;
            case 4: XP_FP8_LAUNCH(4, true); break;
            default: return XP_ERR_SHAPE;
        }
    } else {
        switch (run) {
            case 1: XP_FP8_LAUNCH(1, false); break;
            case 2: XP_FP8_LAUNCH(2, false); break;
            case 4: XP_FP8_LAUNCH(4, false); break;
            default: return XP_ERR_SHAPE;
        }
    }
#undef XP_FP8_LAUNCH
    return launch_status();
}

static int fp8_rows_one(int32_t rows, int32_t n, int32_t k, const void* x, const uint8_t* packed,
                        const float* scales, float* y, int32_t slices, bool f32, void* stream) {
    if (!fp8_shape_ok(n, k) || rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!x || !packed || !scales || !y) return XP_ERR_NULL;
    const xp_fp8_matrix m{n, packed, scales, y};
    return fp8_rows_set(rows, k, x, &m, 1, slices, f32, stream);
}

XP_API int xp_fp8_rows(int32_t rows, int32_t n, int32_t k, const uint16_t* x, const uint8_t* packed,
                       const float* scales, float* y, int32_t slices, void* stream) {
    return fp8_rows_one(rows, n, k, x, packed, scales, y, slices, false, stream);
}

XP_API int xp_fp8_rows_f32(int32_t rows, int32_t n, int32_t k, const float* x, const uint8_t* packed,
                           const float* scales, float* y, int32_t slices, void* stream) {
    return fp8_rows_one(rows, n, k, x, packed, scales, y, slices, true, stream);
}

XP_API int xp_fp8_rows_multi(int32_t rows, int32_t k, const uint16_t* x, const xp_fp8_matrix* mats, int32_t count,
                             int32_t slices, void* stream) {
    return fp8_rows_set(rows, k, x, mats, count, slices, false, stream);
}
