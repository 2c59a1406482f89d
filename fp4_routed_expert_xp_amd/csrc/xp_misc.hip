// xp_misc.hip — combine (router-weighted sum of a row's expert outputs) and
// the one-time weight repack into the kernels' tiled layout.
#include "xp_common.h"

namespace xp {

// y[r][n] = fma chain from +0 over slots j = 0..k-1 of w[r][j] * out[r][j][n];
// Y16 stores it as bf16 (round to nearest even) instead of fp32.
// [#2983, "Receipt": the combine output is the third tensor the probe holds equal]
// Each thread takes V consecutive outputs of a row (V = 4: 16-byte loads of out
// for large batches; V = 1 keeps enough workgroups in flight for small ones).
// H is a multiple of 64, so a run of V never crosses a row.
template <bool Y16, int V>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out, const float* __restrict__ w,
                                                      int R, int H, int k, void* __restrict__ y) {
    typedef __attribute__((ext_vector_type(V))) float fv;
    const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (idx >= (size_t)R * H) return;
    const int r = (int)(idx / H);
    const int n = (int)(idx - (size_t)r * H);
    const float* o = out + (size_t)r * k * H + n;
    const float* wr = w + (size_t)r * k;
    fv s = (fv)0.0f;
    for (int j = 0; j < k; ++j) {
        const float wj = wr[j];
        const fv v = *(const fv*)(o + (size_t)j * H);
#pragma unroll
        for (int c = 0; c < V; ++c) s[c] = __builtin_fmaf(wj, v[c], s[c]);
    }
#pragma unroll
    for (int c = 0; c < V; ++c) {
        if (Y16)
            ((uint16_t*)y)[idx + c] = bf16_rne(s[c]);
        else
            ((float*)y)[idx + c] = s[c];
    }
}

// Batches of at least this many outputs take four per thread.
constexpr size_t kCombineWide = (size_t)4 * 256 * 1024;

// Plain [N][K/2] codes / [N][K/32] scales -> tiles of 64 columns, group-major
// inside a tile (one 1 KiB block of codes and one 64-byte block of scales per
// (tile, group)). One thread moves one (column, group).
__global__ __launch_bounds__(256) void pack_kernel(int N, int K, const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
    const int G = K >> 5;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)N * G) return;
    const int n = (int)(idx / G);
    const int g = (int)(idx - (size_t)n * G);
    const size_t dst = ((size_t)(n / kTile) * G + g) * kTile + (n % kTile);
    const uint4 v = *(const uint4*)(codes + (size_t)n * (K / 2) + (size_t)g * 16);
    *(uint4*)(pcodes + dst * 16) = v;
    pscales[dst] = scales[(size_t)n * G + g];
}

}  // namespace xp

using namespace xp;

static int combine_common(const xp_dims* dims, int32_t rows, const float* out, const float* topk_w, void* y,
                          bool y16, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!out || !topk_w || !y) return XP_ERR_NULL;
    const size_t n = (size_t)rows * dims->hidden;
    hipStream_t s = (hipStream_t)stream;
    const int H = dims->hidden, k = dims->top_k;
    if (n >= kCombineWide) {
        const unsigned grid = (unsigned)((n / 4 + 255) / 256);
        if (y16)
            hipLaunchKernelGGL((combine_kernel<true, 4>), dim3(grid), dim3(256), 0, s, out, topk_w, rows, H, k, y);
        else
            hipLaunchKernelGGL((combine_kernel<false, 4>), dim3(grid), dim3(256), 0, s, out, topk_w, rows, H, k, y);
    } else {
        const unsigned grid = (unsigned)((n + 255) / 256);
        if (y16)
            hipLaunchKernelGGL((combine_kernel<true, 1>), dim3(grid), dim3(256), 0, s, out, topk_w, rows, H, k, y);
        else
            hipLaunchKernelGGL((combine_kernel<false, 1>), dim3(grid), dim3(256), 0, s, out, topk_w, rows, H, k, y);
    }
    return launch_status();
}

XP_API int xp_combine(const xp_dims* dims, int32_t rows, const float* out, const float* topk_w, float* y,
                      void* stream) {
    return combine_common(dims, rows, out, topk_w, y, false, stream);
}

XP_API int xp_combine_y16(const xp_dims* dims, int32_t rows, const float* out, const float* topk_w, uint16_t* y16,
                          void* stream) {
    return combine_common(dims, rows, out, topk_w, y16, true, stream);
}

XP_API int xp_pack_matrix(int32_t n, int32_t k, const uint8_t* codes, const uint8_t* scales, uint8_t* packed_codes,
                          uint8_t* packed_scales, void* stream) {
    if (n <= 0 || k <= 0 || n % kTile != 0 || k % 32 != 0) return XP_ERR_SHAPE;
    if (!codes || !scales || !packed_codes || !packed_scales) return XP_ERR_NULL;
    const size_t items = (size_t)n * (k / 32);
    const unsigned grid = (unsigned)((items + 255) / 256);
    hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, n, k, codes, scales,
                       packed_codes, packed_scales);
    return launch_status();
}
