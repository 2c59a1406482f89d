// synth.hip — device twin of the weight-byte streams of synth/__init__.py.
//
// Integer SplitMix64 only (no floating point), so the bytes equal the host
// generator's exactly. Writes fp4 code bytes and E4M3 scale bytes of one
// matrix of one expert in the plain layout. Input generation only: none of the
// decode method's arithmetic is here, and the product library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define XPS_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t sm(uint64_t x) { return mix64(x + kGolden); }

uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t tensor, uint64_t expert) {
    uint64_t k = sm(seed);
    k = sm(k ^ layer);
    k = sm(k ^ tensor);
    return sm(k ^ expert);
}

// byte b of the codes = byte (b % 8) of output b / 8
__global__ void codes_kernel(uint64_t key, uint64_t nwords, uint64_t* __restrict__ out) {
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (; i < nwords; i += stride) out[i] = mix64(key + (i + 1) * kGolden);
}

__global__ void scales_kernel(uint64_t key, uint64_t n, int emin, uint64_t span, uint8_t* __restrict__ out) {
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        uint64_t w = mix64(key + (i + 1) * kGolden);
        int e = (int)(((w >> 32) * span) >> 32) + emin;
        out[i] = (uint8_t)((e + 7) << 3);
    }
}

// Many experts at once: expert i of the batch uses key keys[i] and is written at out + i*stride.
__global__ void codes_batch_kernel(const uint64_t* __restrict__ keys, int ne, uint64_t nwords, uint64_t stride_words,
                                   uint64_t* __restrict__ out) {
    const uint64_t total = nwords * (uint64_t)ne;
    uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (; t < total; t += step) {
        const uint64_t e = t / nwords, i = t - e * nwords;
        out[e * stride_words + i] = mix64(keys[e] + (i + 1) * kGolden);
    }
}

__global__ void scales_batch_kernel(const uint64_t* __restrict__ keys, int ne, uint64_t n, uint64_t stride, int emin,
                                    uint64_t span, uint8_t* __restrict__ out) {
    const uint64_t total = n * (uint64_t)ne;
    uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (; t < total; t += step) {
        const uint64_t e = t / n, i = t - e * n;
        const uint64_t w = mix64(keys[e] + (i + 1) * kGolden);
        const int x = (int)(((w >> 32) * span) >> 32) + emin;
        out[e * stride + i] = (uint8_t)((x + 7) << 3);
    }
}

}  // namespace

// Codes for experts e0 .. e0+ne-1 (keys_dev: device array of ne stream keys, from
// xps_stream_key). Expert i's [N][K/2] matrix starts at out + i*stride_bytes
// (a multiple of 8).
XPS_API int xps_codes_batch(const uint64_t* keys_dev, int ne, int64_t N, int64_t K, void* out, int64_t stride_bytes,
                            void* stream) {
    uint64_t nbytes = (uint64_t)N * (uint64_t)K / 2;
    if (nbytes % 8 != 0 || stride_bytes % 8 != 0 || !out || !keys_dev || ne <= 0) return -1;
    hipLaunchKernelGGL(codes_batch_kernel, dim3(65536), dim3(256), 0, (hipStream_t)stream, keys_dev, ne, nbytes / 8,
                       (uint64_t)stride_bytes / 8, (uint64_t*)out);
    return (int)hipGetLastError();
}

// Scales for a batch of experts, as xps_codes_batch.
XPS_API int xps_scales_batch(const uint64_t* keys_dev, int ne, int64_t N, int64_t K, int emin, int emax, void* out,
                             int64_t stride_bytes, void* stream) {
    if (!out || !keys_dev || ne <= 0 || emax < emin) return -1;
    uint64_t n = (uint64_t)N * (uint64_t)(K / 32);
    hipLaunchKernelGGL(scales_batch_kernel, dim3(65536), dim3(256), 0, (hipStream_t)stream, keys_dev, ne, n,
                       (uint64_t)stride_bytes, emin, (uint64_t)(emax - emin + 1), (uint8_t*)out);
    return (int)hipGetLastError();
}

// Codes of a [N][K/2] matrix (N*K/2 must be a multiple of 8). Returns 0 or a HIP error.
XPS_API int xps_codes(uint64_t seed, uint64_t layer, uint64_t expert, uint64_t tensor, int64_t N, int64_t K,
                      void* out, void* stream) {
    uint64_t nbytes = (uint64_t)N * (uint64_t)K / 2;
    if (nbytes % 8 != 0 || !out) return -1;
    uint64_t nwords = nbytes / 8;
    uint64_t key = stream_key(seed, layer, tensor, expert);
    unsigned grid = (unsigned)((nwords + 255) / 256);
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(codes_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, key, nwords, (uint64_t*)out);
    return (int)hipGetLastError();
}

// Scales of a [N][K/32] matrix, exponent uniform on {emin..emax}.
XPS_API int xps_scales(uint64_t seed, uint64_t layer, uint64_t expert, uint64_t tensor, int64_t N, int64_t K,
                       int emin, int emax, void* out, void* stream) {
    if (!out || emax < emin) return -1;
    uint64_t n = (uint64_t)N * (uint64_t)(K / 32);
    uint64_t key = stream_key(seed, layer, tensor, expert);
    unsigned grid = (unsigned)((n + 255) / 256);
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(scales_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, key, n, emin,
                       (uint64_t)(emax - emin + 1), (uint8_t*)out);
    return (int)hipGetLastError();
}

// Host copy of the key derivation, for tests that compare against the Python generator.
XPS_API uint64_t xps_stream_key(uint64_t seed, uint64_t layer, uint64_t tensor, uint64_t expert) {
    return stream_key(seed, layer, tensor, expert);
}
