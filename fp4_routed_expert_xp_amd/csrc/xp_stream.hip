// xp_stream.hip — a read-only bandwidth probe over the decode path's weight bytes.
//
// It reads every byte of the packed weights (codes and scales of gate, up and
// down) of a list of experts once, with the decode kernels' load form (16-byte
// non-temporal loads, each wave covering 1 KiB of contiguous bytes per
// instruction), and does no arithmetic on them beyond folding the words into
// one value per thread, so its time is what the memory system needs to deliver
// those bytes: the ceiling against which a decode layer's weight stream is
// measured. It writes nothing unless a folded value equals a fixed constant.
#include "xp_common.h"

namespace xp {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 4;                                      // 16-byte loads per thread per chunk
constexpr size_t kStreamChunk = (size_t)kStreamThreads * 16 * kStreamLoads;  // 16 KiB

typedef const u32x4 __attribute__((address_space(1)))* gvec_t;

// Work item = (expert of the list, matrix, codes or scales, chunk of 16 KiB)
// over the matrices named in `parts` (bit 0 gate, bit 1 up, bit 2 down): per
// matrix seg_codes bytes of codes, then seg_scales bytes of scales; a ragged
// last chunk is bounded per load.
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const xp_expert* __restrict__ experts,
                                                                const int32_t* __restrict__ ids, int n_ids,
                                                                int parts, size_t seg_codes, size_t seg_scales,
                                                                int chunks_codes, int chunks_scales,
                                                                uint32_t* __restrict__ sink) {
    const int per_matrix = chunks_codes + chunks_scales;
    const int n_mat = __builtin_popcount(parts);
    const int item = blockIdx.x;
    const int ei = item / (n_mat * per_matrix);
    if (ei >= n_ids) return;
    int r = item - ei * n_mat * per_matrix;
    const int mi = r / per_matrix;   // mi-th matrix named in parts
    r -= mi * per_matrix;
    int m = 0;
    for (int seen = -1; m < 3; ++m) {
        if ((parts >> m) & 1) ++seen;
        if (seen == mi) break;
    }
    const xp_expert ex = experts[ids[ei]];
    const uint8_t* base;
    size_t len;
    int chunk;
    if (r < chunks_codes) {
        chunk = r;
        base = m == 0 ? ex.gate_codes : m == 1 ? ex.up_codes : ex.down_codes;
        len = seg_codes;
    } else {
        chunk = r - chunks_codes;
        base = m == 0 ? ex.gate_scales : m == 1 ? ex.up_scales : ex.down_scales;
        len = seg_scales;
    }
    const size_t c0 = (size_t)chunk * kStreamChunk;
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kStreamLoads; ++i) {
        const size_t off = c0 + (size_t)i * kStreamThreads * 16 + (size_t)threadIdx.x * 16;
        if (off + 16 <= len) {
            const u32x4 v = __builtin_nontemporal_load((gvec_t)(base + off));
            acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace xp

using namespace xp;

XP_API int xp_stream_weights(const xp_dims* dims, const xp_expert* experts, const int32_t* ids, int32_t n_ids,
                             int32_t parts, uint32_t* sink, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (n_ids < 0 || n_ids > dims->n_experts || parts < 1 || parts > 7) return XP_ERR_SHAPE;
    if (n_ids == 0) return XP_OK;
    if (!experts || !ids || !sink) return XP_ERR_NULL;
    const size_t weights = (size_t)dims->hidden * dims->inter;
    const size_t seg_codes = weights / 2, seg_scales = weights / 32;
    const int cc = (int)((seg_codes + kStreamChunk - 1) / kStreamChunk);
    const int cs = (int)((seg_scales + kStreamChunk - 1) / kStreamChunk);
    const long items = (long)n_ids * __builtin_popcount(parts) * (cc + cs);
    if (items > 0x7fffffffL) return XP_ERR_SHAPE;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)items), dim3(kStreamThreads), 0, (hipStream_t)stream, experts,
                       ids, n_ids, parts, seg_codes, seg_scales, cc, cs, sink);
    return launch_status();
}
