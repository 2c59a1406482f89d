// xp_common.h — internal helpers shared by the libxp HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "xp.h"

#define XP_API extern "C" __attribute__((visibility("default")))

namespace xp {

constexpr int kTile = 64;        // output columns per tile (one wave's lanes)
constexpr int kLeaves = 8;       // partial sums per output: the eight-leaf tree
constexpr int kMaxPass = 8;      // largest pass size the kernels are built for
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kSmallRows = 64;   // route plans up to this many rows in one workgroup
constexpr int kMaxItemsGrid = 8192;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Pass sizes as bit sets: bit p is set when a pass of p rows is allowed (2 <= p <= 8).
struct Tiers {
    uint32_t gu;
    uint32_t dn;
};

// Workspace byte offsets for a plan of up to max_rows rows.
struct WsLayout {
    size_t hdr, count, offset, entry, gu_pass, dn_pass, masks, base, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline bool dims_ok(const xp_dims* d) {
    return d && d->hidden > 0 && d->inter > 0 && d->hidden % 64 == 0 && d->inter % 64 == 0 &&
           d->n_experts >= 1 && d->n_experts <= kMaxExperts;
}

inline int check_dims(const xp_dims* d) {
    if (!d) return XP_ERR_NULL;
    if (d->top_k < 1 || d->top_k > kMaxTopK || (d->n_experts >= 1 && d->top_k > d->n_experts))
        return XP_ERR_TOPK;
    if (!dims_ok(d)) return XP_ERR_SHAPE;
    return XP_OK;
}

inline WsLayout ws_layout(const xp_dims* d, int32_t max_rows) {
    WsLayout L{};
    size_t R = max_rows > 0 ? (size_t)max_rows : 1;
    size_t E = (size_t)d->n_experts;
    size_t entries = R * (size_t)d->top_k;
    size_t nblk = (R + kSmallRows - 1) / kSmallRows;
    size_t o = 0;
    L.hdr = o;     o = align256(o + 64 * sizeof(int32_t));
    L.count = o;   o = align256(o + E * sizeof(int32_t));
    L.offset = o;  o = align256(o + (E + 1) * sizeof(int32_t));
    L.entry = o;   o = align256(o + entries * sizeof(int32_t));
    L.gu_pass = o; o = align256(o + entries * 4 * sizeof(int32_t));
    L.dn_pass = o; o = align256(o + entries * 4 * sizeof(int32_t));
    L.masks = o;   o = align256(o + nblk * E * sizeof(uint64_t));
    L.base = o;    o = align256(o + nblk * E * sizeof(int32_t));
    L.total = o;
    return L;
}

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? XP_OK : XP_ERR_HIP;
}

// Pass sizes in force (set by xp_set_tiers).
Tiers current_tiers();

// Pointers to the fields of one plan inside a workspace.
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

inline WsPtrs ws_ptrs(void* ws, const xp_dims* d, int32_t rows) {
    WsLayout L = ws_layout(d, rows);
    char* b = (char*)ws;
    return WsPtrs{(int32_t*)(b + L.hdr),   (int32_t*)(b + L.count),  (int32_t*)(b + L.offset),
                  (int32_t*)(b + L.entry), (int4*)(b + L.gu_pass),   (int4*)(b + L.dn_pass),
                  (unsigned long long*)(b + L.masks), (int32_t*)(b + L.base)};
}

// Device view of one plan inside a workspace.
struct Plan {
    const int32_t* hdr;
    const int32_t* entry;
    const int4* gu_pass;
    const int4* dn_pass;
};

inline Plan plan_view(const void* ws, const xp_dims* d, int32_t rows) {
    WsLayout L = ws_layout(d, rows);
    const char* b = (const char*)ws;
    return Plan{(const int32_t*)(b + L.hdr), (const int32_t*)(b + L.entry),
                (const int4*)(b + L.gu_pass), (const int4*)(b + L.dn_pass)};
}

}  // namespace xp

// ---------------------------------------------------------------- wave helpers
// Cross-lane steps by DPP (no LDS traffic).
namespace xp {

// v from the DPP source lane; lanes whose source is outside their row, or whose
// row is masked off, get 0 (the identity of a sum).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Largest / smallest unsigned 32-bit value over the wave, returned to every
// lane: six max (min) steps with a DPP source (row shifts 1, 2, 4, 8, then the
// row broadcasts 15 and 31); lanes without a source in a step keep their own
// value, and lane 63 ends with the wave's result. One instruction per step; the
// s_nop pads cover the DPP read-after-VALU-write and EXEC hazards.
#define XP_WAVE_REDUCE_U32(OP)                                              \
    asm volatile("s_nop 4\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t" \
                 "s_nop 1\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t" \
                 "s_nop 1\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t" \
                 "s_nop 1\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t" \
                 "s_nop 1\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t" \
                 "s_nop 1\n\t"                                             \
                 "v_" OP "_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t" \
                 "s_nop 1"                                                   \
                 : "+v"(x))

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    XP_WAVE_REDUCE_U32("max");
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    XP_WAVE_REDUCE_U32("min");
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// fp32 -> bf16 bits, round to nearest, ties to even; a NaN stays a NaN (its
// top half with the quiet bit set).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int wave_incl_sum(int x) {
    x += (int)dpp_or0<0x111, 0xF>((uint32_t)x);
    x += (int)dpp_or0<0x112, 0xF>((uint32_t)x);
    x += (int)dpp_or0<0x114, 0xF>((uint32_t)x);
    x += (int)dpp_or0<0x118, 0xF>((uint32_t)x);
    x += (int)dpp_or0<0x142, 0xA>((uint32_t)x);
    x += (int)dpp_or0<0x143, 0xC>((uint32_t)x);
    return x;
}

}  // namespace xp
