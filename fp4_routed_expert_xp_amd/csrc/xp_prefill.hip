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
// Work items are (expert, block of 128 of its rows, block of output columns);
// for gate/up, an expert's last block of at most 32 rows joins the full block
// before it (an item of up to 160 rows, ten slabs), so those rows do not stream
// the expert's weights a second time. Every wave owns its columns for all of
// the item's rows (up to eight or ten 16-row slabs), so each
// wave decodes only its own columns' weights, and the rows' activations are
// staged once per workgroup in LDS. Gate/up: a wave owns 32 columns (two
// 16-column MFMA tiles) of both matrices, in workgroups of four waves (128
// columns), two per CU. Down: a wave owns 64 columns (one packed tile; its hi
// and lo products share the accumulators), in workgroups of eight waves (512
// columns), one per CU, so each staged act tile serves 512 columns; its act is
// four bytes per element against x's two. The grid is
// persistent; items are laid out expert-major and dealt to the eight XCDs in
// contiguous ranges so the workgroups sharing an expert's rows and weights
// share one L2. Each group's matrix work runs in a generated asm body that
// reads the next two slabs' activation fragments while the current two slabs'
// matrix instructions issue (xp_prefill_asm.h).
#include "xp_common.h"

#include <algorithm>

namespace xp {

constexpr int kPM = 128;        // rows per row block
constexpr int kPMGU = 160;      // rows per gate/up item at most: a full block with a last block of <= 32 rows merged
constexpr int kPN = 128;        // output columns per gate/up item (two packed 64-column tiles)
constexpr int kPThreads = 256;  // four waves

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;

typedef const uint32_t __attribute__((address_space(1)))* gwords_t;
typedef const uint8_t __attribute__((address_space(1)))* gbytes1_t;
typedef const void __attribute__((address_space(1)))* gvoid_t;
typedef void __attribute__((address_space(3)))* lvoid_t;
}  // namespace xp

#include "xp_prefill_asm.h"

namespace xp {

// Keeps the compiler from moving memory operations across this point, so the
// vector-memory counts below follow the program order.
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding): vmcnt N (bits 3:0 and 15:14), expcnt
// and, unless LGKM0, lgkmcnt left at their maxima. Issued through the builtin
// so that the compiler's own wait bookkeeping sees it.
template <int N, bool LGKM0>
constexpr int waitcnt_imm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    return (N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8);
}

// Row blocks of an expert with c rows: 128 each, the last one short.
__device__ __forceinline__ int row_blocks(int c) { return (c + kPM - 1) / kPM; }

// Gate/up's row blocks: the same, except that a last block of at most 32 rows
// after a full one joins it (an item of up to 160 rows), so the weights of the
// expert's columns are streamed once for those rows instead of twice.
__device__ __forceinline__ int gu_blocks(int c) {
    const int nb = row_blocks(c);
    return (nb >= 2 && c - (nb - 1) * kPM <= kPMGU - kPM) ? nb - 1 : nb;
}

// Item bookkeeping shared by both kernels: per-expert row blocks (BLOCKS(c)
// for an expert of c rows) and their prefix, rebuilt by each workgroup from
// the plan's counts. sP[e] = row blocks of experts before e (sP[E] = all); all
// threads call.
template <int NT, typename BLOCKS>
__device__ __forceinline__ int block_prefix(const int32_t* __restrict__ count, int E, int* sP, int* swave,
                                            BLOCKS blocks) {
    static_assert(NT >= 256, "E <= 1024 experts at most four per thread");
    const int t = threadIdx.x;
    const int per = (E + NT - 1) / NT;  // experts per thread
    int loc[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = t * per + j;
        loc[j] = (j < per && e < E) ? blocks(count[e]) : 0;
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
    if (t == NT - 1) sP[E] = run;
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

// The same eight products when the scale is a positive power of two: the
// convert applies only the exponent of its fp32 scale operand (its sign and
// mantissa are not used), which for 2^e is the whole scale, so each bf16 is
// code * 2^e exactly, one instruction per two weights.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 decode8_pow2(uint32_t v, float s) {
    u32x4v r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3));
    return __builtin_bit_cast(bf16x8, r);
}

// True on every lane when the four E4M3 scale bytes a..d (each zero-extended
// to 32 bits) of every lane of the wave are positive normal powers of two: no
// byte has a sign or mantissa bit (their OR has none), and then each byte is
// its exponent field alone, which must be non-zero (their minimum is). Then
// decode8_pow2 is exact for the whole group.
__device__ __forceinline__ bool wave_scales_pow2(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t o = a | b | c | d;
    const uint32_t m = min(min(a, b), min(c, d));
    return (__builtin_amdgcn_ballot_w64((o & 0x87u) == 0u) & __builtin_amdgcn_ballot_w64(m != 0u)) ==
           __builtin_amdgcn_read_exec();
}

// silu(g) = g / (1 + e^-g) with the hardware exponential and reciprocal (a few
// ulp each; this path is held to the per-row tolerance against the float64
// definition, not to the decode chain's bits): six instructions instead of a
// library exp and a correctly rounded division. Large negative g gives -0 or
// 0 (e^-g overflows to +inf), large positive g gives g, NaN stays NaN.
__device__ __forceinline__ float silu_fast(float g) {
    const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Item i -> (expert, first row of the block, rows in the block, column block).
// The last of an expert's blocks takes all its remaining rows (up to 160 with
// gate/up's merged blocks), the others 128.
// An expert's items are contiguous. COL_MAJOR orders them column block first:
// the expert's row blocks of one column block are neighbours, so they are in
// flight together and read that column block's weights through one L2 (the
// gate/up order: 1.5% fewer bytes fetched). Otherwise row block first, so one
// block's act rows are read by neighbouring items (the down order: column block
// first fetched 5% more there).
struct Item {
    int e, m0, rows, nt;
};

template <bool COL_MAJOR>
__device__ __forceinline__ Item item_at(int i, int n_tiles, const int* sP, int E, const int32_t* __restrict__ count) {
    Item it;
    if constexpr (COL_MAJOR) {
        it.e = find_expert(sP, E, i / n_tiles);
        const int nb = sP[it.e + 1] - sP[it.e];      // the expert's row blocks
        const int local = i - sP[it.e] * n_tiles;
        it.nt = local / nb;
        it.m0 = (local - it.nt * nb) * kPM;
    } else {
        const int q = i / n_tiles;
        it.nt = i - q * n_tiles;
        it.e = find_expert(sP, E, q);
        it.m0 = (q - sP[it.e]) * kPM;
    }
    const int nb = sP[it.e + 1] - sP[it.e];
    it.rows = it.m0 == (nb - 1) * kPM ? count[it.e] - it.m0 : kPM;
    return it;
}

// Item dealing. The eight XCDs own contiguous eighths of the item list
// (workgroup b runs on XCD b % 8), so the workgroups that share an expert's
// rows and weights share an L2. Items differ up to tenfold in matrix work (1
// to 10 slabs), so a workgroup takes its next item from its XCD's counter and, once
// that range is done, from the other XCDs' in turn. The counters are int32
// slots of the workspace header, zeroed by pf_counters_zero before each launch.
constexpr int kPfCtrGateUp = 32;   // header slots 32 .. 39
constexpr int kPfCtrDown = 40;     // header slots 40 .. 47

__global__ void pf_counters_zero(int32_t* __restrict__ ctr) {
    if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
}

// Next item of this workgroup, or -1 once every range is done (one thread).
__device__ __forceinline__ int next_item(int32_t* ctr, int total) {
    const int x0 = blockIdx.x & 7;
    for (int j = 0; j < 8; ++j) {
        const int x = (x0 + j) & 7;
        const int lo = (int)(((long long)total * x) >> 3), hi = (int)(((long long)total * (x + 1)) >> 3);
        if (lo >= hi) continue;
        const int v = lo + atomicAdd(&ctr[x], 1);
        if (v < hi) return v;
    }
    return -1;
}

// ------------------------------------------------------------------ gate/up
// The K loops are software-pipelined over 32-wide groups. Gate/up stages every
// operand by buffer loads into LDS, a ring of NB groups (below). Down keeps the
// weight words and scale bytes of the next D groups in flight in a register
// ring, each thread keeps the act of the next kDA groups in flight and stages
// the next two groups (as bf16 hi and lo) in LDS at every other group (one
// barrier per two groups). Where the scales are powers of two the weights are
// decoded inside the generated group bodies while the first activation
// fragments are in flight: gate/up its own group's, down the next group's. The
// loop bodies branch only on that per-group choice of decode, uniform per wave
// (D divides the group count; refills past the end re-read the last group), so
// the wait counts follow the rings exactly. NS = 16-row slabs computed: the
// item's rows rounded up to a multiple of 16.
//
// Per kernel: resident workgroups per CU (gate/up; down's follows from its
// workgroup size), the deepest weight ring and down's activation ring.
#ifndef XP_PF_GU_WAVES
#define XP_PF_GU_WAVES 2
#endif
#ifndef XP_PF_GU_DMAX
#define XP_PF_GU_DMAX 4
#endif
// Down runs one workgroup of XP_PF_DN_WG_WAVES waves per CU when that is 8
// (items of 512 columns: every act tile staged once serves twice the columns),
// else two of four waves (items of 256 columns).
#ifndef XP_PF_DN_WG_WAVES
#define XP_PF_DN_WG_WAVES 8
#endif
#define XP_PF_DN_WAVES (8 / XP_PF_DN_WG_WAVES)
constexpr int kDnWaves = XP_PF_DN_WG_WAVES;
constexpr int kDnThreads = 64 * kDnWaves;
constexpr int kDnCols = 64 * kDnWaves;     // output columns per down item
constexpr int kDnRowsPerWave = kPM / kDnWaves;
constexpr int kAQ = kDnRowsPerWave / 8;    // act loads per thread and group
static_assert(kDnWaves == 4 || kDnWaves == 8, "down workgroup of four or eight waves");
#ifndef XP_PF_DN_DMAX
#define XP_PF_DN_DMAX 2
#endif
#ifndef XP_PF_DN_DA
#define XP_PF_DN_DA 2
#endif

struct GuArgs {
    const uint16_t* x;
    const xp_expert* experts;
    float* act;
    int k, H, I, G;
    uint32_t x_bytes;   // bytes of x (below 4 GiB)
};

// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle or
// stride, so a buffer load reads bytes base + offset, and offsets at or past
// the record count read zero.
constexpr int kBufWord3 = 0x00020000;

// Activation tiles of one 32-wide group: 128 rows (gate/up: 160) x 64 B, no padding; the
// four 16-byte chunks of row r sit at chunk position c ^ swz(r % 16), swz(p) =
// ((p >> 1) ^ (p >> 3)) & 3, so a fragment read (16 rows at one chunk) is free
// of bank conflicts whether the LDS serves 8 lanes a cycle from 32 banks or 16
// lanes from 64.
__device__ __forceinline__ int x_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
constexpr int kXTile = kPM * 64;   // activation bytes per group (down's act halves)
constexpr int kXTileGU = kPMGU * 64;   // gate/up's activation tile per group
constexpr int kWTile = 4 * 1024;   // weight code bytes per group: (matrix, packed tile) x 64 columns x 16 B
constexpr int kSTile = 4 * 64;     // scale bytes per group: (matrix, packed tile) x 64 columns
#ifndef XP_PF_GU_NB
#define XP_PF_GU_NB 4              // LDS buffers per ring (groups staged ahead: NB - 1)
#endif

// A wave's four scale bytes (gate tile 0, gate tile 1, up tile 0, up tile 1 of
// its columns), or its four weight words, from the LDS ring, waited for inside
// the asm block: the reads follow direct global-to-LDS loads whose completion
// the kernel orders itself (vmcnt and a barrier), and the compiler, which
// cannot tell the ring's buffers apart, would otherwise wait for every load in
// flight before each read. The activation fragments are read the same way,
// inside the generated group bodies.
__device__ __forceinline__ void lds_scales(uint32_t saddr, uint32_t (&bs)[4]) {
    asm volatile("ds_read_u8 %0, %4\n\tds_read_u8 %1, %4 offset:16\n\t"
                 "ds_read_u8 %2, %4 offset:128\n\tds_read_u8 %3, %4 offset:144\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(bs[0]), "=&v"(bs[1]), "=&v"(bs[2]), "=&v"(bs[3])
                 : "v"(saddr) : "memory");
}
__device__ __forceinline__ void lds_codes(uint32_t waddr, uint32_t (&bc)[4]) {
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:256\n\t"
                 "ds_read_b32 %2, %4 offset:2048\n\tds_read_b32 %3, %4 offset:2304\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(bc[0]), "=&v"(bc[1]), "=&v"(bc[2]), "=&v"(bc[3])
                 : "v"(waddr) : "memory");
}

// Every operand of a group arrives by buffer loads into LDS (the LDS side is
// M0 plus 16 or 4 bytes per lane), NB - 1 groups ahead, into a ring of NB
// buffers: per wave and group one 16-byte load
// per lane for each of two 16-row halves of its 32 activation rows, one 16-byte
// load per lane of weight codes (wave w fetches the 1 KiB of (matrix w/2,
// packed tile w%2): 64 columns x 16 B) and one 4-byte load on lanes 0-15 of that
// block's 64 scale bytes. Activation lane L of a 1 KiB load writes LDS bytes
// 16L .. 16L+15 of it, i.e. row L/4 of the 16 and chunk position L%4, so it
// reads the row's chunk (L%4) ^ swz(L/4).
// Per group step a wave issues those four loads (compiler fences keep the
// order), reads and decodes the group's weights and runs its matrix
// instructions, waits until its own loads of the next group have landed (a
// fixed vmcnt: the loads issued after them), passes a barrier that publishes
// every wave's, and reads the next group's scale bytes. When every scale byte
// of the wave is a power of two (the vote taken on them), the group body reads
// the code words and the first activation fragments together and decodes the
// words while the fragments are in flight; otherwise the words are read and
// decoded in full before the body. A buffer is refilled only after the barrier
// that follows every wave's last read of it.
template <int NS, int D>
__device__ __forceinline__ void gu_item(const GuArgs& a, const Item& it, uint8_t* sX, uint8_t* sW, uint8_t* sS,
                                        const int* sEntry) {
    constexpr int NB = XP_PF_GU_NB;
    static_assert(NB >= 3 && NB <= 8, "ring");
    constexpr int kPerStep = NS > 8 ? 5 : 4;         // loads per wave per group
    constexpr int kAfter = kPerStep * (NB - 2);      // issued after group g+1's, at step g's wait
    static_assert(kAfter <= 63, "vmcnt range");
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int G = a.G, I = a.I;

    // activation sources of this lane (rows 32w + L/4 and 32w + 16 + L/4)
    const int lrow = lane >> 2;
    const int lchunk = (lane & 3) ^ x_swz(lrow);
    // All loads below are buffer loads into LDS: a per-lane 32-bit offset and
    // the group's step as a scalar offset, so they cost no vector instructions
    // per group (x is below 4 GiB, checked by the entry point).
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)a.x_bytes, kBufWord3);
    const uint32_t xo0 = (uint32_t)(sEntry[32 * wave + lrow] / a.k) * (uint32_t)(a.H * 2) + (uint32_t)(lchunk * 16);
    const uint32_t xo1 = (uint32_t)(sEntry[32 * wave + 16 + lrow] / a.k) * (uint32_t)(a.H * 2) + (uint32_t)(lchunk * 16);
    // rows 128 .. 159 (items of more than 8 slabs): eight more per wave, from its
    // lanes 0 .. 31, at rows 128 + 8w + L/4 of the tile (slab 8 + w/2)
    const int erow = 8 * (wave & 1) + ((lane & 31) >> 2);
    const uint32_t xo2 = (uint32_t)(sEntry[kPM + 8 * wave + ((lane & 31) >> 2)] / a.k) * (uint32_t)(a.H * 2) +
                         (uint32_t)((((lane & 3) ^ x_swz(erow))) * 16);
    // weight block fetched by this wave: matrix wave/2, packed tile it.nt*2 + wave%2
    // (tile 0 when past the last tile: I not a multiple of 128; nothing is stored for it)
    const xp_expert ex = a.experts[it.e];
    const int fpt_raw = it.nt * 2 + (wave & 1);
    const int fpt = fpt_raw * 64 < I ? fpt_raw : 0;
    const uint8_t* wbase = (wave >> 1 ? ex.up_codes : ex.gate_codes) + (size_t)fpt * G * 1024;
    const uint8_t* sbase = (wave >> 1 ? ex.up_scales : ex.gate_scales) + (size_t)fpt * G * 64;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, G * 1024, kBufWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, (short)0, G * 64, kBufWord3);
    const uint32_t woff = (uint32_t)lane * 16, soff = (uint32_t)(lane & 15) * 4;
    auto dma = [&](int g) {
        const int gc = min(g, G - 1);
        const int buf = g % NB;
        uint8_t* dx = sX + (size_t)buf * kXTileGU + wave * 2048;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lvoid_t)dx, 16, xo0, (uint32_t)gc * 64, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lvoid_t)(dx + 1024), 16, xo1, (uint32_t)gc * 64, 0, 0);
        if constexpr (NS > 8) {
            if (lane < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lvoid_t)(sX + (size_t)buf * kXTileGU + 8 * 1024 + wave * 512),
                                                         16, xo2, (uint32_t)gc * 64, 0, 0);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lvoid_t)(sW + (size_t)buf * kWTile + wave * 1024), 16, woff,
                                                 (uint32_t)gc * 1024, 0, 0);
        if (lane < 16)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lvoid_t)(sS + (size_t)buf * kSTile + wave * 64), 4, soff,
                                                     (uint32_t)gc * 64, 0, 0);
    };

    // This wave's columns: packed tile pt, columns c0 .. c0+31 of it. A wave past
    // the last tile (I not a multiple of 128) computes on tile 0 and stores nothing.
    const int pt_raw = it.nt * 2 + (wave >> 1);
    const bool live = pt_raw * 64 < I;
    const int pt = live ? pt_raw : 0;
    const int c0 = (wave & 1) * 32;
    const int word = lane >> 4;        // which 8 k of the 32-group this lane decodes
    // its weights in the ring: block (matrix, wave/2), column c0 + t*16 + lane%16, word `word`
    const uint32_t w_lds = (uint32_t)(size_t)(lvoid_t)sW + (wave >> 1) * 1024 + (c0 + (lane & 15)) * 16 + word * 4;
    const uint32_t s_lds = (uint32_t)(size_t)(lvoid_t)sS + (wave >> 1) * 64 + c0 + (lane & 15);
    uint32_t bs[4];
    // fragment reads: row 16s + (lane & 15), chunk `word`, at its swizzled position
    const int frag_off = (lane & 15) * 64 + ((word ^ x_swz(lane & 15)) * 16);
    const uint32_t x_lds = (uint32_t)(size_t)(lvoid_t)sX + frag_off;   // LDS byte address

    f32x4 acc[NS][2][2];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            acc[s][c][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[s][c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // prologue: groups 0 .. NB-2 into buffers 0 .. NB-2; decode group 0
#pragma unroll
    for (int g = 0; g < NB - 1; ++g) {
        dma(g);
        mem_fence_compiler();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm<0, true>());
    __syncthreads();
    lds_scales(s_lds, bs);
    bool pow2 = wave_scales_pow2(bs[0], bs[1], bs[2], bs[3]);

    for (int g0 = 0; g0 < G; g0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int g = g0 + u;
            // group g + NB - 1 into the buffers group g - 1 used (every wave
            // finished reading them before the last barrier)
            dma(g + NB - 1);
            mem_fence_compiler();
            const uint32_t xb = x_lds + (uint32_t)((g % NB) * kXTileGU), wb = w_lds + (uint32_t)((g % NB) * kWTile);
            bf16x8 b[4];
            u32x4v f[2];
            if (pow2) {
                uint32_t n[4][4];
                PfDec::gateup_dec(xb, wb, bs, n, f);
#pragma unroll
                for (int q = 0; q < 4; ++q) b[q] = __builtin_bit_cast(bf16x8, u32x4v{n[q][0], n[q][1], n[q][2], n[q][3]});
            } else {
                uint32_t bc[4];
                lds_codes(wb, bc);
#pragma unroll
                for (int q = 0; q < 4; ++q) b[q] = decode8(bc[q], e4m3f(bs[q]));
                PfDec::frags(xb, f);
            }
            PfGroup<NS>::gateup_tail(acc, b, f, xb);
            // this wave's loads of group g+1 have landed; the barrier publishes
            // every wave's (a plain barrier: __syncthreads' release fence would
            // wait for every load in flight)
            mem_fence_compiler();
            __builtin_amdgcn_s_waitcnt(waitcnt_imm<kAfter, true>());
            __builtin_amdgcn_s_barrier();
            mem_fence_compiler();
            lds_scales(s_lds + (uint32_t)(((g + 1) % NB) * kSTile), bs);
            pow2 = wave_scales_pow2(bs[0], bs[1], bs[2], bs[3]);
        }
    }
    // no load of this item may still be in flight into the buffers
    __builtin_amdgcn_s_waitcnt(waitcnt_imm<0, false>());
    PfGroup<NS>::drain(acc);

    // Rows past it.rows in the last slab repeat the item's last row (sEntry is
    // clamped), so their results are that row's bits: storing them to its
    // address writes the same values, and needs no per-lane branch.
    if (live) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* dst = a.act + (size_t)sEntry[s * 16 + (lane >> 4) * 4 + r] * I + pt * 64 + c0 + (lane & 15);
#pragma unroll
                for (int c = 0; c < 2; ++c) dst[c * 16] = silu_fast(acc[s][c][0][r]) * acc[s][c][1][r];
            }
        }
    }
}

// Slab count (the item's rows in 16-row slabs, 1 to kNSMax) and ring depth (the
// deepest allowed that divides the group count), then the item.
template <int kDMax, int kNSMax, typename F>
__device__ __forceinline__ void dispatch_item(int rows, int G, F&& f) {
    const int ns = (rows + 15) >> 4;
    // ring depths are even (a step is two groups) and G is even (H and I are
    // multiples of 64): the deepest that divides G, else half of it, else 2
    static_assert(kDMax % 2 == 0, "weight ring depth must be even");
    constexpr int dh = kDMax, dl = (kDMax / 2) % 2 == 0 ? kDMax / 2 : 2;
    const int d = (G % dh == 0) ? dh : (G % dl == 0) ? dl : 2;
#define XP_PF_CASE(NS_, D_) \
    if (ns == NS_ && d == D_) { f.template run<NS_, D_>(); return; }
#define XP_PF_CASES(D_) \
    XP_PF_CASE(1, D_) XP_PF_CASE(2, D_) XP_PF_CASE(3, D_) XP_PF_CASE(4, D_) \
    XP_PF_CASE(5, D_) XP_PF_CASE(6, D_) XP_PF_CASE(7, D_) XP_PF_CASE(8, D_) \
    if constexpr (kNSMax > 8) { XP_PF_CASE(9, D_) XP_PF_CASE(10, D_) }
    XP_PF_CASES(dh)
    if constexpr (dl != dh) {
        XP_PF_CASES(dl)
    }
    if constexpr (dl != 2 && dh != 2) {
        XP_PF_CASES(2)
    }
#undef XP_PF_CASES
#undef XP_PF_CASE
}

struct GuRun {
    const GuArgs& a;
    const Item& it;
    uint8_t* sX;
    uint8_t* sW;
    uint8_t* sS;
    const int* sEntry;
    template <int NS, int D>
    __device__ __forceinline__ void run() const { gu_item<NS, D>(a, it, sX, sW, sS, sEntry); }
};

// act[entry][n] = silu(g) * u for the item's rows and columns, where g and u
// are the rows' products with gate and up (K = hidden).
__global__ __launch_bounds__(kPThreads, XP_PF_GU_WAVES) void prefill_gateup_kernel(
    const xp_expert* __restrict__ experts, const uint16_t* __restrict__ x, const int32_t* __restrict__ count,
    const int32_t* __restrict__ offset, const int32_t* __restrict__ entry, int E, int k, int H, int I,
    uint32_t x_bytes, float* __restrict__ act, int32_t* __restrict__ ctr) {
    __shared__ __attribute__((aligned(1024))) uint8_t sX[XP_PF_GU_NB * kXTileGU];
    __shared__ __attribute__((aligned(1024))) uint8_t sW[XP_PF_GU_NB * kWTile];
    __shared__ __attribute__((aligned(256))) uint8_t sS[XP_PF_GU_NB * kSTile];
    __shared__ int sEntry[kPMGU];
    __shared__ int sP[kMaxExperts + 1];
    __shared__ int swave[4];

    const int t = threadIdx.x;
    const int n_tiles = (I + kPN - 1) / kPN;
    const int total = block_prefix<kPThreads>(count, E, sP, swave, [](int c) { return gu_blocks(c); }) * n_tiles;
    const GuArgs a{x, experts, act, k, H, I, H / 32, x_bytes};
    __shared__ int sItem;

    for (;;) {
        if (t == 0) sItem = next_item(ctr, total);
        __syncthreads();
        const int i = sItem;
        if (i < 0) break;
        Item it = item_at<true>(i, n_tiles, sP, E, count);
        // uniform: the expert table entry and the weight bases are then scalar
        it.e = __builtin_amdgcn_readfirstlane(it.e);
        it.nt = __builtin_amdgcn_readfirstlane(it.nt);
        it.m0 = __builtin_amdgcn_readfirstlane(it.m0);
        it.rows = __builtin_amdgcn_readfirstlane(it.rows);
        if (t < kPMGU) sEntry[t] = entry[offset[it.e] + it.m0 + min(t, it.rows - 1)];
        __syncthreads();
        dispatch_item<XP_PF_GU_DMAX, 10>(it.rows, a.G, GuRun{a, it, sX, sW, sS, sEntry});
        __syncthreads();  // sItem, sEntry and the ring are rewritten by the next item
    }
}

// --------------------------------------------------------------------- down
// act (fp32) split into bf16 hi (top half) and lo (top half of act - hi), two
// values per word.
__device__ __forceinline__ void split_pair(uint32_t a0, uint32_t a1, uint32_t& hi, uint32_t& lo) {
    const float r0 = __uint_as_float(a0) - __uint_as_float(a0 & 0xFFFF0000u);
    const float r1 = __uint_as_float(a1) - __uint_as_float(a1 & 0xFFFF0000u);
    hi = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
    lo = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
}

struct DnArgs {
    const float* act;
    const xp_expert* experts;
    float* out;
    int H, I, G;
};

template <int NS, int D, int kDA>
__device__ __forceinline__ void dn_item(const DnArgs& a, const Item& it, uint8_t* sHi, uint8_t* sLo,
                                        const int* sEntry) {
    static_assert(kDA % 2 == 0 && D % kDA == 0, "rings hold whole steps of two groups");
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int G = a.G, H = a.H, I = a.I;

    // act staging: thread (wave w, lane L) moves floats 4c .. 4c+3 (c = L % 8) of
    // the group for rows R w + 8q + L/8, q = 0 .. R/8 - 1 (R = 128 / waves), so
    // the eight lanes of a row read its 128 bytes together and each load
    // instruction touches eight rows' lines. Each 16 bytes become 8 bytes of hi
    // and 8 of lo at the row's chunk c/2 (at its swizzled position, the tile
    // layout of the gate/up activations; the swizzle follows the row's place in
    // its 16-row slab), half c % 2.
    const int c8 = lane & 7;
    const float* arow_q[kAQ];
    uint32_t soff_q[kAQ];
#pragma unroll
    for (int q = 0; q < kAQ; ++q) {
        const int r = kDnRowsPerWave * wave + 8 * q + (lane >> 3);
        arow_q[q] = a.act + (size_t)sEntry[r] * I + 4 * c8;
        soff_q[q] = (uint32_t)(r * 64 + (((c8 >> 1) ^ x_swz(r & 15)) * 16) + (c8 & 1) * 8);
    }
    // Only the waves whose rows fall in the item's NS slabs stage act: the
    // matrix work reads no other rows (the condition is uniform per wave).
    const bool stage = __builtin_amdgcn_readfirstlane(wave) * kDnRowsPerWave < NS * 16;
    u32x4v ra[kDA][kAQ];
    auto load_a = [&](int slot, int g) {
        if (!stage) return;
        g = min(g, G - 1);
#pragma unroll
        for (int q = 0; q < kAQ; ++q) ra[slot][q] = *(const u32x4v*)(arow_q[q] + 32 * g);
    };
    auto store_a = [&](int buf, int slot, int half) {
        if (!stage) return;
        uint8_t* th = (uint8_t*)sHi + (size_t)(buf * 2 + half) * kXTile;
        uint8_t* tl = (uint8_t*)sLo + (size_t)(buf * 2 + half) * kXTile;
#pragma unroll
        for (int q = 0; q < kAQ; ++q) {
            uint32_t h0, h1, l0, l1;
            split_pair(ra[slot][q][0], ra[slot][q][1], h0, l0);
            split_pair(ra[slot][q][2], ra[slot][q][3], h1, l1);
            *(uint2*)(th + soff_q[q]) = make_uint2(h0, h1);
            *(uint2*)(tl + soff_q[q]) = make_uint2(l0, l1);
        }
    };

    // this wave's columns: packed tile pt, 16-column tiles c = 0 .. 3 of it, column
    // 16 c + lane % 16 (tile 0 when past the last tile: nothing is stored for it)
    const int pt_raw = it.nt * kDnWaves + wave;
    const bool live = pt_raw * 64 < H;
    const int pt = live ? pt_raw : 0;
    const xp_expert ex = a.experts[it.e];
    const int col = lane & 15;
    const int word = lane >> 4;
    const int frag_off = (lane & 15) * 64 + ((word ^ x_swz(lane & 15)) * 16);
    // uniform bases and per-lane 32-bit offsets, so the loads take the
    // scalar-base address form
    gwords_t dc = (gwords_t)(ex.down_codes) + (size_t)pt * G * 256;
    gbytes1_t ds = (gbytes1_t)(ex.down_scales) + (size_t)pt * G * 64;
    const uint32_t dco = (uint32_t)(col * 4 + word), dso = (uint32_t)col;
    uint32_t bc[D][4], bs[D][4];
    auto load_b = [&](int slot, int g) {
        g = min(g, G - 1);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bc[slot][c] = dc[(size_t)(g * 256 + 64 * c) + dco];
            bs[slot][c] = ds[(size_t)(g * 64 + 16 * c) + dso];
        }
    };
    bf16x8 bf[2][4];
    auto decode_b = [&](int buf, int slot) {
        if (wave_scales_pow2(bs[slot][0], bs[slot][1], bs[slot][2], bs[slot][3])) {
#pragma unroll
            for (int c = 0; c < 4; ++c) bf[buf][c] = decode8_pow2(bc[slot][c], e4m3f(bs[slot][c]));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) bf[buf][c] = decode8(bc[slot][c], e4m3f(bs[slot][c]));
        }
    };

    // LDS byte addresses of the two act halves
    const uint32_t hi_lds = (uint32_t)(size_t)(lvoid_t)sHi, lo_lds = (uint32_t)(size_t)(lvoid_t)sLo;
    f32x4 acc[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[s][c] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < D; ++u) load_b(u, u);
#pragma unroll
    for (int u = 0; u < kDA; ++u) load_a(u, u);
    store_a(0, 0, 0);
    store_a(0, 1, 1);
    load_a(0, kDA);
    load_a(1, kDA + 1);
    decode_b(0, 0);
    load_b(0, D);
    __syncthreads();

    for (int g0 = 0; g0 < G; g0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int g = g0 + u;
            const int cur = u & 1;
            const int buf = (g >> 1) & 1;  // LDS buffers hold two groups each
            const uint32_t off = (uint32_t)((buf * 2 + cur) * kXTile + frag_off);
            const int nslot = (u + 1) % D;
            // group g's matrix work, with group g+1's weights decoded inside the
            // same asm body (while its first fragment reads are in flight) by the
            // convert that applies a power-of-two scale; when any scale of the
            // wave is not one, they are decoded again in full after it
            uint32_t n[4][4];
            PfGroup<NS>::down_dec(acc, bf[cur], hi_lds + off, lo_lds + off, bc[nslot], bs[nslot], n);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bf[cur ^ 1][c] = __builtin_bit_cast(bf16x8, u32x4v{n[c][0], n[c][1], n[c][2], n[c][3]});
            if (!wave_scales_pow2(bs[nslot][0], bs[nslot][1], bs[nslot][2], bs[nslot][3])) {
#pragma unroll
                for (int c = 0; c < 4; ++c) bf[cur ^ 1][c] = decode8(bc[nslot][c], e4m3f(bs[nslot][c]));
            }
            load_b(nslot, g + 1 + D);
            if (u & 1) {
                const int s0 = (u + 1) % kDA, s1 = (u + 2) % kDA;
                store_a(buf ^ 1, s0, 0);
                store_a(buf ^ 1, s1, 1);
                load_a(s0, g + 1 + kDA);
                load_a(s1, g + 2 + kDA);
                __syncthreads();
            }
        }
    }

    PfGroup<NS>::drain(acc);
    if (live) {
#pragma unroll
        // rows past it.rows repeat the last row (see gu_item): no per-lane branch
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* dst = a.out + (size_t)sEntry[s * 16 + (lane >> 4) * 4 + r] * H + pt * 64 + (lane & 15);
#pragma unroll
                for (int c = 0; c < 4; ++c) dst[c * 16] = acc[s][c][r];
            }
        }
    }
}

struct DnRun {
    const DnArgs& a;
    const Item& it;
    uint8_t* sHi;
    uint8_t* sLo;
    const int* sEntry;
    template <int NS, int D>
    __device__ __forceinline__ void run() const { dn_item<NS, D, XP_PF_DN_DA>(a, it, sHi, sLo, sEntry); }
};

// out[entry][n] = the rows' act (fp32, as bf16 hi + lo) times down (K = inter).
__global__ __launch_bounds__(kDnThreads, XP_PF_DN_WAVES) void prefill_down_kernel(
    const xp_expert* __restrict__ experts, const float* __restrict__ act, const int32_t* __restrict__ count,
    const int32_t* __restrict__ offset, const int32_t* __restrict__ entry, int E, int H, int I,
    float* __restrict__ out, int32_t* __restrict__ ctr) {
    // act halves, two LDS buffers of two groups each: [buffer][group][128 rows x 64 B], swizzled
    __shared__ __attribute__((aligned(1024))) uint8_t sHi[2 * 2 * kXTile];
    __shared__ __attribute__((aligned(1024))) uint8_t sLo[2 * 2 * kXTile];
    __shared__ int sEntry[kPM];
    __shared__ int sP[kMaxExperts + 1];
    __shared__ int swave[kDnWaves];

    const int t = threadIdx.x;
    const int n_tiles = (H + kDnCols - 1) / kDnCols;
    const int total = block_prefix<kDnThreads>(count, E, sP, swave, [](int c) { return row_blocks(c); }) * n_tiles;
    const DnArgs a{act, experts, out, H, I, I / 32};
    __shared__ int sItem;

    for (;;) {
        if (t == 0) sItem = next_item(ctr, total);
        __syncthreads();
        const int i = sItem;
        if (i < 0) break;
        Item it = item_at<false>(i, n_tiles, sP, E, count);
        // uniform: the expert table entry and the weight bases are then scalar
        it.e = __builtin_amdgcn_readfirstlane(it.e);
        it.nt = __builtin_amdgcn_readfirstlane(it.nt);
        it.m0 = __builtin_amdgcn_readfirstlane(it.m0);
        it.rows = __builtin_amdgcn_readfirstlane(it.rows);
        if (t < kPM) sEntry[t] = entry[offset[it.e] + it.m0 + min(t, it.rows - 1)];
        __syncthreads();
        dispatch_item<XP_PF_DN_DMAX, 8>(it.rows, a.G, DnRun{a, it, sHi, sLo, sEntry});
        __syncthreads();
    }
}

// Persistent grid: per_cu workgroups per CU, a multiple of 8 (one share per XCD),
// never more than an upper bound on the items.
static int prefill_grid(int rows, int k, int E, int n_tiles, int per_cu) {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus = n;
    }
    const int cap = ((per_cu * cus + 7) / 8) * 8;
    const long long nk = (long long)rows * k;
    const long long blocks = (nk + kPM - 1) / kPM + std::min<long long>(E, nk);  // >= sum of ceil(n_e / 128)
    const long long items = blocks * n_tiles;
    const long long g = ((items + 7) / 8) * 8;
    return (int)std::min<long long>(g, cap);
}

}  // namespace xp

using namespace xp;

XP_API int xp_prefill_gateup(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                             void* workspace, size_t ws_bytes, float* act, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!x || !experts || !workspace || !act) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    const unsigned long long x_bytes = (unsigned long long)rows * (unsigned long long)dims->hidden * 2ull;
    if (x_bytes >= (1ull << 32)) return XP_ERR_SHAPE;   // x is addressed with 32-bit offsets
    WsPtrs w = ws_ptrs(workspace, dims, rows);
    const int n_tiles = (dims->inter + kPN - 1) / kPN;
    const int grid = prefill_grid(rows, dims->top_k, dims->n_experts, n_tiles, XP_PF_GU_WAVES);
    int32_t* ctr = w.hdr + kPfCtrGateUp;
    hipLaunchKernelGGL(pf_counters_zero, dim3(1), dim3(64), 0, (hipStream_t)stream, ctr);
    hipLaunchKernelGGL(prefill_gateup_kernel, dim3(grid), dim3(kPThreads), 0, (hipStream_t)stream, experts, x,
                       w.count, w.offset, w.entry, dims->n_experts, dims->top_k, dims->hidden, dims->inter,
                       (uint32_t)x_bytes, act, ctr);
    return launch_status();
}

XP_API int xp_prefill_down(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                           void* workspace, size_t ws_bytes, float* out, void* stream) {
    int st = check_dims(dims);
    if (st != XP_OK) return st;
    if (rows < 0) return XP_ERR_SHAPE;
    if (rows == 0) return XP_OK;
    if (!act || !experts || !workspace || !out) return XP_ERR_NULL;
    if (ws_bytes < ws_layout(dims, rows).total) return XP_ERR_WORKSPACE;
    WsPtrs w = ws_ptrs(workspace, dims, rows);
    const int n_tiles = (dims->hidden + kDnCols - 1) / kDnCols;
    const int grid = prefill_grid(rows, dims->top_k, dims->n_experts, n_tiles, XP_PF_DN_WAVES);
    int32_t* ctr = w.hdr + kPfCtrDown;
    hipLaunchKernelGGL(pf_counters_zero, dim3(1), dim3(64), 0, (hipStream_t)stream, ctr);
    hipLaunchKernelGGL(prefill_down_kernel, dim3(grid), dim3(kDnThreads), 0, (hipStream_t)stream, experts, act,
                       w.count, w.offset, w.entry, dims->n_experts, dims->hidden, dims->inter, out, ctr);
    return launch_status();
}
