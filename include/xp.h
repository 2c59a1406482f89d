/* xp.h — C ABI of libxp.so: the routed-expert decode path of a top-k
 * mixture-of-experts layer over fp4 (e2m1) weights with one E4M3 scale per 32
 * weights, for AMD Instinct MI355X (gfx950).
 *
 * The operation follows the pull-request page "dsv41 metal: decode experts
 * decode an expert's weights once for all of its rows" (TensorFold #2983),
 * cited below as [#2983, <section>]. In short: the rows routed to an expert
 * are grouped into passes whose size follows the rows left (gate/up passes of
 * 2, 4, 6 or 8 rows, down passes of 2 or 4; an expert with one row runs a
 * one-row pass); each pass decodes every 32-weight group of the expert once
 * and applies it to all of the pass's rows; and every row keeps the one-row
 * arithmetic, so a row's output bits do not depend on which other rows share
 * the launch or where they route. [#2983, "What this changes"]
 *
 * Per-row arithmetic (fixed; every pass size runs exactly this per row):
 *   for each group g of 32 consecutive k:
 *       p = +0; for t in 0..31: p = fma(w[32g+t], x[32g+t], p)      (fp32)
 *       part[g mod 8] = fma(p, scale[g], part[g mod 8])             (parts start at +0)
 *   y = ((part0+part1)+(part2+part3))+((part4+part5)+(part6+part7))
 * gate/up epilogue: act = g / (1 + exp(-g)) * u        (fp32, stored as fp32)
 * combine:          y[r] = fma chain from +0 over slots j = 0..k-1 of w[r][j] * out[r][j]
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host". The caller owns and
 *    allocates every buffer; the library allocates nothing on these calls.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls enqueue work
 *    and return without synchronising. Host-visible arguments are validated
 *    synchronously and reported by the return value (an xp_status); device
 *    faults surface at the caller's next synchronisation. XP_ERR_HIP means a
 *    launch was refused by the HIP runtime.
 *  - rows == 0 is valid and enqueues nothing.
 *  - Shapes: hidden and inter are positive multiples of 64; 1 <= top_k <= 16;
 *    top_k <= n_experts <= 1024.
 *  - A workspace holds one routing plan. It is written by xp_route_bucket and
 *    read by the xp_gateup_rows / xp_down_rows calls that follow on the same
 *    stream; use one workspace per plan in flight.
 */
#ifndef XP_H
#define XP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    XP_OK = 0,
    XP_ERR_NULL = -1,      /* a required pointer is NULL */
    XP_ERR_SHAPE = -2,     /* a dimension or row count is out of range */
    XP_ERR_TOPK = -3,      /* top_k out of range */
    XP_ERR_WORKSPACE = -4, /* workspace too small for this many rows */
    XP_ERR_TIERS = -5,     /* malformed pass-size list */
    XP_ERR_HIP = -6        /* the HIP runtime refused a launch */
} xp_status;

/* Layer widths (host struct). */
typedef struct {
    int32_t hidden;    /* H: width of x, y and out */
    int32_t inter;     /* I: expert intermediate width (act) */
    int32_t n_experts; /* E */
    int32_t top_k;     /* k */
} xp_dims;

/* One expert's weights in the PACKED layout (see xp_pack_matrix). gate and up
 * are N = inter columns over K = hidden; down is N = hidden over K = inter.
 * An array of n_experts of these lives in device memory; entries of experts
 * that no row selects are never read and may hold NULL. */
typedef struct {
    const uint8_t* gate_codes;
    const uint8_t* gate_scales;
    const uint8_t* up_codes;
    const uint8_t* up_scales;
    const uint8_t* down_codes;
    const uint8_t* down_scales;
} xp_expert;

/* ---------------------------------------------------------------- weights
 * Weight format [#2983, "What this changes"]: MXFP4-style e2m1 codes, one
 * E4M3FN scale byte per 32 consecutive weights along K.
 *
 * Plain layout (input of xp_pack_matrix): codes [N][K/2] bytes, byte b of
 * column n holds k = 2b in its low nibble and k = 2b+1 in its high nibble;
 * scales [N][K/32] bytes.
 *
 * Packed layout (what the kernels read): columns are taken in tiles of 64;
 * with G = K/32,
 *   codes:  16-byte chunk (n, g) at byte offset ((n/64)*G + g)*1024 + (n%64)*16,
 *           holding the plain bytes 16g .. 16g+15 of column n;
 *   scales: byte (n, g) at ((n/64)*G + g)*64 + n%64.
 * Sizes are those of the plain layout (N*K/2 and N*K/32 bytes). One wave of
 * 64 lanes then reads one group of 64 columns as 1 KiB of contiguous codes
 * and 64 contiguous scale bytes.
 *
 * N must be a positive multiple of 64 and K a positive multiple of 32.
 * In and out buffers must not overlap. */
int xp_pack_matrix(int32_t n, int32_t k, const uint8_t* codes, const uint8_t* scales,
                   uint8_t* packed_codes, uint8_t* packed_scales, void* stream);

/* --------------------------------------------------------------- workspace */

/* Bytes of workspace needed to plan up to max_rows rows (host, pure; 0 on bad dims). */
size_t xp_workspace_bytes(const xp_dims* dims, int32_t max_rows);

/* Byte offsets of the fields of the plan for max_rows rows (host, pure), for
 * callers that read the plan back. A plan made for R rows uses the offsets for
 * R, so the calls that read one plan must pass the same row count:
 *   off[0] header: int32 [0] = gate/up passes, [1] = down passes,
 *                  [32..47] work counters of the prefill calls
 *   off[1] count  int32 [E]          rows per expert
 *   off[2] offset int32 [E+1]        first entry of each expert
 *   off[3] entry  int32 [R*k]        row*k + slot, experts ascending, rows ascending
 *   off[4] gate/up passes int32 [R*k][4] = (expert, first entry, real rows, pass size)
 *   off[5] down passes    int32 [R*k][4]
 * Returns XP_OK or an error for bad dims. */
int xp_workspace_layout(const xp_dims* dims, int32_t max_rows, size_t off[6]);

/* ----------------------------------------------------------- the four calls */

/* Route and bucket rows. For each row: the top_k experts by logit (larger
 * first, equal logits by lower id, NaN after every number) into topk_id
 * [rows][k] int32, and their softmax over the chosen logits, in fp32, into
 * topk_w [rows][k]. Then the plan: a stable bucketing of the rows*k entries by
 * expert and the gate/up and down pass lists under the current pass sizes
 * (xp_set_tiers). logits: [rows][E] fp32.
 * [#2983, "What this changes"; the routing rule itself is not on the page] */
int xp_route_bucket(const xp_dims* dims, int32_t rows, const float* logits, int32_t* topk_id,
                    float* topk_w, void* workspace, size_t ws_bytes, void* stream);

/* Gate/up with the SwiGLU epilogue for every (row, slot) of the plan:
 * act[row][slot][I] fp32 = silu(W_gate x_row) * (W_up x_row). x: [rows][H]
 * bf16 bit patterns. Each pass decodes its expert's groups once for all of
 * its rows; padding rows of a pass repeat its last real row and are never
 * written. [#2983, "What this changes" and the rows commit] */
int xp_gateup_rows(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                   const void* workspace, size_t ws_bytes, float* act, void* stream);

/* Diagnostic twin of xp_gateup_rows: the same passes and per-row chains, but
 * writes the two projections before the epilogue, g and u [rows][k][I] fp32. */
int xp_gateup_rows_split(const xp_dims* dims, int32_t rows, const uint16_t* x,
                         const xp_expert* experts, const void* workspace, size_t ws_bytes,
                         float* g, float* u, void* stream);

/* Down projection for every (row, slot): out[row][slot][H] fp32 = W_down act[row][slot].
 * act: [rows][k][I] fp32 (normally xp_gateup_rows' output). Passes of the
 * down sizes; out is not weighted by the router. [#2983, "What this changes"] */
int xp_down_rows(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                 const void* workspace, size_t ws_bytes, float* out, void* stream);

/* Combine: y[row][H] fp32 = fma chain from +0 over slots in order of
 * topk_w[row][j] * out[row][j]. [#2983, "Receipt": the combine output] */
int xp_combine(const xp_dims* dims, int32_t rows, const float* out, const float* topk_w, float* y,
               void* stream);

/* ------------------------------------------------------------ fused calls
 * The same path in fewer calls, with the same bits. */

/* xp_route_bucket followed by xp_gateup_rows. With one row this is one
 * launch: every workgroup finds the row's expert for its own slot (top-k rounds
 * up to that slot) and starts its weight stream without waiting for a full
 * plan, while one workgroup publishes topk_id, topk_w and the plan exactly as
 * xp_route_bucket writes them. More rows run the two calls. */
int xp_route_gateup(const xp_dims* dims, int32_t rows, const float* logits, const uint16_t* x,
                    const xp_expert* experts, int32_t* topk_id, float* topk_w, void* workspace,
                    size_t ws_bytes, float* act, void* stream);

/* xp_down_rows followed by xp_combine. When rows * top_k <= 64 this is one
 * launch: each workgroup computes 16 output columns of every down pass (the
 * same per-(row, slot, column) chain, leaf order and tree as xp_down_rows),
 * keeps them until every pass is done, then runs the combine for those
 * columns, and writes both out and y. Otherwise the two calls run (two
 * launches on the stream). The bits equal the two calls' in every case. */
int xp_down_combine(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                    const float* topk_w, void* workspace, size_t ws_bytes, float* out, float* y,
                    void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): xp_route_gateup
 * followed by xp_down_combine, the same kernels and the same bits, with no
 * workspace argument. The plan lives in a fixed 1 MiB device array inside the
 * library (each GPU holds its own copy until the process ends); the call makes
 * no allocation. A plan larger than 1 MiB (xp_workspace_bytes(dims, rows) >
 * 1,048,576; for hidden 4096, inter 2048, 256 experts, top-8 that is more than
 * 3,000 rows) is refused with XP_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialised by the caller;
 * calls in order on one stream are safe. The first call on each device looks
 * up the array's address there (make it outside graph capture); XP_ERR_HIP if
 * the runtime refuses. Outputs as the two calls: topk_id/topk_w [rows][k],
 * act [rows][k][I], out [rows][k][H], y [rows][H]. */
int xp_decode_static(const xp_dims* dims, int32_t rows, const float* logits, const uint16_t* x,
                     const xp_expert* experts, int32_t* topk_id, float* topk_w, float* act, float* out,
                     float* y, void* stream);

/* ---------------------------------------------------------- prefill chunk
 * The same layer for a prompt chunk (thousands of rows, about a hundred per
 * expert): gate/up and down as grouped bf16 matrix-core contractions over the
 * plan of xp_route_bucket. Each weight (e2m1 code times its E4M3 scale) is
 * exact in bf16 and x is bf16, so gate/up products are exact with fp32
 * accumulation; act enters down as two bf16 halves (top 16 bits, then the top
 * 16 bits of the remainder), about 16 significant bits. The summation order is
 * the matrix cores', not the decode chain's: results are NOT bit-equal to
 * xp_gateup_rows / xp_down_rows, and meet the per-row tolerance (max |err| /
 * max |ref| <= 1e-3 against the float64 definition) instead. act must be
 * finite for xp_prefill_down (an infinite act gives NaN in out). Any row count
 * is accepted for which x (rows x H bf16) is below 4 GiB: xp_prefill_gateup
 * addresses x with 32-bit offsets and refuses a larger x with XP_ERR_SHAPE
 * (524,287 rows at H = 4096). xp_combine finishes the layer. Each call launches a one-block
 * kernel that zeroes its work counters in the workspace header (int32 slots
 * 32..39 for gate/up, 40..47 for down; the plan is only read), then the
 * contraction, whose workgroups take items from those counters: prefill calls
 * that share a workspace must not overlap. [#2983, "What this changes" for
 * the layer math; the 4,096-row prompt chunk is the serving page's default] */

/* act[row][slot][I] fp32 = silu(W_gate x_row) * (W_up x_row) for every entry of
 * the plan. x: [rows][H] bf16 bit patterns. Same buffers as xp_gateup_rows. */
int xp_prefill_gateup(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                      void* workspace, size_t ws_bytes, float* act, void* stream);

/* out[row][slot][H] fp32 = W_down act[row][slot] for every entry of the plan.
 * Same buffers as xp_down_rows. */
int xp_prefill_down(const xp_dims* dims, int32_t rows, const float* act, const xp_expert* experts,
                    void* workspace, size_t ws_bytes, float* out, void* stream);

/* ------------------------------------------------------ bf16 storage
 * Variants that store act or y as bf16 (the width x arrives in [#2983, "What
 * this changes": bf16 activations into gate/up]) instead of fp32. Each is the
 * fp32 call followed by one rounding, bit for bit: the stored value is the
 * fp32 result rounded to the nearest bf16, ties to even (a NaN stays a NaN,
 * quiet). Same buffers, plans and errors as the fp32 calls they name. */

/* act16[row][slot][I] = bf16 of the act xp_gateup_rows computes. */
int xp_gateup_rows_act16(const xp_dims* dims, int32_t rows, const uint16_t* x, const xp_expert* experts,
                         const void* workspace, size_t ws_bytes, uint16_t* act16, void* stream);

/* out as xp_down_rows computes it from act = act16 widened to fp32 (exact):
 * the same per-row chain, scaled fma and tree. */
int xp_down_rows_act16(const xp_dims* dims, int32_t rows, const uint16_t* act16, const xp_expert* experts,
                       const void* workspace, size_t ws_bytes, float* out, void* stream);

/* y16[row][H] = bf16 of the y xp_combine computes. */
int xp_combine_y16(const xp_dims* dims, int32_t rows, const float* out, const float* topk_w, uint16_t* y16,
                   void* stream);

/* ------------------------------------------------- coded activations
 * Gate/up over activations given as E4M3FN codes [#2983, "What this changes":
 * the chain's 32 products are fp4 weights by E4M3 (or bf16) activations; the
 * commit list registers gate/up kernels over coded activations]. The pages give
 * no activation scale; here each row carries one E8M0 scale per 32 activations
 * (the OCP MX block-scale convention): x[row][k] = e4m3(x_codes[row][k]) *
 * 2^(x_scales[row][k/32] - 127) (scale byte 0xFF is NaN). That value is formed
 * exactly in fp32 and enters the same per-row chain, scaled fma, tree and
 * epilogue as xp_gateup_rows, so the result is bit-equal to xp_gateup_rows on
 * the bf16 activations holding those values (whenever they are bf16 values,
 * i.e. always except below bf16's subnormal range). x_codes: [rows][H] bytes;
 * x_scales: [rows][H/32] bytes. Same plan, workspace, act and errors as
 * xp_gateup_rows. */
int xp_gateup_rows_coded(const xp_dims* dims, int32_t rows, const uint8_t* x_codes, const uint8_t* x_scales,
                         const xp_expert* experts, const void* workspace, size_t ws_bytes, float* act,
                         void* stream);

/* ------------------------------------------------- dense FP8 projections
 * The decode layer's other weight stream: y = x W^T for a dense projection
 * whose weights are E4M3FN bytes with one fp32 scale per 128 x 128 block
 * (value = byte * scale), x bf16 rows, y fp32. A row's result never depends on
 * how many rows share the launch, nor on the `slices` form chosen: [#2983,
 * commit list: the matrix-tile commit for the FP8 projections (#2973), which
 * keeps a row's bits equal to its one-row launch].
 *
 * Arithmetic of y[r][n] (the same in every form and at every row count):
 *   q_j = four v_mfma_f32_16x16x32_bf16 steps from +0 over block j's 128 k, in k order;
 *   c_j = q_j * s[n / 128][j];
 *   y   = pair tree over j in [0, P), P = the power of two >= K/128, with c_j = +0
 *         for j >= K/128, combined level by level as left + right.
 * The products are exact (E4M3FN values are bf16 values) and the sums are the
 * matrix cores' fp32 sums, so y meets the per-row tolerance against the float64
 * definition (max |err| / max |ref| <= 1e-3) and is bit-equal across row counts
 * and forms, not to a sequential fma chain.
 *
 * Shapes: n a positive multiple of 16; k a positive multiple of 128 with
 * k / 128 <= 128. Scales: fp32 [ceil(n/128)][k/128], row-major (a partial last
 * block of columns uses its block's scale). */

/* Bytes of the packed layout of an n x k matrix (n * k), or 0 for a shape the
 * kernels do not take. */
size_t xp_fp8_packed_bytes(int32_t n, int32_t k);

/* Repack w [n][k] (row n = output column n, E4M3FN bytes, k contiguous) into
 * the kernel's layout: per 16-column tile and 128-k block, 2,048 bytes, lane
 * l's 32 bytes at l*32 holding, for g = 0..3, the 8 bytes of column
 * 16*tile + l%16 at k = 128*block + 32g + 8*(l/16) .. +7. One-time setup.
 * w must be 8-byte and packed 16-byte aligned (else XP_ERR_SHAPE). */
int xp_fp8_pack(int32_t n, int32_t k, const uint8_t* w, uint8_t* packed, void* stream);

/* y[rows][n] fp32 = x[rows][k] (bf16 bit patterns) times the packed matrix,
 * scaled per block. x and packed must be 16-byte aligned, scales and y 4-byte
 * aligned (else XP_ERR_SHAPE). slices: 0 picks the form (min(16, P) waves
 * per 16 columns); 1, 2, 4, 8 or 16 forces that many (at most P, and P/slices
 * <= 8), else XP_ERR_SHAPE. Any row count >= 0. */
int xp_fp8_rows(int32_t rows, int32_t n, int32_t k, const uint16_t* x, const uint8_t* packed,
                const float* scales, float* y, int32_t slices, void* stream);

/* The same for fp32 rows x[rows][k] (16-byte aligned). Each x value enters as
 * three bf16 parts whose sum is the value exactly (for |x| >= 2^-110; an
 * infinity or NaN enters as its first part alone), so every product is exact;
 * block root q_j = twelve matrix-core steps from +0: for each 32-k group in k
 * order, its three parts in turn. Same scale, tree, forms, invariance and
 * tolerance as xp_fp8_rows [#2983, commit list: the FP8 commit registers f32
 * and bf16 activation forms]. */
int xp_fp8_rows_f32(int32_t rows, int32_t n, int32_t k, const float* x, const uint8_t* packed,
                    const float* scales, float* y, int32_t slices, void* stream);

/* One launch for several projections that read the same rows x [rows][k]
 * (bf16): matrix i has n = mats[i].n output columns, its packed weights,
 * scales and output y [rows][n] as for xp_fp8_rows. Each matrix's y is bit for
 * bit what xp_fp8_rows gives for it alone with the same `slices` (the form
 * rule and limits of xp_fp8_rows, with k shared by all); the launch saves the
 * fixed cost of one launch per matrix [#2983, commit list: the FP8 commit runs
 * a decode step's dense FP8 projections]. mats: host array of count (1..8)
 * descriptors; errors as xp_fp8_rows, XP_ERR_SHAPE for a count outside 1..8. */
typedef struct {
    int32_t n;
    const uint8_t* packed;
    const float* scales;
    float* y;
} xp_fp8_matrix;

int xp_fp8_rows_multi(int32_t rows, int32_t k, const uint16_t* x, const xp_fp8_matrix* mats, int32_t count,
                      int32_t slices, void* stream);

/* ------------------------------------------------------ measurement probe */

/* Bandwidth probe (not part of the layer): read every byte of the packed
 * weights of the matrices named in `parts` (bit 0 gate, bit 1 up, bit 2 down;
 * 1..7) of the experts ids[0 .. n_ids-1] (device int32, each in [0, n_experts),
 * with non-NULL table entries) once -- codes and scales, hidden * inter *
 * (1/2 + 1/32) bytes per matrix -- with the decode kernels' 16-byte
 * non-temporal loads and no arithmetic on the weights, in one launch of many
 * small workgroups. Its duration is the time the memory system needs to
 * deliver those bytes in one launch: the attainable ceiling a decode launch
 * streaming them (each distinct expert once) is measured against. sink: one
 * device uint32, written only if a folded word equals a fixed constant.
 * n_ids == 0 enqueues nothing; n_ids outside [0, n_experts] or parts outside
 * 1..7 is XP_ERR_SHAPE. */
int xp_stream_weights(const xp_dims* dims, const xp_expert* experts, const int32_t* ids, int32_t n_ids,
                      int32_t parts, uint32_t* sink, void* stream);

/* ------------------------------------------------------------ pass sizes */

/* Set the pass sizes used by later xp_route_bucket calls (host, process-wide,
 * not thread-safe against concurrent route calls). gu: 1..7 strictly
 * increasing sizes in 2..8 for gate/up; dn: the same for down. NULL or a
 * count of 0 restores that list's default ({2,4,6,8} and {2,4}). */
int xp_set_tiers(const int32_t* gu, int32_t n_gu, const int32_t* dn, int32_t n_dn);

/* Current pass sizes (host). gu and dn need room for 8 entries. */
int xp_get_tiers(int32_t* gu, int32_t* n_gu, int32_t* dn, int32_t* n_dn);

/* Human-readable name of a status code (static string). */
const char* xp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* XP_H */
