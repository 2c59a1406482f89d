/* oracle.h — plain CPU reference for the fp4 routed-expert decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library includes, links or
 * calls this code; only the tests, the smoke check and the bench's CPU
 * baseline do. It shares no code, header, table or constant with the GPU path.
 *
 * Source of the method: the pull-request page "dsv41 metal: decode experts
 * decode an expert's weights once for all of its rows" (TensorFold #2983).
 * Weight format: MXFP4-style e2m1 codes with one E4M3 scale per 32 weights
 * along K (that page, "What this changes").
 *
 * Storage layout read here (the plain, unpacked one):
 *   codes  [N][K/2] bytes, byte b of row n holds k = 2b in its low nibble and
 *          k = 2b + 1 in its high nibble;
 *   scales [N][K/32] bytes, one E4M3FN byte per 32 consecutive k.
 * W[n][k] = e2m1(code(n,k)) * e4m3(scale(n, k/32)).
 */
#ifndef XP_ORACLE_H
#define XP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* codecs */
double or_e2m1(unsigned code);
double or_e4m3fn(unsigned byte);
double or_bf16(uint16_t bits);
double or_e8m0(unsigned byte);
void or_dequant_coded(int n, const uint8_t* codes, const uint8_t* scales, double* x);
/* float64 -> nearest bf16 value (ties to even, one rounding), as a double */
double or_round_bf16(double v);

/* routing: top-k by (logit descending, expert id ascending; NaN ranks last),
 * combine weights = softmax over the k chosen logits, in float64. */
void or_route(int R, int E, int k, const float* logits, int32_t* topk_id, double* topk_w);

/* bucketing: stable counting sort of the R*k (row, slot) entries by expert. */
void or_bucket(int R, int E, int k, const int32_t* topk_id, int32_t* count, int32_t* offset,
               int32_t* entry);

/* pass sizes for one expert holding n rows; returns the number of passes. */
int or_passes(int n, const int32_t* tiers, int n_tiers, int32_t* size, int32_t* real, int cap);

/* whole pass plan: rows of (expert, first entry, real rows, pass size), experts ascending. */
int or_plan(int E, const int32_t* count, const int32_t* offset, const int32_t* tiers, int n_tiers,
            int32_t* plan /* [cap][4] */, int cap);

/* float64 definition: y = W x */
void or_matvec(int N, int K, const uint8_t* codes, const uint8_t* scales, const double* x, double* y);
/* act = silu(g) * u, silu(g) = g / (1 + exp(-g)) */
void or_swiglu(int n, const double* g, const double* u, double* act);
/* y = sum_j w[j] * out[j][:] */
void or_combine(int k, int H, const double* w, const double* out, double* y);

/* float64 layer for R rows. experts_* are host arrays of E pointers (NULL allowed
 * for experts no row selects). act [R][k][I], out [R][k][H], y [R][H].
 * act_bf16: act is stored as bf16 (or_round_bf16) before down, as the
 * bf16-storage variant does; act then holds the rounded values.
 * Runs rows x slots over OpenMP threads; returns the thread count used. */
int or_layer(int H, int I, int E, int k, int R, const uint16_t* x_bf16, const float* logits,
             const uint8_t* const* gate_codes, const uint8_t* const* gate_scales,
             const uint8_t* const* up_codes, const uint8_t* const* up_scales,
             const uint8_t* const* down_codes, const uint8_t* const* down_scales,
             int32_t* topk_id, double* topk_w, double* act, double* out, double* y, int act_bf16);
/* or_layer with coded activations: x_codes [R][H] E4M3FN, x_scales [R][H/32] E8M0. */
int or_layer_coded(int H, int I, int E, int k, int R, const uint8_t* x_codes, const uint8_t* x_scales,
                   const float* logits, const uint8_t* const* gate_codes, const uint8_t* const* gate_scales,
                   const uint8_t* const* up_codes, const uint8_t* const* up_scales,
                   const uint8_t* const* down_codes, const uint8_t* const* down_scales,
                   int32_t* topk_id, double* topk_w, double* act, double* out, double* y);

/* fp32 replay of the per-row arithmetic (chain, scaled fma, eight-leaf tree),
 * for x given as float: y[n] for n in [0, N). */
void or_chain32(int N, int K, const uint8_t* codes, const uint8_t* scales, const float* x, float* y);
/* fp32 replay of the combine: fma chain from +0 in slot order */
void or_combine32(int k, int H, const float* w, const float* out, float* y);

/* dense FP8 projection, float64: y [R][N] = x [R][K] (bf16 bits) times the
 * transpose of w [N][K] (E4M3FN bytes) scaled by s [ceil(N/128)][K/128]. */
void or_fp8_proj(int R, int N, int K, const uint16_t* x, const uint8_t* w, const float* s, double* y);
/* the same for fp32 rows x [R][K] */
void or_fp8_proj_f32(int R, int N, int K, const float* x, const uint8_t* w, const float* s, double* y);

int or_omp_threads(void);
void or_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
