/* oracle.c — plain, slow CPU reference for the fp4 routed-expert decode path.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's
 * CPU-baseline leg. The product library never links or calls it, and it
 * shares no code with the GPU kernels.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off -fopenmp (no fast-math).
 *
 * Citations name the page "dsv41 metal: decode experts decode an expert's
 * weights once for all of its rows" (TensorFold pull request #2983), written
 * below as [#2983, <section>]. Where the page is silent, the reading used is
 * stated at the function.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codecs */

/* e2m1 (fp4): bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa;
 * exponent field 0 is subnormal with value m/2. Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
 * [#2983, "What this changes": the expert weights are fp4 products] */
double or_e2m1(unsigned code) {
    code &= 15u;
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E4M3FN (OCP 8-bit float): bit 7 sign, bits 6..3 exponent with bias 7,
 * bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with
 * mantissa 7 is NaN; there is no infinity. [#2983, "What this changes": one
 * E4M3 scale per group of 32 products] */
double or_e4m3fn(unsigned byte) {
    byte &= 255u;
    int sign = (byte >> 7) & 1;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* E8M0 (the OCP MX scale format): an unsigned biased exponent, value
 * 2^(byte - 127); 0xFF is NaN. Reading for coded activations: the pages name a
 * gate/up path over E4M3 activation codes ("32 fp4 by E4M3 (or bf16)
 * products") but give no activation scale; we read one power-of-two scale per
 * 32 activations, stored as E8M0 like an MX block scale. [#2983, "What this
 * changes"; commit list: the gate/up coded kernels] */
double or_e8m0(unsigned byte) {
    byte &= 255u;
    if (byte == 255u) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* Coded activations to float64: x[i] = e4m3fn(code[i]) * e8m0(scale[i / 32]),
 * exact (a 4-significant-bit value times a power of two). */
void or_dequant_coded(int n, const uint8_t* codes, const uint8_t* scales, double* x) {
    for (int i = 0; i < n; ++i) x[i] = or_e4m3fn(codes[i]) * or_e8m0(scales[i / 32]);
}

/* bf16: the high half of an IEEE binary32. */
double or_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round to bf16 precision, to nearest with ties to even, once, from the exact
 * float64 value: 8 significant bits; the exponent range of binary32, so below
 * 2^-126 the step is 2^-133 (bf16 subnormals); a result at or above 2^128
 * becomes infinity. NaN stays NaN, -0 stays -0. Used for the bf16 storage of
 * act and y (reading: the stored value is the float64 definition rounded). */
double or_round_bf16(double v) {
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);                          /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                         /* step: 2^(e-8) gives 8 significant bits */
    if (q < -133) q = -133;                /* bf16 subnormal step */
    double m = ldexp(a, -q);               /* exact: a power-of-two scaling */
    double r = floor(m);
    double frac = m - r;                   /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    double out = ldexp(r, q);
    if (out >= ldexp(1.0, 128)) out = INFINITY;
    return v < 0 ? -out : out;
}

static unsigned code_at(const uint8_t* codes, int K, int n, int k) {
    uint8_t b = codes[(size_t)n * (K / 2) + k / 2];
    return (k & 1) ? (b >> 4) : (b & 15u);
}

static unsigned scale_at(const uint8_t* scales, int K, int n, int k) {
    return scales[(size_t)n * (K / 32) + k / 32];
}

/* --------------------------------------------------------------- routing */

/* Expert a ranks before expert b: larger logit first, equal logits by lower id,
 * NaN after every number. (The pages do not describe routing; this reading is
 * the plain top-k.) */
static int ranks_before(const float* l, int a, int b) {
    int na = isnan(l[a]), nb = isnan(l[b]);
    if (na || nb) {
        if (na && nb) return a < b;
        return nb;
    }
    if (l[a] != l[b]) return l[a] > l[b];
    return a < b;
}

/* Top-k selection, then softmax over the chosen logits as the combine weights. */
void or_route(int R, int E, int k, const float* logits, int32_t* topk_id, double* topk_w) {
    char* taken = (char*)malloc((size_t)E);
    for (int r = 0; r < R; ++r) {
        const float* l = logits + (size_t)r * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(l, e, best))) best = e;
            taken[best] = 1;
            topk_id[(size_t)r * k + j] = best;
        }
        /* softmax over the k chosen logits, shifted by the largest (slot 0) */
        double top = (double)l[topk_id[(size_t)r * k]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp((double)l[topk_id[(size_t)r * k + j]] - top);
        for (int j = 0; j < k; ++j)
            topk_w[(size_t)r * k + j] = exp((double)l[topk_id[(size_t)r * k + j]] - top) / sum;
    }
    free(taken);
}

/* ------------------------------------------------------ bucketing and plan */

/* Entries are e = row*k + slot. Experts ascending; inside an expert, rows
 * ascending (a row selects an expert at most once). [#2983, "What this
 * changes": an expert's rows form its slot] */
void or_bucket(int R, int E, int k, const int32_t* topk_id, int32_t* count, int32_t* offset,
               int32_t* entry) {
    for (int e = 0; e < E; ++e) count[e] = 0;
    for (int i = 0; i < R * k; ++i) count[topk_id[i]]++;
    offset[0] = 0;
    for (int e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) next[e] = offset[e];
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < k; ++j) {
            int e = topk_id[(size_t)r * k + j];
            entry[next[e]++] = r * k + j;
        }
    free(next);
}

/* Pass sizes for an expert with n rows. One row: a single one-row pass.
 * Otherwise, while rows are left: the largest size if at least that many are
 * left, else the smallest size that holds all that are left; the pass takes
 * min(size, left) real rows and pads the rest. Gate/up sizes {2,4,6,8} and
 * down sizes {2,4}: a five-row slot runs gate/up as one pass of 6 and down as
 * a pass of 4 then a pass of 2. [#2983, "What this changes" and the
 * maintainer's review comment on pass sizes] */
int or_passes(int n, const int32_t* tiers, int n_tiers, int32_t* size, int32_t* real, int cap) {
    int np = 0;
    if (n <= 0) return 0;
    if (n == 1) {
        if (cap > 0) { size[0] = 1; real[0] = 1; }
        return 1;
    }
    int largest = tiers[n_tiers - 1];
    int left = n;
    while (left > 0) {
        int p;
        if (left >= largest) {
            p = largest;
        } else {
            p = largest;
            for (int t = 0; t < n_tiers; ++t)
                if (tiers[t] >= left) { p = tiers[t]; break; }
        }
        int take = left < p ? left : p;
        if (np < cap) { size[np] = p; real[np] = take; }
        ++np;
        left -= take;
    }
    return np;
}

int or_plan(int E, const int32_t* count, const int32_t* offset, const int32_t* tiers, int n_tiers,
            int32_t* plan, int cap) {
    int np = 0;
    for (int e = 0; e < E; ++e) {
        int n = count[e];
        if (n <= 0) continue;
        /* an expert with n rows has at most n passes */
        int32_t* size = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
        int32_t* real = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
        int first = offset[e];
        int m = or_passes(n, tiers, n_tiers, size, real, n);
        for (int i = 0; i < m; ++i) {
            if (np < cap) {
                plan[4 * np + 0] = e;
                plan[4 * np + 1] = first;
                plan[4 * np + 2] = real[i];
                plan[4 * np + 3] = size[i];
            }
            ++np;
            first += real[i];
        }
        free(size);
        free(real);
    }
    return np;
}

/* ------------------------------------------------------- float64 layer math */

/* y = W x with W[n][k] = e2m1(code) * e4m3(scale of k's group). */
void or_matvec(int N, int K, const uint8_t* codes, const uint8_t* scales, const double* x, double* y) {
    for (int n = 0; n < N; ++n) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) {
            double w = or_e2m1(code_at(codes, K, n, k)) * or_e4m3fn(scale_at(scales, K, n, k));
            s += w * x[k];
        }
        y[n] = s;
    }
}

/* Gate/up epilogue. The pages only say it is the one-row kernel's; this is the
 * SwiGLU reading: act = g / (1 + exp(-g)) * u. [#2983, "What this changes"] */
void or_swiglu(int n, const double* g, const double* u, double* act) {
    for (int i = 0; i < n; ++i) act[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* Combine output: the router-weighted sum of a row's expert outputs. */
void or_combine(int k, int H, const double* w, const double* out, double* y) {
    for (int n = 0; n < H; ++n) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += w[j] * out[(size_t)j * H + n];
        y[n] = s;
    }
}

int or_omp_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads later parallel regions use (n >= 1); timing only, the results do
 * not depend on it (each (row, slot) pair is computed whole by one thread). */
void or_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* The layer over R rows whose activations are given in float64 (xr: [R][H]). */
static int layer_rows(int H, int I, int E, int k, int R, const double* xr, const float* logits,
                      const uint8_t* const* gate_codes, const uint8_t* const* gate_scales,
                      const uint8_t* const* up_codes, const uint8_t* const* up_scales,
                      const uint8_t* const* down_codes, const uint8_t* const* down_scales,
                      int32_t* topk_id, double* topk_w, double* act, double* out, double* y, int act_bf16) {
    or_route(R, E, k, logits, topk_id, topk_w);
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#endif
    int pairs = R * k;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int p = 0; p < pairs; ++p) {
        int r = p / k;
        int e = topk_id[p];
        const double* x = xr + (size_t)r * H;
        double* g = (double*)malloc(sizeof(double) * (size_t)I);
        double* u = (double*)malloc(sizeof(double) * (size_t)I);
        or_matvec(I, H, gate_codes[e], gate_scales[e], x, g);
        or_matvec(I, H, up_codes[e], up_scales[e], x, u);
        or_swiglu(I, g, u, act + (size_t)p * I);
        if (act_bf16)
            for (int i = 0; i < I; ++i) act[(size_t)p * I + i] = or_round_bf16(act[(size_t)p * I + i]);
        or_matvec(H, I, down_codes[e], down_scales[e], act + (size_t)p * I, out + (size_t)p * H);
        free(g);
        free(u);
    }
    for (int r = 0; r < R; ++r)
        or_combine(k, H, topk_w + (size_t)r * k, out + (size_t)r * k * H, y + (size_t)r * H);
    return used;
}

int or_layer(int H, int I, int E, int k, int R, const uint16_t* x_bf16, const float* logits,
             const uint8_t* const* gate_codes, const uint8_t* const* gate_scales,
             const uint8_t* const* up_codes, const uint8_t* const* up_scales,
             const uint8_t* const* down_codes, const uint8_t* const* down_scales,
             int32_t* topk_id, double* topk_w, double* act, double* out, double* y, int act_bf16) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)R * H);
    for (size_t i = 0; i < (size_t)R * H; ++i) xr[i] = or_bf16(x_bf16[i]);
    int used = layer_rows(H, I, E, k, R, xr, logits, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                          down_scales, topk_id, topk_w, act, out, y, act_bf16);
    free(xr);
    return used;
}

/* The layer with coded activations: row r's x is or_dequant_coded of its H
 * E4M3FN codes and H/32 E8M0 scales; everything after is or_layer's. */
int or_layer_coded(int H, int I, int E, int k, int R, const uint8_t* x_codes, const uint8_t* x_scales,
                   const float* logits, const uint8_t* const* gate_codes, const uint8_t* const* gate_scales,
                   const uint8_t* const* up_codes, const uint8_t* const* up_scales,
                   const uint8_t* const* down_codes, const uint8_t* const* down_scales,
                   int32_t* topk_id, double* topk_w, double* act, double* out, double* y) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)R * H);
    for (int r = 0; r < R; ++r)
        or_dequant_coded(H, x_codes + (size_t)r * H, x_scales + (size_t)r * (H / 32), xr + (size_t)r * H);
    int used = layer_rows(H, I, E, k, R, xr, logits, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                          down_scales, topk_id, topk_w, act, out, y, 0);
    free(xr);
    return used;
}

/* ----------------------------------------------- fp32 replay of the chains */

/* The per-row arithmetic in float: for each group of 32 products, a fused
 * multiply-add chain from +0 in k order, then that group's scale applied by
 * one more fused multiply-add into one of eight partial sums, then a fixed
 * tree over the eight. [#2983, "What this changes" and the rows commit]
 * Readings where the pages are silent: group g goes to partial g mod 8, each
 * partial starts at +0 and takes its groups in ascending order, and the tree
 * is ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)). */
void or_chain32(int N, int K, const uint8_t* codes, const uint8_t* scales, const float* x, float* y) {
    int G = K / 32;
    for (int n = 0; n < N; ++n) {
        float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int g = 0; g < G; ++g) {
            float p = 0.0f;
            for (int t = 0; t < 32; ++t) {
                int k = 32 * g + t;
                float w = (float)or_e2m1(code_at(codes, K, n, k));
                p = fmaf(w, x[k], p);
            }
            float s = (float)or_e4m3fn(scale_at(scales, K, n, 32 * g));
            part[g % 8] = fmaf(p, s, part[g % 8]);
        }
        float a = part[0] + part[1];
        float b = part[2] + part[3];
        float c = part[4] + part[5];
        float d = part[6] + part[7];
        float ab = a + b;
        float cd = c + d;
        y[n] = ab + cd;
    }
}

/* Combine in float: y = fma chain from +0 over the slots in order. */
void or_combine32(int k, int H, const float* w, const float* out, float* y) {
    for (int n = 0; n < H; ++n) {
        float s = 0.0f;
        for (int j = 0; j < k; ++j) s = fmaf(w[j], out[(size_t)j * H + n], s);
        y[n] = s;
    }
}

/* ------------------------------------------------- dense FP8 projections */

/* y[r][n] = sum over k of bf16(x[r][k]) * e4m3fn(w[n][k]) * s[n/128][k/128],
 * in float64 with k ascending; R rows of x [R][K] (bf16 bits), w [N][K] E4M3FN
 * bytes, s [ceil(N/128)][K/128] float. The dense FP8 projections are the
 * other weight stream of a decode layer (the 6-16-row matrix-tile commit,
 * #2973, in [#2983]'s commit list); the pages give no scale layout, so the
 * reading is the released FP8 checkpoints' one: one scale per 128 x 128 block
 * of the weight matrix, multiplying the decoded bytes. */
void or_fp8_proj(int R, int N, int K, const uint16_t* x, const uint8_t* w, const float* s, double* y) {
    const int KB = K / 128;
    for (int r = 0; r < R; ++r)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double wv = or_e4m3fn(w[(size_t)n * K + k]) * (double)s[(size_t)(n / 128) * KB + k / 128];
                acc += or_bf16(x[(size_t)r * K + k]) * wv;
            }
            y[(size_t)r * N + n] = acc;
        }
}

/* The same projection for fp32 rows: y[r][n] = sum over k of x[r][k] *
 * e4m3fn(w[n][k]) * s[n/128][k/128], float64, k ascending (the pages register
 * fp32 and bf16 activation forms of the FP8 projections). */
void or_fp8_proj_f32(int R, int N, int K, const float* x, const uint8_t* w, const float* s, double* y) {
    const int KB = K / 128;
    for (int r = 0; r < R; ++r)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double wv = or_e4m3fn(w[(size_t)n * K + k]) * (double)s[(size_t)(n / 128) * KB + k / 128];
                acc += (double)x[(size_t)r * K + k] * wv;
            }
            y[(size_t)r * N + n] = acc;
        }
}
