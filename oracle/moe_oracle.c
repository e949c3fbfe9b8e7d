/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU reference for the per-token
 * Mixture-of-Experts expert path over affine group-quantised weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file.  Only the tests, the package smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source with the HIP library: it reads the
 * packed format from its written specification (below), not from the packer.
 *
 * Precision: weights are dequantised to fp32 (one rounding, see dequant), every
 * sum is accumulated in fp64, and every activation is carried in fp64.
 *
 * Sources.  The pages ("Flash-MoE" web pages) define:
 *   - the per-element affine dequantisation (nibble * scale + bias) and its FMA
 *     rewrite fma(nibble, scale*x, bias*x):  lilting.ch, "397Bパラメータモデルを
 *     48GB MacBookで動かすFlash-MoE", section "Metal Compute Shaders";
 *   - 4-bit and 2-bit expert matvec kernels, two-pass RMSNorm, and the MoE
 *     combine as a weighted sum of expert outputs: same page, same section, kernel
 *     table;
 *   - 512 experts per layer, 4 active per token, 60 layers: same page, section
 *     "モデルアーキテクチャ" (model architecture);
 *   - ~6.75 MB per 4-bit expert, 4 x 6.75 MB ~= 27 MB per token: same page, section
 *     "コア技術: SSDエキスパートストリーミング" (SSD expert streaming).
 * The pages do not define the router normalisation, top-K rule, SwiGLU, RMSNorm
 * epsilon placement, group size, code order or scale dtype.  This oracle takes the
 * plain readings: softmax over all experts, top-K by logit (ties -> lower index),
 * weights renormalised over the K selected; h = silu(gate) * up with
 * silu(z) = z / (1 + exp(-z)); RMSNorm n = x / sqrt(mean(x^2) + eps) * w_norm;
 * groups of 64 along the input dimension; bf16 (scale, bias) per group.
 *
 * Packed matrix format (rows R = outputs, cols C = inputs, bits b in {2,4}):
 *   code plane  : R * C * b / 8 bytes, row-major.  Code (r, c) lives in byte
 *                 r*(C*b/8) + floor(c*b/8) at bit offset (c*b) mod 8, i.e. the
 *                 lowest bits hold the lowest column (LSB-first).
 *   sb plane    : R * (C/64) pairs of little-endian bf16, pair (r, g) at
 *                 uint16 index 2*(r*(C/64) + g): scale first, then bias.
 *   expert blob : gate.codes, gate.sb, up.codes, up.sb, down.codes, down.sb, each
 *                 plane starting at an offset rounded up to 256 bytes; gate and up
 *                 are I x H, down is H x I.  The blob size is the end of the last
 *                 plane rounded up to 256 bytes.
 *
 * parity pins: every function below is pinned by CPU tests (size identities from
 * the pages, hand-made byte probes, closed forms, brute force, numpy fp64).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 64

static size_t orc_round256(size_t v) { return (v + 255u) & ~(size_t)255u; }

/* Bytes of one code plane: R*C*b/8. */
size_t orc_codes_bytes(int rows, int cols, int bits) {
    return (size_t)rows * (size_t)cols * (size_t)bits / 8u;
}

/* Bytes of one (scale, bias) plane: one bf16 pair per row per group of 64. */
size_t orc_sb_bytes(int rows, int cols) {
    return (size_t)rows * (size_t)(cols / ORC_GROUP) * 4u;
}

/* Plane offsets inside one expert blob: off[0..5] = gate.codes, gate.sb, up.codes,
 * up.sb, down.codes, down.sb; *total = blob size. */
void orc_blob_layout(int H, int I, int bits, size_t off[6], size_t *total) {
    size_t sizes[6];
    sizes[0] = orc_codes_bytes(I, H, bits);
    sizes[1] = orc_sb_bytes(I, H);
    sizes[2] = sizes[0];
    sizes[3] = sizes[1];
    sizes[4] = orc_codes_bytes(H, I, bits);
    sizes[5] = orc_sb_bytes(H, I);
    size_t p = 0;
    for (int i = 0; i < 6; ++i) {
        off[i] = p;
        p = orc_round256(p + sizes[i]);
    }
    *total = p;
}

/* bf16 -> float: the bf16 bits are the top half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t v) {
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Unsigned code of element (r, c) of a packed code plane (LSB-first). */
int orc_code(const uint8_t *codes, int rows, int cols, int bits, int r, int c) {
    (void)rows;
    size_t row_bytes = (size_t)cols * (size_t)bits / 8u;
    size_t bit = (size_t)c * (size_t)bits;
    uint8_t byte = codes[(size_t)r * row_bytes + bit / 8u];
    return (byte >> (bit % 8u)) & ((1 << bits) - 1);
}

/* Affine dequantisation of a whole matrix to fp32: w = q * scale + bias.
 * q * scale is exact in fp32 (at most 4 + 8 significant bits), so the single
 * rounding is that of the addition; the page's fma form gives the same value. */
void orc_dequant(const uint8_t *codes, const uint16_t *sb, int rows, int cols, int bits, float *W) {
    int G = cols / ORC_GROUP;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        for (int c = 0; c < cols; ++c) {
            int g = c / ORC_GROUP;
            float s = orc_bf16_to_f32(sb[2 * ((size_t)r * G + g)]);
            float b = orc_bf16_to_f32(sb[2 * ((size_t)r * G + g) + 1]);
            float q = (float)orc_code(codes, rows, cols, bits, r, c);
            float qs = q * s;
            W[(size_t)r * cols + c] = qs + b;
        }
    }
}

/* y = W x with fp32 W, fp64 x and fp64 accumulation in column order. */
void orc_matvec(const float *W, int rows, int cols, const double *x, double *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        const float *w = W + (size_t)r * cols;
        for (int c = 0; c < cols; ++c) acc += (double)w[c] * x[c];
        y[r] = acc;
    }
}

/* Two-pass RMSNorm (sum of squares, then apply), eps inside the square root,
 * weight applied after normalising. */
void orc_rmsnorm(const double *x, const uint16_t *w_bf16, int H, double eps, double *out) {
    double ss = 0.0;
    for (int c = 0; c < H; ++c) ss += x[c] * x[c];
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int c = 0; c < H; ++c) out[c] = x[c] * inv * (double)orc_bf16_to_f32(w_bf16[c]);
}

/* Router logits l_e = sum_c W_r[e, c] n_c (+ bias_e).  W_r is fp32 or bf16. */
void orc_router_logits(const void *Wr, int wr_is_bf16, int E, int H, const double *n,
                       const float *bias, double *logits) {
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int c = 0; c < H; ++c) {
            double w = wr_is_bf16 ? (double)orc_bf16_to_f32(((const uint16_t *)Wr)[(size_t)e * H + c])
                                  : (double)((const float *)Wr)[(size_t)e * H + c];
            acc += w * n[c];
        }
        logits[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

/* Softmax over all E logits, top-K by logit (descending; equal logits -> lower
 * expert index first), weights renormalised over the K selected.  *margin is the
 * gap between the K-th and (K+1)-th largest logit (+inf when K == E).
 *
 * The pages say nothing about non-finite logits.  Reading taken here: a NaN logit
 * counts as -inf, in the selection and in the softmax alike (so a NaN expert is
 * chosen only after every finite one, and then in index order among the -inf ones,
 * with weight 0).  When every logit is -inf (or NaN) the softmax has no maximum to
 * subtract; the weights are then the limit of K equal logits, 1/K each. */
void orc_route(const double *logits, int E, int K, int32_t *idx, double *w, double *margin) {
    double *lv = (double *)malloc(sizeof(double) * (size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)calloc((size_t)E, 1);
    double mx = -INFINITY;
    for (int e = 0; e < E; ++e) {
        lv[e] = isnan(logits[e]) ? -INFINITY : logits[e];
        if (lv[e] > mx) mx = lv[e];
    }
    /* selection: K passes of "largest remaining logit, lowest index on ties" */
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || lv[e] > lv[best]) best = e;
        }
        taken[best] = 1;
        idx[k] = best;
    }
    if (mx == -INFINITY) {
        for (int k = 0; k < K; ++k) w[k] = 1.0 / (double)K;
    } else {
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp(lv[e] - mx);
            z += p[e];
        }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double sel = 0.0;
        for (int k = 0; k < K; ++k) sel += p[idx[k]];
        for (int k = 0; k < K; ++k) w[k] = p[idx[k]] / sel;
    }
    if (margin) {
        double next = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && lv[e] > next) next = lv[e];
        *margin = (K < E) ? lv[idx[K - 1]] - next : INFINITY;
    }
    free(lv);
    free(p);
    free(taken);
}

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert: g = W_g n, u = W_u n, h = silu(g) * u, y = W_d h.
 * g, u, h have I entries, y has H entries; any of g, u, h may be NULL. */
void orc_expert(const uint8_t *blob, int bits, int H, int I, const double *n,
                double *g_out, double *u_out, double *h_out, double *y) {
    size_t off[6], total;
    orc_blob_layout(H, I, bits, off, &total);
    float *Wg = (float *)malloc(sizeof(float) * (size_t)I * H);
    float *Wu = (float *)malloc(sizeof(float) * (size_t)I * H);
    float *Wd = (float *)malloc(sizeof(float) * (size_t)H * I);
    double *g = (double *)malloc(sizeof(double) * (size_t)I);
    double *u = (double *)malloc(sizeof(double) * (size_t)I);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    orc_dequant(blob + off[0], (const uint16_t *)(blob + off[1]), I, H, bits, Wg);
    orc_dequant(blob + off[2], (const uint16_t *)(blob + off[3]), I, H, bits, Wu);
    orc_dequant(blob + off[4], (const uint16_t *)(blob + off[5]), H, I, bits, Wd);
    orc_matvec(Wg, I, H, n, g);
    orc_matvec(Wu, I, H, n, u);
    for (int j = 0; j < I; ++j) h[j] = orc_silu(g[j]) * u[j];
    orc_matvec(Wd, H, I, h, y);
    if (g_out) memcpy(g_out, g, sizeof(double) * (size_t)I);
    if (u_out) memcpy(u_out, u, sizeof(double) * (size_t)I);
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
    free(Wg); free(Wu); free(Wd); free(g); free(u); free(h);
}

/* Weighted combine out = sum_k w_k y_k (+ residual). y is [K][H]. */
void orc_combine(const double *y, const double *w, int K, int H, const double *residual, double *out) {
    for (int c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += w[k] * y[(size_t)k * H + c];
        out[c] = acc + (residual ? residual[c] : 0.0);
    }
}

/* float -> bf16 bits, round to nearest even (finite inputs). */
static uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Quantise-from-float (the step before packing), group by group along each row.  The pages
 * name an MLX 4-bit affine base (tomo3141592653.github.io, "iPhone 17 Proで400Bパラメータ LLM
 * を動かす「flash-moe」", section "ハイブリッド量子化") and the affine form w = q * scale + bias
 * (lilting.ch page, section "Metal Compute Shaders") but not the rounding; the plain reading:
 *   lo, hi = min and max of the group's 64 weights;
 *   scale  = bf16((hi - lo) / (2^b - 1)),  bias = bf16(lo);
 *   code   = nearest integer, ties to even, to (w - bias) / scale, clamped to [0, 2^b - 1],
 *            and 0 when the bf16 scale is 0 (a constant group),
 * every step in fp32 with the bf16 scale and bias already rounded, so that the stored pair
 * dequantises the codes.  W [rows][cols] finite fp32; codes [rows][cols] one per byte,
 * scale and bias [rows][cols/64] bf16 bits. */
void orc_quantize(const float *W, int rows, int cols, int bits, uint8_t *codes, uint16_t *scale,
                  uint16_t *bias) {
    const int G = cols / ORC_GROUP;
    const float qmax = (float)((1 << bits) - 1);
    for (int r = 0; r < rows; ++r) {
        for (int g = 0; g < G; ++g) {
            const float *w = W + (size_t)r * cols + (size_t)g * ORC_GROUP;
            float lo = w[0], hi = w[0];
            for (int i = 1; i < ORC_GROUP; ++i) {
                if (w[i] < lo) lo = w[i];
                if (w[i] > hi) hi = w[i];
            }
            const uint16_t sb = orc_f32_to_bf16((hi - lo) / qmax);
            const uint16_t bb = orc_f32_to_bf16(lo);
            const float s = orc_bf16_to_f32(sb), b = orc_bf16_to_f32(bb);
            scale[(size_t)r * G + g] = sb;
            bias[(size_t)r * G + g] = bb;
            for (int i = 0; i < ORC_GROUP; ++i) {
                int q = 0;
                if (s > 0.0f) {
                    const float t = w[i] - b;
                    const float u = nearbyintf(t / s);
                    q = u < 0.0f ? 0 : (u > qmax ? (int)qmax : (int)u);
                }
                codes[(size_t)r * cols + (size_t)g * ORC_GROUP + i] = (uint8_t)q;
            }
        }
    }
}

/* silu exported for its own pins. */
double orc_silu_export(double z) { return orc_silu(z); }
