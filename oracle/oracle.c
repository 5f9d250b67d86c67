/*
 * oracle.c -- plain fp64 CPU oracle for the CSA / HCA attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header,
 * table or constant with the HIP library; the two only agree on the byte
 * layouts written down in the C-ABI header, and each side encodes and decodes
 * those layouts with code of its own.
 *
 * Everything here is written for a reader checking it against the method's
 * description by eye: loops in the order of the definitions, fp64 arithmetic,
 * no blocking or fusion.  Sources (the DeepSeek-V4 pages):
 *   - "DeepSeek-V4 ... open-source declaration" (peacm.com), section 3.2
 *     (hybrid attention): the CSA four-step diagram (compress every m tokens to
 *     one KV entry, lightning-indexer top-k, multi-query attention over the
 *     selected blocks, grouped output projection), the HCA paragraph (128:1,
 *     dense attention over every compressed entry) and the list of four tricks
 *     (Q/KV RMSNorm, partial RoPE on the last 64 dims with a -i RoPE on the
 *     output, a 128-token raw sliding window, a learnable sink logit in the
 *     softmax denominator).
 *   - "DeepSeek-V4 technical report digest" (gitcode.csdn.net), section 2.1.4
 *     (KV cache: RoPE dims in BF16, the rest in FP8) and section 3.2 (FP4
 *     E2M1 indexer QK path with 1x32 scales, lossless FP4 -> FP8).
 *   - "DeepSeek V4 (Flash & Pro)" (github wiki article), hybrid-attention
 *     section: HCA compresses KV 128:1 into a dense MQA stream plus a
 *     128-token sliding window.
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* format ids (same numbering as the C-ABI header's csa_dtype) */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2, ORC_FP4_E2M1 = 3 };

/* ======================================================================
 * Number formats.  Each encoder finds the nearest representable value by
 * searching the format's value grid (not by bit manipulation), ties to the
 * code with an even last mantissa bit.
 * ====================================================================== */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
ORC_API double orc_bf16_decode(uint16_t b) {
    int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (e == 0xFF) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -133);            /* m * 2^-7 * 2^-126 */
    else v = ldexp((double)(128 + m), e - 127 - 7);
    return s ? -v : v;
}

/* Round a float to the nearest bf16 value, ties to even.  The grid spacing
 * for |x| in [2^E, 2^(E+1)) is 2^(E-7), and 2^-133 below 2^-126. */
ORC_API uint16_t orc_bf16_encode(float xf) {
    double x = xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7FC0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                       /* a in [2^(ex-1), 2^ex) */
    int q = ex - 1 - 7;
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(a, -q)), q);   /* nearbyint: ties to even */
    if (r >= 0x1p128) return sign | 0x7F80;
    if (r < 0x1p-126) return sign | (uint16_t)(r / 0x1p-133);
    frexp(r, &ex);
    int E = ex - 1;
    int mant = (int)(ldexp(r, -E) * 128.0) - 128;
    return sign | (uint16_t)(((E + 127) << 7) | mant);
}

/* OCP FP8 E4M3FN: bias 7, no infinities, 0x7F / 0xFF are NaN, max 448. */
ORC_API double orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest E4M3FN value, ties to even code, saturating to +-448 (the
 * reading for the FP8 KV cache: finite codes only). */
ORC_API uint8_t orc_e4m3_encode(float xf) {
    double x = xf;
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0) return sign | 126;
    int c = 0;                                 /* largest code with value <= a */
    while (c < 126 && orc_e4m3_decode((uint8_t)(c + 1)) <= a) c++;
    double lo = orc_e4m3_decode((uint8_t)c), hi = orc_e4m3_decode((uint8_t)(c + 1));
    int pick;
    if (a - lo < hi - a) pick = c;
    else if (a - lo > hi - a) pick = c + 1;
    else pick = (c % 2 == 0) ? c : c + 1;
    return sign | (uint8_t)pick;
}

/* OCP FP4 E2M1: values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives. */
ORC_API double orc_e2m1_decode(uint8_t c) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[c & 7];
    return (c & 8) ? -v : v;
}

/* Nearest E2M1 value, ties to even code, saturating to +-6 (OCP MX rule). */
ORC_API uint8_t orc_e2m1_encode(float xf) {
    double x = xf;
    if (isnan(x)) return 0;
    uint8_t sign = signbit(x) ? 8 : 0;
    double a = fabs(x);
    if (a >= 6.0) return sign | 7;
    int c = 0;
    while (c < 7 && orc_e2m1_decode((uint8_t)(c + 1)) <= a) c++;
    double lo = orc_e2m1_decode((uint8_t)c), hi = orc_e2m1_decode((uint8_t)(c + 1));
    int pick;
    if (a - lo < hi - a) pick = c;
    else if (a - lo > hi - a) pick = c + 1;
    else pick = (c % 2 == 0) ? c : c + 1;
    return sign | (uint8_t)pick;
}

/* E8M0 scale: 2^(c - 127); 255 is NaN. */
ORC_API double orc_e8m0_decode(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* FP4 quantisation of one row of n values (n a multiple of 32), in blocks of
 * 32 with one E8M0 scale each (technical-report digest, section 3.2: FP4
 * E2M1 with 1x32 sub-block scales).
 * Per block: e = floor(log2(amax)) - 2 (OCP MX: 2 is E2M1's largest
 * exponent), then clamped to at least e_max(row) - 14 so that every value of
 * the row is exactly representable after the FP4 -> FP8 E4M3 conversion
 * against a common row exponent (the "threshold condition" on the ratio of
 * block scales; reading: the E4M3 grid spans 2^-9 .. 448, and an E2M1 value
 * shifted by 2^delta stays on it exactly for delta in [-8, 6]).
 * An all-zero block takes the row floor e_max - 14; an all-zero row takes 0.
 * codes: n/2 bytes, element 2i in the low nibble; scales: n/32 bytes. */
ORC_API void orc_fp4_quant_row(const float* x, int n, uint8_t* codes, uint8_t* scales) {
    int nb = n / 32;
    int e[64];
    int have = 0, emax = 0;
    for (int b = 0; b < nb; b++) {
        double amax = 0.0;
        for (int i = 0; i < 32; i++) {
            double a = fabs((double)x[b * 32 + i]);
            if (a > amax) amax = a;
        }
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);             /* amax in [2^(ex-1), 2^ex) */
            e[b] = (ex - 1) - 2;
            if (!have || e[b] > emax) emax = e[b];
            have = 1;
        } else {
            e[b] = INT32_MIN;
        }
    }
    for (int b = 0; b < nb; b++) {
        int eb = have ? e[b] : 0;
        if (have && eb < emax - 14) eb = emax - 14;
        if (eb < -127) eb = -127;
        if (eb > 127) eb = 127;
        scales[b] = (uint8_t)(eb + 127);
        for (int i = 0; i < 32; i += 2) {
            float v0 = (float)ldexp((double)x[b * 32 + i], -eb);
            float v1 = (float)ldexp((double)x[b * 32 + i + 1], -eb);
            codes[(b * 32 + i) / 2] = (uint8_t)(orc_e2m1_encode(v0) | (orc_e2m1_encode(v1) << 4));
        }
    }
}

/* ---------------------------------------------------------------------- */
/* KV record layouts (one compressed or window entry of d dims):
 *   F32 : d x f32
 *   BF16: d x bf16
 *   FP8 : (d - dr) x E4M3 codes | dr x bf16 | f32 row scale | zero pad to a
 *         multiple of 16 bytes.   The value of non-RoPE dim i is
 *         e4m3(code_i) * scale; scale = amax(non-RoPE dims) / 448 (1 if the
 *         amax is 0).  (Digest section 2.1.4: RoPE dims BF16, others FP8.)  */
ORC_API int orc_kv_record_bytes(int fmt, int d, int dr) {
    if (fmt == ORC_F32) return 4 * d;
    if (fmt == ORC_BF16) return 2 * d;
    if (fmt == ORC_FP8_E4M3) return ((d - dr) + 2 * dr + 4 + 15) / 16 * 16;
    return -1;
}

/* Encode one entry.  The value is first rounded to fp32 (the precision the
 * quantisation decision is taken in), then quantised. */
ORC_API void orc_kv_encode(const double* v, int fmt, int d, int dr, uint8_t* rec) {
    int nb = orc_kv_record_bytes(fmt, d, dr);
    memset(rec, 0, (size_t)nb);
    if (fmt == ORC_F32) {
        for (int i = 0; i < d; i++) { float f = (float)v[i]; memcpy(rec + 4 * i, &f, 4); }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < d; i++) { uint16_t b = orc_bf16_encode((float)v[i]); memcpy(rec + 2 * i, &b, 2); }
    } else if (fmt == ORC_FP8_E4M3) {
        int dn = d - dr;
        float amax = 0.0f;
        for (int i = 0; i < dn; i++) { float a = fabsf((float)v[i]); if (a > amax) amax = a; }
        float scale = amax > 0.0f ? (float)((double)amax / 448.0) : 1.0f;
        for (int i = 0; i < dn; i++) {
            float q = (float)((double)(float)v[i] / (double)scale);
            rec[i] = orc_e4m3_encode(q);
        }
        for (int i = 0; i < dr; i++) {
            uint16_t b = orc_bf16_encode((float)v[dn + i]);
            memcpy(rec + dn + 2 * i, &b, 2);
        }
        memcpy(rec + dn + 2 * dr, &scale, 4);
    }
}

ORC_API void orc_kv_decode(const uint8_t* rec, int fmt, int d, int dr, double* v) {
    if (fmt == ORC_F32) {
        for (int i = 0; i < d; i++) { float f; memcpy(&f, rec + 4 * i, 4); v[i] = f; }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < d; i++) { uint16_t b; memcpy(&b, rec + 2 * i, 2); v[i] = orc_bf16_decode(b); }
    } else if (fmt == ORC_FP8_E4M3) {
        int dn = d - dr;
        float scale;
        memcpy(&scale, rec + dn + 2 * dr, 4);
        for (int i = 0; i < dn; i++) v[i] = orc_e4m3_decode(rec[i]) * (double)scale;
        for (int i = 0; i < dr; i++) { uint16_t b; memcpy(&b, rec + dn + 2 * i, 2); v[dn + i] = orc_bf16_decode(b); }
    }
}

/* Indexer key / query row layouts (di dims): F32 di x f32; BF16 di x bf16;
 * FP4: di/2 bytes of E2M1 codes (plane 1) and di/32 E8M0 scales (plane 2). */
ORC_API void orc_idx_encode(const double* v, int fmt, int di, uint8_t* codes, uint8_t* scales) {
    if (fmt == ORC_F32) {
        for (int i = 0; i < di; i++) { float f = (float)v[i]; memcpy(codes + 4 * i, &f, 4); }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < di; i++) { uint16_t b = orc_bf16_encode((float)v[i]); memcpy(codes + 2 * i, &b, 2); }
    } else if (fmt == ORC_FP4_E2M1) {
        float tmp[2048];
        for (int i = 0; i < di; i++) tmp[i] = (float)v[i];
        orc_fp4_quant_row(tmp, di, codes, scales);
    }
}

ORC_API void orc_idx_decode(const uint8_t* codes, const uint8_t* scales, int fmt, int di, double* v) {
    if (fmt == ORC_F32) {
        for (int i = 0; i < di; i++) { float f; memcpy(&f, codes + 4 * i, 4); v[i] = f; }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < di; i++) { uint16_t b; memcpy(&b, codes + 2 * i, 2); v[i] = orc_bf16_decode(b); }
    } else if (fmt == ORC_FP4_E2M1) {
        for (int i = 0; i < di; i++) {
            uint8_t byte = codes[i / 2];
            uint8_t c = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
            v[i] = orc_e2m1_decode(c) * orc_e8m0_decode(scales[i / 32]);
        }
    }
}

static int idx_row_code_bytes(int fmt, int di) {
    return fmt == ORC_F32 ? 4 * di : fmt == ORC_BF16 ? 2 * di : di / 2;
}

/* ======================================================================
 * Building blocks of the method.
 * ====================================================================== */

/* Compression of one block (peacm section 3.2, CSA step 1: every m tokens
 * become one KV entry through an attention-like mechanism).  Reading: the
 * block's m tokens are pooled with softmax weights over a learned m-position
 * score vector b, plus an optional content score <u, x_i>:
 *     z_i = b_i + <u, x_i>,  pi = softmax(z),  c = sum_i pi_i x_i.       */
ORC_API void orc_pool(const double* x, int m, int d, const double* b, const double* u,
                      double* c, double* pi) {
    double* z = (double*)malloc(sizeof(double) * (size_t)m);
    double zmax = -INFINITY;
    for (int i = 0; i < m; i++) {
        z[i] = b[i];
        if (u) for (int k = 0; k < d; k++) z[i] += u[k] * x[(size_t)i * d + k];
        if (z[i] > zmax) zmax = z[i];
    }
    double s = 0.0;
    for (int i = 0; i < m; i++) { z[i] = exp(z[i] - zmax); s += z[i]; }
    for (int k = 0; k < d; k++) c[k] = 0.0;
    for (int i = 0; i < m; i++) {
        double p = z[i] / s;
        if (pi) pi[i] = p;
        for (int k = 0; k < d; k++) c[k] += p * x[(size_t)i * d + k];
    }
    free(z);
}

/* RMSNorm (peacm four tricks: Q/KV normalisation before core attention):
 *     n(v) = v / sqrt(mean(v^2) + eps) * gamma      (gamma NULL means 1). */
ORC_API void orc_rmsnorm(const double* v, int d, const double* gamma, double eps, double* out) {
    double ss = 0.0;
    for (int i = 0; i < d; i++) ss += v[i] * v[i];
    double r = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; i++) out[i] = v[i] * r * (gamma ? gamma[i] : 1.0);
}

/* Partial RoPE on the last dr dims (peacm four tricks).  Reading: pairs
 * (v[d-dr+2i], v[d-dr+2i+1]), i < dr/2, are rotated by the angle
 * pos * base^(-2i/dr); the first d-dr dims are untouched.  The angle is
 * formed in fp64 from the integer position. */
ORC_API void orc_rope(double* v, int d, int dr, double pos, double base) {
    int off = d - dr;
    for (int i = 0; i < dr / 2; i++) {
        double theta = pos * pow(base, -2.0 * i / dr);
        double cs = cos(theta), sn = sin(theta);
        double a = v[off + 2 * i], b = v[off + 2 * i + 1];
        v[off + 2 * i] = a * cs - b * sn;
        v[off + 2 * i + 1] = a * sn + b * cs;
    }
}

static double load_scalar(const void* p, int fmt, size_t i) {
    if (fmt == ORC_F32) return ((const float*)p)[i];
    return orc_bf16_decode(((const uint16_t*)p)[i]);
}

/* csa_compress_kv.  x: [B][T][d] raw tokens (f32 or bf16) at absolute
 * positions tok_start[b] .. tok_start[b]+T-1, tok_start a multiple of m.
 * Every complete block i (T/m of them) is block j = tok_start/m + i; it is
 * pooled (orc_pool), normalised (if gamma), rotated to position j*m (if dr),
 * and encoded into slot j (linear cache, skipped if j >= cap) or j mod cap
 * (ring).  out_kind 0: KV records into out_codes ([B][cap] records of
 * out_fmt); out_kind 1: indexer rows (out_codes [B][cap] rows, out_scales
 * [B][cap][d/32] for FP4).  pre_quant, if given, receives the fp64 entry
 * before encoding, [B][cap][d].  Returns the number of blocks written. */
ORC_API long orc_compress(const void* x, int x_fmt, int B, long T, int d, const int* tok_start,
                          int m, const float* b, const float* u, const float* gamma, float eps,
                          int dr, float base, int out_kind, int out_fmt, void* out_codes,
                          uint8_t* out_scales, long cap, int ring, double* pre_quant) {
    long nblk = T / m, written = 0;
    double* bb = (double*)malloc(sizeof(double) * (size_t)m);
    double* uu = u ? (double*)malloc(sizeof(double) * (size_t)d) : NULL;
    double* gg = gamma ? (double*)malloc(sizeof(double) * (size_t)d) : NULL;
    for (int i = 0; i < m; i++) bb[i] = b[i];
    for (int k = 0; k < d; k++) { if (uu) uu[k] = u[k]; if (gg) gg[k] = gamma[k]; }
    int rec = out_kind == 0 ? orc_kv_record_bytes(out_fmt, d, dr) : idx_row_code_bytes(out_fmt, d);
#pragma omp parallel for collapse(2) schedule(static) reduction(+ : written)
    for (int s = 0; s < B; s++) {
        for (long i = 0; i < nblk; i++) {
            long j = tok_start[s] / m + i;
            long slot = ring ? j % cap : j;
            if (!ring && j >= cap) continue;
            double* xs = (double*)malloc(sizeof(double) * (size_t)m * d);
            double* c = (double*)malloc(sizeof(double) * (size_t)d);
            double* e = (double*)malloc(sizeof(double) * (size_t)d);
            for (int t = 0; t < m; t++)
                for (int k = 0; k < d; k++)
                    xs[(size_t)t * d + k] = load_scalar(x, x_fmt, ((size_t)s * T + i * m + t) * d + k);
            orc_pool(xs, m, d, bb, uu, c, NULL);
            if (gg) orc_rmsnorm(c, d, gg, eps, e);
            else memcpy(e, c, sizeof(double) * (size_t)d);
            if (dr > 0) orc_rope(e, d, dr, (double)(j * m), base);
            if (pre_quant) memcpy(pre_quant + ((size_t)s * cap + slot) * d, e, sizeof(double) * (size_t)d);
            size_t r = (size_t)s * cap + slot;
            if (out_kind == 0)
                orc_kv_encode(e, out_fmt, d, dr, (uint8_t*)out_codes + r * rec);
            else
                orc_idx_encode(e, out_fmt, d, (uint8_t*)out_codes + r * rec,
                               out_scales ? out_scales + r * (d / 32) : NULL);
            written++;
            free(xs); free(c); free(e);
        }
    }
    free(bb); free(uu); free(gg);
    return written;
}

/* Lightning-indexer score (peacm section 3.2, CSA step 2: a lightweight
 * indexer scores each query against every compressed block).  Reading:
 *     S_j = sum_h w_h * max(0, <qI_h, key_j>)        for j < n.          */
ORC_API void orc_indexer_scores(const double* qI, const double* w, int Hi, int di,
                                const double* keys, long n, double* S) {
#pragma omp parallel for schedule(static)
    for (long j = 0; j < n; j++) {
        double s = 0.0;
        for (int h = 0; h < Hi; h++) {
            double dot = 0.0;
            for (int k = 0; k < di; k++) dot += qI[h * di + k] * keys[(size_t)j * di + k];
            s += w[h] * (dot > 0.0 ? dot : 0.0);
        }
        S[j] = s;
    }
}

/* Top-k selection (peacm CSA step 2).  Reading: candidates ordered by score
 * descending, ties to the smaller block index; the first min(k, n) are kept
 * and returned in ascending block order, the rest of out[0..k) is -1.
 * Candidates are ranked on the fp64 scores themselves.  NaN ranks below
 * everything. */
typedef struct { double s; long j; } orc_cand;

static int cand_order(const void* a, const void* b) {
    const orc_cand* x = (const orc_cand*)a;
    const orc_cand* y = (const orc_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int index_order(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

ORC_API int orc_topk(const double* S, long n, int k, int32_t* out) {
    orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(n > 0 ? n : 1));
    for (long j = 0; j < n; j++) {
        double s = S[j];
        if (isnan(s)) s = -INFINITY;
        c[j].s = s;
        c[j].j = j;
    }
    qsort(c, (size_t)n, sizeof(orc_cand), cand_order);
    long nsel = n < k ? n : k;
    for (long r = 0; r < nsel; r++) out[r] = (int32_t)c[r].j;
    qsort(out, (size_t)nsel, sizeof(int32_t), index_order);
    for (long r = nsel; r < k; r++) out[r] = -1;
    free(c);
    return (int)nsel;
}

/* csa_indexer_topk for one sequence.  qI rows [Tq][Hi] (format q_fmt, FP4
 * scales in qI_scales), w [Tq][Hi], keys [key_cap] rows.  Query i at
 * position t sees blocks j < min(floor((t+1)/m), key_cap).  out [Tq][k];
 * scores_out (optional) [Tq][key_cap], unset entries left untouched. */
ORC_API void orc_indexer_topk(const uint8_t* qI, const uint8_t* qI_scales, int q_fmt, const float* w,
                              const int32_t* q_pos, int Tq, int Hi, int di,
                              const uint8_t* keys, const uint8_t* key_scales, int key_fmt, long key_cap,
                              int m, int k, int32_t* out, double* scores_out) {
    int qrb = idx_row_code_bytes(q_fmt, di), krb = idx_row_code_bytes(key_fmt, di);
    double* kd = (double*)malloc(sizeof(double) * (size_t)key_cap * di);
#pragma omp parallel for schedule(static)
    for (long j = 0; j < key_cap; j++)
        orc_idx_decode(keys + (size_t)j * krb, key_scales ? key_scales + (size_t)j * (di / 32) : NULL,
                       key_fmt, di, kd + (size_t)j * di);
    double* qd = (double*)malloc(sizeof(double) * (size_t)Hi * di);
    double* wd = (double*)malloc(sizeof(double) * (size_t)Hi);
    double* S = (double*)malloc(sizeof(double) * (size_t)(key_cap > 0 ? key_cap : 1));
    for (int i = 0; i < Tq; i++) {
        for (int h = 0; h < Hi; h++) {
            size_t r = (size_t)i * Hi + h;
            orc_idx_decode(qI + r * qrb, qI_scales ? qI_scales + r * (di / 32) : NULL, q_fmt, di, qd + (size_t)h * di);
            wd[h] = w[r];
        }
        long nt = (q_pos[i] + 1L) / m;
        if (nt > key_cap) nt = key_cap;
        orc_indexer_scores(qd, wd, Hi, di, kd, nt, S);
        if (scores_out) memcpy(scores_out + (size_t)i * key_cap, S, sizeof(double) * (size_t)nt);
        orc_topk(S, nt, k, out + (size_t)i * k);
    }
    free(kd); free(qd); free(wd); free(S);
}

/* ---- array helpers for the test harness ---- */
ORC_API void orc_bf16_encode_n(const float* x, long n, uint16_t* o) { for (long i = 0; i < n; i++) o[i] = orc_bf16_encode(x[i]); }
ORC_API void orc_bf16_decode_n(const uint16_t* x, long n, double* o) { for (long i = 0; i < n; i++) o[i] = orc_bf16_decode(x[i]); }
ORC_API void orc_e4m3_encode_n(const float* x, long n, uint8_t* o) { for (long i = 0; i < n; i++) o[i] = orc_e4m3_encode(x[i]); }
ORC_API void orc_e4m3_decode_n(const uint8_t* x, long n, double* o) { for (long i = 0; i < n; i++) o[i] = orc_e4m3_decode(x[i]); }
ORC_API void orc_e2m1_encode_n(const float* x, long n, uint8_t* o) { for (long i = 0; i < n; i++) o[i] = orc_e2m1_encode(x[i]); }
ORC_API void orc_kv_encode_n(const double* v, long n, int fmt, int d, int dr, uint8_t* recs) {
    int rb = orc_kv_record_bytes(fmt, d, dr);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; i++) orc_kv_encode(v + (size_t)i * d, fmt, d, dr, recs + (size_t)i * rb);
}
ORC_API void orc_kv_decode_n(const uint8_t* recs, long n, int fmt, int d, int dr, double* v) {
    int rb = orc_kv_record_bytes(fmt, d, dr);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; i++) orc_kv_decode(recs + (size_t)i * rb, fmt, d, dr, v + (size_t)i * d);
}
ORC_API void orc_idx_encode_n(const double* v, long n, int fmt, int di, uint8_t* codes, uint8_t* scales) {
    int rb = idx_row_code_bytes(fmt, di);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; i++)
        orc_idx_encode(v + (size_t)i * di, fmt, di, codes + (size_t)i * rb, scales ? scales + (size_t)i * (di / 32) : NULL);
}
ORC_API void orc_idx_decode_n(const uint8_t* codes, const uint8_t* scales, long n, int fmt, int di, double* v) {
    int rb = idx_row_code_bytes(fmt, di);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; i++)
        orc_idx_decode(codes + (size_t)i * rb, scales ? scales + (size_t)i * (di / 32) : NULL, fmt, di, v + (size_t)i * di);
}

/* ----------------------------------------------------------------------
 * Attention for one sequence.
 *
 * Per query token t (position q_pos[i]) and head h (peacm four tricks and
 * CSA step 3; the wiki article's HCA paragraph):
 *   q^ = RoPE_t(RMSNorm(q_{t,h}))
 *   E  = compressed entries (CSA: the top-k list of that token; HCA: every
 *        complete block j < floor((t+1)/m), capped at the cache size)
 *        together with the raw window entries of positions
 *        max(0, t-W+1) .. t (kept even where they overlap a block: the
 *        window is additionally visible).
 *   z_e = scale * <q^, e>
 *   p_e = exp(z_e) / (exp(sink_h) + sum_e' exp(z_e'))    (sink: denominator only)
 *   o   = sum_e p_e e   (one vector per entry is both key and value: MQA)
 *   o[d-dr:] = RoPE_{-t}(o[d-dr:])
 * With no entries o = 0.
 * ---------------------------------------------------------------------- */
typedef struct {
    int d, dr, window, m;
    double base, scale, eps;
} orc_attn_params;

/* fill the entry list of one query; returns the count.  Entries are refs:
 * kind 0 = compressed slot, kind 1 = window slot. */
static long entry_list(long t, const int32_t* topk_row, int k, long comp_cap, int m, long win_cap,
                       int W, long* slots, char* kinds) {
    long n = 0;
    long nt = (t + 1) / m;
    if (nt > comp_cap) nt = comp_cap;
    if (topk_row) {
        for (int i = 0; i < k; i++) {
            long j = topk_row[i];
            if (j < 0 || j >= nt) continue;
            slots[n] = j; kinds[n] = 0; n++;
        }
    } else {
        for (long j = 0; j < nt; j++) { slots[n] = j; kinds[n] = 0; n++; }
    }
    long s0 = t - W + 1;
    if (s0 < 0) s0 = 0;
    for (long s = s0; s <= t; s++) { slots[n] = s % win_cap; kinds[n] = 1; n++; }
    return n;
}

static void attend_one(const double* qhat, const double* ents, long n, int d, double scale,
                       double sink, double* o, double* p_out, double* p_sink_out) {
    double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double zmax = sink;
    for (long e = 0; e < n; e++) {
        double dot = 0.0;
        for (int k = 0; k < d; k++) dot += qhat[k] * ents[(size_t)e * d + k];
        z[e] = scale * dot;
        if (z[e] > zmax) zmax = z[e];
    }
    for (int k = 0; k < d; k++) o[k] = 0.0;
    if (n == 0) {
        if (p_sink_out) *p_sink_out = 1.0;
        free(z);
        return;
    }
    double den = exp(sink - zmax);
    for (long e = 0; e < n; e++) den += exp(z[e] - zmax);
    for (long e = 0; e < n; e++) {
        double p = exp(z[e] - zmax) / den;
        if (p_out) p_out[e] = p;
        for (int k = 0; k < d; k++) o[k] += p * ents[(size_t)e * d + k];
    }
    if (p_sink_out) *p_sink_out = exp(sink - zmax) / den;
    free(z);
}

/* q: [Tq][H][d] (q_fmt f32 / bf16); comp / win: record arrays of one
 * sequence; topk: [Tq][k] or NULL for dense (HCA); out: [Tq][H][d] fp64.
 * p_out / p_sink_out (optional, for tests): weights of query 0, head 0 in
 * entry-list order, and its sink weight. Returns the entry count of the last
 * query. */
ORC_API long orc_attention(const void* q, int q_fmt, const int32_t* q_pos, int Tq, int H,
                           const float* gamma_q, const float* sink, const orc_attn_params* P,
                           const uint8_t* comp, int comp_fmt, long comp_cap,
                           const uint8_t* win, int win_fmt, long win_cap,
                           const int32_t* topk, int k, double* out,
                           double* p_out, double* p_sink_out) {
    int d = P->d, dr = P->dr;
    int crec = orc_kv_record_bytes(comp_fmt, d, dr), wrec = orc_kv_record_bytes(win_fmt, d, dr);
    long maxn = (topk ? k : comp_cap) + P->window + 1;
    long* slots = (long*)malloc(sizeof(long) * (size_t)maxn);
    char* kinds = (char*)malloc((size_t)maxn);
    double* ents = (double*)malloc(sizeof(double) * (size_t)maxn * d);
    double* gq = (double*)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < d; i++) gq[i] = gamma_q ? gamma_q[i] : 1.0;
    long n = 0;
    for (int i = 0; i < Tq; i++) {
        long t = q_pos[i];
        n = entry_list(t, topk ? topk + (size_t)i * k : NULL, k, comp_cap, P->m, win_cap,
                       P->window, slots, kinds);
#pragma omp parallel for schedule(static)
        for (long e = 0; e < n; e++) {
            if (kinds[e] == 0) orc_kv_decode(comp + (size_t)slots[e] * crec, comp_fmt, d, dr, ents + (size_t)e * d);
            else orc_kv_decode(win + (size_t)slots[e] * wrec, win_fmt, d, dr, ents + (size_t)e * d);
        }
#pragma omp parallel for schedule(static)
        for (int h = 0; h < H; h++) {
            double* qv = (double*)malloc(sizeof(double) * (size_t)d);
            double* qh = (double*)malloc(sizeof(double) * (size_t)d);
            for (int c = 0; c < d; c++) qv[c] = load_scalar(q, q_fmt, ((size_t)i * H + h) * d + c);
            orc_rmsnorm(qv, d, gq, P->eps, qh);
            orc_rope(qh, d, dr, (double)t, P->base);
            double* o = out + ((size_t)i * H + h) * d;
            int first = (i == 0 && h == 0);
            attend_one(qh, ents, n, d, P->scale, (double)sink[h], o, first ? p_out : NULL,
                       first ? p_sink_out : NULL);
            orc_rope(o, d, dr, -(double)t, P->base);
            free(qv); free(qh);
        }
    }
    free(slots); free(kinds); free(ents); free(gq);
    return n;
}

/* Grouped output projection (peacm CSA step 4: the head-dim-512 outputs are
 * projected in groups).  Reading: block-diagonal, heads grouped
 * consecutively, no bias:
 *   y[r, g*(D/G) + i] = sum_c o[r, g*(Hd/G) + c] * W[g][i][c].            */
ORC_API void orc_out_proj(const double* o, const double* W, long M, int Hd, int D, int G, double* y) {
    int dg = D / G, cg = Hd / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (long r = 0; r < M; r++)
        for (int g = 0; g < G; g++)
            for (int i = 0; i < dg; i++) {
                double s = 0.0;
                for (int c = 0; c < cg; c++)
                    s += o[(size_t)r * Hd + (size_t)g * cg + c] * W[((size_t)g * dg + i) * cg + c];
                y[(size_t)r * D + (size_t)g * dg + i] = s;
            }
}

/* ======================================================================
 * Projections with FP8 weights.  The pages fix the precision of every
 * parameter outside the MoE experts as FP8 ("DeepSeek-V4 preview review"
 * (deepseek.csdn.net), section 6.2 on precision and deployment; "DeepSeek V4
 * (Flash & Pro)" (github wiki article), specification table: FP4 + FP8 mixed
 * precision).  They say nothing of the scaling granularity or of the
 * activations.  Reading: a weight matrix is stored as E4M3 codes with one
 * fp32 scale per output row (value = e4m3(code) * scale, the per-row rule of
 * the FP8 KV records); activations are not quantised; no bias.
 * ====================================================================== */

/* Preparing weights (test input generation, not a step of the path): row n of
 * W [N][K] gets scale = max|W[n][:]| / 448 as an fp32 number (1 for an
 * all-zero row) and codes = nearest E4M3 of W[n][c] / scale. */
ORC_API void orc_fp8_rows_quant(const float* W, long N, int K, uint8_t* codes, float* scale) {
    for (long n = 0; n < N; n++) {
        double amax = 0.0;
        for (int c = 0; c < K; c++) {
            double a = fabs((double)W[(size_t)n * K + c]);
            if (a > amax) amax = a;
        }
        float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
        scale[n] = s;
        for (int c = 0; c < K; c++)
            codes[(size_t)n * K + c] = orc_e4m3_encode((float)((double)W[(size_t)n * K + c] / (double)s));
    }
}

/* A projection with FP8 weights, G groups of consecutive rows (G = 1: a dense
 * map, as the input projections; G > 1: the block-diagonal grouped output
 * projection of CSA step 4):
 *   y[r][g*(N/G) + i] = scale[g*(N/G) + i]
 *                       * sum_c x[r][g*(K/G) + c] * e4m3(W[g*(N/G) + i][c])
 * x [M][K], W [N][K/G] codes, scale [N], y [M][N]. */
ORC_API void orc_linear_fp8(const double* x, long M, int K, const uint8_t* W, const float* scale, int N,
                            int G, double* y) {
    int ng = N / G, kg = K / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (long r = 0; r < M; r++)
        for (int n = 0; n < N; n++) {
            int g = n / ng;
            double s = 0.0;
            for (int c = 0; c < kg; c++)
                s += x[(size_t)r * K + (size_t)g * kg + c] * orc_e4m3_decode(W[(size_t)n * kg + c]);
            y[(size_t)r * N + n] = (double)scale[n] * s;
        }
}
