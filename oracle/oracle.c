/*
 * Plain CPU oracle for the S3D8 weight-decode-fused linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads
 * or calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Sources (cited by page title and section/equation):
 *   [BLOG]  "11 billion parameters on a phone" (Graphcore Research blog),
 *           sections "S3D8: a 2.7-bit weight format for fast decoding",
 *           "Bit layout", "Output channel packing", "Fused matrix-vector
 *           product", "QAT details".
 *   [PAPER] "Llama-Mobile: Efficient 2.7-Bit Quantization of VLMs" (arXiv),
 *           Sec. 3.4 "The S3D8 Format" (Eq. 1 and the "Quantization"
 *           equations), Sec. 4 (channel-scaled INT8 activations),
 *           Appendix A.3.
 *
 * Every routine is the plain definition written out: scalar loops, no
 * blocking, no intrinsics.  Floating point is fp32 exactly where the pages
 * fix it (the activation scale is a float, the epilogue multiplies floats,
 * channel scales are bfloat16) and fp64 elsewhere (centroid fitting and
 * nearest-centroid assignment).  Build with -ffp-contract=off so that no
 * multiply-add is fused.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - activation scale is one fp32 absmax/127 per token (row of X);
 *   - activation rounding is round-half-to-even of the IEEE fp32 quotient,
 *     clamped to [-127, 127]; an all-zero row has scale 0 and codes 0;
 *   - channel scale alpha = bf16_rne(max|W| / 127.0f), and the stored bf16
 *     value is the one used to normalise weights for fitting/assignment;
 *   - padded channels (n rounded up to a multiple of 3) have alpha = 0,
 *     normalised value 0 and sign selector 0;
 *   - nearest-centroid ties go to the lowest index;
 *   - k-means++ draws come from SplitMix64 (counter form); Lloyd stops when
 *     no assignment changes or after max_iters; an empty cluster keeps its
 *     centroid; centroids are rounded half-to-even and clamped to [0,127];
 *   - 3D8 (the unstructured format the blog compares S3D8 with) keeps S3D8's
 *     channel packing, scales and matrix layout; its table is int8 [256][3],
 *     row-major, entries in [-127, 127], and the whole byte is the row index;
 *   - bfloat16 output is the round-to-nearest-even of the fp32 epilogue value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bfloat16 <-> fp32                                                   */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 word. */
float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even of a finite fp32 to bf16: keep the upper 16 bits,
 * rounding on the discarded lower 16 bits, ties to the even upper half. */
uint16_t oracle_f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* ------------------------------------------------------------------ */
/* Format: byte fields and Eq. 1                                       */
/* ------------------------------------------------------------------ */

/* [BLOG] "Bit layout": the physical byte is [S2 xor S0, S1, Q4..Q0, S0]
 * from bit 7 down to bit 0: S0 in bit 0, the 5-bit shared index Q in bits
 * 5..1, S1 in bit 6 and the sign difference S2 xor S0 in bit 7.  A sign
 * selector of 1 selects the negative value. */
void oracle_byte_fields(uint8_t b, int32_t *q, int32_t *s0, int32_t *s1, int32_t *s2) {
    int32_t bit0 = b & 1;
    int32_t bit6 = (b >> 6) & 1;
    int32_t bit7 = (b >> 7) & 1;
    *q = (b >> 1) & 31;
    *s0 = bit0;
    *s1 = bit6;
    *s2 = bit7 ^ bit0;
}

/* The inverse: fields -> physical byte, per the same layout. */
uint8_t oracle_byte_from_fields(int32_t q, int32_t s0, int32_t s1, int32_t s2) {
    uint32_t b = 0;
    b |= (uint32_t)(s0 & 1);
    b |= ((uint32_t)(q & 31)) << 1;
    b |= ((uint32_t)(s1 & 1)) << 6;
    b |= ((uint32_t)((s2 ^ s0) & 1)) << 7;
    return (uint8_t)b;
}

/* [PAPER] Eq. 1 without the channel scale: the channel-INT8 weight
 *   w_ij = s_ij * C[q_{floor(i/3), j}][i mod 3]
 * with the packed matrix stored as ceil(n/3) rows of k bytes, each byte
 * holding output channels 3t, 3t+1, 3t+2 at input column j ([BLOG]
 * "Output channel packing"; k-contiguous per channel triple as in the
 * [BLOG] fused matrix-vector listing).  C is 32 x 3, row-major. */
int32_t oracle_decode_weight(const uint8_t *packed, const uint8_t *C, int64_t K,
                             int64_t i, int64_t j) {
    int64_t t = i / 3;
    int32_t d = (int32_t)(i % 3);
    uint8_t b = packed[t * K + j];
    int32_t q, s0, s1, s2;
    oracle_byte_fields(b, &q, &s0, &s1, &s2);
    int32_t s = (d == 0) ? s0 : (d == 1) ? s1 : s2;
    int32_t c = (int32_t)C[q * 3 + d];
    return s ? -c : c;
}

/* Decode the whole matrix, one weight at a time: w is [N][K] int8. */
void oracle_decode(const uint8_t *packed, const uint8_t *C, int64_t N, int64_t K, int8_t *w) {
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < K; ++j)
            w[i * K + j] = (int8_t)oracle_decode_weight(packed, C, K, i, j);
}

/* ------------------------------------------------------------------ */
/* 3D8: the unstructured 3-weights-per-byte format                     */
/* ------------------------------------------------------------------ */

/* [BLOG] "S3D8: a 2.7-bit weight format for fast decoding" and "S3D8
 * design notes": the plain 3-values-per-byte vector format uses the whole
 * byte as an 8-bit index into a (256, 3) table of signed values (768
 * bytes), with no separate sign selectors.  Channel packing, scales and
 * the packed matrix layout are those of S3D8; only the byte -> weights
 * step differs:  w_ij = T[b][i mod 3], b = packed[floor(i/3)][j], with T
 * row-major int8 [256][3]. */
int32_t oracle_decode_weight_3d8(const uint8_t *packed, const int8_t *T3, int64_t K,
                                 int64_t i, int64_t j) {
    int64_t t = i / 3;
    int32_t d = (int32_t)(i % 3);
    uint8_t b = packed[t * K + j];
    return (int32_t)T3[(int64_t)b * 3 + d];
}

/* The whole 3D8 matrix, one weight at a time: w is [N][K] int8. */
void oracle_decode_3d8(const uint8_t *packed, const int8_t *T3, int64_t N, int64_t K, int8_t *w) {
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < K; ++j)
            w[i * K + j] = (int8_t)oracle_decode_weight_3d8(packed, T3, K, i, j);
}

/* ------------------------------------------------------------------ */
/* Activation quantisation (per-token channel-scaled INT8)             */
/* ------------------------------------------------------------------ */

/* [PAPER] Sec. 4 / A.3 and [BLOG] "QAT details": activations are
 * channel-scaled INT8 with absmax scaling; the [BLOG] fused listing takes
 * one float scale per activation vector.  Per row m:
 *   a = max_j |x_mj|;  s_m = a / 127 (fp32);
 *   xq_mj = clamp(round_half_even(x_mj / s_m), -127, 127);
 * and s_m = 0, xq = 0 for an all-zero row. */
void oracle_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs) {
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * K;
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float v = fabsf(row[j]);
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            xs[m] = 0.0f;
            for (int64_t j = 0; j < K; ++j) xq[m * K + j] = 0;
            continue;
        }
        volatile float s = a / 127.0f;
        xs[m] = s;
        for (int64_t j = 0; j < K; ++j) {
            volatile float quot = row[j] / s;
            float r = nearbyintf(quot); /* default rounding mode: half to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[m * K + j] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------------------ */
/* INT8 x INT8 -> INT32 products and the fp32 epilogue                 */
/* ------------------------------------------------------------------ */

/* One output element: acc = sum_j xq[j] * w[n][j], every weight decoded by
 * Eq. 1 on the fly, summed in int64. */
int64_t oracle_acc_one(const int8_t *xq_row, const uint8_t *packed, const uint8_t *C,
                       int64_t K, int64_t n) {
    int64_t acc = 0;
    for (int64_t j = 0; j < K; ++j)
        acc += (int64_t)xq_row[j] * (int64_t)oracle_decode_weight(packed, C, K, n, j);
    return acc;
}

/* acc[M][N] = xq[M][K] . w[N][K]^T with w decoded one weight at a time.
 * Sums are int64; returns 0 if every |acc| <= K*127*127 (so the value fits
 * INT32 exactly), else 1.  Output rows n run in parallel (OpenMP), each
 * dot product is a plain sequential loop. */
int32_t oracle_linear_acc(const int8_t *xq, int64_t M, int64_t K, int64_t N,
                          const uint8_t *packed, const uint8_t *C, int32_t *acc) {
    const int64_t bound = K * 127 * 127;
    int32_t bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        int8_t *wrow = (int8_t *)malloc((size_t)(K > 0 ? K : 1));
        for (int64_t j = 0; j < K; ++j) wrow[j] = (int8_t)oracle_decode_weight(packed, C, K, n, j);
        for (int64_t m = 0; m < M; ++m) {
            int64_t s = 0;
            const int8_t *xr = xq + m * K;
            for (int64_t j = 0; j < K; ++j) s += (int64_t)xr[j] * (int64_t)wrow[j];
            if (s > bound || s < -bound || s > INT32_MAX || s < INT32_MIN) bad |= 1;
            acc[m * N + n] = (int32_t)s;
        }
        free(wrow);
    }
    return bad;
}

/* acc[M][N] = xq[M][K] . w[N][K]^T for an already decoded int8 weight
 * matrix (any format), summed in int64; returns 1 if some |acc| exceeds
 * K*127*127, else 0. */
int32_t oracle_linear_acc_decoded(const int8_t *xq, int64_t M, int64_t K, int64_t N,
                                  const int8_t *w, int32_t *acc) {
    const int64_t bound = K * 127 * 127;
    int32_t bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *wrow = w + n * K;
        for (int64_t m = 0; m < M; ++m) {
            int64_t s = 0;
            const int8_t *xr = xq + m * K;
            for (int64_t j = 0; j < K; ++j) s += (int64_t)xr[j] * (int64_t)wrow[j];
            if (s > bound || s < -bound) bad |= 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad;
}

/* [BLOG] "Fused matrix-vector product": y = x_s * float(acc) * float(W_s),
 * evaluated left to right in fp32 with the bf16 channel scale widened to
 * fp32.  y is [M][N]. */
void oracle_epilogue(const int32_t *acc, const float *xs, const uint16_t *alpha_bf16,
                     int64_t M, int64_t N, float *y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            volatile float a = (float)acc[m * N + n];
            volatile float t = xs[m] * a;
            volatile float r = t * oracle_bf16_to_f32(alpha_bf16[n]);
            y[m * N + n] = r;
        }
}

/* [BLOG] "Fused matrix-vector product": the blog's kernel converts each
 * fp32 result to bfloat16 on the way out.  y16[e] = bf16_rne(y[e]) for the
 * fp32 epilogue values y (round to nearest even, as the conversion above). */
void oracle_to_bf16(const float *y, int64_t n, uint16_t *y16) {
    for (int64_t e = 0; e < n; ++e) y16[e] = oracle_f32_to_bf16_rne(y[e]);
}

/* ------------------------------------------------------------------ */
/* Channel scales, normalisation, signs, nearest-centroid assignment   */
/* ------------------------------------------------------------------ */

int64_t oracle_num_triples(int64_t N) { return (N + 2) / 3; }

/* [PAPER] Sec. 3.4 "Quantization": alpha_i = max_j |W_ij| / 127, stored in
 * bfloat16 ([BLOG] "S3D8" list; A.3 "scale is stored in bfloat16").  The
 * division is fp32; padded channels get 0.  alpha has 3*ceil(N/3) entries. */
void oracle_channel_scales(const float *W, int64_t N, int64_t K, uint16_t *alpha) {
    int64_t npad = 3 * oracle_num_triples(N);
    for (int64_t i = 0; i < npad; ++i) {
        if (i >= N) { alpha[i] = 0; continue; }
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float v = fabsf(W[i * K + j]);
            if (v > a) a = v;
        }
        volatile float s = a / 127.0f;
        alpha[i] = oracle_f32_to_bf16_rne(s);
    }
}

/* W'_{i'jd} = |W_{3i'+d, j}| / alpha_{3i'+d} in fp64, with the stored
 * (bf16) alpha; 0 for padded channels and for alpha = 0. */
static double normalised(const float *W, int64_t N, int64_t K, const uint16_t *alpha,
                         int64_t t, int32_t d, int64_t j) {
    int64_t i = 3 * t + d;
    if (i >= N) return 0.0;
    double a = (double)oracle_bf16_to_f32(alpha[i]);
    if (a == 0.0) return 0.0;
    return fabs((double)W[i * K + j]) / a;
}

/* Squared Euclidean distance, summed in component order 0, 1, 2. */
static double dist3(const double *c, const double *v) {
    double e0 = c[0] - v[0];
    double e1 = c[1] - v[1];
    double e2 = c[2] - v[2];
    return e0 * e0 + e1 * e1 + e2 * e2;
}

/* q = argmin_l ||C_l - W'||_2 over l = 0..31, lowest index on ties. */
static int32_t nearest(const double *cent /*[32*3]*/, const double *v) {
    int32_t best = 0;
    double bd = dist3(cent, v);
    for (int32_t l = 1; l < 32; ++l) {
        double dd = dist3(cent + 3 * l, v);
        if (dd < bd) { bd = dd; best = l; }
    }
    return best;
}

/* [PAPER] Sec. 3.4, QAT phase with frozen centroids: scale as above,
 * s_ij = +1 if W_ij >= 0 else -1, q = nearest integer centroid to the
 * scaled-absolute 3-vector; then pack per the [BLOG] bit layout.  Signs of
 * padded channels are +1. */
void oracle_encode(const float *W, int64_t N, int64_t K, const uint8_t *C,
                   uint16_t *alpha, uint8_t *packed) {
    int64_t T = oracle_num_triples(N);
    double cent[96];
    for (int32_t e = 0; e < 96; ++e) cent[e] = (double)C[e];
    oracle_channel_scales(W, N, K, alpha);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j) {
            double v[3];
            int32_t s[3];
            for (int32_t d = 0; d < 3; ++d) {
                int64_t i = 3 * t + d;
                v[d] = normalised(W, N, K, alpha, t, d, j);
                s[d] = (i < N && W[i * K + j] < 0.0f) ? 1 : 0;
            }
            int32_t q = nearest(cent, v);
            packed[t * K + j] = oracle_byte_from_fields(q, s[0], s[1], s[2]);
        }
}

/* ------------------------------------------------------------------ */
/* Centroid fit: k-means++ seeding, Lloyd-Max iterations, rounding      */
/* ------------------------------------------------------------------ */

/* SplitMix64 in counter form (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): draw number c (c >= 1) is
 * the mix of seed + c * gamma.  A uniform double in [0,1) takes the top 53
 * bits. */
static uint64_t splitmix64_draw(uint64_t seed, uint64_t c) {
    uint64_t z = seed + c * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform01(uint64_t seed, uint64_t c) {
    return (double)(splitmix64_draw(seed, c) >> 11) * (1.0 / 9007199254740992.0);
}
uint64_t oracle_splitmix64(uint64_t seed, uint64_t c) { return splitmix64_draw(seed, c); }

/* Round half to even for a finite double. */
static double round_half_even(double v) {
    double f = floor(v);
    double r = v - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* [PAPER] Sec. 3.4 "Quantization": normalise each output channel by its
 * absmax scale, take absolute values, zero-pad to a multiple of 3 channels
 * and reshape into 3-vectors (one per channel triple and input column);
 * seed 32 centroids with k-means++ (each new centre drawn with probability
 * proportional to the squared distance to the nearest chosen centre, the
 * first uniformly); run Lloyd-Max (assign every vector to its nearest
 * centre, move every centre to the mean of its vectors) until no
 * assignment changes or max_iters; C = Round(centres), clamped to [0,127].
 *
 * Draw numbering: k-means++ pick p (0..31) uses draw p+1.  If every
 * remaining squared distance is 0 (fewer than 32 distinct vectors), the
 * pick is uniform, like the first.
 *
 * Outputs: C (32x3 uint8), centres_real (32x3 fp64, before rounding),
 * distortion[0..iters] = sum of squared distances to the nearest centre
 * after seeding (index 0) and after each Lloyd update, iterations run.
 * alpha must already hold the bf16 scales (oracle_channel_scales).
 * Returns the number of Lloyd iterations run, or -1 on allocation failure. */
int32_t oracle_fit_centroids(const float *W, int64_t N, int64_t K, const uint16_t *alpha,
                             uint64_t seed, int32_t max_iters, uint8_t *C,
                             double *centres_real, double *distortion) {
    int64_t T = oracle_num_triples(N);
    int64_t P = T * K; /* number of 3-vectors */
    double *pts = (double *)malloc((size_t)P * 3 * sizeof(double));
    double *d2 = (double *)malloc((size_t)P * sizeof(double));
    int32_t *asg = (int32_t *)malloc((size_t)P * sizeof(int32_t));
    if (!pts || !d2 || !asg) { free(pts); free(d2); free(asg); return -1; }

    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j)
            for (int32_t d = 0; d < 3; ++d)
                pts[(t * K + j) * 3 + d] = normalised(W, N, K, alpha, t, d, j);

    double cent[96];
    /* k-means++ seeding */
    int64_t first = (int64_t)(uniform01(seed, 1) * (double)P);
    if (first >= P) first = P - 1;
    for (int32_t d = 0; d < 3; ++d) cent[d] = pts[first * 3 + d];
    for (int64_t p = 0; p < P; ++p) d2[p] = dist3(cent, pts + p * 3);
    for (int32_t l = 1; l < 32; ++l) {
        double total = 0.0;
        for (int64_t p = 0; p < P; ++p) total += d2[p];
        double u = uniform01(seed, (uint64_t)l + 1);
        int64_t pick;
        if (total > 0.0) {
            double target = u * total;
            double run = 0.0;
            pick = P - 1;
            for (int64_t p = 0; p < P; ++p) {
                run += d2[p];
                if (run > target) { pick = p; break; }
            }
        } else {
            pick = (int64_t)(u * (double)P);
            if (pick >= P) pick = P - 1;
        }
        for (int32_t d = 0; d < 3; ++d) cent[3 * l + d] = pts[pick * 3 + d];
        for (int64_t p = 0; p < P; ++p) {
            double dd = dist3(cent + 3 * l, pts + p * 3);
            if (dd < d2[p]) d2[p] = dd;
        }
    }

    /* Lloyd-Max iterations */
    double dist0 = 0.0;
    for (int64_t p = 0; p < P; ++p) {
        asg[p] = nearest(cent, pts + p * 3);
        dist0 += dist3(cent + 3 * asg[p], pts + p * 3);
    }
    if (distortion) distortion[0] = dist0;
    int32_t it = 0;
    while (it < max_iters) {
        double sum[96];
        int64_t cnt[32];
        for (int32_t e = 0; e < 96; ++e) sum[e] = 0.0;
        for (int32_t l = 0; l < 32; ++l) cnt[l] = 0;
        for (int64_t p = 0; p < P; ++p) {
            int32_t l = asg[p];
            cnt[l] += 1;
            for (int32_t d = 0; d < 3; ++d) sum[3 * l + d] += pts[p * 3 + d];
        }
        for (int32_t l = 0; l < 32; ++l)
            if (cnt[l] > 0)
                for (int32_t d = 0; d < 3; ++d) cent[3 * l + d] = sum[3 * l + d] / (double)cnt[l];
        ++it;
        int64_t changed = 0;
        double dist = 0.0;
        for (int64_t p = 0; p < P; ++p) {
            int32_t l = nearest(cent, pts + p * 3);
            if (l != asg[p]) { ++changed; asg[p] = l; }
            dist += dist3(cent + 3 * l, pts + p * 3);
        }
        if (distortion) distortion[it] = dist;
        if (changed == 0) break;
    }

    for (int32_t e = 0; e < 96; ++e) {
        if (centres_real) centres_real[e] = cent[e];
        double r = round_half_even(cent[e]);
        if (r < 0.0) r = 0.0;
        if (r > 127.0) r = 127.0;
        C[e] = (uint8_t)r;
    }
    free(pts);
    free(d2);
    free(asg);
    return it;
}
