// Host side of libs3d8: error reporting, size helpers, and the offline
// packer (centroid fit + frozen-centroid encode).
//
// The packer follows "Llama-Mobile: Efficient 2.7-Bit Quantization of VLMs",
// Sec. 3.4 "Quantization": channel absmax scales stored in bfloat16,
// normalised absolute values grouped into 3-vectors over consecutive output
// channels, k-means++ seeding and Lloyd-Max iterations, rounded integer
// centroids, then nearest-centroid assignment and sign extraction.  The byte
// layout is the one of the Graphcore blog "11 billion parameters on a phone",
// section "Bit layout".
//
// Determinism: every reduction runs over fixed chunks of kChunk vectors, each
// summed in vector order, and the chunk partials are combined in chunk order.
// The result therefore does not depend on the number of threads.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "s3d8.h"
#include "s3d8_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kChunk = 1 << 16;  // vectors per reduction chunk
constexpr int kCentroids = 32;

int resolve_threads(int32_t requested) {
    if (requested > 0) return requested;
    unsigned hc = std::thread::hardware_concurrency();
    return hc ? (int)hc : 1;
}

// Run fn(chunk) for chunk in [0, nchunks) on nthreads threads; chunks are
// handed out dynamically, each writes only its own outputs.
void parallel_chunks(int64_t nchunks, int nthreads, const std::function<void(int64_t)> &fn) {
    if (nchunks <= 0) return;
    int nt = (int)std::min<int64_t>(nthreads, nchunks);
    if (nt <= 1) {
        for (int64_t c = 0; c < nchunks; ++c) fn(c);
        return;
    }
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (;;) {
            int64_t c = next.fetch_add(1, std::memory_order_relaxed);
            if (c >= nchunks) break;
            fn(c);
        }
    };
    std::vector<std::thread> pool;
    pool.reserve(nt - 1);
    for (int i = 0; i < nt - 1; ++i) pool.emplace_back(worker);
    worker();
    for (auto &t : pool) t.join();
}

// fp32 -> bfloat16 bit pattern, round to nearest even (finite inputs).
uint16_t bf16_from_f32(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)((u + rounding) >> 16);
}

float f32_from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// SplitMix64, counter form: draw c is the output mix of seed + c * gamma
// (Steele, Lea, Flood, OOPSLA 2014).
uint64_t splitmix(uint64_t seed, uint64_t c) {
    uint64_t z = seed + c * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
double unit_draw(uint64_t seed, uint64_t c) {
    return (double)(splitmix(seed, c) >> 11) * 0x1.0p-53;
}

// The scaled-absolute 3-vectors, structure of arrays (one array per
// component), vector p = t*K + j.
struct Vectors {
    int64_t P = 0;
    std::vector<double> v[3];
};

int validate_host(const void *W, int64_t N, int64_t K, const void *a, const void *b, const void *c) {
    if (!W || !a || !b || !c) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    if (N <= 0 || K <= 0) return s3d8::fail(S3D8_ERR_INVALID_ARG, "N and K must be positive");
    if (K % 16 != 0) return s3d8::fail(S3D8_ERR_SHAPE, "K must be a multiple of 16");
    if (N > (int64_t(1) << 40) / K) return s3d8::fail(S3D8_ERR_SHAPE, "N*K too large");
    return S3D8_OK;
}

// alpha_i = bf16(max_j |W_ij| / 127.0f) for i < N, 0 for padded channels.
void channel_scales(const float *W, int64_t N, int64_t K, int nthreads, uint16_t *alpha) {
    const int64_t T = (N + 2) / 3;
    const int64_t rows_per = 64;
    parallel_chunks((3 * T + rows_per - 1) / rows_per, nthreads, [&](int64_t c) {
        int64_t i0 = c * rows_per, i1 = std::min<int64_t>(3 * T, i0 + rows_per);
        for (int64_t i = i0; i < i1; ++i) {
            if (i >= N) { alpha[i] = 0; continue; }
            const float *row = W + i * K;
            float a = 0.0f;
            for (int64_t j = 0; j < K; ++j) a = std::max(a, std::fabs(row[j]));
            volatile float s = a / 127.0f;
            alpha[i] = bf16_from_f32(s);
        }
    });
}

// W'_{t,j,d} = |W_{3t+d, j}| / alpha_{3t+d} in fp64 with the stored bf16
// scale; 0 for padded channels and zero scales.
bool make_vectors(const float *W, int64_t N, int64_t K, const uint16_t *alpha, int nthreads,
                  Vectors &out) {
    const int64_t T = (N + 2) / 3;
    out.P = T * K;
    try {
        for (int d = 0; d < 3; ++d) out.v[d].assign((size_t)out.P, 0.0);
    } catch (const std::bad_alloc &) {
        return false;
    }
    parallel_chunks(T, nthreads, [&](int64_t t) {
        for (int d = 0; d < 3; ++d) {
            int64_t i = 3 * t + d;
            double *dst = out.v[d].data() + t * K;
            if (i >= N) continue;
            double a = (double)f32_from_bf16(alpha[i]);
            if (a == 0.0) continue;
            const float *row = W + i * K;
            for (int64_t j = 0; j < K; ++j) dst[j] = std::fabs((double)row[j]) / a;
        }
    });
    return true;
}

// Squared distance with the components summed in order 0, 1, 2 and no
// fused multiply-add (this file is compiled with -ffp-contract=off).
inline double sqdist(double c0, double c1, double c2, double x0, double x1, double x2) {
    double e0 = c0 - x0, e1 = c1 - x1, e2 = c2 - x2;
    return e0 * e0 + e1 * e1 + e2 * e2;
}

// Nearest centre (lowest index on ties) for vectors [p0, p1), written to
// asg[p - p0]; the distance of each vector to its centre goes to
// dist[p - p0] when dist is non-null.  The loop runs centre-outer over a block of vectors so that the
// inner loop vectorises across vectors; each vector sees the same sequence
// of strict comparisons as a plain scan over l = 0..31.
void assign_block(const Vectors &V, const double *cent, int64_t p0, int64_t p1, int32_t *asg,
                  double *dist) {
    constexpr int B = 256;
    double bd[B];
    int32_t bl[B];
    for (int64_t s = p0; s < p1; s += B) {
        int n = (int)std::min<int64_t>(B, p1 - s);
        const double *x0 = V.v[0].data() + s, *x1 = V.v[1].data() + s, *x2 = V.v[2].data() + s;
        {
            double c0 = cent[0], c1 = cent[1], c2 = cent[2];
            for (int i = 0; i < n; ++i) {
                bd[i] = sqdist(c0, c1, c2, x0[i], x1[i], x2[i]);
                bl[i] = 0;
            }
        }
        for (int l = 1; l < kCentroids; ++l) {
            double c0 = cent[3 * l], c1 = cent[3 * l + 1], c2 = cent[3 * l + 2];
            for (int i = 0; i < n; ++i) {
                double dd = sqdist(c0, c1, c2, x0[i], x1[i], x2[i]);
                bool better = dd < bd[i];
                bd[i] = better ? dd : bd[i];
                bl[i] = better ? l : bl[i];
            }
        }
        for (int i = 0; i < n; ++i) asg[s - p0 + i] = bl[i];
        if (dist)
            for (int i = 0; i < n; ++i) dist[s - p0 + i] = bd[i];
    }
}

struct ChunkStats {
    double sum[3 * kCentroids];
    int64_t cnt[kCentroids];
    double dist;
    int64_t changed;
};

// One assignment pass: new nearest centres, per-chunk distortion, changed
// count and per-cluster sums (for the next Lloyd update), each accumulated
// in vector order inside the chunk.
void assignment_pass(const Vectors &V, const double *cent, int nthreads, std::vector<int32_t> &asg,
                     std::vector<double> &scratch, std::vector<ChunkStats> &stats, bool first) {
    const int64_t nchunks = (V.P + kChunk - 1) / kChunk;
    stats.assign((size_t)nchunks, ChunkStats{});
    parallel_chunks(nchunks, nthreads, [&](int64_t c) {
        int64_t p0 = c * kChunk, p1 = std::min<int64_t>(V.P, p0 + kChunk);
        ChunkStats &st = stats[(size_t)c];
        std::memset(&st, 0, sizeof(st));
        std::vector<int32_t> na((size_t)(p1 - p0));
        assign_block(V, cent, p0, p1, na.data(), scratch.data() + p0);
        for (int64_t p = p0; p < p1; ++p) {
            int32_t l = na[(size_t)(p - p0)];
            if (!first && l != asg[(size_t)p]) ++st.changed;
            asg[(size_t)p] = l;
            st.dist += scratch[(size_t)p];
        }
        for (int64_t p = p0; p < p1; ++p) {
            int32_t l = asg[(size_t)p];
            st.cnt[l] += 1;
            st.sum[3 * l + 0] += V.v[0][(size_t)p];
            st.sum[3 * l + 1] += V.v[1][(size_t)p];
            st.sum[3 * l + 2] += V.v[2][(size_t)p];
        }
    });
}

// k-means++ seeding ("k-means++: the advantages of careful seeding",
// Arthur and Vassilvitskii, 2007): the first centre uniform over the
// vectors, each next one drawn with probability proportional to the squared
// distance to the nearest chosen centre.  Pick l uses draw l + 1; if every
// squared distance is zero the pick is uniform.
void kmeanspp(const Vectors &V, uint64_t seed, int nthreads, double *cent,
              std::vector<double> &d2) {
    const int64_t P = V.P;
    const int64_t nchunks = (P + kChunk - 1) / kChunk;
    auto pick_uniform = [&](double u) {
        int64_t p = (int64_t)(u * (double)P);
        return p >= P ? P - 1 : p;
    };
    int64_t first = pick_uniform(unit_draw(seed, 1));
    for (int d = 0; d < 3; ++d) cent[d] = V.v[d][(size_t)first];
    std::vector<double> csum((size_t)nchunks);
    parallel_chunks(nchunks, nthreads, [&](int64_t c) {
        int64_t p0 = c * kChunk, p1 = std::min<int64_t>(P, p0 + kChunk);
        double s = 0.0;
        for (int64_t p = p0; p < p1; ++p) {
            double dd = sqdist(cent[0], cent[1], cent[2], V.v[0][(size_t)p], V.v[1][(size_t)p],
                               V.v[2][(size_t)p]);
            d2[(size_t)p] = dd;
            s += dd;
        }
        csum[(size_t)c] = s;
    });
    for (int l = 1; l < kCentroids; ++l) {
        double total = 0.0;
        for (int64_t c = 0; c < nchunks; ++c) total += csum[(size_t)c];
        double u = unit_draw(seed, (uint64_t)l + 1);
        int64_t pick = P - 1;
        if (total > 0.0) {
            double target = u * total;
            double run = 0.0;
            for (int64_t c = 0; c < nchunks; ++c) {
                if (run + csum[(size_t)c] > target) {
                    int64_t p0 = c * kChunk, p1 = std::min<int64_t>(P, p0 + kChunk);
                    bool hit = false;
                    for (int64_t p = p0; p < p1; ++p) {
                        run += d2[(size_t)p];
                        if (run > target) { pick = p; hit = true; break; }
                    }
                    if (hit) break;
                    // rounding left the chunk's running total at the target:
                    // keep scanning the following chunks
                    continue;
                }
                run += csum[(size_t)c];
            }
        } else {
            pick = pick_uniform(u);
        }
        double *cl = cent + 3 * l;
        for (int d = 0; d < 3; ++d) cl[d] = V.v[d][(size_t)pick];
        parallel_chunks(nchunks, nthreads, [&](int64_t c) {
            int64_t p0 = c * kChunk, p1 = std::min<int64_t>(P, p0 + kChunk);
            double s = 0.0;
            for (int64_t p = p0; p < p1; ++p) {
                double dd = sqdist(cl[0], cl[1], cl[2], V.v[0][(size_t)p], V.v[1][(size_t)p],
                                   V.v[2][(size_t)p]);
                double cur = d2[(size_t)p];
                cur = dd < cur ? dd : cur;
                d2[(size_t)p] = cur;
                s += cur;
            }
            csum[(size_t)c] = s;
        });
    }
}

void encode_bytes(const float *W, int64_t N, int64_t K, const Vectors &V, const double *cent,
                  int nthreads, uint8_t *packed) {
    const int64_t T = (N + 2) / 3;
    parallel_chunks(T, nthreads, [&](int64_t t) {
        std::vector<int32_t> q((size_t)K);
        assign_block(V, cent, t * K, (t + 1) * K, q.data(), nullptr);
        for (int64_t j = 0; j < K; ++j) {
            uint32_t s[3];
            for (int d = 0; d < 3; ++d) {
                int64_t i = 3 * t + d;
                s[d] = (i < N && W[i * K + j] < 0.0f) ? 1u : 0u;
            }
            // [S2 xor S0, S1, Q4..Q0, S0], bit 7 down to bit 0
            uint32_t b = s[0] | ((uint32_t)q[(size_t)j] << 1) | (s[1] << 6) | ((s[2] ^ s[0]) << 7);
            packed[t * K + j] = (uint8_t)b;
        }
    });
}

}  // namespace

namespace s3d8 {
int fail(int code, const char *msg) {
    g_last_error = msg;
    return code;
}
void clear_error() { g_last_error.clear(); }
}  // namespace s3d8

extern "C" {

int32_t s3d8_version(void) { return 20100; }

int64_t s3d8_num_triples(int64_t N) { return N > 0 ? (N + 2) / 3 : -1; }

int64_t s3d8_packed_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return -1;
    return s3d8_num_triples(N) * K;
}

int64_t s3d8_format_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return -1;
    int64_t T = s3d8_num_triples(N);
    return T * K + 2 * (3 * T) + 96;
}

const char *s3d8_last_error(void) { return g_last_error.c_str(); }

int32_t s3d8_encode(const float *W, int64_t N, int64_t K, const uint8_t *centroids,
                    int32_t num_threads, uint16_t *scales_bf16, uint8_t *packed) {
    int rc = validate_host(W, N, K, centroids, scales_bf16, packed);
    if (rc) return rc;
    for (int e = 0; e < 96; ++e)
        if (centroids[e] > 127) return s3d8::fail(S3D8_ERR_INVALID_ARG, "centroid entry above 127");
    try {
        const int nt = resolve_threads(num_threads);
        channel_scales(W, N, K, nt, scales_bf16);
        Vectors V;
        if (!make_vectors(W, N, K, scales_bf16, nt, V))
            return s3d8::fail(S3D8_ERR_NOMEM, "host allocation failed");
        double cent[96];
        for (int e = 0; e < 96; ++e) cent[e] = (double)centroids[e];
        encode_bytes(W, N, K, V, cent, nt, packed);
    } catch (const std::bad_alloc &) {
        return s3d8::fail(S3D8_ERR_NOMEM, "host allocation failed");
    } catch (...) {
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "unexpected host exception");
    }
    s3d8::clear_error();
    return S3D8_OK;
}

int32_t s3d8_pack(const float *W, int64_t N, int64_t K, uint64_t seed, int32_t max_iters,
                  int32_t num_threads, uint8_t *centroids, uint16_t *scales_bf16,
                  uint8_t *packed, double *distortion, int32_t *iterations) {
    int rc = validate_host(W, N, K, centroids, scales_bf16, packed);
    if (rc) return rc;
    if (max_iters < 0) return s3d8::fail(S3D8_ERR_INVALID_ARG, "max_iters must be >= 0");
    try {
        const int nt = resolve_threads(num_threads);
        channel_scales(W, N, K, nt, scales_bf16);
        Vectors V;
        if (!make_vectors(W, N, K, scales_bf16, nt, V))
            return s3d8::fail(S3D8_ERR_NOMEM, "host allocation failed");
        std::vector<double> scratch((size_t)V.P);
        std::vector<int32_t> asg((size_t)V.P);
        double cent[96];
        kmeanspp(V, seed, nt, cent, scratch);

        std::vector<ChunkStats> stats;
        auto reduce = [&](double &dist, int64_t &changed, double *sum, int64_t *cnt) {
            dist = 0.0;
            changed = 0;
            std::fill(sum, sum + 96, 0.0);
            std::fill(cnt, cnt + 32, 0);
            for (const ChunkStats &st : stats) {
                dist += st.dist;
                changed += st.changed;
                for (int e = 0; e < 96; ++e) sum[e] += st.sum[e];
                for (int l = 0; l < 32; ++l) cnt[l] += st.cnt[l];
            }
        };
        double dist, sum[96];
        int64_t changed, cnt[32];
        assignment_pass(V, cent, nt, asg, scratch, stats, true);
        reduce(dist, changed, sum, cnt);
        if (distortion) distortion[0] = dist;
        int32_t it = 0;
        while (it < max_iters) {
            for (int l = 0; l < 32; ++l)
                if (cnt[l] > 0)
                    for (int d = 0; d < 3; ++d) cent[3 * l + d] = sum[3 * l + d] / (double)cnt[l];
            ++it;
            assignment_pass(V, cent, nt, asg, scratch, stats, false);
            reduce(dist, changed, sum, cnt);
            if (distortion) distortion[it] = dist;
            if (changed == 0) break;
        }
        if (iterations) *iterations = it;

        double rc_cent[96];
        for (int e = 0; e < 96; ++e) {
            double r = std::nearbyint(cent[e]);  // default mode: half to even
            r = std::min(127.0, std::max(0.0, r));
            centroids[e] = (uint8_t)r;
            rc_cent[e] = r;
        }
        encode_bytes(W, N, K, V, rc_cent, nt, packed);
    } catch (const std::bad_alloc &) {
        return s3d8::fail(S3D8_ERR_NOMEM, "host allocation failed");
    } catch (...) {
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "unexpected host exception");
    }
    s3d8::clear_error();
    return S3D8_OK;
}

}  // extern "C"
