// Device side of libs3d8 for gfx950 (CDNA4): activation quantisation, the
// S3D8 decode, the fused decode GEMV/GEMM and the standalone dequantiser,
// plus the device entry points of the C ABI.
//
// Format and arithmetic follow "Llama-Mobile: Efficient 2.7-Bit Quantization
// of VLMs" (Sec. 3.4, Eq. 1) and the Graphcore blog "11 billion parameters
// on a phone" ("Bit layout", "Output channel packing", "Fused matrix-vector
// product").
//
// Decode on the GPU.  The blog folds the sign selectors into three signed
// 64-entry lookup tables so that no separate sign step is needed.  Here the
// same idea is taken one step further for LDS: one 256-entry table indexed by
// the whole packed byte returns the three signed INT8 weights of the byte in
// one dword, [w0, w1, w2, 0].  It is built in LDS by every workgroup from the
// 96-byte centroid table.  To make random lookups from 64 lanes free of bank
// conflicts the table is stored 64 times, interleaved so that lane L always
// reads copy L: entry b of copy L sits at byte address (b << 8) | (L << 2).
// That address is a single v_perm_b32 of the packed dword and the lane
// offset.  Four lookups give a 4x3 byte block; seven more v_perm_b32 turn it
// into one dword of four consecutive-k weights per output channel, which is
// exactly the INT8 operand layout of the MFMA instructions.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "s3d8.h"
#include "s3d8_internal.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kTabEntries = 256;
constexpr int kTabCopies = 64;
constexpr int kTabWords = kTabEntries * kTabCopies;  // 64 KiB of LDS

// --------------------------------------------------------------- decode

// Signed weights of packed byte b as bytes [w0, w1, w2, 0]: q = bits 5..1,
// S0 = bit 0, S1 = bit 6, S2 = bit 7 xor bit 0 (blog "Bit layout");
// w_d = (S_d ? -1 : +1) * C[q][d] (paper Eq. 1 without alpha).
__device__ __forceinline__ uint32_t signed_triple(uint32_t b, const uint8_t *C) {
    const uint32_t q = (b >> 1) & 31u;
    const uint32_t s0 = b & 1u, s1 = (b >> 6) & 1u, s2 = ((b >> 7) ^ b) & 1u;
    const int32_t c0 = C[3 * q], c1 = C[3 * q + 1], c2 = C[3 * q + 2];
    const int32_t w0 = s0 ? -c0 : c0, w1 = s1 ? -c1 : c1, w2 = s2 ? -c2 : c2;
    return (uint32_t)(w0 & 0xFF) | ((uint32_t)(w1 & 0xFF) << 8) | ((uint32_t)(w2 & 0xFF) << 16);
}

// Build the lane-interleaved signed table.  Every wave writes one entry to
// 64 consecutive dwords per step.  Ends with a barrier.
__device__ __forceinline__ void build_table(uint32_t *tab, uint8_t *cl, const uint8_t *C) {
    const int tid = threadIdx.x, nth = blockDim.x;
    if (tid < 96) cl[tid] = C[tid];
    __syncthreads();
    for (int idx = tid; idx < kTabWords; idx += nth) tab[idx] = signed_triple((uint32_t)idx >> 6, cl);
    __syncthreads();
}

// Decode 16 packed bytes (k = 0..15 of one channel triple) into three
// 16-byte INT8 vectors, one per channel of the triple: o_d byte k = w_d(k).
__device__ __forceinline__ void decode16(const uint4 p, const uint32_t lane_off, const uint32_t *tab,
                                         v4i &o0, v4i &o1, v4i &o2) {
    const char *tb = reinterpret_cast<const char *>(tab);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t dw = w[c];
        // address = (byte_i << 8) | lane_off
        const uint32_t a0 = __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0400u);
        const uint32_t a1 = __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0500u);
        const uint32_t a2 = __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0600u);
        const uint32_t a3 = __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0700u);
        const uint32_t r0 = *reinterpret_cast<const uint32_t *>(tb + a0);
        const uint32_t r1 = *reinterpret_cast<const uint32_t *>(tb + a1);
        const uint32_t r2 = *reinterpret_cast<const uint32_t *>(tb + a2);
        const uint32_t r3 = *reinterpret_cast<const uint32_t *>(tb + a3);
        // 4x3 byte transpose: r_i = [w0, w1, w2, 0] of byte i
        const uint32_t p01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.w0 r1.w0 r0.w1 r1.w1
        const uint32_t p23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
        const uint32_t q01 = __builtin_amdgcn_perm(r1, r0, 0x0C0C0602u);  // r0.w2 r1.w2 0 0
        const uint32_t q23 = __builtin_amdgcn_perm(r3, r2, 0x0C0C0602u);
        o0[c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x05040100u);
        o1[c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x07060302u);
        o2[c] = (int32_t)__builtin_amdgcn_perm(q23, q01, 0x05040100u);
    }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// --------------------------------------------------------------- quant_act

// One workgroup per token row: absmax reduction, then s = a / 127 and
// xq = clamp(rne(x / s), -127, 127) with IEEE fp32 division (the paper's
// channel-scaled INT8 activations, one scale per token).
constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const float *__restrict__ x, int K,
                                                                  int8_t *__restrict__ xq,
                                                                  float *__restrict__ xs) {
    __shared__ float wmax[kQuantThreads / 64];
    const int64_t row = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + row * K);
    const int n4 = K >> 2;
    float a = 0.0f;
    for (int i = threadIdx.x; i < n4; i += kQuantThreads) {
        const float4 v = xr[i];
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
    __syncthreads();
    a = wmax[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) a = fmaxf(a, wmax[w]);
    const float s = a / 127.0f;
    if (threadIdx.x == 0) xs[row] = (a == 0.0f) ? 0.0f : s;
    char4 *qr = reinterpret_cast<char4 *>(xq + row * K);
    for (int i = threadIdx.x; i < n4; i += kQuantThreads) {
        const float4 v = xr[i];
        char4 o;
        if (a == 0.0f) {
            o = make_char4(0, 0, 0, 0);
        } else {
            o.x = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(v.x / s)));
            o.y = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(v.y / s)));
            o.z = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(v.z / s)));
            o.w = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(v.w / s)));
        }
        qr[i] = o;
    }
}

// --------------------------------------------------------------- GEMV

// Decode GEMV for up to 16 token rows (and, tiled over blockIdx.y, any M).
//
// Workgroup = kGemvWaves waves sharing one tile of 16 channel triples (48
// output channels) and splitting K between them.  Each wave runs
// v_mfma_i32_16x16x64_i8: the A operand holds the 16 token rows of X, the B
// operand the decoded weights of the 16 triples for one channel d of the
// triple, so three MFMAs (d = 0, 1, 2) consume one 64-column block of the
// packed matrix.  Lane L = n + 16*g holds A row n / B column n and bytes
// [16g, 16g + 16) of the 64-column block: its packed bytes are one 16-byte
// load of triple row n, and after decode16 they are already in B layout.
// Partial sums of the waves are added in LDS; the epilogue multiplies by
// the token scale and the bf16 channel scale and writes fp32.
constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = kGemvWaves * 64;
constexpr int kGemvUnroll = 4;

__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ xs, int M, int K, int N, int T,
    const uint8_t *__restrict__ packed, const uint8_t *__restrict__ centroids,
    const uint16_t *__restrict__ scales, float *__restrict__ y, int32_t *__restrict__ acc_out,
    int kb_per_wave) {
    __shared__ uint32_t tab[kTabWords];
    __shared__ uint8_t cl[96];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int t = blockIdx.x * 16 + n;   // triple of B column n
    const int m = blockIdx.y * 16 + n;   // token row of A row n
    const int KB = (K + 63) >> 6;
    const int kb0 = wave * kb_per_wave;
    const int kb1 = min(KB, kb0 + kb_per_wave);
    const bool tvalid = t < T, mvalid = m < M;
    const uint8_t *prow = packed + (int64_t)(tvalid ? t : 0) * K + g * 16;
    const int8_t *xrow = xq + (int64_t)(mvalid ? m : 0) * K + g * 16;
    const uint32_t lane_off = (uint32_t)lane << 2;

    // first block of loads goes out before the table is built
    uint4 pk[kGemvUnroll];
    v4i xa[kGemvUnroll];
    auto load = [&](int kb) {
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) {
            const int b = kb + u;
            const bool ok = b < kb1 && (b * 64 + g * 16) < K;
            pk[u] = (ok && tvalid) ? *reinterpret_cast<const uint4 *>(prow + (int64_t)b * 64)
                                   : make_uint4(0, 0, 0, 0);
            xa[u] = (ok && mvalid) ? *reinterpret_cast<const v4i *>(xrow + (int64_t)b * 64)
                                   : v4i{0, 0, 0, 0};
        }
    };
    if (kb0 < kb1) load(kb0);

    build_table(tab, cl, centroids);

    v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
    for (int kb = kb0; kb < kb1; kb += kGemvUnroll) {
        if (kb != kb0) load(kb);
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) {
            v4i b0, b1, b2;
            decode16(pk[u], lane_off, tab, b0, b1, b2);
            acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[u], b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[u], b1, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[u], b2, acc2, 0, 0, 0);
        }
    }

    // cross-wave reduction in LDS (the table is dead from here on)
    __syncthreads();
    int32_t *red = reinterpret_cast<int32_t *>(tab);  // [wave][d][i][lane]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        red[((wave * 3 + 0) * 4 + i) * 64 + lane] = acc0[i];
        red[((wave * 3 + 1) * 4 + i) * 64 + lane] = acc1[i];
        red[((wave * 3 + 2) * 4 + i) * 64 + lane] = acc2[i];
    }
    __syncthreads();

    // D[row r][col n] of the 16x16 MFMA result sits in lane n + 16*(r/4),
    // element r%4.  Output channel of (col n, d) is 48*tile + 3n + d.
    const int rows = min(16, M - (int)blockIdx.y * 16);
    for (int idx = tid; idx < rows * 48; idx += kGemvThreads) {
        const int r = idx / 48, c = idx - r * 48;
        const int col = c / 3, d = c - col * 3;
        const int src = (d * 4 + (r & 3)) * 64 + col + 16 * (r >> 2);
        int32_t s = 0;
        for (int w = 0; w < kGemvWaves; ++w) s += red[w * 3 * 4 * 64 + src];
        const int ch = blockIdx.x * 48 + c;
        const int row = blockIdx.y * 16 + r;
        if (ch < N) {
            const float v = (xs[row] * (float)s) * bf16_to_f32(scales[ch]);
            y[(int64_t)row * N + ch] = v;
            if (acc_out) acc_out[(int64_t)row * N + ch] = s;
        }
    }
}

// --------------------------------------------------------------- dequant

// Standalone S3D8 -> channel-INT8 decode (the blog's dequantisation kernel).
// Persistent workgroups build the table once and stride over 16-byte chunks.
constexpr int kDequantThreads = 512;

__global__ __launch_bounds__(kDequantThreads) void dequant_kernel(
    const uint8_t *__restrict__ packed, const uint8_t *__restrict__ centroids, int K, int N,
    int64_t nchunks, int8_t *__restrict__ w) {
    __shared__ uint32_t tab[kTabWords];
    __shared__ uint8_t cl[96];
    build_table(tab, cl, centroids);
    const uint32_t lane_off = (uint32_t)(threadIdx.x & 63) << 2;
    const int cpr = K >> 4;  // 16-byte chunks per triple row
    for (int64_t c = (int64_t)blockIdx.x * kDequantThreads + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * kDequantThreads) {
        const int64_t t = c / cpr;
        const int j = (int)(c - t * cpr) * 16;
        const uint4 p = *reinterpret_cast<const uint4 *>(packed + t * K + j);
        v4i o[3];
        decode16(p, lane_off, tab, o[0], o[1], o[2]);
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const int64_t i = 3 * t + d;
            if (i < N) *reinterpret_cast<v4i *>(w + i * K + j) = o[d];
        }
    }
}

// --------------------------------------------------------------- host glue

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return s3d8::fail(S3D8_ERR_INVALID_ARG, "sizes must be positive");
    if (K % 16 != 0) return s3d8::fail(S3D8_ERR_SHAPE, "K must be a multiple of 16");
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (M > lim || K > lim || N > lim || (N + 2) / 3 > lim / K || M > lim / K || M > lim / N)
        return s3d8::fail(S3D8_ERR_SHAPE, "tensor too large (more than 2^31 elements)");
    return S3D8_OK;
}

// gfx950 check, cached per device.
int check_device(int *num_cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return s3d8::fail(S3D8_ERR_HIP, "hipGetDevice failed");
    static std::atomic<int> state[64];  // 0 unknown, >0 CU count (gfx950), -1 other
    if (dev < 0 || dev >= 64) return s3d8::fail(S3D8_ERR_DEVICE, "device ordinal out of range");
    int st = state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return s3d8::fail(S3D8_ERR_HIP, "hipGetDeviceProperties failed");
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? prop.multiProcessorCount : -1;
        if (st == 0) st = -1;
        state[dev].store(st, std::memory_order_release);
    }
    if (st < 0) return s3d8::fail(S3D8_ERR_DEVICE, "the current device is not a gfx950 (MI355X) GPU");
    if (num_cus) *num_cus = st;
    return S3D8_OK;
}

int launch_status() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return s3d8::fail(S3D8_ERR_HIP, hipGetErrorString(e));
    s3d8::clear_error();
    return S3D8_OK;
}

}  // namespace

extern "C" {

int32_t s3d8_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs, void *stream) {
    if (!x || !xq || !xs) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(M, K, 1);
    if (rc) return rc;
    if (!aligned16(x) || !aligned16(xq)) return s3d8::fail(S3D8_ERR_ALIGN, "x and xq must be 16-byte aligned");
    if (M > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "M too large");
    rc = check_device(nullptr);
    if (rc) return rc;
    hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)M), dim3(kQuantThreads), 0,
                       (hipStream_t)stream, x, (int)K, xq, xs);
    return launch_status();
}

int32_t s3d8_linear(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                    const uint8_t *packed, const uint8_t *centroids, const uint16_t *scales_bf16,
                    float *y, int32_t *acc_out, void *stream) {
    if (!xq || !xs || !packed || !centroids || !scales_bf16 || !y)
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(M, K, N);
    if (rc) return rc;
    if (!aligned16(xq) || !aligned16(packed))
        return s3d8::fail(S3D8_ERR_ALIGN, "xq and packed must be 16-byte aligned");
    const int64_t mtiles = (M + 15) / 16;
    if (mtiles > 65535) return s3d8::fail(S3D8_ERR_SHAPE, "M too large");
    rc = check_device(nullptr);
    if (rc) return rc;
    const int64_t T = (N + 2) / 3;
    const int KB = (int)((K + 63) / 64);
    const int kbpw = (KB + kGemvWaves - 1) / kGemvWaves;
    dim3 grid((unsigned)((T + 15) / 16), (unsigned)mtiles);
    hipLaunchKernelGGL(gemv_kernel, grid, dim3(kGemvThreads), 0, (hipStream_t)stream, xq, xs,
                       (int)M, (int)K, (int)N, (int)T, packed, centroids, scales_bf16, y, acc_out,
                       kbpw);
    return launch_status();
}

int32_t s3d8_dequant(const uint8_t *packed, const uint8_t *centroids, int64_t N, int64_t K, int8_t *w,
                     void *stream) {
    if (!packed || !centroids || !w) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(1, K, N);
    if (rc) return rc;
    if (!aligned16(packed) || !aligned16(w)) return s3d8::fail(S3D8_ERR_ALIGN, "packed and w must be 16-byte aligned");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const int64_t T = (N + 2) / 3;
    const int64_t nchunks = T * (K / 16);
    int64_t blocks = (nchunks + kDequantThreads - 1) / kDequantThreads;
    const int64_t cap = (int64_t)cus * 2;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(kDequantThreads), 0,
                       (hipStream_t)stream, packed, centroids, (int)K, (int)N, nchunks, w);
    return launch_status();
}

}  // extern "C"
