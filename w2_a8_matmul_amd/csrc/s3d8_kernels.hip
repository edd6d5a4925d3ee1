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

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "s3d8.h"
#include "s3d8_internal.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef int32_t v8i __attribute__((ext_vector_type(8)));

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

// Row b of a 3D8 table as bytes [w0, w1, w2, 0].  3D8 is the unstructured
// format the blog sets beside S3D8 ("S3D8: a 2.7-bit weight format for fast
// decoding"): the whole byte indexes a (256, 3) table of signed values,
// here int8, row-major, 768 bytes.  Channel packing, scales and layout are
// those of S3D8, so both formats decode through the same 256-entry table.
__device__ __forceinline__ uint32_t row_3d8(uint32_t b, const uint8_t *T) {
    return (uint32_t)T[3 * b] | ((uint32_t)T[3 * b + 1] << 8) | ((uint32_t)T[3 * b + 2] << 16);
}
constexpr int kTableWords3D8 = 192;  // 768 bytes (the S3D8 table is 24 words)

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

// Position, inside the streaming GEMV's per-wave code slice, of the code of
// column c (a multiple of 4): blocks of 64 stay in place, and inside a block
// the 8-byte chunks of columns [0, 8), [16, 24), [32, 40), [48, 56) come
// first, then those of [8, 16), [24, 32), [40, 48), [56, 64); i.e. column
// bits 5..3 become bits 4, 3, 5.  The 16 bytes at 16 G of a block are then
// the codes that A lane group G of the sparse product needs.
__device__ __forceinline__ int code_pos(int c) {
    return (c & ~63) | ((c >> 1) & 0x18) | ((c << 2) & 0x20) | (c & 7);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Round to nearest even of a finite fp32 to bfloat16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Raw buffer loads (buffer_load_dwordx4): an offset at or past the buffer
// size returns zeros without touching memory, so predicated-off lanes need no
// branch around the load.  kOOB is past every buffer (sizes are < 2^31).
constexpr uint32_t kOOB = 0x80000000u;
constexpr int32_t kRsrcWord3 = 0x00020000;  // gfx9 family: raw, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS byte offset of a __shared__ object (the value M0 takes for an
// LDS-destination buffer load).
#define S3D8_LDS_OFFSET(p) ((uint32_t)(size_t)((__attribute__((address_space(3))) const char *)(p)))

// Buffer resource as four SGPRs for inline assembly (raw, no swizzle).
__device__ __forceinline__ v4i rsrc_words(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    return v4i{(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xFFFFu), (int32_t)bytes, kRsrcWord3};
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 *
// lane (buffer_load_dwordx4 with the LDS bit; M0 holds the LDS base and is
// restored afterwards).  soff, the instruction's scalar offset, lets per-lane
// offsets stay loop-invariant.  A lane whose voff is at or past the buffer
// size (kOOB) writes zeros; callers keep soff below 2^31 so that voff + soff
// never wraps, and keep voff + soff inside the buffer for every other lane.
// The load counts in vmcnt like any vector load; the compiler does not see
// it, so the caller waits for it explicitly.
__device__ __forceinline__ void load_to_lds16_so(uint32_t lds, uint32_t voff, uint32_t soff, v4i rsrc) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

// The LDS-DMA loads of one GEMM block in one go: activation loads a0..a(NA-1)
// from buffer ra with scalar offset sa, then weight loads w0, w1 from buffer
// rw with scalar offset sw (the block's byte offset rides in the loads' soffset
// field, so the per-lane offsets stay loop-invariant), each into LDS at its
// own base (through M0, saved once around the batch).  Offsets and waits as
// for load_to_lds16_so.
template <int NA>
__device__ __forceinline__ void load_block_to_lds(const uint32_t (&lds)[NA + 2], const uint32_t (&voff)[NA + 2],
                                                  v4i ra, uint32_t sa, v4i rw, uint32_t sw) {
    uint32_t saved;
    static_assert(NA >= 1 && NA <= 3, "one to three activation loads per block");
    if constexpr (NA == 1) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %7, %8 offen lds\n\t"
            "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %9, %10 offen lds\n\t"
            "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %9, %10 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds[0]), "s"(lds[1]), "s"(lds[2]), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "s"(ra), "s"(sa),
              "s"(rw), "s"(sw)
            : "memory");
    } else if constexpr (NA == 3) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %11, %12 offen lds\n\t"
            "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %11, %12 offen lds\n\t"
            "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %8, %11, %12 offen lds\n\t"
            "s_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %9, %13, %14 offen lds\n\t"
            "s_mov_b32 m0, %5\n\ts_nop 0\n\tbuffer_load_dwordx4 %10, %13, %14 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds[0]), "s"(lds[1]), "s"(lds[2]), "s"(lds[3]), "s"(lds[4]), "v"(voff[0]), "v"(voff[1]),
              "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "s"(ra), "s"(sa), "s"(rw), "s"(sw)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %9, %10 offen lds\n\t"
            "s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %9, %10 offen lds\n\t"
            "s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %11, %12 offen lds\n\t"
            "s_mov_b32 m0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %8, %11, %12 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(lds[0]), "s"(lds[1]), "s"(lds[2]), "s"(lds[3]), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]),
              "v"(voff[3]), "s"(ra), "s"(sa), "s"(rw), "s"(sw)
            : "memory");
    }
}

// Stage the weight table into LDS (clw: kTableWords3D8 words), then build the
// lane-interleaved signed table.  S3D8: the 96-byte centroid table, read
// through the scalar cache so that it does not queue behind vector loads
// already in flight; 3D8 (f3d8): the 768-byte signed table, one word per
// thread.  C32 must be 4-byte aligned.  Contains barriers.  kThreads: the
// workgroup size (a constant, so that no load of it from the argument
// segment is waited for first)
template <int kThreads>
__device__ __forceinline__ void stage_and_build_table(uint32_t *tab, uint32_t *clw, const uint32_t *__restrict__ C32,
                                                      bool f3d8) {
    if (f3d8) {
        for (int i = threadIdx.x; i < kTableWords3D8; i += kThreads) clw[i] = C32[i];
    } else {
        uint32_t cw[24];
#pragma unroll
        for (int i = 0; i < 24; ++i) cw[i] = C32[i];
        if (threadIdx.x == 0) {
#pragma unroll
            for (int i = 0; i < 6; ++i)
                reinterpret_cast<uint4 *>(clw)[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
        }
    }
    __syncthreads();
    const uint8_t *cl = reinterpret_cast<const uint8_t *>(clw);
    for (int idx = threadIdx.x; idx < kTabWords / 4; idx += kThreads) {
        const uint32_t b = (uint32_t)idx >> 4;
        const uint32_t v = f3d8 ? row_3d8(b, cl) : signed_triple(b, cl);
        reinterpret_cast<uint4 *>(tab)[idx] = make_uint4(v, v, v, v);
    }
    __syncthreads();
}

// --------------------------------------------------------------- quant_act

// One workgroup per token row: absmax reduction, then s = a / 127 and
// xq = clamp(rne(x / s), -127, 127) with IEEE fp32 division (the paper's
// channel-scaled INT8 activations, one scale per token).  NV > 0: the row is
// read once, NV float4 per thread held in registers between the reduction
// and the quantisation (K <= 1024 NV); NV = 0: any K, the row is read twice.
// (1024 threads: one float4 per thread at K = 4096, so the serial chain of
// IEEE divisions per thread is short; 0.07 to 0.09 us faster than 256
// threads at 1, 8 and 64 rows, K = 4096, alternating on one box)
constexpr int kQuantThreads = 1024;

template <int NV>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const float *__restrict__ x, int K,
                                                                  int8_t *__restrict__ xq,
                                                                  float *__restrict__ xs) {
    __shared__ float wmax[kQuantThreads / 64];
    const int64_t row = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + row * K);
    const int n4 = K >> 2;
    float4 v[NV > 0 ? NV : 1];
    float a = 0.0f;
    auto amax4 = [](float4 q) { return fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))); };
    if constexpr (NV > 0) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = threadIdx.x + j * kQuantThreads;
            v[j] = i < n4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) a = fmaxf(a, amax4(v[j]));
    } else {
        for (int i = threadIdx.x; i < n4; i += kQuantThreads) a = fmaxf(a, amax4(xr[i]));
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
    auto quant4 = [&](float4 q) {
        if (a == 0.0f) return make_char4(0, 0, 0, 0);
        char4 o;
        o.x = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(q.x / s)));
        o.y = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(q.y / s)));
        o.z = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(q.z / s)));
        o.w = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(q.w / s)));
        return o;
    };
    if constexpr (NV > 0) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = threadIdx.x + j * kQuantThreads;
            if (i < n4) qr[i] = quant4(v[j]);
        }
    } else {
        for (int i = threadIdx.x; i < n4; i += kQuantThreads) qr[i] = quant4(xr[i]);
    }
}

// Launch of quant_act_kernel: the one-read build when the row fits 16
// float4 per thread (K <= 65536), else the two-read build.
void launch_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs, hipStream_t stream) {
    const int64_t nv = (K / 4 + kQuantThreads - 1) / kQuantThreads;
    typedef void (*QFn)(const float *, int, int8_t *, float *);
    QFn fn = quant_act_kernel<0>;
    if (nv <= 1) fn = quant_act_kernel<1>;
    else if (nv <= 2) fn = quant_act_kernel<2>;
    else if (nv <= 4) fn = quant_act_kernel<4>;
    else if (nv <= 8) fn = quant_act_kernel<8>;
    else if (nv <= 16) fn = quant_act_kernel<16>;
    hipLaunchKernelGGL(fn, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, x, (int)K, xq, xs);
}

// --------------------------------------------------------------- tiled layout

// The device weight layout that the linear kernels read.  The canonical
// matrix (triple rows of K bytes) is cut into fragments of 16 triples x 64
// columns; fragment (tile i, block b) is stored as 1 KiB at byte offset
// (i * KB + b) * 1024 with KB = ceil(K/64), and inside it lane L = n + 16g of
// a wave owns bytes [16L, 16L+16) = packed[16i + n][64b + 16g .. +15] (zero
// past the last triple or past K).  That is the B-operand layout of
// v_mfma_i32_16x16x64_i8 for 16 triples, so a wave reads each fragment as
// one fully contiguous 1 KiB load.  Like the blog's table permutation, the
// re-layout is done once before the weights are used.
constexpr int kTileThreads = 256;

__global__ __launch_bounds__(kTileThreads) void tile_kernel(const uint8_t *__restrict__ packed, int K, int T,
                                                            int KB, int64_t nchunks,
                                                            uint8_t *__restrict__ tiled) {
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(packed, (uint32_t)T * (uint32_t)K);
    for (int64_t c = (int64_t)blockIdx.x * kTileThreads + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * kTileThreads) {
        const int64_t frag = c >> 6;
        const int l = (int)(c & 63);
        const int64_t tile = frag / KB;
        const int blk = (int)(frag - tile * KB);
        const int64_t t = tile * 16 + (l & 15);
        const int k = blk * 64 + (l >> 4) * 16;
        const uint32_t off = (t < T && k < K) ? (uint32_t)t * (uint32_t)K + (uint32_t)k : kOOB;
        *reinterpret_cast<uint4 *>(tiled + c * 16) = bload16(rp, off);
    }
}

// --------------------------------------------------------------- GEMV

// Decode GEMV for up to 16 token rows.
//
// Work item = one tile of 16 channel triples (48 output channels).  A
// workgroup of WAVES waves builds the decode table once, then loops over
// tiles (persistent when there are more tiles than resident workgroups).
// Its waves split K: wave w owns 64-column blocks [w*kbw, (w+1)*kbw).  Each
// wave runs v_mfma_i32_16x16x64_i8 with the (up to) 16 token rows of X as
// the A operand and the decoded weights of the 16 triples for channel d of
// the triple as the B operand: three MFMAs (d = 0, 1, 2) per 64-column
// block.  Lane L = n + 16*g holds A row n / B column n and bytes
// [16g, 16g+16) of the block; its weight bytes are one contiguous 16-byte
// slice of the fragment, already in B layout after decode16.
//
// Each wave walks its (tile, chunk of U blocks) steps with two register
// buffers: the loads of the next step (possibly the next tile's first chunk)
// are in flight while the current one is decoded.  Every wave has the same
// number of steps per tile (blocks past its range are predicated off), so
// the per-tile barriers line up.  Wave partial sums meet in LDS through
// integer atomics (exact, order-free); the epilogue multiplies by the token
// scale and the bf16 channel scale and writes fp32.
//
// FUSED (M <= 4): the kernel also quantises the fp32 activations.  Each wave
// loads its own K range of x first (before any weight load, since vector
// loads retire in order), the workgroup reduces the row absmax through LDS,
// and each wave writes its INT8 codes to a private LDS slice from which the
// A operands are read.  Workgroup 0 also stores xq and xs for the caller.
template <int U>
struct GemvBuf {
    uint4 p[U];
    v4i x[U];
};

constexpr int kFusedMaxRows = 4;
constexpr int kFusedXF4 = 4;  // at most this many float4 of x per lane in the fused prologue

template <int WAVES, int U, bool FUSED>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ xs, const float *__restrict__ xf,
    int8_t *__restrict__ xq_out, float *__restrict__ xs_out, int M, int K, int N, int T,
    const uint8_t *__restrict__ tiled, const uint32_t *__restrict__ centroids,
    const uint16_t *__restrict__ scales, void *__restrict__ y, int32_t *__restrict__ acc_out,
    int kbw, int f3d8, int obf) {
    constexpr int kThreads = WAVES * 64;
    __shared__ uint32_t tab[kTabWords];
    __shared__ int32_t red[16 * 48];
    __shared__ uint32_t clw[kTableWords3D8];
    __shared__ float rmax[FUSED ? WAVES * kFusedMaxRows : 1];
    __shared__ float srow[FUSED ? kFusedMaxRows : 1];
    extern __shared__ int8_t xw[];  // FUSED: [WAVES][M][64 * kbw] INT8 codes, then 16 zero bytes

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int KB = (K + 63) >> 6;
    const int tiles = (T + 15) >> 4;
    const int kb0 = min(KB, wave * kbw);
    const int kb1 = min(KB, kb0 + kbw);
    const int nchunks = (kbw + U - 1) / U;  // uniform across the workgroup
    const uint32_t lane_off = (uint32_t)lane << 2;

    // The small inputs on every workgroup's critical path go out first, ahead
    // of the weight stream: the centroid table (scalar loads), this thread's
    // epilogue scales, and (fused) the wave's slice of x.
    uint32_t cw[24];
#pragma unroll
    for (int i = 0; i < 24; ++i) cw[i] = centroids[i];
    const uint32_t c3 = (f3d8 && tid < kTableWords3D8) ? centroids[tid] : 0u;  // 3D8: one word per thread
    // epilogue: output idx = tid + j * kThreads is (row idx / 48, channel
    // idx % 48 of the tile); its scales are fetched a tile ahead
    constexpr int kEp = (16 * 48 + kThreads - 1) / kThreads;
    float ep_sx[kEp], ep_a[kEp];
    auto ep_scale = [&](int t16, int j) {
        const int idx = tid + j * kThreads;
        const int ch = t16 * 48 + idx % 48;
        return (idx < M * 48 && ch < N) ? bf16_to_f32(scales[ch]) : 0.0f;
    };
#pragma unroll
    for (int j = 0; j < kEp; ++j) {
        const int idx = tid + j * kThreads;
        ep_sx[j] = 0.0f;
        if constexpr (!FUSED) {
            if (idx < M * 48) ep_sx[j] = xs[idx / 48];
        }
        ep_a[j] = blockIdx.x < (unsigned)((T + 15) >> 4) ? ep_scale(blockIdx.x, j) : 0.0f;
    }

    // fused prologue, part 1: this wave's slice of x
    float4 xv[kFusedXF4];
    const int span4 = 16 * kbw;                   // float4 per row in the wave's K range
    const int nf4 = (M * span4 + 63) >> 6;        // float4 per lane actually used (<= kFusedXF4)
    if constexpr (FUSED) {
        const __amdgpu_buffer_rsrc_t rf = make_rsrc(xf, (uint32_t)M * (uint32_t)K * 4u);
#pragma unroll
        for (int i = 0; i < kFusedXF4; ++i) {
            if (i < nf4) {
                const int f = lane + 64 * i;
                const int m = f / span4, r = f - m * span4;
                const int k = kb0 * 64 + 4 * r;
                const bool ok = m < M && k < K;
                xv[i] = __builtin_bit_cast(
                    float4, bload16(rf, ok ? ((uint32_t)m * (uint32_t)K + (uint32_t)k) * 4u : kOOB));
            }
        }
    }

    for (int i = tid; i < 16 * 48; i += kThreads) red[i] = 0;
    if constexpr (FUSED) {
        if (tid < 4) reinterpret_cast<uint32_t *>(xw + WAVES * M * 64 * kbw)[tid] = 0u;  // zero block
    }

    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tiled, (uint32_t)tiles * (uint32_t)KB * 1024u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq, FUSED ? 0u : (uint32_t)M * (uint32_t)K);
    const uint32_t xbase = (!FUSED && n < M) ? (uint32_t)n * (uint32_t)K + g * 16 : kOOB;
    auto load = [&](GemvBuf<U> &b, int tile, int c) {
        const uint32_t fbase = ((uint32_t)tile * (uint32_t)KB + (uint32_t)(kb0 + c * U)) * 1024u + (uint32_t)lane * 16u;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int blk = kb0 + c * U + u;  // wave-uniform
            if (blk < kb1) {
                b.p[u] = bload16(rt, fbase + u * 1024u);
                if constexpr (!FUSED)
                    b.x[u] = __builtin_bit_cast(
                        v4i, bload16(rx, (blk * 64 + g * 16 < K) ? xbase + (uint32_t)blk * 64 : kOOB));
            }
        }
    };

    // fused prologue, part 2: per-row absmax of the wave's slice.  This waits
    // for x before the first weight load is issued: behind the weight stream
    // of all CUs, x would arrive much later, and every wave of the workgroup
    // needs it before the decode can start.
    float lm[kFusedMaxRows] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < kFusedXF4; ++i) {
            if (i < nf4) {
                const int m = (lane + 64 * i) / span4;
                const float a = fmaxf(fmaxf(fabsf(xv[i].x), fabsf(xv[i].y)), fmaxf(fabsf(xv[i].z), fabsf(xv[i].w)));
#pragma unroll
                for (int r = 0; r < kFusedMaxRows; ++r) lm[r] = (m == r) ? fmaxf(lm[r], a) : lm[r];
            }
        }
#pragma unroll
        for (int r = 0; r < kFusedMaxRows; ++r) {
            if (r < M) {
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) lm[r] = fmaxf(lm[r], __shfl_xor(lm[r], off, 64));
            }
        }
    }

    GemvBuf<U> A, B;
    int tile = blockIdx.x;
    if (tile < tiles) load(A, tile, 0);

    // signed table from the table words loaded at the top
    if (f3d8) {
        if (tid < kTableWords3D8) clw[tid] = c3;
    } else if (tid == 0) {
#pragma unroll
        for (int i = 0; i < 6; ++i)
            reinterpret_cast<uint4 *>(clw)[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
    }
    __syncthreads();
    {
        const uint8_t *cl = reinterpret_cast<const uint8_t *>(clw);
        for (int idx = tid; idx < kTabWords / 4; idx += kThreads) {
            const uint32_t b = (uint32_t)idx >> 4;
            const uint32_t v = f3d8 ? row_3d8(b, cl) : signed_triple(b, cl);
            reinterpret_cast<uint4 *>(tab)[idx] = make_uint4(v, v, v, v);
        }
    }
    if constexpr (FUSED) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < kFusedMaxRows; ++r)
                if (r < M) rmax[wave * kFusedMaxRows + r] = lm[r];
        }
    }
    __syncthreads();
    if constexpr (FUSED) {
        // fused prologue, part 3: scales, INT8 codes into this wave's LDS slice
        float srow_r[kFusedMaxRows];
#pragma unroll
        for (int r = 0; r < kFusedMaxRows; ++r) {
            float a = 0.0f;
            if (r < M)
                for (int w = 0; w < WAVES; ++w) a = fmaxf(a, rmax[w * kFusedMaxRows + r]);
            srow_r[r] = (a == 0.0f) ? 0.0f : a / 127.0f;
        }
        if (tid < kFusedMaxRows) srow[tid] = srow_r[tid];
        if (blockIdx.x == 0 && tid < M && xs_out) xs_out[tid] = srow_r[tid];
#pragma unroll
        for (int i = 0; i < kFusedXF4; ++i) {
            if (i < nf4) {
                const int f = lane + 64 * i;
                const int m = f / span4, r = f - m * span4;
                if (m < M) {
                    float s = srow_r[0];
#pragma unroll
                    for (int rr = 1; rr < kFusedMaxRows; ++rr) s = (m == rr) ? srow_r[rr] : s;
                    char4 o;
                    if (s == 0.0f) {
                        o = make_char4(0, 0, 0, 0);
                    } else {
                        o.x = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(xv[i].x / s)));
                        o.y = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(xv[i].y / s)));
                        o.z = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(xv[i].z / s)));
                        o.w = (signed char)fminf(127.0f, fmaxf(-127.0f, rintf(xv[i].w / s)));
                    }
                    *reinterpret_cast<char4 *>(xw + ((wave * M + m) * 64 * kbw + 4 * r)) = o;
                    const int k = kb0 * 64 + 4 * r;
                    if (blockIdx.x == 0 && xq_out && k < K)
                        *reinterpret_cast<char4 *>(xq_out + (int64_t)m * K + k) = o;
                }
            }
        }
    }

    // fused A operand: lanes of rows < M read their codes, the others read a
    // zero block (stride 0)
    const int xa_base = n < M ? (wave * M + n) * 64 * kbw + g * 16 : WAVES * M * 64 * kbw;
    const int xa_step = n < M ? 64 : 0;

    v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
    auto process = [&](const GemvBuf<U> &b, int c) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int bl = c * U + u;
            if (kb0 + bl >= kb1) continue;  // wave-uniform: past this wave's range
            v4i a;
            if constexpr (FUSED) {
                a = *reinterpret_cast<const v4i *>(xw + (xa_base + bl * xa_step));
            } else {
                a = b.x[u];
            }
            v4i b0, b1, b2;
            decode16(b.p[u], lane_off, tab, b0, b1, b2);
            acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b1, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b2, acc2, 0, 0, 0);
        }
    };

    // after the last chunk of a tile: reduce across waves, epilogue
    auto finish = [&](int t16) {
        // D[row r][col n] sits in lane n + 16*(r/4), element r%4; the channel
        // of (col n, d) within the tile is 3n + d.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            if (r < M && kb0 < kb1) {
                atomicAdd(&red[r * 48 + 3 * n + 0], acc0[i]);
                atomicAdd(&red[r * 48 + 3 * n + 1], acc1[i]);
                atomicAdd(&red[r * 48 + 3 * n + 2], acc2[i]);
            }
        }
        acc0 = v4i{0, 0, 0, 0};
        acc1 = v4i{0, 0, 0, 0};
        acc2 = v4i{0, 0, 0, 0};
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kEp; ++j) {
            const int idx = tid + j * kThreads;
            const float a_cur = ep_a[j];
            if (t16 + (int)gridDim.x < ((T + 15) >> 4)) ep_a[j] = ep_scale(t16 + gridDim.x, j);
            if (idx < M * 48) {
                const int r = idx / 48;
                const int32_t sum = red[idx];
                red[idx] = 0;
                const int ch = t16 * 48 + idx % 48;
                if (ch < N) {
                    const float sx = FUSED ? srow[r] : ep_sx[j];
                    const float v = (sx * (float)sum) * a_cur;
                    if (obf)
                        static_cast<uint16_t *>(y)[(int64_t)r * N + ch] = f32_to_bf16_rne(v);
                    else
                        static_cast<float *>(y)[(int64_t)r * N + ch] = v;
                    if (acc_out) acc_out[(int64_t)r * N + ch] = sum;
                }
            }
        }
        __syncthreads();
    };

    // steps (tile, c), c = 0 .. nchunks-1, alternating buffers A and B
    int c = 0;
    bool in_a = true;
    while (tile < tiles) {
        int ntile = tile, nc = c + 1;
        if (nc == nchunks) {
            nc = 0;
            ntile = tile + gridDim.x;
        }
        const bool more = ntile < tiles;
        if (in_a) {
            if (more) load(B, ntile, nc);
            process(A, c);
        } else {
            if (more) load(A, ntile, nc);
            process(B, c);
        }
        if (nc == 0) finish(tile);
        tile = ntile;
        c = nc;
        in_a = !in_a;
    }
}

// --------------------------------------------------------------- streaming fused GEMV

// Quantise + decode GEMV for 1..4 token rows, the weight stream started at
// kernel entry.
//
// At one token the layer is a single read of the packed matrix; what limits
// it is how early that read starts, how long the chain in front of the first
// decode is, and how evenly the bytes are spread.  Every wave issues first
// one load of the centroid row its lanes need for the table and its share of
// the fp32 activations, then (after a barrier that lets every wave's small
// loads go ahead) its first two weight fragments (16 bytes per lane each,
// into a ring of registers: a lane's bytes are its own, so they need not
// pass through LDS).  The table is then built from registers, the row
// absmax is reduced with DPP, and after one workgroup barrier the last two
// fragments of the ring are issued, the activations are quantised and the
// decode starts.  The main loop has no barriers: each step takes the oldest
// fragment, looks up its 16 packed bytes, runs two sparse products
// v_smfmac_i32_16x16x128_i8 on the raw lookup dwords (see the loop) and
// refills the ring entry kStreamSlots steps ahead.
//
// Work split: a workgroup takes tiles of 16 triples (its index, + grid,
// ...), its 16 waves split K into ranges of kbw 64-column blocks.  Partial
// sums of a tile meet in LDS through integer atomics (exact, order-free) and
// stay there until the end; every global store (y, the optional
// accumulators, xq and xs) happens after the last weight load has landed.
constexpr int kStreamMaxTiles = 16;  // tiles per workgroup (results held in LDS)

// Maxima of non-negative floats (absolute values and their maxima, never
// NaN): for x >= +0 the IEEE bit patterns order like the values, so the
// reductions compare them as unsigned integers (0 is the identity, and the
// DPP moves fold into the max instructions).
// max over each row of 16 lanes, result in every lane of the row (DPP:
// swap neighbours, swap pairs, mirror halves of 8, mirror the row)
__device__ __forceinline__ float row16_max(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));
    return __uint_as_float(u);
}
// max over the wave, wave-uniform
__device__ __forceinline__ float wave_max(float v) {
    const uint32_t u = __float_as_uint(row16_max(v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)u, 0), (uint32_t)__builtin_amdgcn_readlane((int)u, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)u, 32), (uint32_t)__builtin_amdgcn_readlane((int)u, 48));
    return __uint_as_float(max(a, b));
}

// One launch can serve up to kStreamBatch independent matrices (e.g. the
// seven linears of a decoder layer, each with its own activations, table
// and scales): workgroups [wg0[p], wg0[p + 1]) work on matrix p, each on its
// own tiles, as if launched alone with grid = wg0[p + 1] - wg0[p].  The
// workgroup starts (first in the arguments, so that they arrive in
// preloaded SGPRs) pick the matrix; its parameters are then read from the
// kernel argument segment.
//
// One instantiation per row count MR (the per-row code folds away) and
// wave count W (8 or 16; the launch uses 16).  Each wave's prologue is a
// fixed cost that all W waves pay on a CU's four SIMDs.
constexpr int kStreamBatch = 8;
struct StreamProb {
    const float *xf;
    const uint8_t *tiled;
    const uint8_t *centroids;
    const uint16_t *scales;
    float *y;
    int32_t *acc_out;
    int8_t *xq_out;
    float *xs_out;
    int K, N, T, kbw, ntw_q, ntw_r;  // ntw_q, ntw_r: tiles of the matrix over its workgroups
};
struct StreamBatch {
    int wg0[kStreamBatch + 1];  // first workgroup of each matrix; unused entries INT32_MAX
    StreamProb p[kStreamBatch];
};

// The streaming kernels' decode table, built without staging it in LDS:
// thread t of kThreads (1024) writes uint4 t + kThreads i (i < 4) of the
// 64-copy table, entry b = t / 16 + 64 i.  For S3D8 all four entries use
// centroid row (t / 32) % 32 (bits 1..5 of b come from t) and S0 = bit 4 of
// t, while S1 and the bit-7 selector come from i; for 3D8 entry b is row b
// of the 768-byte signed table.  Each thread loads the 8 bytes around its
// row(s) from a 4-aligned offset (one row for S3D8, four for 3D8) with
// asm loads that the caller waits for; build_stream_table then writes the
// entries from registers.
typedef uint32_t u2v_t __attribute__((ext_vector_type(2)));
template <bool F3>
struct StreamTableRows {
    static constexpr int kRows = F3 ? kTabWords / 4 / 1024 : 1;
    u2v_t cpair[kRows];
    int cshift[kRows];
};

template <bool F3>
__device__ __forceinline__ void load_stream_table_rows(StreamTableRows<F3> &t, const uint8_t *centroids, int tid) {
    const v4i rcen = rsrc_words(centroids, F3 ? 768u : 96u);
#pragma unroll
    for (int k = 0; k < StreamTableRows<F3>::kRows; ++k) {
        const int trow = F3 ? (tid >> 4) + k * (1024 >> 4) : ((tid >> 5) + k * (1024 >> 5)) & 31;
        const int cbase = min((3 * trow) & ~3, F3 ? 760 : 88);
        t.cshift[k] = 8 * (3 * trow - cbase);
        asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen" : "=v"(t.cpair[k]) : "v"((uint32_t)cbase), "s"(rcen)
                     : "memory");
    }
}

template <bool F3>
__device__ __forceinline__ void build_stream_table(uint32_t *tab, const StreamTableRows<F3> &t, int tid) {
    constexpr int kThreads = 1024;
    constexpr int kPasses = kTabWords / 4 / kThreads;
    if constexpr (F3) {
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const uint32_t v = (uint32_t)((((uint64_t)t.cpair[i].y << 32) | t.cpair[i].x) >> t.cshift[i]) & 0xFFFFFFu;
            reinterpret_cast<uint4 *>(tab)[tid + kThreads * i] = make_uint4(v, v, v, v);
        }
    } else {
        const bool s0 = (tid >> 4) & 1;
        const uint64_t cv = (((uint64_t)t.cpair[0].y << 32) | t.cpair[0].x) >> t.cshift[0];
        const uint32_t c0 = (uint32_t)cv & 0xFFu, c1 = (uint32_t)(cv >> 8) & 0xFFu, c2 = (uint32_t)(cv >> 16) & 0xFFu;
        const uint32_t w0 = (s0 ? 0u - c0 : c0) & 0xFFu;
        const uint32_t lo[2] = {w0 | (c1 << 8), w0 | (((0u - c1) & 0xFFu) << 8)};
        const uint32_t hp = c2 << 16, hn = ((0u - c2) & 0xFFu) << 16;
        const uint32_t hi[2] = {s0 ? hn : hp, s0 ? hp : hn};  // bit 7 clear: S2 = S0
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const int hib = (kThreads / 16) * i;  // bits 6.. of b contributed by the pass
            const uint32_t v = lo[(hib >> 6) & 1] | hi[(hib >> 7) & 1];
            reinterpret_cast<uint4 *>(tab)[tid + kThreads * i] = make_uint4(v, v, v, v);
        }
    }
}

template <int MR, int W, int NF, bool F3>
__device__ __forceinline__ void gemv_stream_body(
    const float *__restrict__ xf, const uint8_t *__restrict__ tiled, const uint8_t *__restrict__ centroids,
    const uint16_t *__restrict__ scales, int K, int N, int bid, int grid, int ntw_q, int ntw_r,
    void *__restrict__ y, int32_t *__restrict__ acc_out, int8_t *__restrict__ xq_out, float *__restrict__ xs_out,
    int obf) {
    static_assert(MR >= 1 && MR <= kFusedMaxRows, "1 to 4 token rows");
    const int T = (N + 2) / 3;
    const int kbw = (((K + 63) >> 6) + W - 1) / W;  // 64-column blocks per wave
    static_assert(W == 8 || W == 16, "8 or 16 waves");
    static_assert(NF >= 1 && NF <= kFusedXF4, "1 to 4 float4 of activations per lane");
    constexpr int M = MR;
    constexpr int kStreamWaves = W;
    constexpr int kStreamSlots = 64 / W;  // fragments in flight per wave (registers)
    constexpr int kStreamEp = (kStreamMaxTiles * MR * 48 + W * 64 - 1) / (W * 64);  // outputs per thread
    constexpr int kThreads = W * 64;
    typedef float f4v __attribute__((ext_vector_type(4)));
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(16))) uint32_t tab[kTabWords];
    __shared__ __attribute__((aligned(16))) int8_t xw[kStreamWaves][16384 / W];
    __shared__ __attribute__((aligned(16))) int8_t zero16[16];
    __shared__ int32_t ybuf[kStreamMaxTiles * kFusedMaxRows * 48];
    __shared__ float rmax[kStreamWaves * kFusedMaxRows];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int KB = (K + 63) >> 6;
    const int tiles = (T + 15) >> 4;
    const int kb0 = wave * kbw;
    const int ntw = ntw_q + (bid < ntw_r);  // tiles of this workgroup, >= 1
    const int nout = ntw * M * 48;                                 // outputs of this workgroup

    // 1. epilogue scales (the compiler's loads, issued first: the explicit
    //    vmcnt counts below never wait for them).  Output idx = tid + q *
    //    kThreads is (tile j, row r, channel c), j = idx / (48 M).
    const uint32_t invM = 0x10000u / (uint32_t)M + 1u;  // (x * invM) >> 16 == x / M for x < 64
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scales, (uint32_t)N * 2u);
    uint16_t ep_a[kStreamEp];
    int ep_j[kStreamEp], ep_r[kStreamEp], ep_c[kStreamEp];
#pragma unroll
    for (int q = 0; q < kStreamEp; ++q) {
        const int idx = tid + q * kThreads;
        const int i48 = idx / 48, c = idx - 48 * i48;
        const int j = (int)(((uint32_t)i48 * invM) >> 16), r = i48 - j * M;
        ep_j[q] = j;
        ep_r[q] = r;
        ep_c[q] = c;
        const int ch = (bid + j * grid) * 48 + c;
        ep_a[q] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (idx < nout && ch < N) ? (uint32_t)ch * 2u : kOOB, 0, 0);
    }

    // 2. the table rows of this thread's table entries (load_stream_table_rows)
    static_assert(W == 16, "the table build assumes 1024 threads");
    StreamTableRows<F3> trows;
    load_stream_table_rows<F3>(trows, centroids, tid);

    // 3. activations: this wave's K range of every row, up to 4 float4 per
    //    lane; float4 f of the range is row f / (16 kbw)
    const v4i rx = rsrc_words(xf, (uint32_t)M * (uint32_t)K * 4u);
    const int span4 = 16 * kbw;
    const int nf4 = (M * span4 + 63) >> 6;  // float4 per lane in use (<= 4)
    f4v xv[NF];
    int xm[NF], xr[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = lane + 64 * i;
        int m = 0;  // row of float4 f; M means past the rows
#pragma unroll
        for (int q = 1; q <= M; ++q) m += f >= q * span4;
        const int r = f - m * span4;
        xm[i] = m;
        xr[i] = r;
        // unconditional: a register written by these loads must not pass
        // through a branch merge (the compiler would copy it before it lands)
        const int k = kb0 * 64 + 4 * r;
        const uint32_t off = (i < nf4 && m < M && k < K) ? ((uint32_t)m * (uint32_t)K + (uint32_t)k) * 4u : kOOB;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(xv[i]) : "v"(off), "s"(rx) : "memory");
    }

    // every wave's small loads enter the CU's memory queue before any
    // fragment load does
    asm volatile("s_barrier" ::: "memory");

    // 4. weight fragments, straight into registers (each lane's 16 bytes of
    //    a fragment are its own: nothing to share through LDS): step s of
    //    this wave = tile j = s / kbw of the workgroup, block kb0 + s % kbw,
    //    kStreamSlots steps in flight in a ring of registers; steps past the
    //    end read zeros (out-of-range offsets)
    const v4i rw = rsrc_words(tiled, (uint32_t)tiles * (uint32_t)KB * 1024u);
    int is_j = 0, is_b = 0;  // (tile, block) of the next step to issue
    auto next_off = [&]() {
        const int kb = kb0 + is_b;
        const bool live = is_j < ntw && kb < KB;
        const uint32_t tile = (uint32_t)(bid + is_j * grid);
        const uint32_t off = live ? (tile * (uint32_t)KB + (uint32_t)kb) * 1024u + (uint32_t)lane * 16u : kOOB;
        if (++is_b == kbw) {
            is_b = 0;
            ++is_j;
        }
        return off;
    };
    // The ring loads are issued from inline assembly and waited for
    // explicitly (the compiler's own count at the loop header is not exact:
    // it waits for every load in flight there).  Each load's destination is
    // tied to its ring entry ("+v"), so no copy of an entry can be read
    // before the load lands; every entry is waited for with vmcnt(slots - 1)
    // before use: the younger loads in flight are the other entries.
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v pr[kStreamSlots];
    auto ring_load = [&](u4v &dst, uint32_t off) {
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "+v"(dst) : "v"(off), "s"(rw) : "memory");
    };
    // the first kEarly entries now, the rest after the workgroup barrier
    // below: a wave stalled issuing weight loads behind the memory
    // system's backlog reaches its absmax late and holds up the barrier.
    // Measured at K = 4096, N = 14336: one token row 6.77 us with three
    // entries early against 6.97 with two (7.35 with one, 7.20 with four;
    // also faster for 3D8, the lm_head and the batched layer); four rows
    // 10.43 us with two against 10.57 with three.
    constexpr int kEarly = MR == 1 ? 3 : 2;
#pragma unroll
    for (int sl = 0; sl < kEarly; ++sl) {
        asm volatile("" : "=v"(pr[sl]));  // defined, with no code: the load below overwrites it
        ring_load(pr[sl], next_off());
    }

    // lane constants of the products' A operand (described with the loop
    // below), computed here while the loads are in flight rather than after
    // the barrier, where every wave of the CU is busy quantising
    const int arw = lane & 15;
    const bool arow = arw < 3 * M;
    const int8_t *xa = arow ? &xw[wave][(arw / 3) * 64 * kbw + g * 16] : zero16;
    const int xa_step = arow ? 64 : 0;
    // sparsity indices: 2-bit field e of a word is the position, inside its
    // table dword, that compressed A byte e multiplies; the first product
    // takes the even bytes to channel d = m % 3 of the row and the odd ones
    // to position 3 (always zero), the second the other way round
    const uint32_t dsel = (uint32_t)(arw % 3);
    const int idx_even = (int)(dsel * 0x11111111u + 0xCCCCCCCCu);
    const int idx_odd = (int)(0x33333333u + dsel * 0x44444444u);
    asm volatile("" ::"v"(idx_even), "v"(idx_odd), "v"(xa), "v"(xa_step));

    for (int i = tid; i < ntw * kFusedMaxRows * 48; i += kThreads) ybuf[i] = 0;
    if (tid < 4) reinterpret_cast<uint32_t *>(zero16)[tid] = 0u;

    // table: entry b holds [w0, w1, w2, 0] with w_d = +-C[q][d], q = (b >> 1)
    // % 32, sign selectors S0 = bit 0, S1 = bit 6, S2 = bit 7 xor bit 0
    // (build_stream_table, from the rows loaded above).
    // (the empty statements after the wait keep every use of the rows behind it)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kEarly + NF) : "memory");
#pragma unroll
    for (int k = 0; k < StreamTableRows<F3>::kRows; ++k) asm volatile("" : "+v"(trows.cpair[k]));
    build_stream_table<F3>(tab, trows, tid);

    // activations landed (only fragment loads behind them)
    if constexpr (NF == 1) {
        asm volatile("s_waitcnt vmcnt(%1)" : "+v"(xv[0]) : "n"(kEarly) : "memory");
    } else if constexpr (NF == 2) {
        asm volatile("s_waitcnt vmcnt(%2)" : "+v"(xv[0]), "+v"(xv[1]) : "n"(kEarly) : "memory");
    } else if constexpr (NF == 3) {
        asm volatile("s_waitcnt vmcnt(%3)" : "+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]) : "n"(kEarly) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(%4)" : "+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]) : "n"(kEarly)
                     : "memory");
    }
    // (16 waves share a CU's four SIMDs: every VALU operation here costs
    // four of them, so only the nf4 float4 in use are touched; lanes past
    // the rows hold zeros)
    float am[kFusedMaxRows] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        if (i < nf4) {  // uniform
            const float a4 = fmaxf(fmaxf(fabsf(xv[i].x), fabsf(xv[i].y)), fmaxf(fabsf(xv[i].z), fabsf(xv[i].w)));
#pragma unroll
            for (int r = 0; r < M; ++r) am[r] = fmaxf(am[r], (M == 1 || xm[i] == r) ? a4 : 0.0f);
        }
    }
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const float a = wave_max(am[r]);
        if (lane == 0) rmax[wave * kFusedMaxRows + r] = a;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // table, rmax, ybuf complete
#pragma unroll
    for (int sl = kEarly; sl < kStreamSlots; ++sl) {
        asm volatile("" : "=v"(pr[sl]));
        ring_load(pr[sl], next_off());
    }

    // per-token scale s = a / 127 (lane w of each row reads wave w's maximum),
    // codes clamp(rne(x / s), -127, 127) into this wave's slice of xw
    float srow[kFusedMaxRows] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < kFusedMaxRows; ++r) {
        if (r < M) {  // uniform
            const float a = row16_max(n < kStreamWaves ? rmax[n * kFusedMaxRows + r] : 0.0f);
            srow[r] = (a == 0.0f) ? 0.0f : a / 127.0f;
        }
    }
    // rne(x / s) through t = x * rcp(s), rcp the hardware reciprocal (error
    // below 1 ulp): |t - x / s| < 2.5e-7 |x / s| <= 3.2e-5, so whenever t is
    // more than 1e-4 away from a half-integer, t, the exact quotient and its
    // fp32 rounding lie in the same rounding interval and rint(t) is the
    // code.  A lane with an element within 2e-4 of a half-integer (|t -
    // rint(t)| >= 0.4998), or of a row whose s is below 1e-30, takes the
    // IEEE quotient for all its elements instead, in a pass the wave runs
    // only when one of its lanes needs it.
    float rcp[kFusedMaxRows] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < M; ++r) rcp[r] = srow[r] >= 1e-30f ? __builtin_amdgcn_rcpf(srow[r]) : 0.0f;
    float qv[NF][4];
    float scv[NF];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        scv[i] = 0.0f;
        if (i < nf4) {  // uniform
            float sc = srow[0], rc = rcp[0];
#pragma unroll
            for (int rr = 1; rr < M; ++rr) {
                sc = (xm[i] == rr) ? srow[rr] : sc;
                rc = (xm[i] == rr) ? rcp[rr] : rc;
            }
            scv[i] = sc;
            const float xe[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            slow = slow || (rc == 0.0f && sc != 0.0f);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float t = xe[e] * rc;
                qv[i][e] = rintf(t);
                slow = slow || fabsf(t - qv[i][e]) >= 0.4998f;
            }
        }
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
        if (slow) {
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                const float xe[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) qv[i][e] = rintf(xe[e] / scv[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        if (i >= nf4) break;  // uniform
        if (xm[i] < M) {
            uint32_t o = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o |= ((uint32_t)(int32_t)__builtin_amdgcn_fmed3f(qv[i][e], -127.0f, 127.0f) & 0xFFu) << (8 * e);
            *reinterpret_cast<uint32_t *>(&xw[wave][xm[i] * 64 * kbw + code_pos(4 * xr[i])]) = scv[i] != 0.0f ? o : 0u;
        }
    }

    // The products run without the byte transpose of decode16.  A table
    // lookup gives the dword [w0, w1, w2, 0] of packed byte k, and eight of
    // them are used as they are as the B operand of the sparse product
    // v_smfmac_i32_16x16x128_i8, whose 128-deep sum runs over (byte,
    // position) pairs.  Row m = 3r + d (token r, channel d) of its A operand
    // has one non-zero per dword-sized group of K: token r's code of that
    // byte, at position d.  The instruction takes A compressed (two values
    // per group of four, each with a 2-bit position in an index register),
    // so A is just 16 codes per lane; D[3r + d][n] = sum_k x_rk w_d(k) for
    // triple n: two products per 64 x 16 fragment, one accumulator.
    //   Operand layout of the instruction (lane l = (row or column l % 16,
    //   group G = l / 16)): A byte e of lane group G meets B dword
    //   4 (G / 2) + (e % 8) / 2 of lane group 2 (G % 2) + e / 8.  The first
    //   product's B dword w is the table dword of lane byte 2w, the second's
    //   of byte 2w + 1, so A byte e must hold the code of block column
    //   32 (G % 2) + 16 (e / 8) + 8 (G / 2) + e % 8: the 16 bytes at
    //   16 G of the block when the codes are stored permuted (code_pos).
    //   Both products read that one A register; the index word of the first
    //   sends its even bytes to position d and its odd ones to position 3
    //   (a zero of every table dword), the second the reverse.
    // (arw, arow, xa, xa_step and the index words are set up before the
    // wait for x)
    const uint32_t lane_off = (uint32_t)lane << 2;
    const char *tb = reinterpret_cast<const char *>(tab);
    const int nsteps = ntw * kbw;  // fragments per wave

    v4i acc = {0, 0, 0, 0};
    v4i a = {0, 0, 0, 0};  // this step's codes (A operand)
    int bl = 0, j = 0;
    // One loop for every workgroup, without branches around it: a ring
    // entry that reaches a loop in other registers than it was loaded into
    // is copied there before its load lands.
#pragma unroll 1
    for (int st0 = 0; st0 < nsteps; st0 += kStreamSlots) {
#pragma unroll
        for (int u = 0; u < kStreamSlots; ++u) {
            if (st0 + u >= nsteps) break;  // uniform
            asm volatile("s_waitcnt vmcnt(%1)" : "+v"(pr[u]) : "n"(kStreamSlots - 1) : "memory");
            const u4v p = pr[u];
            // rows m >= 3M keep the zeros set before the loop
            if (arow) a = *reinterpret_cast<const v4i *>(xa + bl * xa_step);
            const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
            v8i be, bo;  // table dwords of the lane's even / odd bytes
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t t = *reinterpret_cast<const int32_t *>(
                        tb + __builtin_amdgcn_perm(pw[jj], lane_off, 0x0C0C0400u + ((uint32_t)i << 8)));
                    if (i & 1)
                        bo[2 * jj + (i >> 1)] = t;
                    else
                        be[2 * jj + (i >> 1)] = t;
                }
            }
            acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, be, acc, idx_even, 0, 0);
            acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, bo, acc, idx_odd, 0, 0);
            // refill the entry once its bytes are consumed (so the new load
            // writes the same registers and the loop carries no copies)
            ring_load(pr[u], next_off());
            if (++bl == kbw) {
                // tile j done for this wave: lane (n, g) holds rows 4 g + i,
                // row m = 3r + d is channel 3n + d of token r within the tile
                if (kb0 < KB) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * g + i;
                        if (m < 3 * M) atomicAdd(&ybuf[(j * kFusedMaxRows + m / 3) * 48 + 3 * n + m % 3], acc[i]);
                    }
                }
                acc = v4i{0, 0, 0, 0};
                bl = 0;
                ++j;
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The ring registers stay allocated to this point: the compiler takes
    // an asm load as complete when issued, so without this it could give a
    // register to another value while a load past the end still writes it.
#pragma unroll
    for (int sl = 0; sl < kStreamSlots; ++sl) asm volatile("" ::"v"(pr[sl]));

    // epilogue
#pragma unroll
    for (int q = 0; q < kStreamEp; ++q) {
        const int jj = ep_j[q], r = ep_r[q], c = ep_c[q];
        const int ch = (bid + jj * grid) * 48 + c;
        if (jj < ntw && ch < N) {
            float sx = srow[0];
#pragma unroll
            for (int rr = 1; rr < kFusedMaxRows; ++rr) sx = (r == rr) ? srow[rr] : sx;
            const int32_t sum = ybuf[(jj * kFusedMaxRows + r) * 48 + c];
            const float v = (sx * (float)sum) * bf16_to_f32(ep_a[q]);
            if (obf)
                static_cast<uint16_t *>(y)[(int64_t)r * N + ch] = f32_to_bf16_rne(v);
            else
                static_cast<float *>(y)[(int64_t)r * N + ch] = v;
            if (acc_out) acc_out[(int64_t)r * N + ch] = sum;
        }
    }
    if (bid == 0) {
        if (tid < M && xs_out) {
            float sx = srow[0];
#pragma unroll
            for (int rr = 1; rr < kFusedMaxRows; ++rr) sx = (tid == rr) ? srow[rr] : sx;
            xs_out[tid] = sx;
        }
        if (xq_out) {
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                const int k = kb0 * 64 + 4 * xr[i];
                if (i < nf4 && xm[i] < M && k < K)
                    *reinterpret_cast<char4 *>(xq_out + (int64_t)xm[i] * K + k) =
                        *reinterpret_cast<const char4 *>(&xw[wave][xm[i] * 64 * kbw + code_pos(4 * xr[i])]);
            }
        }
    }
}

// One matrix: the arguments used before the first loads come first, so that
// they are among the kernel arguments preloaded into SGPRs.
template <int MR, int W, int NF, bool F3>
__global__ __launch_bounds__(W * 64) void gemv_stream_kernel(
    const float *__restrict__ xf, const uint8_t *__restrict__ tiled, const uint8_t *__restrict__ centroids,
    const uint16_t *__restrict__ scales, int K, int N, int grid, int ntw_q, int ntw_r, void *__restrict__ y,
    int32_t *__restrict__ acc_out, int8_t *__restrict__ xq_out, float *__restrict__ xs_out, int obf) {
    gemv_stream_body<MR, W, NF, F3>(xf, tiled, centroids, scales, K, N, (int)blockIdx.x, grid, ntw_q, ntw_r, y,
                                    acc_out, xq_out, xs_out, obf);
}

// Several matrices: this workgroup's matrix is the last p with wg0[p] <=
// blockIdx.x; its parameters come from the argument segment.
template <int MR, int W, int NF>
__global__ __launch_bounds__(W * 64) void gemv_stream_batch_kernel(const StreamBatch B) {
    int pi = 0;
#pragma unroll
    for (int q = 1; q < kStreamBatch; ++q) pi += (int)blockIdx.x >= B.wg0[q];
    const StreamProb &P = B.p[pi];
    gemv_stream_body<MR, W, NF, false>(P.xf, P.tiled, P.centroids, P.scales, P.K, P.N,
                                       (int)blockIdx.x - B.wg0[pi], B.wg0[pi + 1] - B.wg0[pi], P.ntw_q, P.ntw_r,
                                       P.y, P.acc_out, P.xq_out, P.xs_out, 0);
}

// --------------------------------------------------------------- streaming GEMV on INT8 codes

// The streaming GEMV's decode and sparse products for 1 to 8 token rows
// whose INT8 codes and scales are already computed: s3d8_linear at M <= 8,
// and s3d8_forward from five tokens on (after s3d8_quant_act, whose codes
// every workgroup then reads instead of the fp32 rows).
//
// The sparse product v_smfmac_i32_16x16x128_i8 has 16 A rows; token r,
// channel d takes row 3 r' + d of row group r / 5 (r' = r % 5), so five
// tokens fill one group and six to eight tokens use two.  Both groups
// multiply the same table-lookup dwords: the lookups, which dominate a
// step, are shared, and a step runs two sparse products per group.  As in
// the fused kernel the codes sit in LDS permuted in 8-byte chunks (code_pos)
// so that one 16-byte read per lane is a group's A operand, and each lane
// reads rows of its group only (others keep zeros); the weight fragments
// stream through a ring of registers, kCodesSlots ahead.
//
// Work split as in the fused kernel: workgroup b takes tiles b, b + grid,
// ... (at most kCodesMaxTiles), its 16 waves split K in ranges of kbw
// 64-column blocks, partial sums meet in LDS through integer atomics.
constexpr int kCodesMaxRows = 8;
constexpr int kCodesWaveBytes = 4096;  // codes per wave: M * 64 * kbw <= 4096
constexpr int kCodesMaxTiles = 16;
constexpr int kCodesSlots = 4;

// (the arguments used before the first loads come first, the grid size
// among them, so that all of them are preloaded into SGPRs: gridDim.x would
// be a load from the argument segment, waited for before any other load)
template <int MR, int NCL, bool F3>
__global__ __launch_bounds__(1024) void gemv_codes_kernel(const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                          const uint8_t *__restrict__ tiled,
                                                          const uint8_t *__restrict__ table,
                                                          const uint16_t *__restrict__ scales, int K, int N, int grid,
                                                          int ntw_q, int ntw_r, void *__restrict__ y,
                                                          int32_t *__restrict__ acc_out, int obf) {
    static_assert(MR >= 1 && MR <= kCodesMaxRows, "1 to 8 token rows");
    static_assert(NCL >= 1 && NCL * 16 * 64 <= kCodesWaveBytes, "code loads per lane");
    constexpr int W = 16, kThreads = W * 64;
    constexpr int NG = MR > 5 ? 2 : 1;  // row groups of the sparse product (five tokens each)
    constexpr int kEp = (kCodesMaxTiles * MR * 48 + kThreads - 1) / kThreads;
    // ring entries issued before the first barrier: measured at K = 4096,
    // N = 14336 (alternating on one box) 7.13 / 7.79 / 9.14 us at M = 1 / 4 / 8
    // with three, against 7.44 / 8.03 / 9.45 with two and 7.10 / 7.83 / 9.50
    // with four
    constexpr int kEarly = 3;
    __shared__ __attribute__((aligned(16))) uint32_t tab[kTabWords];
    // codes slice per wave: NCL loads of 16 bytes per lane, 1024 NCL bytes
    __shared__ __attribute__((aligned(16))) int8_t xw[W][1024 * NCL];
    __shared__ __attribute__((aligned(16))) int8_t zero16[16];
    __shared__ int32_t ybuf[kCodesMaxTiles * MR * 48];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int T = (N + 2) / 3, KB = (K + 63) >> 6, tiles = (T + 15) >> 4;
    const int kbw = (KB + W - 1) / W;
    const int kb0 = wave * kbw;
    const int bid = (int)blockIdx.x;
    const int ntw = ntw_q + (bid < ntw_r);  // tiles of this workgroup, >= 1
    const int nout = ntw * MR * 48;

    // 1. epilogue operands (the compiler's loads, issued first: the explicit
    //    vmcnt counts below never wait for them); output idx = tid + q *
    //    kThreads is (tile j, row r, channel c)
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scales, (uint32_t)N * 2u);
    uint16_t ep_a[kEp];
    float ep_s[kEp];
#pragma unroll
    for (int q = 0; q < kEp; ++q) {
        const int idx = tid + q * kThreads;
        const int j = idx / (MR * 48), rc = idx - j * (MR * 48), r = rc / 48, c = rc - r * 48;
        const int ch = (bid + j * grid) * 48 + c;
        const bool ok = idx < nout && ch < N;
        ep_a[q] = __builtin_amdgcn_raw_buffer_load_b16(rsc, ok ? (uint32_t)ch * 2u : kOOB, 0, 0);
        ep_s[q] = ok ? xs[r] : 0.0f;
    }

    // 2. the small loads: this thread's table rows (load_stream_table_rows)
    //    and this wave's codes, NCL 16-byte chunks per lane: chunk q of the
    //    wave's slice is (row q / (4 kbw), columns 16 (q % (4 kbw)) ..)
    StreamTableRows<F3> trows;
    load_stream_table_rows<F3>(trows, reinterpret_cast<const uint8_t *>(table), tid);
    const v4i rx = rsrc_words(xq, (uint32_t)MR * (uint32_t)K);
    const int nq = MR * 4 * kbw;
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v cv[NCL];
#pragma unroll
    for (int i = 0; i < NCL; ++i) {
        const int q = lane + 64 * i;
        const int r = q / (4 * kbw), c16 = q - r * 4 * kbw;
        const int k = kb0 * 64 + 16 * c16;
        const uint32_t off = (q < nq && k < K) ? (uint32_t)r * (uint32_t)K + (uint32_t)k : kOOB;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(cv[i]) : "v"(off), "s"(rx) : "memory");
    }
    // every wave's small loads enter the CU's memory queue before any
    // fragment load does
    asm volatile("s_barrier" ::: "memory");

    // 3. weight fragments into a ring of registers: step s of this wave =
    //    tile j = s / kbw of the workgroup, block kb0 + s % kbw; steps past
    //    the end read zeros.  Each entry is tied to its registers ("+v") and
    //    waited for with vmcnt(slots - 1) before use (the younger loads are
    //    the other entries).  kEarly entries now, the rest after the
    //    workgroup barrier (a wave stalled issuing weight loads behind the
    //    memory backlog would reach the barrier late).
    const v4i rw = rsrc_words(tiled, (uint32_t)tiles * (uint32_t)KB * 1024u);
    int is_j = 0, is_b = 0;  // (tile, block) of the next step to issue
    auto next_off = [&]() {
        const int kb = kb0 + is_b;
        const bool live = is_j < ntw && kb < KB;
        const uint32_t tile = (uint32_t)(bid + is_j * grid);
        const uint32_t off = live ? (tile * (uint32_t)KB + (uint32_t)kb) * 1024u + (uint32_t)lane * 16u : kOOB;
        if (++is_b == kbw) {
            is_b = 0;
            ++is_j;
        }
        return off;
    };
    u4v pr[kCodesSlots];
    auto ring_load = [&](u4v &dst, uint32_t off) {
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "+v"(dst) : "v"(off), "s"(rw) : "memory");
    };
#pragma unroll
    for (int sl = 0; sl < kEarly; ++sl) {
        asm volatile("" : "=v"(pr[sl]));
        ring_load(pr[sl], next_off());
    }

    // 4. the table from the rows (only the codes and fragments may still be
    //    in flight), then the codes (only fragments) into this wave's LDS
    //    slice, 8-byte chunks at their permuted positions (read by this wave
    //    only); the workgroup barrier completes the table and the zeroed sums
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kEarly + NCL) : "memory");
#pragma unroll
    for (int k = 0; k < StreamTableRows<F3>::kRows; ++k) asm volatile("" : "+v"(trows.cpair[k]));
    build_stream_table<F3>(tab, trows, tid);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kEarly) : "memory");
#pragma unroll
    for (int i = 0; i < NCL; ++i) asm volatile("" : "+v"(cv[i]));
#pragma unroll
    for (int i = 0; i < NCL; ++i) {
        const int q = lane + 64 * i;
        if (q < nq) {
            const int r = q / (4 * kbw), c16 = q - r * 4 * kbw;
            int8_t *row = &xw[wave][r * 64 * kbw];
            *reinterpret_cast<uint2 *>(row + code_pos(16 * c16)) = make_uint2(cv[i].x, cv[i].y);
            *reinterpret_cast<uint2 *>(row + code_pos(16 * c16 + 8)) = make_uint2(cv[i].z, cv[i].w);
        }
    }
    for (int i = tid; i < ntw * MR * 48; i += kThreads) ybuf[i] = 0;
    if (tid < 4) reinterpret_cast<uint32_t *>(zero16)[tid] = 0u;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int sl = kEarly; sl < kCodesSlots; ++sl) {
        asm volatile("" : "=v"(pr[sl]));
        ring_load(pr[sl], next_off());
    }

    // A operand of group gr: lane row arw = 3 r' + d holds token 5 gr + r'
    // (rows past the tokens read zeros); sparsity index words as in the
    // fused kernel (the first product sends the even code bytes to position
    // d and the odd ones to position 3, a zero of every table dword; the
    // second the reverse)
    const int arw = lane & 15;
    const uint32_t dsel = (uint32_t)(arw % 3);
    const int idx_even = (int)(dsel * 0x11111111u + 0xCCCCCCCCu);
    const int idx_odd = (int)(0x33333333u + dsel * 0x44444444u);
    const int8_t *xa[NG];
    int xa_step[NG];
    bool arow[NG];
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
        const int tok = 5 * gr + arw / 3;
        arow[gr] = arw < 15 && tok < MR;
        xa[gr] = arow[gr] ? &xw[wave][tok * 64 * kbw + g * 16] : zero16;
        xa_step[gr] = arow[gr] ? 64 : 0;
    }
    const uint32_t lane_off = (uint32_t)lane << 2;
    const char *tb = reinterpret_cast<const char *>(tab);
    const int nsteps = ntw * kbw;

    v4i acc[NG], a[NG];
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
        acc[gr] = v4i{0, 0, 0, 0};
        a[gr] = v4i{0, 0, 0, 0};
    }
    int bl = 0, j = 0;
#pragma unroll 1
    for (int st0 = 0; st0 < nsteps; st0 += kCodesSlots) {
#pragma unroll
        for (int u = 0; u < kCodesSlots; ++u) {
            if (st0 + u >= nsteps) break;  // uniform
            asm volatile("s_waitcnt vmcnt(%1)" : "+v"(pr[u]) : "n"(kCodesSlots - 1) : "memory");
            const u4v p = pr[u];
#pragma unroll
            for (int gr = 0; gr < NG; ++gr)
                if (arow[gr]) a[gr] = *reinterpret_cast<const v4i *>(xa[gr] + bl * xa_step[gr]);
            const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
            v8i be, bo;  // table dwords of the lane's even / odd bytes
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t t = *reinterpret_cast<const int32_t *>(
                        tb + __builtin_amdgcn_perm(pw[jj], lane_off, 0x0C0C0400u + ((uint32_t)i << 8)));
                    if (i & 1)
                        bo[2 * jj + (i >> 1)] = t;
                    else
                        be[2 * jj + (i >> 1)] = t;
                }
            }
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                acc[gr] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[gr], be, acc[gr], idx_even, 0, 0);
                acc[gr] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[gr], bo, acc[gr], idx_odd, 0, 0);
            }
            ring_load(pr[u], next_off());
            if (++bl == kbw) {
                // tile j done for this wave: lane (n, g) holds rows 4 g + i of
                // each group, row 3 r' + d = channel 3 n + d of token 5 gr + r'
                if (kb0 < KB) {
#pragma unroll
                    for (int gr = 0; gr < NG; ++gr)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int m = 4 * g + i, tok = 5 * gr + m / 3;
                            if (m < 15 && tok < MR) atomicAdd(&ybuf[(j * MR + tok) * 48 + 3 * n + m % 3], acc[gr][i]);
                        }
                }
#pragma unroll
                for (int gr = 0; gr < NG; ++gr) acc[gr] = v4i{0, 0, 0, 0};
                bl = 0;
                ++j;
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // (the ring registers stay allocated until every load into them landed)
#pragma unroll
    for (int sl = 0; sl < kCodesSlots; ++sl) asm volatile("" ::"v"(pr[sl]));

#pragma unroll
    for (int q = 0; q < kEp; ++q) {
        const int idx = tid + q * kThreads;
        const int jj = idx / (MR * 48), rc = idx - jj * (MR * 48), r = rc / 48, c = rc - r * 48;
        const int ch = (bid + jj * grid) * 48 + c;
        if (idx < nout && ch < N) {
            const int32_t sum = ybuf[(jj * MR + r) * 48 + c];
            const float v = (ep_s[q] * (float)sum) * bf16_to_f32(ep_a[q]);
            if (obf)
                static_cast<uint16_t *>(y)[(int64_t)r * N + ch] = f32_to_bf16_rne(v);
            else
                static_cast<float *>(y)[(int64_t)r * N + ch] = v;
            if (acc_out) acc_out[(int64_t)r * N + ch] = sum;
        }
    }
}

// --------------------------------------------------------------- GEMM

// Prefill GEMM for many token rows: INT8 activations x decoded S3D8 weights
// on v_mfma_i32_32x32x32_i8 (INT32 accumulation), one wave per SIMD.  The
// library runs it for 64-row tiles and for every split-K launch; 128- and
// 160-row tiles without split-K run on the eight-wave kernel further down.
//
// Workgroup tile = 32 RT token rows x 128 channel triples (384 output
// channels), RT = 2, 4 or 5; 4 waves side by side along N, each 32 RT rows x
// 32 triples = RT row tiles x 3 channels of the triple = 3 RT accumulators
// of 32 x 32 (96, 192 or 240 AGPRs, one wave per SIMD).  Per 64-column block of K:
//  - activations (32 RT x 64 INT8) and the packed weights (128 triples x 64)
//    are copied straight from memory into LDS by buffer loads with the LDS
//    destination bit (no registers involved), four blocks ahead of use, into
//    a ring of five LDS slots.  The wait for a block is an explicit vmcnt
//    count, so the loads of later blocks stay in flight;
//  - the activation tile is stored with its 16-byte chunks XOR-swizzled by
//    row so that the MFMA operand reads (16 rows x 16 bytes per quarter
//    wave) hit distinct LDS banks;
//  - each wave reads its own 2 KiB of packed weights of block kb + 1 and
//    decodes them (LDS lookup table, see decode16) into B operands while the
//    MFMAs of block kb run.
// Epilogue: lane (c, h) of a 32 x 32 accumulator holds column c, i.e. the
// three channels of triple c, for rows 8 (v / 4) + 4 h + v % 4; each row's
// three outputs go out as one 12-byte store, 384 contiguous bytes per row and
// half wave.
//
// Workgroups are mapped XCD-aware and in groups (gemm_tile), so that the
// tiles resident on one XCD share activation and weight tiles in its L2.
constexpr int kGemmBF = 8;        // weight fragments (16 triples) per workgroup
constexpr int kGemmSlots = 5;     // LDS ring slots
constexpr int kGemmAhead = kGemmSlots - 1;  // blocks in flight ahead of use
constexpr int kXcds = 8;
// a workgroup's rows of fp32 output stay under 2^31 bytes (32-bit store offsets)
constexpr int kGemmMaxRT = 5;     // most 32-row tiles per wave of any GEMM variant
constexpr int64_t kGemmMaxN = (int64_t(1) << 31) / (4 * 32 * kGemmMaxRT) - 1;

typedef int32_t v16i __attribute__((ext_vector_type(16)));

// Tile of workgroup blockIdx.x.  Workgroup w runs on XCD w % 8; each XCD
// takes a contiguous range of tile indices, and tile indices run over
// groups of kGroupM row blocks, row block fastest within a group and
// column block next: the ~32 workgroups resident on one XCD then cover
// about 8 row blocks x 4 column blocks, so their activation and weight
// tiles are shared through that XCD's L2 instead of each workgroup
// streaming its own weight stripe.
//
// With the input columns split into `splits` ranges, the range index ks is
// the slowest: an XCD's workgroups then share a k range as well.
constexpr int kGroupM = 8;
__device__ __forceinline__ bool gemm_tile(int nbm, int nbn, int splits, int &bm, int &bn, int &ks) {
    const int nt = nbm * nbn;
    const int nwg = nt * splits;
    const int per_xcd = (nwg + kXcds - 1) / kXcds;
    const int L0 = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (L0 >= nwg) return false;
    ks = L0 / nt;
    const int L = L0 - ks * nt;
    const int group = L / (kGroupM * nbn), r = L - group * (kGroupM * nbn);
    const int gm = min(kGroupM, nbm - group * kGroupM);
    bm = group * kGroupM + r % gm;
    bn = r / gm;
    return true;
}
__device__ __forceinline__ bool gemm_tile(int nbm, int nbn, int &bm, int &bn) {
    int ks;
    return gemm_tile(nbm, nbn, 1, bm, bn, ks);
}

// s_waitcnt vmcnt(N) for the loads the compiler does not see (LDS-DMA), and
// the same followed by lgkmcnt(0) and a workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint16_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Epilogue of a wave's block of 32 RT rows: y[row][col_j] = (xs[row] * acc) *
// sc[j] for the three 32 x 32 accumulator columns j of each row tile i
// (and, kAcc, the accumulators themselves into acc_out).  Lane (c, h) holds
// rows 32 i + 8 (v / 4) + 4 h + v % 4 of accumulator register v; coff[j] is
// the byte offset of its column j within a row of y (kOOB for a column past
// N) and sc[j] that column's channel scale.
//
// Branch-free: the lane's 16 token scales arrive as four 16-byte buffer
// loads per row tile (rows past M read as zero), and every store is a
// buffer store whose offset has bit 31 set (out of range: dropped) for a row
// past M or a column past N.  kTriple: the three columns are channels 3t,
// 3t + 1, 3t + 2 of one triple and go out as one 12-byte store; a lane whose
// triple straddles N (at most one per matrix) stores its valid channels one
// by one instead, in a second pass only its wave runs.  Offsets stay below
// 2^32: the caller keeps 128 rows of y under 2^31 bytes.
//
// kBF: y is bfloat16 (round to nearest even of the fp32 value, as the
// blog's fused kernel writes its results); every channel goes out as its
// own 2-byte store.  kNT: the stores of y are non-temporal (they stream past
// the caches; measured faster for the plain INT8 GEMM, slower for the fused
// one).
template <bool kTriple, bool kAcc, int RT, bool kBF = false, bool kNT = false>
__device__ __forceinline__ void store_tile_rows(const v16i (&acc)[RT][3], const float *__restrict__ xs, int M,
                                                int N, int row0, int h, const float (&sc)[3], const uint32_t (&coff)[3],
                                                void *__restrict__ y, int32_t *__restrict__ acc_out) {
    const int nrows = min(M - row0, 32 * RT);
    const uint32_t rowb = 4u * (uint32_t)N;
    constexpr int kYAux = kNT ? 2 : 0;  // cache policy bits of the y stores (2: non-temporal)
    const auto rxs = make_rsrc(xs + row0, 4u * (uint32_t)nrows);
    float4 sx[RT][4];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            sx[i][g] = __builtin_bit_cast(float4, bload16(rxs, 4u * (uint32_t)(32 * i + 8 * g + 4 * h)));
    const auto ra = make_rsrc(acc_out + (int64_t)row0 * N, kAcc ? rowb * (uint32_t)nrows : 0u);
    uint32_t base[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) base[j] = coff[j] + (uint32_t)(4 * h) * rowb;
    // bit 31 when row 32 i + 8 (v / 4) + v % 4 + 4 h is past M
    auto dead = [&](int r) { return (uint32_t)(nrows - 1 - r - 4 * h) & kOOB; };
    auto outf = [&](int i, int v, int j) { return (sx[i][v >> 2][v & 3] * (float)acc[i][j][v]) * sc[j]; };
    auto out = [&](int i, int v, int j) { return __float_as_uint(outf(i, v, j)); };
    if constexpr (kBF) {
        const uint32_t yrowb = 2u * (uint32_t)N;
        const auto ry = make_rsrc(static_cast<uint16_t *>(y) + (int64_t)row0 * N, yrowb * (uint32_t)nrows);
        uint32_t ybase[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) ybase[j] = (coff[j] == kOOB ? kOOB : coff[j] >> 1) + (uint32_t)(4 * h) * yrowb;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + (v & 3);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(outf(i, v, j)), ry,
                                                          (ybase[j] + (uint32_t)r * yrowb) | dead(r), 0, kYAux);
                    if constexpr (kAcc)
                        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc[i][j][v], ra,
                                                              (base[j] + (uint32_t)r * rowb) | dead(r), 0, 0);
                }
            }
        return;
    }
    const auto ry = make_rsrc(static_cast<float *>(y) + (int64_t)row0 * N, rowb * (uint32_t)nrows);
    if constexpr (kTriple) {
        typedef uint32_t u3 __attribute__((ext_vector_type(3)));
        const bool split = coff[0] != kOOB && coff[2] == kOOB;
        const uint32_t base3 = split ? kOOB : base[0];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + (v & 3);
                const uint32_t off = (base3 + (uint32_t)r * rowb) | dead(r);
                __builtin_amdgcn_raw_buffer_store_b96(u3{out(i, v, 0), out(i, v, 1), out(i, v, 2)}, ry, off, 0, kYAux);
                if constexpr (kAcc)
                    __builtin_amdgcn_raw_buffer_store_b96(
                        u3{(uint32_t)acc[i][0][v], (uint32_t)acc[i][1][v], (uint32_t)acc[i][2][v]}, ra, off, 0, 0);
            }
        if (__builtin_amdgcn_ballot_w64(split) == 0) return;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + (v & 3);
                const uint32_t d = dead(r) | (split ? 0u : kOOB);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint32_t off = (base[j] + (uint32_t)r * rowb) | d;
                    __builtin_amdgcn_raw_buffer_store_b32(out(i, v, j), ry, off, 0, kYAux);
                    if constexpr (kAcc) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc[i][j][v], ra, off, 0, 0);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + (v & 3);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const uint32_t off = (base[j] + (uint32_t)r * rowb) | dead(r);
                    __builtin_amdgcn_raw_buffer_store_b32(out(i, v, j), ry, off, 0, kYAux);
                    if constexpr (kAcc) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc[i][j][v], ra, off, 0, 0);
                }
            }
    }
}

// Split-K (splits > 1): the ceil(K/64) column blocks are cut into ranges of
// kbper blocks and workgroup (tile, ks) runs range ks only.  Its INT32 sums
// are exact partial sums of the tile's accumulators, so adding the ranges'
// sums in any order gives the accumulators of the whole product.  The
// workgroups of a tile meet through two counters per tile in ws_cnt: each
// takes an arrival number from the first and stores its partial sums in slot
// `arrival` of the tile in ws_part (`splits` slots per tile,
// part_wave_bytes(RT) per wave; on 64-row tiles the last arrival stores
// nothing); all but the last then count themselves done in the second; the
// last waits for splits - 1 done, sets both counters back to zero for the
// next call, and runs the epilogue on the sum of all the tile's partial
// sums.  It only waits
// for workgroups that have already arrived (so
// are running and wait for nothing), and the wait is bounded: counters that
// do not start at zero give wrong results, never a hang.  Loads and stores
// in ws_part are range-checked against part_bytes.
//
// Visibility across XCDs (each has its own L2) without fences: a fence at
// device scope writes back and invalidates the whole L2 of the XCD, which
// also throws away the operand tiles of every other workgroup there (the
// first version, with fences and an acquiring spin, ran the vision
// down-projection 1.5 to 2.7 times slower than without split-K).  Instead
// the partial sums are stored and loaded with device scope (the SC1 cache
// policy bit), which makes those accesses themselves coherent across the
// device; every wave waits for its stores to complete (vmcnt(0)) before the
// workgroup barrier that precedes the done count, and the counters are
// relaxed device-scope atomics.
constexpr int kScopeDevice = 16;      // cache policy SC1 (SC0 = 0): device scope
constexpr uint32_t kPartQuad = 1024;  // one 16-byte quarter of an accumulator, all 64 lanes
constexpr int kSpinLimit = 1 << 20;   // about 0.2 s of s_sleep 8
__host__ __device__ constexpr uint32_t part_wave_bytes(int rt) { return 3u * 4u * kPartQuad * (uint32_t)rt; }

// (the arguments the prologue uses come first, so that they are all among
// the 16 argument dwords preloaded into SGPRs; the epilogue's follow)
template <int RT, bool kAcc, bool kBF, bool kSplit>
__global__ __launch_bounds__(256) void gemm_kernel(const int8_t *__restrict__ xq, const uint8_t *__restrict__ tiled,
                                                   const uint32_t *__restrict__ centroids, int M, int K, int N,
                                                   int T, int nbm, int nbn, int f3d8, int splits, int kbper,
                                                   const float *__restrict__ xs,
                                                   const uint16_t *__restrict__ scales, void *__restrict__ y,
                                                   int32_t *__restrict__ acc_out, int32_t *__restrict__ ws_cnt,
                                                   int32_t *__restrict__ ws_part, uint32_t part_bytes) {
    __shared__ __attribute__((aligned(16))) uint32_t tab[kTabWords];
    constexpr int BM = 32 * RT;          // token rows per workgroup
    constexpr int NA = (2 * RT + 3) / 4;  // activation loads per wave and block
    constexpr int ND = NA + 2;            // all loads per wave and block
    __shared__ __attribute__((aligned(16))) int8_t abuf[kGemmSlots][BM * 64];
    __shared__ __attribute__((aligned(16))) int8_t spill[(4 * NA > 2 * RT) ? 1024 : 16];
    __shared__ __attribute__((aligned(16))) int8_t wbuf[kGemmSlots][kGemmBF * 1024];
    __shared__ uint32_t clw[kTableWords3D8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, h = lane >> 5;
    const int KB = (K + 63) >> 6;
    const int tiles16 = (T + 15) >> 4;
    const uint32_t lane_off = (uint32_t)lane << 2;

    // (the builds without split-K keep one range: they compile to the plain
    // kernel, with no trace of the split-K code)
    if constexpr (!kSplit) splits = 1;
    int bm, bn, ks;
    if (!gemm_tile(nbm, nbn, splits, bm, bn, ks)) return;  // padding workgroup (grid rounded up to a multiple of 8)
    const int row0 = bm * BM;
    const int frag0 = bn * kGemmBF + wave * 2;
    // this workgroup's column blocks: kb0 .. kb0 + nkb - 1 (the host makes
    // every range non-empty)
    const int kb0 = kSplit ? ks * kbper : 0;
    const int nkb = kSplit ? min(kbper, KB - kb0) : KB;

    // the table: S3D8's 96 bytes through the scalar cache; 3D8's 768 bytes as
    // one word per thread (an explicit load, waited for below; an
    // out-of-range offset reads nothing for S3D8)
    uint32_t cw[24];
#pragma unroll
    for (int i = 0; i < 24; ++i) cw[i] = centroids[i];
    uint32_t c3;
    {
        const v4i rc3 = rsrc_words(centroids, 768u);
        const uint32_t off = (f3d8 && tid < kTableWords3D8) ? 4u * (uint32_t)tid : kOOB;
        asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(c3) : "v"(off), "s"(rc3) : "memory");
    }

    const v4i rx = rsrc_words(xq, (uint32_t)M * (uint32_t)K);
    const v4i rw = rsrc_words(tiled, (uint32_t)tiles16 * (uint32_t)KB * 1024u);

    // activation copy: wave w moves 16-byte units u = 64 (NA w + j) + lane of
    // the BM x 64 tile; unit u holds row u / 4, chunk (u % 4) ^ ((row / 4) % 4).
    // Loads past the tile (when 4 NA > 2 RT) read nothing into `spill`.
    uint32_t aoff[NA];
    int acol[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int u = 64 * (NA * wave + j) + lane;
        const int row = u >> 2;
        const int chunk = (u & 3) ^ ((row >> 2) & 3);
        aoff[j] = row < BM && row0 + row < M ? (uint32_t)(row0 + row) * (uint32_t)K + 16u * chunk : kOOB;
        acol[j] = 16 * chunk;
    }
    // weight copy: lane (c, h), k-half kh takes triple c of the wave at
    // k = 32 kh + 16 h .. + 15, i.e. fragment lane (c % 16) + 16 (2 kh + h)
    const int wfr = frag0 + (c32 >> 4);
    uint32_t woff[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
        woff[kh] = wfr < tiles16 ? (uint32_t)wfr * (uint32_t)KB * 1024u + (uint32_t)((c32 & 15) + 16 * (2 * kh + h)) * 16u
                                 : kOOB;

    const uint32_t abase = S3D8_LDS_OFFSET(&abuf[0][0]), wbase = S3D8_LDS_OFFSET(&wbuf[0][0]);
    const uint32_t sbase = S3D8_LDS_OFFSET(&spill[0]);
    // In the last block the activation chunks at or past K must read zeros
    // (the weights there decode to +-C[0], not to zero): atail holds the
    // per-lane offsets of that block.
    const int ktail = K - 64 * (KB - 1);
    uint32_t atail[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) atail[j] = acol[j] < ktail ? aoff[j] : kOOB;
    // ND loads per wave and block, also for the blocks past the end of the
    // range, so that every wait below counts the same: those re-read the
    // range's last block into a slot that is never read.  kb counts from the
    // range's start.  The per-lane offsets are block 0's; the block's byte
    // offset goes in the scalar offset of the loads.
    auto issue = [&](int kb, int slot) {
        const int kbc = kb0 + (kb < nkb ? kb : nkb - 1);
        const bool tail = kbc >= KB - 1;
        uint32_t lds[ND], vo[ND];
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            lds[j] = NA * wave + j < 2 * RT ? abase + (uint32_t)(BM * 64) * slot + 1024u * (NA * wave + j) : sbase;
            vo[j] = tail ? atail[j] : aoff[j];
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            lds[NA + kh] = wbase + (uint32_t)(kGemmBF * 1024) * slot + 2048u * wave + 1024u * kh;
            vo[NA + kh] = woff[kh];
        }
        load_block_to_lds<NA>(lds, vo, rx, 64u * (uint32_t)kbc, rw, 1024u * (uint32_t)kbc);
    };

    // A operand of row tile i, k-half kh: row 32 i + c32, chunk 2 kh + h
    const int swz = (c32 >> 2) & 3;
    const int ard0 = c32 * 64 + 16 * (h ^ swz), ard1 = c32 * 64 + 16 * ((h ^ swz) ^ 2);

    // decode of packed dword p (k-half p / 4, dword p % 4) of the raw
    // weights, in two halves that the block below schedules apart: the four
    // table lookups, and the 4 x 3 byte transpose into operand set bs
    auto lookups = [&](const uint4 (&ps)[2], int p, uint32_t (&q)[4]) {
        const char *tb = reinterpret_cast<const char *>(tab);
        const int kh = p >> 2, c = p & 3;
        const uint32_t dw = c == 0 ? ps[kh].x : c == 1 ? ps[kh].y : c == 2 ? ps[kh].z : ps[kh].w;
        q[0] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0400u));
        q[1] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0500u));
        q[2] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0600u));
        q[3] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0700u));
    };
    auto transpose = [&](const uint32_t (&q)[4], v4i (&bs)[2][3], int p) {
        const int kh = p >> 2, c = p & 3;
        const uint32_t p01 = __builtin_amdgcn_perm(q[1], q[0], 0x05010400u);
        const uint32_t p23 = __builtin_amdgcn_perm(q[3], q[2], 0x05010400u);
        const uint32_t s01 = __builtin_amdgcn_perm(q[1], q[0], 0x0C0C0602u);
        const uint32_t s23 = __builtin_amdgcn_perm(q[3], q[2], 0x0C0C0602u);
        bs[kh][0][c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x05040100u);
        bs[kh][1][c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x07060302u);
        bs[kh][2][c] = (int32_t)__builtin_amdgcn_perm(s23, s01, 0x05040100u);
    };
    auto read_w = [&](uint4 (&ps)[2], int slot) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
            ps[kh] = *reinterpret_cast<const uint4 *>(&wbuf[slot][2048 * wave + 1024 * kh + 16 * lane]);
    };

    // prologue: blocks 0 and 1 in flight, build the table, wait for block 0,
    // then blocks 2 and 3 (every workgroup starts at once: with only two
    // blocks each in the first burst, block 0 lands sooner; measured
    // alternating on one box, c3 133.6 against 133.9 us, vision up 25.0
    // against 25.2 us, the other prefill shapes 0.1 to 0.4 us faster; three
    // blocks first gained nothing)
#pragma unroll
    for (int s = 0; s < 2; ++s) issue(s, s);
    // (the table word is the oldest load: waiting until only the blocks'
    // loads are in flight covers it)
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(c3) : "n"(2 * ND) : "memory");
    if (f3d8) {
        if (tid < kTableWords3D8) clw[tid] = c3;
    } else if (tid == 0) {
#pragma unroll
        for (int i = 0; i < 6; ++i)
            reinterpret_cast<uint4 *>(clw)[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
    }
    __syncthreads();
    {
        const uint8_t *cl = reinterpret_cast<const uint8_t *>(clw);
        for (int idx = tid; idx < kTabWords / 4; idx += 256) {
            const uint32_t b = (uint32_t)idx >> 4;
            const uint32_t v = f3d8 ? row_3d8(b, cl) : signed_triple(b, cl);
            reinterpret_cast<uint4 *>(tab)[idx] = make_uint4(v, v, v, v);
        }
    }
    static_assert(kGemmAhead == 4, "the waits below assume four blocks in flight");
    wait_vmcnt<ND>();  // this wave's block 0 is in LDS
    __syncthreads();   // everyone's block 0, and the table
    issue(2, 2);
    issue(3, 3);

    v16i acc[RT][3];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int d = 0; d < 3; ++d) acc[i][d] = v16i{};

    // operands of block 0 (A from LDS, B decoded)
    auto read_a = [&](v4i (&a)[RT][2], int slot, int i) {
        const int8_t *ab = abuf[slot];
        a[i][0] = *reinterpret_cast<const v4i *>(ab + 2048 * i + ard0);
        a[i][1] = *reinterpret_cast<const v4i *>(ab + 2048 * i + ard1);
    };
    v4i a0[RT][2], a1[RT][2];
    v4i b0[2][3], b1[2][3];
    {
        uint4 w0[2];
        read_w(w0, 0);
#pragma unroll
        for (int i = 0; i < RT; ++i) read_a(a0, 0, i);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint32_t q[4];
            lookups(w0, p, q);
            transpose(q, b0, p);
        }
    }

    // block kb (LDS slot `slot`): wait until blocks <= kb + 1 are in LDS for
    // every wave (2 ND loads = blocks kb + 2, kb + 3 may stay in flight),
    // refill the slot of block kb - 1 with block kb + 4, then the 6 RT MFMAs
    // of A(kb) x B(kb) in 2 RT groups of three, with the operands of block
    // kb + 1 prepared between them.  Group g carries: the raw weights (g = 0),
    // A row tile i (g = i % 4), the lookups of dwords 2 (g - LK0) and
    // 2 (g - LK0) + 1, and the transposes of dwords 2 (g - TR0) and
    // 2 (g - TR0) + 1.  At RT = 5 (ten groups) LK0 = 2 and TR0 = 6: the raw
    // weights have two groups of MFMAs to land behind and every lookup four
    // (measured at c3 about 2.5 % faster than LK0 = 1, TR0 = 3, which is all
    // that the eight groups at RT = 4 leave room for).  RT = 2 (64-row tiles,
    // for shapes with few output tiles) has four groups: the lookups of
    // dwords 0..3 in group 1 and of 4..7 in group 2, their transposes one
    // group later.
    // Inside a group
    // each MFMA is followed by a share of the VALU and LDS work, since one
    // wave per SIMD only overlaps what lies between its MFMAs; sched_barrier
    // keeps the compiler from regrouping across groups.
    static_assert(RT == 2 || 2 * RT >= 7, "the block schedule needs seven groups, or the four of RT = 2");
    constexpr int kGrpValu = RT == 2 ? 8 : 6, kGrpLds = RT == 2 ? 6 : 4;
    auto block = [&](const v4i (&ac)[RT][2], v4i (&an)[RT][2], const v4i (&bc)[2][3], v4i (&bnx)[2][3], int kb,
                     int slot) {
        wait_vmcnt_barrier<2 * ND>();
        const int next = slot == kGemmSlots - 1 ? 0 : slot + 1;
        const int prev = slot == 0 ? kGemmSlots - 1 : slot - 1;
        issue(kb + kGemmAhead, prev);
        uint4 wn[2];
        uint32_t q[8][4];
#pragma unroll
        for (int g = 0; g < 2 * RT; ++g) {
            const int kh = g / RT, i = g % RT;
#pragma unroll
            for (int d = 0; d < 3; ++d)
                acc[i][d] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ac[i][kh], bc[kh][d], acc[i][d], 0, 0, 0);
            if (g == 0) read_w(wn, next);
#pragma unroll
            for (int r = 0; r < RT; ++r)
                if (g == r % 4) read_a(an, next, r);
            if constexpr (RT == 2) {
                if (g == 1 || g == 2)
#pragma unroll
                    for (int p = 4 * (g - 1); p < 4 * g; ++p) lookups(wn, p, q[p]);
                if (g == 2 || g == 3)
#pragma unroll
                    for (int p = 4 * (g - 2); p < 4 * (g - 1); ++p) transpose(q[p], bnx, p);
            } else {
                constexpr int LK0 = RT == 5 ? 2 : 1;
                if (g >= LK0 && g <= LK0 + 3) {
                    lookups(wn, 2 * (g - LK0), q[2 * (g - LK0)]);
                    lookups(wn, 2 * (g - LK0) + 1, q[2 * (g - LK0) + 1]);
                }
                constexpr int TR0 = RT == 5 ? 6 : 3;
                if (g >= TR0 && g <= TR0 + 3) {
                    transpose(q[2 * (g - TR0)], bnx, 2 * (g - TR0));
                    transpose(q[2 * (g - TR0) + 1], bnx, 2 * (g - TR0) + 1);
                }
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, kGrpValu, 0);  // a share of the VALU
                __builtin_amdgcn_sched_group_barrier(0x100, kGrpLds, 0);   // and of the LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int kb = 0, slot = 0;
#pragma unroll 1
    for (; kb + 1 < nkb; kb += 2) {
        block(a0, a1, b0, b1, kb, slot);
        slot = slot == kGemmSlots - 1 ? 0 : slot + 1;
        block(a1, a0, b1, b0, kb + 1, slot);
        slot = slot == kGemmSlots - 1 ? 0 : slot + 1;
    }
    if (kb < nkb) block(a0, a1, b0, b1, kb, slot);
    // loads of blocks past the end are still in flight: drain before exit
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // kKeepOwn: the last workgroup of a tile adds the other slots to its own
    // accumulators (row tiles unrolled, so that the accumulators are indexed
    // at compile time); otherwise it stores its sums like the others and
    // adds all slots in a run-time row-tile loop.  Only the 64-row tiles
    // take the first form: with 128 or 160 rows the compiler moves part of
    // the accumulators through scratch memory for it, as much traffic as the
    // slot it saves.  (Adding into the accumulators, or indexing them with a
    // run-time row tile, made it spill inside the main loop.)
    constexpr bool kKeepOwn = RT == 2;
    if (kSplit && splits > 1) {
        __shared__ int arrival;
        const int tile = bm * nbn + bn;
        if (tid == 0)
            arrival = __hip_atomic_fetch_add(ws_cnt + 2 * tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int arr = min(max(arrival, 0), splits - 1);
        auto store_own = [&]() {
            const auto rp = make_rsrc(ws_part, part_bytes);
            const uint32_t pb =
                ((uint32_t)(tile * splits + arr) * 4u + (uint32_t)wave) * part_wave_bytes(RT) + 16u * lane;
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int d = 0; d < 3; ++d)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4i v{acc[i][d][4 * q], acc[i][d][4 * q + 1], acc[i][d][4 * q + 2],
                                    acc[i][d][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rp,
                                                               pb + (uint32_t)((i * 3 + d) * 4 + q) * kPartQuad, 0,
                                                               kScopeDevice);
                    }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's sums are stored at device scope
            __syncthreads();
        };
        if constexpr (!kKeepOwn) store_own();
        if (arr < splits - 1) {
            if constexpr (kKeepOwn) store_own();
            if (tid == 0) __hip_atomic_fetch_add(ws_cnt + 2 * tile + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (tid == 0) {
            int spins = 0;
            while (__hip_atomic_load(ws_cnt + 2 * tile + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < splits - 1 &&
                   ++spins < kSpinLimit)
                __builtin_amdgcn_s_sleep(8);
            __hip_atomic_store(ws_cnt + 2 * tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ws_cnt + 2 * tile + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }

    // epilogue: y = (xs[row] * acc) * alpha[ch] for channels 3 (16 frag0 +
    // c) + d, the three contiguous channels of lane c's triple
    const int ch0 = 3 * (16 * frag0 + c32);
    float sc[3];
    uint32_t coff[3];
    const auto rsc = make_rsrc(scales, (uint32_t)N * 2u);
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const bool ok = ch0 + d < N;
        coff[d] = ok ? 4u * (uint32_t)(ch0 + d) : kOOB;
        sc[d] = bf16_to_f32(bload2(rsc, ok ? 2u * (uint32_t)(ch0 + d) : kOOB));
    }
    if (!kSplit || splits == 1) {
        store_tile_rows<true, kAcc, RT, kBF>(acc, xs, M, N, row0, h, sc, coff, y, acc_out);
        return;
    }
    // split-K, last workgroup of the tile: one 32-row tile at a time, the
    // slots added to its own sums (kKeepOwn: slots 0 .. splits - 2 to the
    // accumulators; else all slots, its own included, to zero), two slots'
    // loads (24 per lane) in flight at a time (the loads come from other
    // XCDs' writes at device scope: one at a time they cost about half a
    // microsecond each)
    const auto rp = make_rsrc(ws_part, part_bytes);
    const int tile = bm * nbn + bn;
    const int rows = min(RT, (M - row0 + 31) / 32);
    if constexpr (kKeepOwn) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            if (i >= rows) break;  // uniform
            v16i sum[1][3] = {{acc[i][0], acc[i][1], acc[i][2]}};
#pragma unroll 1
            for (int s = 0; s < splits - 1; s += 2) {
                uint4 v[2][12];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    // a missing second slot reads zeros (out-of-range offset)
                    const uint32_t pb = s + u < splits - 1
                                            ? ((uint32_t)(tile * splits + s + u) * 4u + (uint32_t)wave) *
                                                      part_wave_bytes(RT) +
                                                  16u * lane + (uint32_t)(12 * i) * kPartQuad
                                            : kOOB;
#pragma unroll
                    for (int j = 0; j < 12; ++j)
                        v[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                rp, pb == kOOB ? kOOB : pb + (uint32_t)j * kPartQuad,
                                                                0, kScopeDevice));
                }
                __builtin_amdgcn_sched_barrier(0);  // all 24 loads issued before the first add waits
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int j = 0; j < 12; ++j) {
                        const int d = j >> 2, q = j & 3;
                        sum[0][d][4 * q] += (int32_t)v[u][j].x;
                        sum[0][d][4 * q + 1] += (int32_t)v[u][j].y;
                        sum[0][d][4 * q + 2] += (int32_t)v[u][j].z;
                        sum[0][d][4 * q + 3] += (int32_t)v[u][j].w;
                    }
            }
            store_tile_rows<true, kAcc, 1, kBF>(sum, xs, M, N, row0 + 32 * i, h, sc, coff, y, acc_out);
        }
        return;
    }
#pragma unroll 1
    for (int i = 0; i < rows; ++i) {
        v16i sum[1][3] = {};
#pragma unroll 1
        for (int s = 0; s < splits; s += 2) {
            uint4 v[2][12];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                // a missing second slot reads zeros (out-of-range offset)
                const uint32_t pb =
                    s + u < splits
                        ? ((uint32_t)(tile * splits + s + u) * 4u + (uint32_t)wave) * part_wave_bytes(RT) + 16u * lane +
                              (uint32_t)(12 * i) * kPartQuad
                        : kOOB;
#pragma unroll
                for (int j = 0; j < 12; ++j)
                    v[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            rp, pb == kOOB ? kOOB : pb + (uint32_t)j * kPartQuad, 0,
                                                            kScopeDevice));
            }
            __builtin_amdgcn_sched_barrier(0);  // all 24 loads issued before the first add waits
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 12; ++j) {
                    const int d = j >> 2, q = j & 3;
                    sum[0][d][4 * q] += (int32_t)v[u][j].x;
                    sum[0][d][4 * q + 1] += (int32_t)v[u][j].y;
                    sum[0][d][4 * q + 2] += (int32_t)v[u][j].z;
                    sum[0][d][4 * q + 3] += (int32_t)v[u][j].w;
                }
        }
        store_tile_rows<true, kAcc, 1, kBF>(sum, xs, M, N, row0 + 32 * i, h, sc, coff, y, acc_out);
    }
}

// --------------------------------------------------------------- GEMM, eight waves

// The fused GEMM's workgroup tile (16 R token rows x 128 triples, R = 8 or
// 10) split by columns over eight waves, two per SIMD: wave w owns weight
// fragment w of the tile (16 triples, 48 channels) over all 16 R rows, on
// v_mfma_i32_16x16x64_i8: R row tiles x the 3 channels of the triple = 3 R
// accumulators of 16 x 16 (120 registers at R = 10).  Each wave decodes only its own
// fragment (16 table lookups per lane and block, half of gemm_kernel's at
// the same tile) and reads the whole activation tile (R ds_read_b128 per
// block).  With two waves per SIMD one wave's lookups, reads and decode run
// beside the other wave's MFMAs, which one wave per SIMD cannot do.
//
// Operand layouts of the 16 x 16 x 64 product: B lane (t, g) = t + 16 g
// holds column t at k = 16 g .. 16 g + 15, which is how the tiled layout
// stores a fragment's block (one ds_read_b128 at 16 lane gives a wave its
// raw weights); A lane (r, g) holds row r of the row tile, 16-byte chunk g of
// the block; the result lane (t, g) holds triple t for rows 4 g .. 4 g + 3.
//
// Copies as in gemm_kernel (LDS-DMA, five slots, four blocks ahead): the R
// activation loads and 8 weight loads of a block go to waves w (activation
// load w and weight load w) and, for w + 8 < R, activation load 8 + w as
// well.  The activation tile is laid out in LDS as the A operand wants it:
// KiB i holds rows 16 i .. 16 i + 15, chunk g of row 16 i + r at 256 g + 16 r,
// so that a row tile's operand is one contiguous ds_read_b128 (16 lane).
// (gemm_kernel's row-swizzled layout, read in this operand's lane pattern,
// measured a two-way bank conflict on every such read: SQ_LDS_BANK_CONFLICT
// at a third of SQ_LDS_IDX_ACTIVE over the whole kernel.)
constexpr int kW8Threads = 512;

// Epilogue of the eight-wave GEMM for one wave: y[row][3 t + d] = (xs[row] *
// acc) * sc[d] for rows 16 i + 4 g + v of accumulator acc[i][d] (element v),
// with xs[row0 + r] read from xsl[r] in LDS;
// coff[d] is the byte offset of channel 3 t + d within a row of y (kOOB
// past N).  Branch-free as store_tile_rows: rows past M and channels past N
// get an out-of-range offset and their stores are dropped; a lane whose
// triple straddles N stores its valid channels one by one in a second pass.
// kBF: bfloat16 outputs, a 4-byte and a 2-byte store per row (one 2-byte
// store per channel when the accumulators are stored as well).
template <int R, bool kAcc, bool kBF>
__device__ __forceinline__ void store_rows16(const v4i (&acc)[R][3], const float *xsl, int M, int N,
                                             int row0, int g, const float (&sc)[3], const uint32_t (&coff)[3],
                                             void *__restrict__ y, int32_t *__restrict__ acc_out) {
    const int nrows = min(M - row0, 16 * R);
    const uint32_t rowb = 4u * (uint32_t)N;
    float4 sx[R];
#pragma unroll
    for (int i = 0; i < R; ++i) sx[i] = *reinterpret_cast<const float4 *>(&xsl[16 * i + 4 * g]);
    const auto ra = make_rsrc(acc_out + (int64_t)row0 * N, kAcc ? rowb * (uint32_t)nrows : 0u);
    auto dead = [&](int r) { return (uint32_t)(nrows - 1 - r) & kOOB; };
    auto outf = [&](int i, int v, int d) { return (sx[i][v] * (float)acc[i][d][v]) * sc[d]; };
    auto out = [&](int i, int v, int d) { return __float_as_uint(outf(i, v, d)); };
    typedef uint32_t u3 __attribute__((ext_vector_type(3)));
    const bool split = coff[0] != kOOB && coff[2] == kOOB;
    if constexpr (kBF && kAcc) {
        // with the accumulators as well: one 2-byte store per channel beside
        // each accumulator (the packed stores below made this build spill)
        const uint32_t yrowb = 2u * (uint32_t)N;
        const auto ry = make_rsrc(static_cast<uint16_t *>(y) + (int64_t)row0 * N, yrowb * (uint32_t)nrows);
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * g + v;
#pragma unroll
                for (int d = 0; d < 3; ++d) {
                    const uint32_t yo = coff[d] == kOOB ? kOOB : coff[d] >> 1;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(outf(i, v, d)), ry,
                                                          (yo + (uint32_t)r * yrowb) | dead(r), 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc[i][d][v], ra,
                                                          (coff[d] + (uint32_t)r * rowb) | dead(r), 0, 0);
                }
            }
        return;
    } else if constexpr (kBF) {
        // Triple t's three bf16 channels are bytes 6t .. 6t + 5 of a row: for
        // even t a 4-byte-aligned pair (channels 0, 1) and a halfword, for
        // odd t a halfword and an aligned pair (channels 1, 2), so two stores
        // per row instead of three.  (Lane parity is triple parity: the
        // wave's first triple is a multiple of 16.)  A triple that straddles
        // N stores its valid channels one by one in a second pass.
        const uint32_t yrowb = 2u * (uint32_t)N;
        const auto ry = make_rsrc(static_cast<uint16_t *>(y) + (int64_t)row0 * N, yrowb * (uint32_t)nrows);
        const bool odd = (threadIdx.x & 1) != 0;
        const uint32_t b0 = split ? kOOB : (coff[0] == kOOB ? kOOB : coff[0] >> 1);
        const uint32_t o32 = odd ? b0 + 2u : b0, o16 = odd ? b0 : b0 + 4u;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * g + v;
                const uint32_t h0 = f32_to_bf16_rne(outf(i, v, 0)), h1 = f32_to_bf16_rne(outf(i, v, 1)),
                               h2 = f32_to_bf16_rne(outf(i, v, 2));
                const uint32_t pair = odd ? (h1 | (h2 << 16)) : (h0 | (h1 << 16));
                __builtin_amdgcn_raw_buffer_store_b32(pair, ry, (o32 + (uint32_t)r * yrowb) | dead(r), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(odd ? h0 : h2), ry,
                                                      (o16 + (uint32_t)r * yrowb) | dead(r), 0, 0);
            }
        if (__builtin_amdgcn_ballot_w64(split) == 0) return;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * i + 4 * g + v;
                const uint32_t dd = dead(r) | (split ? 0u : kOOB);
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const uint32_t yo = coff[d] == kOOB ? kOOB : coff[d] >> 1;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(outf(i, v, d)), ry,
                                                          (yo + (uint32_t)r * yrowb) | dd, 0, 0);
                }
            }
        return;
    }
    const auto ry = make_rsrc(static_cast<float *>(y) + (int64_t)row0 * N, rowb * (uint32_t)nrows);
    const uint32_t base3 = split ? kOOB : coff[0];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * i + 4 * g + v;
            const uint32_t off = (base3 + (uint32_t)r * rowb) | dead(r);
            __builtin_amdgcn_raw_buffer_store_b96(u3{out(i, v, 0), out(i, v, 1), out(i, v, 2)}, ry, off, 0, 0);
            if constexpr (kAcc)
                __builtin_amdgcn_raw_buffer_store_b96(
                    u3{(uint32_t)acc[i][0][v], (uint32_t)acc[i][1][v], (uint32_t)acc[i][2][v]}, ra, off, 0, 0);
        }
    if (__builtin_amdgcn_ballot_w64(split) == 0) return;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * i + 4 * g + v;
            const uint32_t dd = dead(r) | (split ? 0u : kOOB);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const uint32_t off = (coff[d] + (uint32_t)r * rowb) | dd;
                __builtin_amdgcn_raw_buffer_store_b32(out(i, v, d), ry, off, 0, 0);
                if constexpr (kAcc) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)acc[i][d][v], ra, off, 0, 0);
            }
        }
}

// vmcnt waits of the eight-wave GEMM, where a wave issues one weight load
// and one or two activation loads per block (two for w + 8 < R): wait until
// at most kBlocks blocks of this wave's loads are in flight (then, kBar,
// lgkmcnt(0) and a workgroup barrier)
template <int R, int kBlocks, bool kBar>
__device__ __forceinline__ void w8_wait(int wave) {
    static_assert(R >= 8 && R <= 16, "every wave takes at least one activation load");
    if (wave + 8 < R) {
        if constexpr (kBar) wait_vmcnt_barrier<3 * kBlocks>(); else wait_vmcnt<3 * kBlocks>();
    } else {
        if constexpr (kBar) wait_vmcnt_barrier<2 * kBlocks>(); else wait_vmcnt<2 * kBlocks>();
    }
}

template <int R, bool kAcc, bool kBF>
__global__ __launch_bounds__(kW8Threads) void gemm_w8_kernel(const int8_t *__restrict__ xq,
                                                             const uint8_t *__restrict__ tiled,
                                                             const uint32_t *__restrict__ centroids, int M, int K,
                                                             int N, int T, int nbm, int nbn, int f3d8,
                                                             const float *__restrict__ xs,
                                                             const uint16_t *__restrict__ scales,
                                                             void *__restrict__ y, int32_t *__restrict__ acc_out) {
    static_assert(R == 8 || R == 10, "128 or 160 token rows (the block schedule and the LDS ring are sized for them)");
    constexpr int BM = 16 * R;
    __shared__ __attribute__((aligned(16))) uint32_t tab[kTabWords];
    __shared__ __attribute__((aligned(16))) int8_t abuf[kGemmSlots][BM * 64];
    __shared__ __attribute__((aligned(16))) int8_t wbuf[kGemmSlots][kGemmBF * 1024];
    __shared__ uint32_t clw[kTableWords3D8];
    __shared__ __attribute__((aligned(16))) float xsl[4 * 64];  // the tile's token scales (one LDS-DMA load)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = (K + 63) >> 6;
    const int tiles16 = (T + 15) >> 4;
    const uint32_t lane_off = (uint32_t)lane << 2;

    int bm, bn;
    if (!gemm_tile(nbm, nbn, bm, bn)) return;  // padding workgroup (grid rounded up to a multiple of 8)
    const int row0 = bm * BM;
    const int frag = bn * kGemmBF + wave;

    // wave 0 copies the tile's token scales xs[row0 ..] into xsl first of all
    // its loads (so that every later wait covers it); rows past M read zero
    if (wave == 0)
        load_to_lds16_so(S3D8_LDS_OFFSET(&xsl[0]), lane < 4 * R ? 16u * (uint32_t)lane : kOOB, 0u,
                         rsrc_words(xs + row0, 4u * (uint32_t)(M - row0)));

    const v4i rx = rsrc_words(xq, (uint32_t)M * (uint32_t)K);
    const v4i rw = rsrc_words(tiled, (uint32_t)tiles16 * (uint32_t)KB * 1024u);

    // activation loads of this wave: load index L = wave (+ 8 for w + 8 < R)
    // moves rows 16 L .. 16 L + 15; lane l takes row 16 L + l % 16, chunk
    // l / 16, stored at 16 l of the load's KiB
    uint32_t aoff[2], atail[2];
    const int ktail = K - 64 * (KB - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * (wave + 8 * j) + (lane & 15);
        const int chunk = lane >> 4;
        aoff[j] = wave + 8 * j < R && row0 + row < M ? (uint32_t)(row0 + row) * (uint32_t)K + 16u * chunk : kOOB;
        atail[j] = 16 * chunk < ktail ? aoff[j] : kOOB;
    }
    // weight load: the wave's own fragment, 16 bytes per lane in place
    const uint32_t woff = frag < tiles16 ? (uint32_t)frag * (uint32_t)KB * 1024u + 16u * lane : kOOB;
    const uint32_t abase = S3D8_LDS_OFFSET(&abuf[0][0]), wbase = S3D8_LDS_OFFSET(&wbuf[0][0]);
    // blocks past the end re-read the last block into a slot never read, so
    // that every wait counts the same
    auto issue = [&](int kb, int slot) {
        const int kbc = kb < KB ? kb : KB - 1;
        const bool tail = kbc >= KB - 1;
        const uint32_t ab = abase + (uint32_t)(BM * 64) * slot;
        load_to_lds16_so(ab + 1024u * wave, tail ? atail[0] : aoff[0], 64u * (uint32_t)kbc, rx);
        if (wave + 8 < R) load_to_lds16_so(ab + 1024u * (8 + wave), tail ? atail[1] : aoff[1], 64u * (uint32_t)kbc, rx);
        load_to_lds16_so(wbase + (uint32_t)(kGemmBF * 1024) * slot + 1024u * wave, woff, 1024u * (uint32_t)kbc, rw);
    };

    // A operand of row tile i: row 16 i + l % 16, chunk l / 16, at 16 l
    auto read_a = [&](int slot, int i) { return *reinterpret_cast<const v4i *>(&abuf[slot][1024 * i + 16 * lane]); };
    auto read_w = [&](int slot) { return *reinterpret_cast<const uint4 *>(&wbuf[slot][1024 * wave + 16 * lane]); };
    // decode of raw dword c (k = 16 g + 4 c .. + 3): four table lookups, then
    // the 4 x 3 byte transpose into dword c of the three B operands
    auto lookups = [&](const uint4 &w, int c, uint32_t (&q)[4]) {
        const char *tb = reinterpret_cast<const char *>(tab);
        const uint32_t dw = c == 0 ? w.x : c == 1 ? w.y : c == 2 ? w.z : w.w;
        q[0] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0400u));
        q[1] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0500u));
        q[2] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0600u));
        q[3] = *reinterpret_cast<const uint32_t *>(tb + __builtin_amdgcn_perm(dw, lane_off, 0x0C0C0700u));
    };
    auto transpose = [&](const uint32_t (&q)[4], v4i (&b)[3], int c) {
        const uint32_t p01 = __builtin_amdgcn_perm(q[1], q[0], 0x05010400u);
        const uint32_t p23 = __builtin_amdgcn_perm(q[3], q[2], 0x05010400u);
        const uint32_t s01 = __builtin_amdgcn_perm(q[1], q[0], 0x0C0C0602u);
        const uint32_t s23 = __builtin_amdgcn_perm(q[3], q[2], 0x0C0C0602u);
        b[0][c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x05040100u);
        b[1][c] = (int32_t)__builtin_amdgcn_perm(p23, p01, 0x07060302u);
        b[2][c] = (int32_t)__builtin_amdgcn_perm(s23, s01, 0x05040100u);
    };

    // prologue as gemm_kernel's: blocks 0 and 1 in flight, the table, block 0
    // waited for, then blocks 2 and 3.  3D8: the 768-byte table as one word
    // per thread, loaded before the blocks and waited for (oldest load, four
    // younger ones in flight for every wave) in the same branch, so that its
    // register is neither copied nor reused while the load is in flight;
    // S3D8: the 96-byte table through the scalar cache, no vector wait.
    if (f3d8) {
        uint32_t c3;
        const uint32_t off = tid < kTableWords3D8 ? 4u * (uint32_t)tid : kOOB;
        asm volatile("buffer_load_dword %0, %1, %2, 0 offen" : "=v"(c3) : "v"(off), "s"(rsrc_words(centroids, 768u))
                     : "memory");
        issue(0, 0);
        issue(1, 1);
        asm volatile("s_waitcnt vmcnt(4)" : "+v"(c3)::"memory");
        if (tid < kTableWords3D8) clw[tid] = c3;
    } else {
        uint32_t cw[24];
#pragma unroll
        for (int i = 0; i < 24; ++i) cw[i] = centroids[i];
        issue(0, 0);
        issue(1, 1);
        if (tid == 0)
#pragma unroll
            for (int i = 0; i < 6; ++i)
                reinterpret_cast<uint4 *>(clw)[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
    }
    __syncthreads();
    {
        // thread t computes entry t / 2 once and writes its copies
        // 32 (t % 2) .. + 31 as eight 16-byte stores, in an order rotated by
        // t / 2 so that the eight lanes of a store cycle hit distinct banks
        static_assert(kW8Threads == 2 * kTabEntries && kTabCopies == 64, "two threads per table entry");
        const uint8_t *cl = reinterpret_cast<const uint8_t *>(clw);
        const uint32_t b = (uint32_t)tid >> 1;
        const uint32_t v = f3d8 ? row_3d8(b, cl) : signed_triple(b, cl);
        uint4 *row = reinterpret_cast<uint4 *>(tab) + 16 * b + 8 * (tid & 1);
#pragma unroll
        for (int k = 0; k < 8; ++k) row[(k + (tid >> 1)) & 7] = make_uint4(v, v, v, v);
    }
    static_assert(kGemmAhead == 4, "the waits below assume four blocks in flight");
    w8_wait<R, 1, false>(wave);  // this wave's block 0 is in LDS
    __syncthreads();          // everyone's block 0, and the table
    issue(2, 2);
    issue(3, 3);

    v4i acc[R][3];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int d = 0; d < 3; ++d) acc[i][d] = v4i{0, 0, 0, 0};

    // operands of block 0: A row tiles 0 and 1 (the rest are read during the
    // block), B decoded
    v4i an[2] = {read_a(0, 0), read_a(0, 1)};
    v4i b0[3], b1[3];
    {
        const uint4 w0 = read_w(0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t q[4];
            lookups(w0, c, q);
            transpose(q, b0, c);
        }
    }

    // block kb (slot `slot`): wait until blocks <= kb + 1 are in LDS for
    // every wave, refill the slot of block kb - 1 with block kb + 4, then R
    // groups of three MFMAs (row tile i x the three B operands).  Group i
    // reads A row tile i + 2 (of block kb + 1 for the last two groups); the
    // raw weights of block kb + 1 come in group 0, the lookups of raw dword c
    // in group LK0 + c and its transpose in group R - 4 + c (LK0 = 2 at
    // R = 10, 1 at R = 8: three groups between them either way).
    auto block = [&](v4i (&anx)[2], const v4i (&bc)[3], v4i (&bnx)[3], int kb, int slot) {
        w8_wait<R, 2, true>(wave);
        const int next = slot == kGemmSlots - 1 ? 0 : slot + 1;
        const int prev = slot == 0 ? kGemmSlots - 1 : slot - 1;
        issue(kb + kGemmAhead, prev);
        v4i a[R];
        a[0] = anx[0];
        a[1] = anx[1];
        uint4 wn;
        uint32_t q[4][4];
#pragma unroll
        for (int i = 0; i < R; ++i) {
#pragma unroll
            for (int d = 0; d < 3; ++d) acc[i][d] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bc[d], acc[i][d], 0, 0, 0);
            if (i == 0) wn = read_w(next);
            if (i + 2 < R)
                a[i + 2] = read_a(slot, i + 2);
            else
                anx[i + 2 - R] = read_a(next, i + 2 - R);
            constexpr int LK0 = R >= 10 ? 2 : 1;
            if (i >= LK0 && i < LK0 + 4) lookups(wn, i - LK0, q[i - LK0]);
            if (i >= R - 4) transpose(q[i - (R - 4)], bnx, i - (R - 4));
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // a share of the VALU
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // and of the LDS reads
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int kb = 0, slot = 0;
#pragma unroll 1
    for (; kb + 1 < KB; kb += 2) {
        block(an, b0, b1, kb, slot);
        slot = slot == kGemmSlots - 1 ? 0 : slot + 1;
        block(an, b1, b0, kb + 1, slot);
        slot = slot == kGemmSlots - 1 ? 0 : slot + 1;
    }
    if (kb < KB) block(an, b0, b1, kb, slot);

    // epilogue: lane (t, g) holds channels 3 (16 frag + t) + d (their scales
    // loaded before the loads of blocks past the end are drained)
    const int ch0 = 3 * (16 * frag + (lane & 15));
    float sc[3];
    uint32_t coff[3];
    const auto rsc = make_rsrc(scales, (uint32_t)N * 2u);
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const bool ok = ch0 + d < N;
        coff[d] = ok ? 4u * (uint32_t)(ch0 + d) : kOOB;
        sc[d] = bf16_to_f32(bload2(rsc, ok ? 2u * (uint32_t)(ch0 + d) : kOOB));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads of blocks past the end
    store_rows16<R, kAcc, kBF>(acc, xsl, M, N, row0, lane >> 4, sc, coff, y, acc_out);
}

// --------------------------------------------------------------- matrix-core rate probe

// A measurement utility, not part of the method: the INT8 matrix-core rate
// this part sustains, against which the fused GEMM is read.  Each wave runs
// `iters` rounds of four independent v_mfma_i32_32x32x32_i8 (one chain per
// accumulator, so an instruction never waits for the previous one's result)
// on register operands whose bytes all equal v; nothing else is in the loop.
// Every accumulator element gains 32 v^2 per round, so lane t of workgroup w
// stores 4 x 16 x 32 v^2 iters = 2048 v^2 iters (mod 2^32).
constexpr int kRateThreads = 256;
__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(int iters, int v, int32_t *__restrict__ out) {
    const int32_t w = (int32_t)(((uint32_t)v & 0xFFu) * 0x01010101u);
    const v4i a = {w, w, w, w};
    v16i acc[4] = {};
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[c], 0, 0, 0);
    }
    uint32_t sum = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += (uint32_t)acc[c][r];
    out[(int64_t)blockIdx.x * kRateThreads + threadIdx.x] = (int32_t)sum;
}

// --------------------------------------------------------------- HBM read probe

// A measurement utility, not part of the method: how fast the chip streams a
// buffer of a given size out of memory, the ceiling a memory-bound kernel of
// that size is read against (the decode GEMV reads 19.6 MB per call, a size
// at which start-up and drain weigh as much as the bandwidth).  Workgroup w of
// G reads the 16-byte chunks c with (c / 256) % G == w, four loads in flight
// per thread, and stores the XOR of every 32-bit word it read into out[w], so
// that no load can be dropped.
constexpr int kReadThreads = 256;
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const uint4 *__restrict__ p, int64_t nchunks,
                                                                uint32_t *__restrict__ out) {
    __shared__ uint32_t part[kReadThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t c = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t v = 0;
    for (; c + 3 * stride < nchunks; c += 4 * stride) {
        const uint4 a = p[c], b = p[c + stride], d = p[c + 2 * stride], e = p[c + 3 * stride];
        v ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ d.x ^ d.y ^ d.z ^ d.w ^ e.x ^ e.y ^ e.z ^ e.w;
    }
    for (; c < nchunks; c += stride) {
        const uint4 a = p[c];
        v ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int m = 32; m >= 1; m >>= 1) v ^= (uint32_t)__shfl_xor((int)v, m, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// --------------------------------------------------------------- dequant

// Standalone S3D8 -> channel-INT8 decode (the blog's dequantisation kernel).
// Persistent workgroups build the table once and stride over 16-byte chunks.
constexpr int kDequantThreads = 512;

__global__ __launch_bounds__(kDequantThreads) void dequant_kernel(
    const uint8_t *__restrict__ packed, const uint32_t *__restrict__ centroids, int K, int N,
    int64_t nchunks, int8_t *__restrict__ w, int f3d8) {
    __shared__ uint32_t tab[kTabWords];
    __shared__ uint32_t clw[kTableWords3D8];
    stage_and_build_table<kDequantThreads>(tab, clw, centroids, f3d8 != 0);
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

// --------------------------------------------------------------- unfused prefill

// The pages' strategy for many token rows: decode the matrix once per call to
// channel-INT8 in HBM, then run a plain INT8 GEMM.  Each weight byte is then
// decoded once per call, instead of once per 128-row tile of the fused GEMM.

// Tiled S3D8 -> channel-INT8 in the B-operand order of the INT8 GEMM: the
// decoded matrix is cut into fragments of 32 channels x 64 input columns,
// fragment (channel tile ct, block b) at byte (ct * KB + b) * 2048; inside
// it, 16-byte unit (kh * 64 + c + 32 h) holds channel 32 ct + c at columns
// 64 b + 32 kh + 16 h .. + 15 (the B operand of v_mfma_i32_32x32x32_i8 for
// lane c + 32 h, k-half kh).  Channels past 3T and columns past K are not
// written: they only meet zero activations or outputs that are never
// stored.  Thread c handles 16-byte chunk c of the tiled matrix: fragment
// c / 64, lane c % 64 = triple n + 16 g of the fragment, columns 16 g ..
// (grid = gridDim.x, passed so that it arrives preloaded with the other
// arguments instead of through a load from the argument segment)
__global__ __launch_bounds__(kDequantThreads) void dequant_tiled_kernel(
    const uint8_t *__restrict__ tiled, const uint32_t *__restrict__ centroids, int K, int T, int KB, int grid,
    int64_t nchunks, int8_t *__restrict__ w8, int f3d8) {
    __shared__ uint32_t tab[kTabWords];
    __shared__ uint32_t clw[kTableWords3D8];
    stage_and_build_table<kDequantThreads>(tab, clw, centroids, f3d8 != 0);
    const uint32_t lane_off = (uint32_t)(threadIdx.x & 63) << 2;
    for (int64_t c = (int64_t)blockIdx.x * kDequantThreads + threadIdx.x; c < nchunks;
         c += (int64_t)grid * kDequantThreads) {
        const int64_t frag = c >> 6;
        const int l = (int)(c & 63);
        const int64_t tile = frag / KB;
        const int blk = (int)(frag - tile * KB);
        const int64_t t = tile * 16 + (l & 15);
        const int g = l >> 4;
        if (t >= T || blk * 64 + g * 16 >= K) continue;
        const uint4 p = *reinterpret_cast<const uint4 *>(tiled + c * 16);
        v4i o[3];
        decode16(p, lane_off, tab, o[0], o[1], o[2]);
        const int kh = g >> 1, h = g & 1;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const int64_t ch = 3 * t + d;
            const int64_t ct = ch >> 5;
            const int cc = (int)(ch & 31);
            *reinterpret_cast<v4i *>(w8 + (ct * KB + blk) * 2048 + kh * 1024 + (cc + 32 * h) * 16) = o[d];
        }
    }
}

// INT8 x INT8 GEMM on v_mfma_i32_32x32x32_i8: y = (xs * acc) * alpha.
// Workgroup tile 32 RT token rows x 384 channels, 4 waves side by side
// along N, wave tile 32 RT x 96 (RT x 3 accumulators of 32 x 32).  Per
// 64-column block the activation tile (XOR-swizzled as in the fused GEMM)
// and the weight fragments (already in B-operand lane order, 1 KiB
// contiguous per load) are copied into an LDS ring of kSlots slots,
// kSlots - 1 blocks ahead (five slots at RT = 4, four at RT = 5, whose
// larger activation tile leaves room for no more); the MFMAs read both
// operands from LDS.
template <int RT, bool kAcc, bool kBF>
__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t *__restrict__ xq, const int8_t *__restrict__ w8,
                                                      int M, int K, int N, int NP, int nbm, int nbn,
                                                      const float *__restrict__ xs,
                                                      const uint16_t *__restrict__ scales, void *__restrict__ y,
                                                      int32_t *__restrict__ acc_out) {
    static_assert(RT == 4 || RT == 5, "4 or 5 row tiles per wave");
    constexpr int BM = 32 * RT;
    constexpr int kSlots = RT == 4 ? 5 : 4;
    constexpr int kAhead = kSlots - 1;
    constexpr int NA = (2 * RT + 3) / 4;  // activation loads per wave and block
    constexpr int ND = NA + 6;            // all loads per wave and block
    // activation slots, then (only when 4 NA > 2 RT) 1 KiB that loads past
    // the tile fill
    constexpr int kSpill = (4 * NA > 2 * RT) ? 1024 : 0;
    __shared__ __attribute__((aligned(16))) int8_t abuf[kSlots * BM * 64 + kSpill];
    __shared__ __attribute__((aligned(16))) int8_t bbuf[kSlots][4 * 6 * 1024];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, h = lane >> 5;
    const int KB = (K + 63) >> 6;

    int bm, bn;
    if (!gemm_tile(nbm, nbn, bm, bn)) return;
    const int row0 = bm * BM;
    const int ch0 = bn * 384 + wave * 96;  // first channel of this wave

    const v4i rx = rsrc_words(xq, (uint32_t)M * (uint32_t)K);
    const v4i rw = rsrc_words(w8, (uint32_t)((NP + 31) / 32) * (uint32_t)KB * 2048u);

    // activation copy: wave w moves 16-byte units u = 64 (NA w + j) + lane
    // of the BM x 64 tile (row u / 4, chunk (u % 4) ^ ((row / 4) % 4));
    // units past the tile (4 NA > 2 RT) read nothing into `spill`
    uint32_t aoff[NA];
    int acol[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int u = 64 * (NA * wave + j) + lane;
        const int row = u >> 2;
        const int chunk = (u & 3) ^ ((row >> 2) & 3);
        aoff[j] = row < BM && row0 + row < M ? (uint32_t)(row0 + row) * (uint32_t)K + 16u * chunk : kOOB;
        acol[j] = 16 * chunk;
    }
    // B operand (column tile ct, k-half kh) of lane L: 16 bytes at unit
    // kh * 64 + L of fragment (channel tile ch0 / 32 + ct, block kb)
    uint32_t boff[3];
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
        const int ctile = ch0 / 32 + ct;
        boff[ct] = 32 * ctile < NP ? (uint32_t)ctile * (uint32_t)KB * 2048u + 16u * lane : kOOB;
    }
    const uint32_t abase = S3D8_LDS_OFFSET(&abuf[0]), bbase = S3D8_LDS_OFFSET(&bbuf[0][0]);
    const uint32_t sbase = abase + (uint32_t)(kSlots * BM * 64);
    // activation chunks at or past K in the last block read zeros (the
    // workspace bytes there are not written by the decode)
    const int ktail = K - 64 * (KB - 1);
    uint32_t atail[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) atail[j] = acol[j] < ktail ? aoff[j] : kOOB;
    // ND loads per wave and block, also for the blocks past the end, so that
    // every wait below counts the same: those re-read the last block into a
    // slot that is never read.  The block's byte offset goes in the scalar
    // offset of the loads; the per-lane offsets are block 0's.
    auto issue = [&](int kb, int slot) {
        const int kbc = kb < KB ? kb : KB - 1;
        const bool tail = kb >= KB - 1;
#pragma unroll
        for (int j = 0; j < NA; ++j)
            load_to_lds16_so(NA * wave + j < 2 * RT ? abase + (uint32_t)(BM * 64) * slot + 1024u * (NA * wave + j)
                                                    : sbase,
                             tail ? atail[j] : aoff[j], 64u * (uint32_t)kbc, rx);
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                load_to_lds16_so(bbase + (uint32_t)(4 * 6 * 1024) * slot + 6144u * wave + 1024u * (2 * ct + kh),
                                 boff[ct] + 1024u * kh, 2048u * (uint32_t)kbc, rw);
    };

    const int swz = (c32 >> 2) & 3;
    const int ard0 = c32 * 64 + 16 * (h ^ swz), ard1 = c32 * 64 + 16 * ((h ^ swz) ^ 2);

#pragma unroll
    for (int sl = 0; sl < kAhead; ++sl) issue(sl, sl);

    v16i acc[RT][3];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int d = 0; d < 3; ++d) acc[i][d] = v16i{};

    // operands of one block: A for RT row tiles x 2 k-halves, B for 3
    // column tiles x 2 k-halves (2 RT + 6 times 16 bytes per lane)
    struct Ops {
        v4i a[RT][2], b[3][2];
    };
    auto read_ops = [&](Ops &o, int slot) {
        const int8_t *ab = abuf + slot * (BM * 64);
        const int8_t *bb = bbuf[slot] + 6144 * wave + 16 * lane;
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            o.a[i][0] = *reinterpret_cast<const v4i *>(ab + 2048 * i + ard0);
            o.a[i][1] = *reinterpret_cast<const v4i *>(ab + 2048 * i + ard1);
        }
#pragma unroll
        for (int ct = 0; ct < 3; ++ct)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) o.b[ct][kh] = *reinterpret_cast<const v4i *>(bb + 1024 * (2 * ct + kh));
    };
    auto mfmas = [&](const Ops &o) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int ct = 0; ct < 3; ++ct)
                    acc[i][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.a[i][kh], o.b[ct][kh], acc[i][ct], 0, 0, 0);
    };

    // block kb (operands already in registers `cur`): wait until blocks <=
    // kb + 1 are in LDS for every wave (the loads of blocks kb + 2 ..
    // kb + kAhead - 1 may still fly), refill the slot of block kb - 1 with
    // block kb + kAhead, read block kb + 1's operands into `nxt` while the
    // MFMAs of block kb run
    auto block = [&](const Ops &cur, Ops &nxt, int kb, int slot) {
        wait_vmcnt_barrier<(kAhead - 2) * ND>();
        issue(kb + kAhead, slot == 0 ? kSlots - 1 : slot - 1);
        read_ops(nxt, slot == kSlots - 1 ? 0 : slot + 1);
        mfmas(cur);
        // interleave the 2 RT + 6 operand reads of the next block with the
        // first MFMAs of this one, so that their LDS latency hides behind them
#pragma unroll
        for (int q = 0; q < 2 * RT + 6; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6 * RT - (2 * RT + 6), 0);
    };

    Ops o0, o1;
    wait_vmcnt_barrier<(kAhead - 1) * ND>();  // block 0 in LDS for every wave
    read_ops(o0, 0);
    int kb = 0, slot = 0;
#pragma unroll 1
    for (; kb + 1 < KB; kb += 2) {
        block(o0, o1, kb, slot);
        slot = slot == kSlots - 1 ? 0 : slot + 1;
        block(o1, o0, kb + 1, slot);
        slot = slot == kSlots - 1 ? 0 : slot + 1;
    }
    if (kb < KB) block(o0, o1, kb, slot);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // epilogue: lane (c, h) holds column c of each column tile for rows
    // 32 i + 8 (v / 4) + 4 h + v % 4 (store_tile_rows)
    float sc[3];
    uint32_t coff[3];
    const auto rsc = make_rsrc(scales, (uint32_t)N * 2u);
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
        const int ch = ch0 + 32 * ct + c32;
        coff[ct] = ch < N ? 4u * (uint32_t)ch : kOOB;
        sc[ct] = bf16_to_f32(bload2(rsc, ch < N ? 2u * (uint32_t)ch : kOOB));
    }
    store_tile_rows<false, kAcc, RT, kBF, true>(acc, xs, M, N, row0, h, sc, coff, y, acc_out);
}

// --------------------------------------------------------------- encode on the device

// The frozen-centroid quantiser of the paper (Sec. 3.4, "Quantization", the
// QAT-phase Q(.)) on the GPU, with the same arithmetic as the host encoder:
// alpha_i = bf16_rne(fp32(max_j |W_ij|) / 127.0f); W'_{t,j,d} = |W_{3t+d,j}|
// / alpha in fp64 (0 for padded channels and zero scales); q = the first
// centroid row with the smallest squared distance (components summed in
// order 0, 1, 2, no fused multiply-add); S_d = W < 0; byte per the blog's
// "Bit layout".

// One workgroup per (padded) channel row: the absmax and its bf16 scale.
constexpr int kScaleThreads = 256;
__global__ __launch_bounds__(kScaleThreads) void channel_scale_kernel(const float *__restrict__ W, int N, int K,
                                                                      uint16_t *__restrict__ alpha) {
    __shared__ float red[kScaleThreads / 64];
    const int i = blockIdx.x;
    float a = 0.0f;
    if (i < N)
        for (int j = threadIdx.x; j < K; j += kScaleThreads) a = fmaxf(a, fabsf(W[(int64_t)i * K + j]));
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
#pragma unroll
        for (int w = 1; w < kScaleThreads / 64; ++w) m = fmaxf(m, red[w]);
        const float s = m / 127.0f;  // IEEE division
        const uint32_t u = __float_as_uint(s);
        // round to nearest even on the upper 16 bits (s is finite and >= 0)
        alpha[i] = f32_to_bf16_rne(__uint_as_float(u));
    }
}

// One thread per packed byte (triple t, column j).
constexpr int kEncodeThreads = 256;
__global__ __launch_bounds__(kEncodeThreads) void encode_kernel(const float *__restrict__ W, int N, int K, int T,
                                                                const uint16_t *__restrict__ alpha,
                                                                const uint8_t *__restrict__ centroids,
                                                                uint8_t *__restrict__ packed) {
    __shared__ double cent[96];
    if (threadIdx.x < 96) cent[threadIdx.x] = (double)centroids[threadIdx.x];
    __syncthreads();
    const int64_t p = (int64_t)blockIdx.x * kEncodeThreads + threadIdx.x;
    if (p >= (int64_t)T * K) return;
    const int t = (int)(p / K), j = (int)(p - (int64_t)t * K);
    double x[3];
    uint32_t sg[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int i = 3 * t + d;
        x[d] = 0.0;
        sg[d] = 0;
        if (i < N) {
            const float w = W[(int64_t)i * K + j];
            sg[d] = w < 0.0f ? 1u : 0u;
            const double a = (double)bf16_to_f32(alpha[i]);
            if (a != 0.0) x[d] = fabs((double)w) / a;
        }
    }
    double best = 0.0;
    uint32_t q = 0;
#pragma unroll 4
    for (int l = 0; l < 32; ++l) {
        const double e0 = cent[3 * l] - x[0], e1 = cent[3 * l + 1] - x[1], e2 = cent[3 * l + 2] - x[2];
        const double dd = e0 * e0 + e1 * e1 + e2 * e2;
        if (l == 0 || dd < best) {
            best = dd;
            q = (uint32_t)l;
        }
    }
    packed[p] = (uint8_t)(sg[0] | (q << 1) | (sg[1] << 6) | ((sg[2] ^ sg[0]) << 7));
}

// --------------------------------------------------------------- host glue

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t lim_int() { return (int64_t(1) << 31) - 1; }

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

// Launch shapes of the GEMV: waves per workgroup, blocks per load batch, and
// resident workgroups per CU (two 64 KiB tables fit in LDS; 16-wave groups
// are limited to one per CU by registers).
struct GemvConfig {
    int waves, unroll, wgs_per_cu;
};
constexpr GemvConfig kGemvDefault = {16, 2, 1};

struct GemvArgs {
    const int8_t *xq;
    const float *xs;
    const float *xf;
    int8_t *xq_out;
    float *xs_out;
    int M, K, N, T;
    const uint8_t *tiled;
    const uint32_t *centroids;
    const uint16_t *scales;
    void *y;
    int32_t *acc_out;
    int f3d8, obf;  // 3D8 table; bf16 output
};

// kbw = 64-column blocks per wave; the fused prologue needs M * kbw <= 16
// (four float4 of x per lane).
int gemv_kbw(int K, int waves) { return ((K + 63) / 64 + waves - 1) / waves; }
bool gemv_fusable(int M, int K, GemvConfig cfg) { return M <= kFusedMaxRows && M * gemv_kbw(K, cfg.waves) <= 16; }

// Returns false (and launches nothing) if a fused launch is asked for a shape
// the fused prologue cannot hold.
bool launch_gemv(GemvConfig cfg, bool fused, const GemvArgs &a, int cus, hipStream_t stream) {
    if (a.M > 16 || (fused && !gemv_fusable(a.M, a.K, cfg))) return false;
    const int kbw = gemv_kbw(a.K, cfg.waves);
    const int64_t tiles = (a.T + 15) / 16;
    const int64_t cap = (int64_t)cus * cfg.wgs_per_cu;
    const int grid = (int)(tiles < cap ? tiles : cap);
    const size_t xw_bytes = fused ? (size_t)cfg.waves * a.M * 64 * kbw + 16 : 0;
#define S3D8_GEMV_CASE(W, U, F)                                                                          \
    if (cfg.waves == W && cfg.unroll == U && fused == F) {                                               \
        hipLaunchKernelGGL((gemv_kernel<W, U, F>), dim3(grid), dim3(W * 64), xw_bytes, stream, a.xq, a.xs, \
                           a.xf, a.xq_out, a.xs_out, a.M, a.K, a.N, a.T, a.tiled, a.centroids, a.scales,  \
                           a.y, a.acc_out, kbw, a.f3d8, a.obf);                                          \
        return true;                                                                                     \
    }
    S3D8_GEMV_CASE(16, 2, false)
    S3D8_GEMV_CASE(16, 2, true)
    S3D8_GEMV_CASE(8, 2, false)
    S3D8_GEMV_CASE(8, 2, true)
#undef S3D8_GEMV_CASE
    return false;
}

int64_t tiled_bytes(int64_t N, int64_t K) { return ((N + 2) / 3 + 15) / 16 * ((K + 63) / 64) * 1024; }

// The streaming fused GEMV takes M <= 4 rows whose per-wave activation slice
// fits four float4 per lane, and at most kStreamMaxTiles tiles per workgroup
// (one workgroup per CU).  Returns false (launching nothing) otherwise.
// Workgroups for a batch of stream-GEMV matrices: one per CU in all, shared
// out so that the largest per-workgroup work (tiles x K) is smallest; each
// matrix gets at least one workgroup and at most one per tile.  Returns
// false if some matrix would need more than kStreamMaxTiles tiles on one
// workgroup.
bool stream_split(int count, const int64_t *tiles, const int64_t *K, int cus, int *groups) {
    int used = 0;
    for (int p = 0; p < count; ++p) {
        groups[p] = 1;
        ++used;
    }
    auto load = [&](int p, int g) { return (tiles[p] + g - 1) / g * K[p]; };
    while (used < cus) {
        int best = -1;
        for (int p = 0; p < count; ++p)
            if (groups[p] < tiles[p] && (best < 0 || load(p, groups[p]) > load(best, groups[best]))) best = p;
        if (best < 0) break;
        ++groups[best];
        ++used;
    }
    for (int p = 0; p < count; ++p)
        if ((tiles[p] + groups[p] - 1) / groups[p] > kStreamMaxTiles) return false;
    return true;
}

// One launch of gemv_stream_kernel over `count` matrices that share M; false
// (nothing launched) if a matrix does not fit the kernel.  A single matrix
// may be 3D8 (f3d8) and write bf16 (obf); a batch is S3D8 with fp32 output.
bool launch_gemv_stream_batch(int count, const s3d8_forward_item *items, int cus, hipStream_t stream,
                              bool f3d8 = false, int obf = 0) {
    if (count < 1 || count > kStreamBatch) return false;
    if (count > 1 && (f3d8 || obf)) return false;
    const int64_t M = items[0].M;
    if (M < 1 || M > kFusedMaxRows) return false;
    // 16 waves (8 were measured slower at K = 4096, with the dense product
    // and again with the sparse one, 8.3 against 7.3 us: the shorter
    // prologue is outweighed by half as many waves hiding the lookups' LDS
    // latency; 8 waves also take K = 14336 out of the M * kbw <= 16 range)
    constexpr int W = 16;
    int64_t tiles[kStreamBatch], Ks[kStreamBatch];
    for (int p = 0; p < count; ++p) {
        if (items[p].M != M || M * gemv_kbw((int)items[p].K, W) > 16) return false;
        tiles[p] = ((items[p].N + 2) / 3 + 15) / 16;
        Ks[p] = items[p].K;
    }
    int groups[kStreamBatch];
    if (!stream_split(count, tiles, Ks, cus, groups)) return false;
    StreamBatch B;
    int wg = 0;
    for (int p = 0; p < kStreamBatch; ++p) {
        B.wg0[p] = p < count ? wg : INT32_MAX;
        if (p >= count) {
            B.p[p] = StreamProb{};
            continue;
        }
        const s3d8_forward_item &it = items[p];
        B.p[p] = StreamProb{it.x, it.tiled, it.centroids, it.scales_bf16, it.y, it.acc_out, it.xq, it.xs,
                            (int)it.K, (int)it.N, (int)((it.N + 2) / 3), gemv_kbw((int)it.K, W),
                            (int)(tiles[p] / groups[p]), (int)(tiles[p] % groups[p])};
        wg += groups[p];
    }
    for (int p = count; p <= kStreamBatch; ++p) B.wg0[p] = INT32_MAX;
    B.wg0[count] = wg;  // end of the last matrix
    // float4 of activations per lane: ceil(M * kbw / 4) for the widest K
    int NF = 1;
    for (int p = 0; p < count; ++p) NF = std::max(NF, (int)((M * B.p[p].kbw + 3) / 4));
    typedef void (*Single)(const float *, const uint8_t *, const uint8_t *, const uint16_t *, int, int, int, int, int,
                           void *, int32_t *, int8_t *, float *, int);
    typedef void (*Batched)(StreamBatch);
#define S3D8_ROW(m, f) {gemv_stream_kernel<m, W, 1, f>, gemv_stream_kernel<m, W, 2, f>, \
                         gemv_stream_kernel<m, W, 3, f>, gemv_stream_kernel<m, W, 4, f>}
    static const Single single[2][4][4] = {
        {S3D8_ROW(1, false), S3D8_ROW(2, false), S3D8_ROW(3, false), S3D8_ROW(4, false)},
        {S3D8_ROW(1, true), S3D8_ROW(2, true), S3D8_ROW(3, true), S3D8_ROW(4, true)}};
#undef S3D8_ROW
#define S3D8_ROW(m) {gemv_stream_batch_kernel<m, W, 1>, gemv_stream_batch_kernel<m, W, 2>, \
                      gemv_stream_batch_kernel<m, W, 3>, gemv_stream_batch_kernel<m, W, 4>}
    static const Batched batched[4][4] = {S3D8_ROW(1), S3D8_ROW(2), S3D8_ROW(3), S3D8_ROW(4)};
#undef S3D8_ROW
    if (count == 1) {
        const StreamProb &P = B.p[0];
        hipLaunchKernelGGL(single[f3d8 ? 1 : 0][M - 1][NF - 1], dim3((unsigned)wg), dim3(W * 64), 0, stream, P.xf,
                           P.tiled, P.centroids, P.scales, P.K, P.N, wg, P.ntw_q, P.ntw_r, (void *)P.y, P.acc_out,
                           P.xq_out, P.xs_out, obf);
        return true;
    }
    auto kern = batched[M - 1][NF - 1];
    hipLaunchKernelGGL(kern, dim3((unsigned)wg), dim3(W * 64), 0, stream, B);
    return true;
}

// The streaming GEMV on INT8 codes (gemv_codes_kernel) for 1 to 8 token
// rows: taken when every wave's codes fit its LDS slice (M * 64 * kbw <=
// 4096 bytes, kbw = ceil(ceil(K/64) / 16)) and no workgroup needs more than
// kCodesMaxTiles tiles (one workgroup per CU).  Returns false, launching
// nothing, otherwise.
bool launch_gemv_codes(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                       const void *table, bool f3d8, const uint16_t *scales, void *y, bool obf, int32_t *acc_out,
                       int cus, hipStream_t stream) {
    if (M < 1 || M > kCodesMaxRows) return false;
    const int64_t KB = (K + 63) / 64, kbw = (KB + 15) / 16;
    if (M * 64 * kbw > kCodesWaveBytes) return false;
    const int64_t tiles = ((N + 2) / 3 + 15) / 16;
    const int64_t grid = tiles < cus ? tiles : cus;
    if ((tiles + grid - 1) / grid > kCodesMaxTiles) return false;
    typedef void (*CodesFn)(const int8_t *, const float *, const uint8_t *, const uint8_t *, const uint16_t *, int,
                            int, int, int, int, void *, int32_t *, int);
    // 16-byte code loads per lane: M * 4 * kbw chunks over 64 lanes (1, 2 or 4)
    const int64_t ncl = (M * 4 * kbw + 63) / 64;
    const int cl = ncl <= 1 ? 0 : ncl <= 2 ? 1 : 2;
#define S3D8_CODES(m, f) {gemv_codes_kernel<m, 1, f>, gemv_codes_kernel<m, 2, f>, gemv_codes_kernel<m, 4, f>}
#define S3D8_CODES_ROWS(f) {S3D8_CODES(1, f), S3D8_CODES(2, f), S3D8_CODES(3, f), S3D8_CODES(4, f), \
                            S3D8_CODES(5, f), S3D8_CODES(6, f), S3D8_CODES(7, f), S3D8_CODES(8, f)}
    static const CodesFn fns[2][kCodesMaxRows][3] = {S3D8_CODES_ROWS(false), S3D8_CODES_ROWS(true)};
#undef S3D8_CODES_ROWS
#undef S3D8_CODES
    hipLaunchKernelGGL(fns[f3d8 ? 1 : 0][M - 1][cl], dim3((unsigned)grid), dim3(1024), 0, stream, xq, xs, tiled,
                       static_cast<const uint8_t *>(table), scales, (int)K, (int)N, (int)grid, (int)(tiles / grid),
                       (int)(tiles % grid), y, acc_out, (int)obf);
    return true;
}

bool launch_gemv_stream(const float *x, int8_t *xq, float *xs, int64_t M, int64_t K, int64_t N,
                        const uint8_t *tiled, const uint8_t *centroids, const uint16_t *scales, void *y,
                        int32_t *acc_out, int cus, hipStream_t stream, bool f3d8, int obf) {
    // (the item's y is only passed on: the kernel stores through it as bf16 when obf)
    const s3d8_forward_item it{x, M, K, N, tiled, tiled_bytes(N, K), centroids, scales, static_cast<float *>(y), xq, xs,
                               acc_out};
    return launch_gemv_stream_batch(1, &it, cus, stream, f3d8, obf);
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
    launch_quant_act(x, M, K, xq, xs, (hipStream_t)stream);
    return launch_status();
}

int64_t s3d8_tiled_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return -1;
    return tiled_bytes(N, K);
}

int32_t s3d8_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled, void *stream) {
    if (!packed || !tiled) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(1, K, N);
    if (rc) return rc;
    if (tiled_bytes(N, K) > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "tiled weights over 2^31 bytes");
    if (!aligned16(tiled)) return s3d8::fail(S3D8_ERR_ALIGN, "tiled must be 16-byte aligned");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const int64_t T = (N + 2) / 3;
    const int KB = (int)((K + 63) / 64);
    const int64_t nchunks = tiled_bytes(N, K) / 16;
    int64_t blocks = (nchunks + kTileThreads - 1) / kTileThreads;
    if (blocks > (int64_t)cus * 8) blocks = (int64_t)cus * 8;
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)blocks), dim3(kTileThreads), 0, (hipStream_t)stream, packed,
                       (int)K, (int)T, KB, nchunks, tiled);
    return launch_status();
}

namespace {
// Launch plan of the fused GEMM (M > 16).
//   rt      32-row tiles per wave (2, 4 or 5, gemm_rt);
//   splits  column-block ranges per tile (split-K), kbper blocks each;
//   ws_cnt_bytes, ws_part_bytes: the split-K workspace (two counters per
//           tile, padded to 256 bytes; `splits` partial-sum slots per tile).
struct GemmPlan {
    int rt, nbm, nbn, splits, kbper;
    int64_t grid, ws_cnt_bytes, ws_part_bytes;
};
constexpr int kMaxSplits = 16;
constexpr int64_t kClkBlockRT2 = 1250;  // clocks per 64-column block at 64-row tiles (measured)

GemmPlan gemm_plan_rt(int64_t M, int64_t K, int64_t N, int rt, int splits) {
    GemmPlan p{};
    const int64_t T = (N + 2) / 3;
    const int KB = (int)((K + 63) / 64);
    p.rt = rt;
    p.nbn = (int)(((T + 15) / 16 + kGemmBF - 1) / kGemmBF);
    p.nbm = (int)((M + 32 * rt - 1) / (32 * rt));
    const int s = splits < 1 ? 1 : splits > KB ? KB : splits;
    p.kbper = (KB + s - 1) / s;
    p.splits = (KB + p.kbper - 1) / p.kbper;  // every range non-empty
    const int64_t tiles = (int64_t)p.nbm * p.nbn;
    p.grid = (tiles * p.splits + kXcds - 1) / kXcds * kXcds;
    p.ws_cnt_bytes = p.splits > 1 ? (2 * 4 * tiles + 255) / 256 * 256 : 0;
    p.ws_part_bytes = p.splits > 1 ? tiles * p.splits * 4 * (int64_t)part_wave_bytes(rt) : 0;
    return p;
}

// Tile height: 64, 128 or 160 token rows (rt = 2, 4, 5: the four-wave
// kernel's 32-row tiles per wave; 128 and 160 rows run on the eight-wave
// kernel).  When the 64-row tiles all fit one round on the CUs, they are
// taken: the kernel then lasts one workgroup's time, which is least for the
// smallest tile (the vision down-projection, 104 tiles of 64 rows: 46.7 us
// against 51.2 us on 52 tiles of 128).  Otherwise the one with the least
// estimated time at one workgroup per CU: workgroup rounds x (64-column
// blocks x clocks per block + a fixed prologue and epilogue), with the
// clocks measured on this part (the eight-wave figures from timestamps
// inside the kernel: 1283 and 1612 clk per block, 12500 and 14000 fixed).
// Taller tiles reuse each decoded weight over more rows; shorter ones make
// more workgroups, which pays when the taller tiles leave CUs idle.
int gemm_rt(int64_t M, int64_t K, int64_t N, int cus) {
    const int64_t T = (N + 2) / 3;
    const int64_t nbn = ((T + 15) / 16 + kGemmBF - 1) / kGemmBF;
    const int64_t KB = (K + 63) / 64;
    if ((M + 63) / 64 * nbn <= cus) return 2;
    auto cost = [&](int rt, int64_t clk_block, int64_t clk_fixed) {
        const int64_t tiles = (M + 32 * rt - 1) / (32 * rt) * nbn;
        return (tiles + cus - 1) / cus * (KB * clk_block + clk_fixed);
    };
    const int64_t c2 = cost(2, kClkBlockRT2, 18000), c4 = cost(4, 1283, 12500), c5 = cost(5, 1612, 14000);
    return c5 < c4 && c5 < c2 ? 5 : c2 < c4 ? 2 : 4;
}

// The automatic split count.  A split into S ranges runs ceil(KB/S) blocks
// per workgroup and then a fixup whose cost grows with S: the last
// workgroup of a tile reads all S slots of partial sums.  Measured on the
// vision down-projection (80 blocks, 52 tiles of 128 rows): each slot costs
// about as much as 9 column blocks of the main loop (44.0 / 42.3 / 46.5 us
// at S = 2 / 3 / 4, against 57.1 us unsplit), so S minimises
// ceil(KB/S) + 9 S over the counts whose workgroups fit one round on the
// CUs (tiles x S <= CUs), at most 16.
constexpr int kSplitSlotBlocks = 9;
int gemm_auto_splits(int64_t M, int64_t K, int64_t N, int cus) {
    if (M <= 16) return 1;
    const GemmPlan p = gemm_plan_rt(M, K, N, gemm_rt(M, K, N, cus), 1);
    const int64_t tiles = (int64_t)p.nbm * p.nbn;
    const int64_t KB = (K + 63) / 64;
    int best = 1;
    int64_t best_cost = KB + kSplitSlotBlocks;
    for (int64_t s = 2; s <= kMaxSplits && s <= KB && tiles * s <= cus; ++s) {
        const int64_t cost = (KB + s - 1) / s + kSplitSlotBlocks * s;
        if (cost < best_cost) best = (int)s, best_cost = cost;
    }
    return best;
}

typedef void (*GemmFn)(const int8_t *, const uint8_t *, const uint32_t *, int, int, int, int, int, int, int, int, int,
                       const float *, const uint16_t *, void *, int32_t *, int32_t *, int32_t *, uint32_t);

// Enqueue the fused GEMM under plan p (workspace checked by the caller).
int launch_gemm(const GemmPlan &p, const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                const uint8_t *tiled, const uint32_t *table32, bool f3d8, const uint16_t *scales_bf16, void *y,
                bool obf, int32_t *acc_out, void *ws, hipStream_t stream) {
    if (p.grid > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "problem too large");
    const bool split = p.splits > 1;
    // 128- and 160-row tiles without split-K: the eight-wave kernel
    if ((p.rt == 4 || p.rt == 5) && !split) {
        typedef void (*W8Fn)(const int8_t *, const uint8_t *, const uint32_t *, int, int, int, int, int, int, int,
                             const float *, const uint16_t *, void *, int32_t *);
#define S3D8_W8(r)                                                                    \
    {{gemm_w8_kernel<r, false, false>, gemm_w8_kernel<r, false, true>},              \
     {gemm_w8_kernel<r, true, false>, gemm_w8_kernel<r, true, true>}}
        static const W8Fn w8[2][2][2] = {S3D8_W8(8), S3D8_W8(10)};
#undef S3D8_W8
        hipLaunchKernelGGL(w8[p.rt == 5][acc_out != nullptr][obf], dim3((unsigned)p.grid), dim3(kW8Threads), 0,
                           stream, xq, tiled, table32, (int)M, (int)K, (int)N, (int)((N + 2) / 3), p.nbm, p.nbn,
                           (int)f3d8, xs, scales_bf16, y, acc_out);
        return launch_status();
    }
    // the four-wave kernel: 64-row tiles, and every split-K launch
#define S3D8_GEMM_RT(rt, sk)                                                         \
    {{gemm_kernel<rt, false, false, sk>, gemm_kernel<rt, false, true, sk>},          \
     {gemm_kernel<rt, true, false, sk>, gemm_kernel<rt, true, true, sk>}}
    static const GemmFn fns[4][2][2] = {S3D8_GEMM_RT(2, false), S3D8_GEMM_RT(2, true), S3D8_GEMM_RT(4, true),
                                        S3D8_GEMM_RT(5, true)};
#undef S3D8_GEMM_RT
    int32_t *cnt = split ? static_cast<int32_t *>(ws) : nullptr;
    int32_t *part = split ? reinterpret_cast<int32_t *>(static_cast<char *>(ws) + p.ws_cnt_bytes) : nullptr;
    const int variant = split ? (p.rt == 2 ? 1 : p.rt == 4 ? 2 : 3) : 0;
    hipLaunchKernelGGL(fns[variant][acc_out != nullptr][obf], dim3((unsigned)p.grid),
                       dim3(256), 0, stream,
                       xq, tiled, table32, (int)M, (int)K, (int)N, (int)((N + 2) / 3), p.nbm, p.nbn, (int)f3d8,
                       p.splits, p.kbper, xs, scales_bf16, y, acc_out, cnt, part, (uint32_t)p.ws_part_bytes);
    return launch_status();
}

int check_linear_args(const void *tiled, int64_t tiled_size, const void *table, const uint16_t *scales,
                      const void *y, int64_t M, int64_t K, int64_t N) {
    if (!tiled || !table || !scales || !y) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(M, K, N);
    if (rc) return rc;
    if (tiled_bytes(N, K) > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "tiled weights over 2^31 bytes");
    if (tiled_size < tiled_bytes(N, K))
        return s3d8::fail(S3D8_ERR_INVALID_ARG,
                          "tiled_bytes below s3d8_tiled_bytes(N, K): pass the matrix in the tiled layout "
                          "(s3d8_tile), not the canonical packed bytes");
    if (!aligned16(tiled)) return s3d8::fail(S3D8_ERR_ALIGN, "tiled weights must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(table) & 3u)
        return s3d8::fail(S3D8_ERR_ALIGN, "the centroid table must be 4-byte aligned");
    return S3D8_OK;
}

int check_variant(int32_t format, int32_t out_type) {
    if (format != S3D8_FORMAT_S3D8 && format != S3D8_FORMAT_3D8)
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "unknown weight format");
    if (out_type != S3D8_OUT_F32 && out_type != S3D8_OUT_BF16)
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "unknown output type");
    return S3D8_OK;
}

int linear_impl(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                int64_t tiled_size, const void *table, bool f3d8, const uint16_t *scales_bf16, void *y, bool obf,
                int32_t *acc_out, void *stream) {
    if (!xq || !xs) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_linear_args(tiled, tiled_size, table, scales_bf16, y, M, K, N);
    if (rc) return rc;
    if (!aligned16(xq)) return s3d8::fail(S3D8_ERR_ALIGN, "xq must be 16-byte aligned");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const uint32_t *table32 = reinterpret_cast<const uint32_t *>(table);
    if (M > 16) {
        if (N > kGemmMaxN) return s3d8::fail(S3D8_ERR_SHAPE, "N over 3355442 is not supported for M > 16");
        const GemmPlan p = gemm_plan_rt(M, K, N, gemm_rt(M, K, N, cus), 1);
        return launch_gemm(p, xq, xs, M, K, N, tiled, table32, f3d8, scales_bf16, y, obf, acc_out, nullptr,
                           (hipStream_t)stream);
    }
    // up to 8 token rows: the streaming GEMV on the codes, when they fit it
    if (launch_gemv_codes(xq, xs, M, K, N, tiled, table, f3d8, scales_bf16, y, obf, acc_out, cus,
                          (hipStream_t)stream))
        return launch_status();
    // otherwise the token-row GEMV, up to 16 token rows per launch
    const size_t ysize = obf ? 2 : 4;
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int mrows = (int)(M - m0 < 16 ? M - m0 : 16);
        GemvArgs a{xq + m0 * K, xs + m0, nullptr, nullptr, nullptr, mrows, (int)K, (int)N, (int)((N + 2) / 3),
                   tiled, table32, scales_bf16, static_cast<char *>(y) + m0 * N * ysize,
                   acc_out ? acc_out + m0 * N : nullptr, (int)f3d8, (int)obf};
        if (!launch_gemv(kGemvDefault, false, a, cus, (hipStream_t)stream))
            return s3d8::fail(S3D8_ERR_INVALID_ARG, "no GEMV variant for this launch shape");
    }
    return launch_status();
}

int splitk_impl(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                int64_t tiled_size, const void *table, bool f3d8, const uint16_t *scales_bf16, void *y, bool obf,
                int32_t *acc_out, int32_t splits, void *ws, int64_t ws_bytes, void *stream) {
    if (splits < 0) return s3d8::fail(S3D8_ERR_INVALID_ARG, "splits must be 0 (automatic) or positive");
    if (M <= 16)  // the GEMV paths: no split, no workspace
        return linear_impl(xq, xs, M, K, N, tiled, tiled_size, table, f3d8, scales_bf16, y, obf, acc_out, stream);
    if (!xq || !xs) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_linear_args(tiled, tiled_size, table, scales_bf16, y, M, K, N);
    if (rc) return rc;
    if (!aligned16(xq)) return s3d8::fail(S3D8_ERR_ALIGN, "xq must be 16-byte aligned");
    if (N > kGemmMaxN) return s3d8::fail(S3D8_ERR_SHAPE, "N over 3355442 is not supported for M > 16");
    // the workspace against the documented size (the largest of the three
    // tile heights' needs), checked before the device for an explicit count
    auto check_ws = [&](int s) {
        const int64_t need = s3d8_splitk_workspace_bytes(M, K, N, s);
        if (need == 0) return (int)S3D8_OK;
        for (int rt : {2, 4, 5})
            if (gemm_plan_rt(M, K, N, rt, s).ws_part_bytes > 2147483647)
                return s3d8::fail(S3D8_ERR_SHAPE, "split-K partial sums over 2^31 bytes: use fewer splits");
        if (!ws) return s3d8::fail(S3D8_ERR_INVALID_ARG, "split-K needs a workspace");
        if (ws_bytes < need)
            return s3d8::fail(S3D8_ERR_INVALID_ARG, "workspace below s3d8_splitk_workspace_bytes(M, K, N, splits)");
        if (reinterpret_cast<uintptr_t>(ws) & 255u)
            return s3d8::fail(S3D8_ERR_ALIGN, "the split-K workspace must be 256-byte aligned");
        return (int)S3D8_OK;
    };
    if (splits > 0 && (rc = check_ws(splits))) return rc;
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const int s = splits == 0 ? gemm_auto_splits(M, K, N, cus) : splits;
    if (splits == 0 && (rc = check_ws(s))) return rc;
    const GemmPlan p = gemm_plan_rt(M, K, N, gemm_rt(M, K, N, cus), s);
    return launch_gemm(p, xq, xs, M, K, N, tiled, reinterpret_cast<const uint32_t *>(table), f3d8, scales_bf16, y, obf,
                       acc_out, ws, (hipStream_t)stream);
}

int forward_impl(const float *x, int64_t M, int64_t K, int64_t N, const uint8_t *tiled, int64_t tiled_size,
                 const void *table, bool f3d8, const uint16_t *scales_bf16, void *y, bool obf, int8_t *xq, float *xs,
                 int32_t *acc_out, void *stream) {
    if (!x || !xq || !xs) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_linear_args(tiled, tiled_size, table, scales_bf16, y, M, K, N);
    if (rc) return rc;
    if (!aligned16(x) || !aligned16(xq)) return s3d8::fail(S3D8_ERR_ALIGN, "x and xq must be 16-byte aligned");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const uint8_t *table8 = static_cast<const uint8_t *>(table);
    if (launch_gemv_stream(x, xq, xs, M, K, N, tiled, table8, scales_bf16, y, acc_out, cus, (hipStream_t)stream,
                           f3d8, (int)obf))
        return launch_status();
    if (gemv_fusable((int)M, (int)K, kGemvDefault)) {
        GemvArgs a{nullptr, nullptr, x, xq, xs, (int)M, (int)K, (int)N, (int)((N + 2) / 3), tiled,
                   reinterpret_cast<const uint32_t *>(table), scales_bf16, y, acc_out, (int)f3d8, (int)obf};
        if (!launch_gemv(kGemvDefault, true, a, cus, (hipStream_t)stream))
            return s3d8::fail(S3D8_ERR_INVALID_ARG, "no fused GEMV variant for this launch shape");
        return launch_status();
    }
    rc = s3d8_quant_act(x, M, K, xq, xs, stream);
    if (rc) return rc;
    return linear_impl(xq, xs, M, K, N, tiled, tiled_size, table, f3d8, scales_bf16, y, obf, acc_out, stream);
}
}  // namespace

int32_t s3d8_linear(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                    const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                    const uint16_t *scales_bf16, float *y, int32_t *acc_out, void *stream) {
    return linear_impl(xq, xs, M, K, N, tiled, tiled_bytes, centroids, false, scales_bf16, y, false, acc_out,
                       stream);
}

int32_t s3d8_linear_ex(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                       int64_t tiled_bytes, const void *table, int32_t format, const uint16_t *scales_bf16, void *y,
                       int32_t out_type, int32_t *acc_out, void *stream) {
    int rc = check_variant(format, out_type);
    if (rc) return rc;
    return linear_impl(xq, xs, M, K, N, tiled, tiled_bytes, table, format == S3D8_FORMAT_3D8, scales_bf16, y,
                       out_type == S3D8_OUT_BF16, acc_out, stream);
}

int32_t s3d8_splitk_auto(int64_t M, int64_t K, int64_t N, int32_t num_cus) {
    if (M <= 0 || K <= 0 || N <= 0 || num_cus < 1) return -1;
    return gemm_auto_splits(M, K, N, num_cus);
}

int64_t s3d8_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t splits) {
    if (M <= 0 || K <= 0 || N <= 0 || splits < 1) return -1;
    if (M <= 16) return 0;
    int64_t most = 0;
    for (int rt : {2, 4, 5}) {
        const GemmPlan p = gemm_plan_rt(M, K, N, rt, splits);
        most = std::max(most, p.ws_cnt_bytes + p.ws_part_bytes);
    }
    return most;
}

int32_t s3d8_linear_splitk(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                           int64_t tiled_bytes, const void *table, int32_t format, const uint16_t *scales_bf16,
                           void *y, int32_t out_type, int32_t *acc_out, int32_t splits, void *workspace,
                           int64_t workspace_bytes, void *stream) {
    int rc = check_variant(format, out_type);
    if (rc) return rc;
    return splitk_impl(xq, xs, M, K, N, tiled, tiled_bytes, table, format == S3D8_FORMAT_3D8, scales_bf16, y,
                       out_type == S3D8_OUT_BF16, acc_out, splits, workspace, workspace_bytes, stream);
}

int32_t s3d8_forward(const float *x, int64_t M, int64_t K, int64_t N, const uint8_t *tiled, int64_t tiled_bytes,
                     const uint8_t *centroids, const uint16_t *scales_bf16, float *y, int8_t *xq, float *xs,
                     int32_t *acc_out, void *stream) {
    return forward_impl(x, M, K, N, tiled, tiled_bytes, centroids, false, scales_bf16, y, false, xq, xs, acc_out,
                        stream);
}

int32_t s3d8_forward_ex(const float *x, int64_t M, int64_t K, int64_t N, const uint8_t *tiled, int64_t tiled_bytes,
                        const void *table, int32_t format, const uint16_t *scales_bf16, void *y, int32_t out_type,
                        int8_t *xq, float *xs, int32_t *acc_out, void *stream) {
    int rc = check_variant(format, out_type);
    if (rc) return rc;
    return forward_impl(x, M, K, N, tiled, tiled_bytes, table, format == S3D8_FORMAT_3D8, scales_bf16, y,
                        out_type == S3D8_OUT_BF16, xq, xs, acc_out, stream);
}

int32_t s3d8_forward_batch(int32_t count, const s3d8_forward_item *items, void *stream) {
    if (count < 0 || (count > 0 && !items)) return s3d8::fail(S3D8_ERR_INVALID_ARG, "bad item list");
    for (int32_t i = 0; i < count; ++i) {
        const s3d8_forward_item &it = items[i];
        if (!it.x || !it.xq || !it.xs) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
        int rc = check_linear_args(it.tiled, it.tiled_bytes, it.centroids, it.scales_bf16, it.y, it.M, it.K, it.N);
        if (rc) return rc;
        if (!aligned16(it.x) || !aligned16(it.xq)) return s3d8::fail(S3D8_ERR_ALIGN, "x and xq must be 16-byte aligned");
    }
    if (count == 0) return S3D8_OK;
    int cus = 0;
    int rc = check_device(&cus);
    if (rc) return rc;
    if (launch_gemv_stream_batch(count, items, cus, (hipStream_t)stream)) return launch_status();
    for (int32_t i = 0; i < count; ++i) {
        const s3d8_forward_item &it = items[i];
        rc = s3d8_forward(it.x, it.M, it.K, it.N, it.tiled, it.tiled_bytes, it.centroids, it.scales_bf16, it.y,
                          it.xq, it.xs, it.acc_out, stream);
        if (rc) return rc;
    }
    return S3D8_OK;
}

int32_t s3d8_encode_device(const float *W, int64_t N, int64_t K, const uint8_t *centroids, uint16_t *scales_bf16,
                           uint8_t *packed, void *stream) {
    if (!W || !centroids || !scales_bf16 || !packed) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(1, K, N);
    if (rc) return rc;
    if (reinterpret_cast<uintptr_t>(W) & 3u) return s3d8::fail(S3D8_ERR_ALIGN, "W must be 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(scales_bf16) & 1u)
        return s3d8::fail(S3D8_ERR_ALIGN, "scales_bf16 must be 2-byte aligned");
    if (N > lim_int() / K) return s3d8::fail(S3D8_ERR_SHAPE, "N * K over 2^31");
    rc = check_device(nullptr);
    if (rc) return rc;
    const int64_t T = (N + 2) / 3;
    hipLaunchKernelGGL(channel_scale_kernel, dim3((unsigned)(3 * T)), dim3(kScaleThreads), 0, (hipStream_t)stream, W,
                       (int)N, (int)K, scales_bf16);
    const int64_t nbytes = T * K;
    hipLaunchKernelGGL(encode_kernel, dim3((unsigned)((nbytes + kEncodeThreads - 1) / kEncodeThreads)),
                       dim3(kEncodeThreads), 0, (hipStream_t)stream, W, (int)N, (int)K, (int)T, scales_bf16, centroids,
                       packed);
    return launch_status();
}

int64_t s3d8_unfused_workspace_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return -1;
    return (3 * ((N + 2) / 3) + 31) / 32 * ((K + 63) / 64) * 2048;
}

// ------------------------------------------------- no-allocation unfused path

// Device-side workspace of s3d8_linear_unfused_noalloc: the decoded INT8
// matrix lives in this file-scope array instead of a caller's buffer, for
// callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol, never a device address: the address is looked up
// once per device with hipGetSymbolAddress (noalloc_scratch) and only that
// pointer is handed to kernels.  Every call on one GPU shares its copy, so
// calls that overlap on one GPU (different streams) race.  What a previous
// call left there needs no clearing: the decode overwrites every byte of the
// matrix, and the bytes it leaves alone (channels past the last triple,
// columns past K in the last 64-column block) only meet zero activations or
// feed outputs that are never stored.
constexpr int64_t kNoAllocScratchBytes = S3D8_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes == int64_t(64) << 20, "the header states 64 MiB");
static __device__ __align__(256) int8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;

// The current device's copy of `scratch`, looked up on the first call on
// that device (after check_device has accepted the device).
int noalloc_scratch(int8_t **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return s3d8::fail(S3D8_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return s3d8::fail(S3D8_ERR_DEVICE, "device ordinal out of range");
    static std::mutex mu;
    static int8_t *ptr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return s3d8::fail(S3D8_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
        ptr[dev] = static_cast<int8_t *>(p);
    }
    *out = ptr[dev];
    return S3D8_OK;
}

// noalloc: the workspace is the library's scratch array (workspace and
// workspace_bytes are ignored), looked up once the arguments are validated.
int unfused_impl(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                 int64_t tiled_size, const void *table, bool f3d8, const uint16_t *scales_bf16, void *y, bool obf,
                 int32_t *acc_out, int8_t *workspace, int64_t workspace_bytes, void *stream, bool noalloc = false) {
    if (!xq || !xs || (!noalloc && !workspace)) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_linear_args(tiled, tiled_size, table, scales_bf16, y, M, K, N);
    if (rc) return rc;
    if (!aligned16(xq) || (!noalloc && !aligned16(workspace)))
        return s3d8::fail(S3D8_ERR_ALIGN, "xq and workspace must be 16-byte aligned");
    if (N > kGemmMaxN) return s3d8::fail(S3D8_ERR_SHAPE, "N over 3355442 is not supported");
    const int64_t T = (N + 2) / 3;
    const int64_t wbytes = s3d8_unfused_workspace_bytes(N, K);
    if (wbytes > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "decoded matrix over 2^31 bytes");
    if (noalloc && wbytes > kNoAllocScratchBytes)
        return s3d8::fail(S3D8_ERR_SHAPE,
                          "the decoded matrix exceeds the 64 MiB device scratch of s3d8_linear_unfused_noalloc "
                          "(s3d8_unfused_workspace_bytes(N, K) > S3D8_NOALLOC_SCRATCH_BYTES); use "
                          "s3d8_linear_unfused with a workspace");
    if (!noalloc && workspace_bytes < wbytes)
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "workspace smaller than s3d8_unfused_workspace_bytes");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    if (noalloc) {
        rc = noalloc_scratch(&workspace);
        if (rc) return rc;
    }
    const int KB = (int)((K + 63) / 64);
    const int64_t nchunks = tiled_bytes(N, K) / 16;
    int64_t blocks = (nchunks + kDequantThreads - 1) / kDequantThreads;
    if (blocks > (int64_t)cus * 2) blocks = (int64_t)cus * 2;
    hipLaunchKernelGGL(dequant_tiled_kernel, dim3((unsigned)blocks), dim3(kDequantThreads), 0, (hipStream_t)stream,
                       tiled, reinterpret_cast<const uint32_t *>(table), (int)K, (int)T, KB, (int)blocks, nchunks,
                       workspace, (int)f3d8);
    const int nbn = (int)((3 * T + 383) / 384);
    // 4 or 5 row tiles per wave: the one that needs fewer workgroup rounds,
    // counted in units of row-tile work (this kernel has no 64-row build)
    auto cost = [&](int rt) {
        const int64_t tiles = (M + 32 * rt - 1) / (32 * rt) * nbn;
        return (tiles + cus - 1) / cus * rt;
    };
    const int rt = cost(5) < cost(4) ? 5 : 4;
    const int nbm = (int)((M + 32 * rt - 1) / (32 * rt));
    const int64_t nwg = (int64_t)nbm * nbn;
    const int64_t grid = (nwg + kXcds - 1) / kXcds * kXcds;
    if (grid > 2147483647) return s3d8::fail(S3D8_ERR_SHAPE, "problem too large");
    typedef void (*I8Fn)(const int8_t *, const int8_t *, int, int, int, int, int, int, const float *,
                         const uint16_t *, void *, int32_t *);
    static const I8Fn fns[2][2][2] = {
        {{gemm_i8_kernel<4, false, false>, gemm_i8_kernel<4, false, true>},
         {gemm_i8_kernel<4, true, false>, gemm_i8_kernel<4, true, true>}},
        {{gemm_i8_kernel<5, false, false>, gemm_i8_kernel<5, false, true>},
         {gemm_i8_kernel<5, true, false>, gemm_i8_kernel<5, true, true>}}};
    hipLaunchKernelGGL(fns[rt == 5][acc_out != nullptr][obf], dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, xq,
                       workspace, (int)M, (int)K, (int)N, (int)(3 * T), nbm, nbn, xs, scales_bf16, y, acc_out);
    return launch_status();
}

int dequant_impl(const uint8_t *packed, const void *table, bool f3d8, int64_t N, int64_t K, int8_t *w,
                 void *stream) {
    if (!packed || !table || !w) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    int rc = check_sizes(1, K, N);
    if (rc) return rc;
    if (!aligned16(packed) || !aligned16(w)) return s3d8::fail(S3D8_ERR_ALIGN, "packed and w must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(table) & 3u)
        return s3d8::fail(S3D8_ERR_ALIGN, "the centroid table must be 4-byte aligned");
    int cus = 0;
    rc = check_device(&cus);
    if (rc) return rc;
    const int64_t T = (N + 2) / 3;
    const int64_t nchunks = T * (K / 16);
    int64_t blocks = (nchunks + kDequantThreads - 1) / kDequantThreads;
    const int64_t cap = (int64_t)cus * 2;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(kDequantThreads), 0, (hipStream_t)stream, packed,
                       reinterpret_cast<const uint32_t *>(table), (int)K, (int)N, nchunks, w, (int)f3d8);
    return launch_status();
}
}  // namespace

int32_t s3d8_linear_unfused(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                            const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                            const uint16_t *scales_bf16, float *y, int32_t *acc_out, int8_t *workspace,
                            int64_t workspace_bytes, void *stream) {
    return unfused_impl(xq, xs, M, K, N, tiled, tiled_bytes, centroids, false, scales_bf16, y, false, acc_out,
                        workspace, workspace_bytes, stream);
}

int32_t s3d8_linear_unfused_ex(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                               const uint8_t *tiled, int64_t tiled_bytes, const void *table, int32_t format,
                               const uint16_t *scales_bf16, void *y, int32_t out_type, int32_t *acc_out,
                               int8_t *workspace, int64_t workspace_bytes, void *stream) {
    int rc = check_variant(format, out_type);
    if (rc) return rc;
    return unfused_impl(xq, xs, M, K, N, tiled, tiled_bytes, table, format == S3D8_FORMAT_3D8, scales_bf16, y,
                        out_type == S3D8_OUT_BF16, acc_out, workspace, workspace_bytes, stream);
}

int32_t s3d8_linear_unfused_noalloc(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                                    const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                                    const uint16_t *scales_bf16, float *y, int32_t *acc_out, void *stream) {
    return unfused_impl(xq, xs, M, K, N, tiled, tiled_bytes, centroids, false, scales_bf16, y, false, acc_out,
                        nullptr, 0, stream, true);
}

int32_t s3d8_dequant(const uint8_t *packed, const uint8_t *centroids, int64_t N, int64_t K, int8_t *w,
                     void *stream) {
    return dequant_impl(packed, centroids, false, N, K, w, stream);
}

int32_t s3d8_dequant_ex(const uint8_t *packed, const void *table, int32_t format, int64_t N, int64_t K, int8_t *w,
                        void *stream) {
    int rc = check_variant(format, S3D8_OUT_F32);
    if (rc) return rc;
    return dequant_impl(packed, table, format == S3D8_FORMAT_3D8, N, K, w, stream);
}

int32_t s3d8_mfma_rate_probe(int32_t iters, int32_t workgroups, int32_t v, int32_t *out, void *stream) {
    if (!out) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    if (iters < 1 || workgroups < 1 || workgroups > 65536 || v < -128 || v > 127)
        return s3d8::fail(S3D8_ERR_INVALID_ARG, "iters >= 1, 1 <= workgroups <= 65536, -128 <= v <= 127");
    if (reinterpret_cast<uintptr_t>(out) & 3u) return s3d8::fail(S3D8_ERR_ALIGN, "out must be 4-byte aligned");
    int rc = check_device(nullptr);
    if (rc) return rc;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)workgroups), dim3(kRateThreads), 0, (hipStream_t)stream,
                       (int)iters, (int)v, out);
    return launch_status();
}

int32_t s3d8_hbm_read_probe(const void *p, int64_t bytes, int32_t workgroups, uint32_t *out, void *stream) {
    if (!p || !out) return s3d8::fail(S3D8_ERR_INVALID_ARG, "null pointer argument");
    if (bytes <= 0 || bytes % 16 != 0) return s3d8::fail(S3D8_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (workgroups < 1 || workgroups > 65536) return s3d8::fail(S3D8_ERR_INVALID_ARG, "1 <= workgroups <= 65536");
    if (!aligned16(p)) return s3d8::fail(S3D8_ERR_ALIGN, "p must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(out) & 3u) return s3d8::fail(S3D8_ERR_ALIGN, "out must be 4-byte aligned");
    int rc = check_device(nullptr);
    if (rc) return rc;
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4 *>(p), bytes / 16, out);
    return launch_status();
}

}  // extern "C"
