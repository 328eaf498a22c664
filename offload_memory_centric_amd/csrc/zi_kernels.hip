// zi_kernels.hip -- gfx950 kernels of the tiled linear operator.
//
// One MFMA GEMM template covers the three products of a weight tile
// (memory-centric tiling of Y = XW, ZeRO-Infinity transformer-math page,
// section "Memory-centric tiling: operators bigger than the device"):
//   forward   Y_i  = X W_i          both operands reduction-contiguous
//   dX       dX   += dY_i W_i^T     the tile operand is read across its rows
//   dW       dW_i  = X^T dY_i       both operands are read across their rows
// The output C[p][q] is row-major with q contiguous.  The MFMA "A" operand is
// the one indexed by q (called Q), the "B" operand the one indexed by p
// (called P), so each lane's four consecutive accumulator registers land on
// four consecutive q, and every epilogue store is one 8- or 16-byte vector.
//
// Workgroup: 256 threads = 4 wave64s in a 2 x 2 arrangement over a
// 256 (p) x 256 (q) macro-tile; each wave owns 128 x 128 = 4 x 4 MFMA blocks
// of 32 x 32 (v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulators: 256 per lane,
// which is why the kernel runs one wave per SIMD).  The reduction advances 64
// at a time through two LDS stages (2 x 64 KiB): global loads of step k+1 are
// issued before the MFMAs of step k and written to the other stage after
// them, one barrier per step.
//
// LDS rows hold 64 reduction elements (128 B = 8 chunks of 16 B).  Chunk c of
// row r sits at physical chunk c ^ ((r ^ (r >> 3)) & 7): the MFMA fragment
// reads (32 consecutive rows, same chunk), the row-contiguous writes (one row,
// 8 chunks) and the transposed writes (rows 8 apart, same chunk) each touch 8
// distinct chunk positions per 8 lanes.
//
// An operand whose reduction index is strided in memory is loaded as 8 x 8
// blocks of 16-bit values (8 reduction rows of 8 contiguous elements, one
// 16-byte load each, coalesced along the contiguous dimension) and transposed
// in registers before it is written to LDS in the same reduction-contiguous
// layout, so the MFMA side never sees the difference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zi_internal.h"

namespace zi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int BK = 64;                        // reduction elements per main-loop step
constexpr int kRowBytes = BK * 2;             // one LDS row: 8 chunks of 16 B
constexpr int kOperandBytes = 256 * kRowBytes;  // 32 KiB: one operand, one stage
constexpr int kStageBytes = 2 * kOperandBytes;  // Q and P
constexpr int kLdsBytes = 2 * kStageBytes;      // two stages: 128 KiB

enum Epi { EPI_LP = 0, EPI_F32 = 1, EPI_GELU = 2, EPI_ACC = 3 };

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// ---- global -> registers ----------------------------------------------------

// Reduction-contiguous operand: element (r, k) at M[r * ld + k].  Thread t
// loads chunk (t & 7) of rows (t >> 3) + 32 j, j < 8.  red % 8 == 0, so a
// 16-byte chunk is entirely inside or entirely outside the reduction range.
__device__ __forceinline__ void load_rc(const uint16_t *__restrict__ M, int64_t ld, int64_t r0,
                                        int64_t rext, int64_t k0, int64_t red, int tid,
                                        u32x4 (&v)[8]) {
    const int c = tid & 7;
    const int rb = tid >> 3;
    const int64_t k = k0 + c * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = r0 + rb + 32 * j;
        if (r < rext && k < red)
            v[j] = *reinterpret_cast<const u32x4 *>(M + r * ld + k);
        else
            v[j] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Reduction-strided operand: element (r, k) at M[k * ld + r].  Thread t loads
// the 8 x 8 block of reduction rows 8 (t >> 5) .. +7 and elements
// r0 + 8 (t & 31) .. +7; rext % 8 == 0.
__device__ __forceinline__ void load_rs(const uint16_t *__restrict__ M, int64_t ld, int64_t r0,
                                        int64_t rext, int64_t k0, int64_t red, int tid,
                                        u32x4 (&v)[8]) {
    const int rg = tid & 31;
    const int kg = tid >> 5;
    const int64_t r = r0 + rg * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t k = k0 + kg * 8 + q;
        if (r < rext && k < red)
            v[q] = *reinterpret_cast<const u32x4 *>(M + k * ld + r);
        else
            v[q] = u32x4{0u, 0u, 0u, 0u};
    }
}

// ---- registers -> LDS --------------------------------------------------------

__device__ __forceinline__ void store_rc(char *lds, int tid, const u32x4 (&v)[8]) {
    const int c = tid & 7;
    const int rb = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = rb + 32 * j;
        *reinterpret_cast<u32x4 *>(lds + row * kRowBytes + ((c ^ swz(row)) << 4)) = v[j];
    }
}

// Transpose the thread's 8 x 8 block (v[q] = reduction row q, 8 elements) into
// 8 rows of 8 reduction values and write each as chunk (t >> 5) of its row.
__device__ __forceinline__ void store_rs(char *lds, int tid, const u32x4 (&v)[8]) {
    const int rg = tid & 31;
    const int kg = tid >> 5;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4 u;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = v[2 * p][c >> 1];
            const uint32_t hi = v[2 * p + 1][c >> 1];
            u[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int row = rg * 8 + c;
        *reinterpret_cast<u32x4 *>(lds + row * kRowBytes + ((kg ^ swz(row)) << 4)) = u;
    }
}

__device__ __forceinline__ u32x4 lds_frag(const char *lds, int row, int chunk) {
    return *reinterpret_cast<const u32x4 *>(lds + row * kRowBytes + ((chunk ^ swz(row)) << 4));
}

// ---- MFMA ------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<_Float16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- conversions and GeLU ---------------------------------------------------------

// One round-to-nearest-even conversion (v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
template <typename T>
__device__ __forceinline__ uint32_t bits16(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (T)x);
}

template <typename T>
__device__ __forceinline__ float value16(uint32_t b) {
    return (float)__builtin_bit_cast(T, (uint16_t)b);
}

// GeLU(a) = a * Phi(a), Phi(a) = erfc(-a / sqrt 2) / 2 (exact erf form).
__device__ __forceinline__ float gelu_f32(float a) {
    return a * (0.5f * erfcf(-a * 0.70710678118654752f));
}

// GeLU'(a) = Phi(a) + a * phi(a), phi(a) = exp(-a^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f32(float a) {
    const float cdf = 0.5f * erfcf(-a * 0.70710678118654752f);
    const float pdf = 0.39894228040143268f * expf(-0.5f * a * a);
    return cdf + a * pdf;
}

// ---- workgroup -> macro-tile ------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8).  When the tile count allows it, XCD x is given the contiguous
// range of tiles [x * nt/8, (x+1) * nt/8), so the workgroups that share an L2
// also share operand tiles; inside a range, tiles go in column groups 8
// macro-rows tall (8 P tiles reuse one Q tile, 8 consecutive groups reuse P).
__device__ __forceinline__ void tile_coords(int w, int tiles_p, int tiles_q, int &tp, int &tq) {
    const int nt = tiles_p * tiles_q;
    int t = w;
    if ((nt & 7) == 0) t = (w & 7) * (nt >> 3) + (w >> 3);
    constexpr int G = 8;
    const int per_group = G * tiles_q;
    const int g = t / per_group;
    const int first = g * G;
    const int gsz = min(tiles_p - first, G);
    const int r = t - g * per_group;
    tp = first + r % gsz;
    tq = r / gsz;
}

// ---- the GEMM ---------------------------------------------------------------------

template <typename T, bool Q_RS, bool P_RS, int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs a, int tiles_p, int tiles_q) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wq = wave & 1;
    const int wp = wave >> 1;

    int tp, tq;
    tile_coords(blockIdx.x, tiles_p, tiles_q, tp, tq);
    const int64_t p0 = (int64_t)tp * 256;
    const int64_t q0 = (int64_t)tq * 256;

    const uint16_t *__restrict__ Q = static_cast<const uint16_t *>(a.Q);
    const uint16_t *__restrict__ P = static_cast<const uint16_t *>(a.P);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    u32x4 vq[8], vp[8];
    const int64_t ksteps = (a.red + BK - 1) / BK;

    auto load = [&](int64_t k0) {
        if constexpr (Q_RS)
            load_rs(Q, a.ldq, q0, a.cols, k0, a.red, tid, vq);
        else
            load_rc(Q, a.ldq, q0, a.cols, k0, a.red, tid, vq);
        if constexpr (P_RS)
            load_rs(P, a.ldp, p0, a.rows, k0, a.red, tid, vp);
        else
            load_rc(P, a.ldp, p0, a.rows, k0, a.red, tid, vp);
    };
    auto store = [&](char *stage) {
        if constexpr (Q_RS)
            store_rs(stage, tid, vq);
        else
            store_rc(stage, tid, vq);
        if constexpr (P_RS)
            store_rs(stage + kOperandBytes, tid, vp);
        else
            store_rc(stage + kOperandBytes, tid, vp);
    };

    load(0);
    store(lds);
    __syncthreads();

    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    for (int64_t kt = 0; kt < ksteps; ++kt) {
        const char *cur = lds + (kt & 1) * kStageBytes;
        const bool more = kt + 1 < ksteps;
        if (more) load((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int chunk = ks * 2 + fhalf;
            u32x4 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = lds_frag(cur, wq * 128 + i * 32 + frow, chunk);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fb[j] = lds_frag(cur + kOperandBytes, wp * 128 + j * 32 + frow, chunk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32<T>(fa[i], fb[j], acc[i][j]);
        }
        if (more) store(lds + ((kt + 1) & 1) * kStageBytes);
        __syncthreads();
    }

    // Epilogue.  Accumulator register 4g + e of block (i, j) holds
    // C[p][q] with p = j-block row (lane & 31) and q = 8 g + 4 (lane >> 5) + e.
    const int64_t pb = p0 + wp * 128 + frow;
    const int64_t qb = q0 + wq * 128 + 4 * fhalf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t p = pb + j * 32;
            if (p >= a.rows) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t q = qb + i * 32 + 8 * g;
                if (q >= a.cols) continue;
                f32x4 v = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
                const int64_t off = p * a.ldc + q;
                if constexpr (EPI == EPI_F32) {
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.C) + off) = v;
                } else if constexpr (EPI == EPI_ACC) {
                    f32x4 *c = reinterpret_cast<f32x4 *>(static_cast<float *>(a.C) + off);
                    if (a.accumulate) v += *c;
                    *c = v;
                } else if constexpr (EPI == EPI_LP) {
                    u32x2 o = {bits16<T>(v[0]) | (bits16<T>(v[1]) << 16),
                               bits16<T>(v[2]) | (bits16<T>(v[3]) << 16)};
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C) + off) = o;
                } else {  // EPI_GELU: A = RNE(acc); H = RNE(GeLU(A))
                    uint32_t b[4], h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        b[e] = bits16<T>(v[e]);
                        h[e] = bits16<T>(gelu_f32(value16<T>(b[e])));
                    }
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C) + off) =
                        u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C2) + off) =
                        u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                }
            }
        }
    }
}

// ---- dA = RNE(dH * GeLU'(A)) ----------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void gelu_bwd_kernel(const float *__restrict__ dH,
                                                       const uint16_t *__restrict__ A,
                                                       uint16_t *__restrict__ dA, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < count; i += stride) {
        if (i + 8 <= count) {
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(dH + i);
            const f32x4 g1 = *reinterpret_cast<const f32x4 *>(dH + i + 4);
            const u32x4 av = *reinterpret_cast<const u32x4 *>(A + i);
            const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a0 = value16<T>(av[w] & 0xffffu);
                const float a1 = value16<T>(av[w] >> 16);
                o[w] = bits16<T>(g[2 * w] * gelu_grad_f32(a0)) |
                       (bits16<T>(g[2 * w + 1] * gelu_grad_f32(a1)) << 16);
            }
            *reinterpret_cast<u32x4 *>(dA + i) = o;
        } else {
            for (int64_t e = i; e < count; ++e)
                dA[e] = (uint16_t)bits16<T>(dH[e] * gelu_grad_f32(value16<T>(A[e])));
        }
    }
}

template <typename T, bool Q_RS, bool P_RS, int EPI>
hipError_t run(const GemmArgs &a, hipStream_t s) {
    const int tiles_p = (int)((a.rows + kTileP - 1) / kTileP);
    const int tiles_q = (int)((a.cols + kTileQ - 1) / kTileQ);
    const int64_t nt = (int64_t)tiles_p * tiles_q;
    if (nt <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<T, Q_RS, P_RS, EPI>), dim3((unsigned)nt), dim3(kThreads), 0, s,
                       a, tiles_p, tiles_q);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(GemmOp op, const GemmArgs &a, hipStream_t s) {
    switch (op) {
        case GemmOp::Fwd:
            return a.out_f32 ? run<T, false, false, EPI_F32>(a, s) : run<T, false, false, EPI_LP>(a, s);
        case GemmOp::FwdGelu:
            return run<T, false, false, EPI_GELU>(a, s);
        case GemmOp::Dx:
            return run<T, true, false, EPI_ACC>(a, s);
        case GemmOp::Dw:
            return a.out_f32 ? run<T, true, true, EPI_F32>(a, s) : run<T, true, true, EPI_LP>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(GemmOp op, int dtype, const GemmArgs &a, hipStream_t stream) {
    if (dtype == 1) return dispatch<_Float16>(op, a, stream);
    if (dtype == 2) return dispatch<__bf16>(op, a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gelu_bwd(int dtype, const float *dH, const void *A, void *dA, int64_t count,
                           hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t threads = (count + 7) / 8;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    const uint16_t *a16 = static_cast<const uint16_t *>(A);
    uint16_t *d16 = static_cast<uint16_t *>(dA);
    if (dtype == 1)
        hipLaunchKernelGGL(gelu_bwd_kernel<_Float16>, dim3((unsigned)blocks), dim3(256), 0, stream, dH,
                           a16, d16, count);
    else if (dtype == 2)
        hipLaunchKernelGGL(gelu_bwd_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, dH,
                           a16, d16, count);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace zi
