// zi_internal.h -- declarations shared by the library's own translation units
// (host API, ring model, kernels).  Not installed; the public ABI is zi.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace zi {

// Which product a GEMM launch forms.  The output C[p][q] is row-major with q
// contiguous; "Q" is the operand indexed by q, "P" the operand indexed by p.
enum class GemmOp : int {
    Fwd = 0,      // Y_i[t][m]  = sum_k X[t][k] W^t_i[m][k]      (Q = W slot, P = X)
    FwdGelu = 1,  // same product; stores A = RNE(acc) (fp32 acc with out_f32) and H = RNE(GeLU(RNE(acc)))
    Dx = 2,       // dX[t][k]  (+)= sum_r dY[t][i*n+r] W^t_i[r][k] (Q = W slot^T, P = dY)
    Dw = 3,       // dW^t_i[m][k] = sum_t dY[t][i*n+m] X[t][k]    (Q = X^T,      P = dY^T)
};

struct GemmArgs {
    const void *Q;  // 16-bit elements
    int64_t ldq;
    const void *P;  // 16-bit elements
    int64_t ldp;
    void *C;        // output: 16-bit, or fp32 when out_f32 / Dx
    int64_t ldc;
    void *C2;       // FwdGelu: H output (same layout as C)
    int64_t rows;   // extent of p
    int64_t cols;   // extent of q (multiple of 8)
    int64_t red;    // reduction length
    int accumulate; // Dx only: 0 = overwrite, 1 = add into C
    int out_f32;    // Fwd / Dw: write fp32 instead of the 16-bit format; FwdGelu: A in fp32
    // Two weight tiles held in different ring slots, consumed by one launch.
    // Dx: reduction rows k >= qsplit of Q come from Q2 (row k - qsplit);
    // qsplit a multiple of the kernel's step (64).  Fwd: output columns
    // q >= qsplit come from Q2 (row q - qsplit); qsplit a multiple of the
    // launch's macro-tile width (gemm_tile).  Q2 = null: no split.
    const void *Q2;
    int64_t qsplit;
    // Dx: at most this many workgroups (a multiple of 8), each taking several
    // output tiles in turn, the next tile's first copies and C loads issued
    // under the finished tile's stores; 0 = one workgroup per output tile.
    int32_t wg_cap;
    // FwdGelu: fp32 half-sums and arrival counters (workspace of
    // kSplitBytes, counters zero between launches) for splitting the
    // reduction of the launch's last, partial round of tiles between two
    // workgroups each, when at most half of split_cap (the workgroups that run
    // at once) would be busy in it; null: no split.  split_tail is set by the
    // launch: the number of such tiles.
    float *split_part;
    uint32_t *split_cnt;
    int32_t split_cap;
    int32_t split_tail;
};

// dtype: 1 = fp16, 2 = bf16.  Returns the launch status (hipGetLastError).
hipError_t launch_gemm(GemmOp op, int dtype, const GemmArgs &a, hipStream_t stream);

// Workgroups (one macro-tile each) that launch_gemm runs for a product with
// `rows` output rows and `cols` output columns: the macro-tile is 256 x 256,
// or 192 x 320 / 320 x 192 (rows x columns) where that tile covers a forward's
// columns or a gradient's rows with clearly less padding.
int64_t gemm_workgroups(GemmOp op, int64_t rows, int64_t cols);
// That macro-tile: output rows and columns of one workgroup.
void gemm_tile(GemmOp op, int64_t rows, int64_t cols, int *tile_rows, int *tile_cols);

// Builds the per-device tables H = RNE16(GeLU(A)) over every 16-bit A (fp16
// and bf16) that the forward GeLU epilogue reads; enqueued on `stream`.
hipError_t build_gelu_tables(hipStream_t stream);

// dA[i] = RNE(dH[i] * GeLU'(A[i])), i < count; with out_f32 the fp32 product
// itself (dA then holds fp32 elements).
hipError_t launch_gelu_bwd(int dtype, const float *dH, const void *A, void *dA, int64_t count,
                           bool out_f32, hipStream_t stream);

// Reduction values per pipeline step of the GEMM kernels.
constexpr int kGemmStep = 64;

// Split GeLU forward: at most kSplitTiles tiles, each two fp32 half-sums of
// 256 x 256 (256 KiB), then one 32-bit counter per tile.
constexpr int kSplitTiles = 128;
constexpr uint64_t kSplitPartBytes = (uint64_t)kSplitTiles * 2 * 256 * 256 * 4;
constexpr uint64_t kSplitBytes = kSplitPartBytes + 512;

}  // namespace zi
