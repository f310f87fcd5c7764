// Internal interface of the fp32 matrix-core GEMM kernel with epilogues and
// the MSE kernel (gemm_kernels.hip), used by the MLP C-ABI layer
// (mlp_api.hip) and by the GEMM-form CfC weight gradient (cfc_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm {

constexpr int kGemmThreads = 512;   // 8 wave64: 4 (rows) x 2 (columns) over the tile
constexpr int kTile = 64;           // output tile: 64 rows x 64 columns
constexpr int kBK = 32;             // reduction indices staged per chunk
constexpr int kLdsPitch = 32;       // floats per staged row; its 8 float4 columns are XOR-swizzled by row
constexpr int kMaxTasks = 8;
constexpr int kMseThreads = 256;

enum Epilogue { kEpiFwd = 0, kEpiDx = 1, kEpiDw = 2 };

// An operand as rows r (m for A, n for B) by reduction index k.
struct Operand {
    const float* p;
    int64_t ld;
    int kc;    // 1: element (r, k) at p[r * ld + k]; 0: at p[k * ld + r] (fixed by the epilogue)
    int vec;   // 1: 16-byte loads along the contiguous index: ld and that index's
               //    extent multiples of 4, p 16-byte aligned
};

// One matrix product C[m, n] = sum_k A(m, k) B(n, k) over the tiles of one
// launch, with its epilogue.
struct GemmTask {
    Operand A, B;
    int M, N, K;
    int a_ext;             // > 0: A's contiguous index may be read up to a_ext (its entries past
                           //      K or M are zero in memory), so 16-byte loads cover the tail
    int k_split;           // reduction length of one split (multiple of kBK)
    int n_mt, n_nt, n_s;   // row tiles, column tiles, splits
    int epi, relu;
    const float* bias;     // kEpiFwd: [N] added before the ReLU (nullable)
    const float* mask;     // kEpiDx: [M, ldm], keep where > 0 (nullable)
    int64_t ldm;
    float* out;            // kEpiFwd / kEpiDx: [M, ldo]; kEpiDw: split s at out + s * split_stride
    int64_t ldo;
    int64_t split_stride;
    float* colsum;         // kEpiDw: sums of A(m, k) over the split's k, [M] at colsum + s * colsum_stride (nullable)
    int64_t colsum_stride;
    int64_t zlo[2], zhi[2];   // kEpiDw: floats [zlo, zhi) after out + s * split_stride to zero (layout gaps)
};

struct GemmBatch {
    GemmTask t[kMaxTasks];
    int64_t start[kMaxTasks + 1];   // prefix sums of the tasks' workgroups n_mt * n_nt * n_s
    int ntask;
};

struct MseArgs {
    const float* Y;
    const float* T;
    float* dY;
    int64_t M;
    int N;
    int64_t ldd;          // row pitch of dY
    float gscale;         // 2 / (M N), rounded once
    double lscale;        // 1 / (M N)
    float* lossp;         // [S] partial losses
    int S;
    int64_t rows_per;
};

// Fill the tile counts and start offsets of a batch from its tasks.
void finish_batch(GemmBatch& g);
hipError_t launch_gemm(const GemmBatch& g, hipStream_t s);
hipError_t launch_mse(const MseArgs& a, hipStream_t s);

}  // namespace gemm
