// Internal interface between the C-ABI layer (cfc_api.hip) and the gfx950
// kernels (cfc_kernels.hip).  Not installed; include/cfc.h is the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cfc {

constexpr int kThreads = 256;          // step, fill and reduce kernels: 4 wave64 per workgroup
constexpr int kGroup = 16;             // lanes that share one forward dot product (one DPP row)
constexpr int kGroups = kThreads / kGroup;
constexpr int kSlices = 16;            // backward W^T dp: 16 slices x 4 row groups = 64 groups
constexpr int kCols = kThreads / kSlices;
constexpr int kMaxReduceSegs = 2;
constexpr int kPersistThreads = 512;   // persistent K-loop kernel: 8 wave64, 64 groups of 8 lanes
constexpr int kFillTile = 64;          // scratch fill: 64 rows x 64 columns per workgroup
constexpr int kFillSteps = 64;         // time steps staged in LDS per pass

struct FwdArgs {
    const float* u_t;     // [B, n_x]
    const float* h_prev;  // [B, C]
    const float* W;       // [3, C, n_in]
    const float* bias;    // [3, C]
    float* h_t;           // [B, C]
    float* act_t;         // [3, B, C]
    float* h_prev_copy;   // nullable [B, C]: receives h_prev (h_hist[0] = h0 in the K-loop)
    int B, C, n_x, CT, n_ctiles, ldu, ldh;
};

struct BwdArgs {
    const float* u_t;
    const float* h_prev;
    const float* h_t;
    const float* y_t;
    const float* W;
    const float* act_t;
    const float* dh_in;   // nullable: zero carry
    float* dh_out;
    float* du_t;          // nullable
    float* gW_s;          // [B, 3, C, n_in] accumulated (when dp_out is null)
    float* gb_s;          // [B, 3, C]       accumulated (when dp_out is null)
    float* dp_out;        // nullable [B, 3C]: store dp instead of updating the scratch
    int B, C, n_x, CT, n_ctiles, ldz;
};

struct FillArgs {
    const float* dp;      // [K, B, 3C]
    const float* u;       // [K, B, n_x]
    const float* h_hist;  // [K+1, B, C]
    float* gW_s;          // [B, 3C, n_in] overwritten
    float* gb_s;          // [B, 3C]       overwritten
    int B, C, n_x, K, n_rt, n_kt;
};

struct XprojArgs {
    const float* u;       // [M, n_x], rows (t, b)
    const float* W;       // [3C, n_in]; columns 0 .. n_x - 1 are used
    const float* bias;    // [3C]
    float* X;             // [M, N]
    int64_t M;            // K * B
    int N;                // 3C
    int n_x, n_in, n_ntiles;
};

struct PersistArgs {
    const float* X;       // [K, B, 3C] input projection (bias included)
    const float* y;       // [K, B, C]
    const float* h0;      // [B, C]
    const float* W;       // [3, C, n_in]
    const float* bias;    // [3, C]
    float* h_hist;        // [K+1, B, C]
    float* act;           // [K, 3, B, C]
    float* dp;            // [K, B, 3C]
    int B, C, n_x, K;
};

struct ReduceSeg {
    const float* in;      // [B, N]
    float* out;           // [N]
    int64_t N;
    int64_t groups;       // column groups of V columns: ceil(N / V)
};

struct ReduceArgs {
    ReduceSeg seg[kMaxReduceSegs];
    int nseg;
    int64_t B;
    int R;                // row slices per column (a function of B only)
    int64_t rows_per_slice;
};

// Tiling of the step kernels, chosen on the host.  No choice here changes
// the arithmetic of any output (see cfc_math.h).
struct StepPlan {
    int BT;        // samples per workgroup
    int CT;        // channels per workgroup
    int n_ctiles;  // ceil(C / CT)
    int n_btiles;  // ceil(B / BT)
    int Vf;        // forward: 4 = float4 reads of W's recurrent columns (n_x, n_in % 4 == 0, W aligned), else 1
    int Vb;        // backward: 4 = float4 scratch updates (n_in % 4 == 0, scratch aligned), else 1
    int ldz;       // backward LDS row pitch of z (n_in rounded up to 4)
    int ldu, ldh;  // forward LDS row pitches of u and h (n_x and C rounded up to 4)
    size_t fwd_smem, bwd_smem;
};

int reduce_slices(int64_t B);

// Persistent K-loop kernel: returns the LDS bytes it needs for C channels,
// or 0 if no instantiation holds the recurrent W in registers (C > 128).
size_t persist_smem(int C);

hipError_t launch_fwd(const FwdArgs& a, const StepPlan& p, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, const StepPlan& p, hipStream_t s);
hipError_t launch_fill(const FillArgs& a, hipStream_t s);
hipError_t launch_xproj(const XprojArgs& a, hipStream_t s);
hipError_t launch_persist(const PersistArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceSeg* segs, int nseg, int64_t B, int V, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

}  // namespace cfc
