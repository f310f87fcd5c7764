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
// [persistent kernel source: begin]
constexpr int kPersistThreads = 512;   // persistent K-loop kernel: 8 wave64, 64 groups of 8 lanes
// [persistent kernel source: end]
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
    int kt_per;           // column tiles per workgroup (chosen by launch_fill)
};

// MFMA step path (the K-loop's step kernels at large B).  W is re-laid once
// per K-loop call into two operand layouts in the workspace:
//  Wf [3C][ldf]: row r = W[r] with the input columns as they are (zero padded
//     to nxp = round_up(n_x, 16)) followed by the recurrent columns of each
//     block of 32 permuted as  Wf[r][nxp + 32 i + 8 e + j] = W[r][n_x + 32 i + 4 j + e]
//     (zero past C), so that MFMA k-slot e of the eight recurrent partitions
//     j is one 32-byte run;
//  Wb [C][64][4][4]: Wb[k][g][kk][p] = W[row of element 4 p + kk of dz group
//     g][n_x + k] (zero past the group), the carry columns transposed so that
//     a lane's four k-slots of a group are one float4.
struct MfmaLayout {
    int nxp;   // input columns, padded to 16
    int cp;    // recurrent columns, padded to 32
    int ldf;   // nxp + cp
    int pg;    // MFMA instructions per dz group: ceil(3 cpg / 4) (<= 4)
};

struct PermuteArgs {
    const float* W;       // [3, C, n_in]
    float* Wf;            // [3C, ldf]
    float* Wb;            // [C, 64, 4, 4]
    int C, n_x;
    MfmaLayout L;
};

struct FwdMfmaArgs {
    const float* u_t;     // [B, n_x]
    const float* h_prev;  // [B, C]
    const float* Wf;      // MFMA forward layout
    const float* bias;    // [3, C]
    float* h_t;           // [B, C]
    float* act_t;         // [3, B, C]
    float* h_prev_copy;   // nullable [B, C]
    int B, C, n_x, n_ctiles;
    MfmaLayout L;
};

struct BwdMfmaArgs {
    const float* h_t;     // [B, C]      (read when dp_in is null)
    const float* y_t;     // [B, C]      (read when dp_in is null)
    const float* act_t;   // [3, B, C]   (read when dp_in is null)
    const float* dh_in;   // nullable [B, C]: carry into this step (read when dp_in is null)
    const float* Wb;      // MFMA backward layout
    float* dh_out;        // nullable [B, C]: carry to step t - 1
    float* dp_out;        // [B, 3C] dp of this step, the tile's channels (written when dp_in is null)
    int B, C, n_ctiles;
    MfmaLayout L;
    const float* dp_in;   // nullable [B, 3C]: dp of this step, formed by the launch of step t + 1
    const float* h_prev;  // [B, C] h_{t-1}       (when dp_prev_out is not null)
    const float* y_prev;  // [B, C] y_{t-1}
    const float* act_prev;  // [3, B, C] act_{t-1}
    float* dp_prev_out;   // nullable [B, 3C]: dp of step t - 1 for the tile's channels
    // resident kernel only: dp_t and dp_{t-1} of the sample tile in the
    // staged layout ([16][64 groups][16]), at agent scope
    const float* dpx;
    float* dpx_out;
};

// Resident MFMA K-loop (one cooperative launch): workgroup (btile, ctile)
// runs the forward step and then the backward step of its tile for every t,
// its W operands held in registers throughout; the workgroups of a sample
// tile hand h_t, act_t and dp_t to one another through memory, each step
// gated by their step counters in `flags`.
constexpr int kResFlagStride = 32;   // ints between the resident kernel's counters
struct ResidentArgs {
    const float* u;       // [K, B, n_x]
    const float* y;       // [K, B, C]
    const float* h0;      // [B, C]
    const float* Wf;      // MFMA forward layout
    const float* Wb;      // MFMA backward layout
    const float* bias;    // [3, C]
    float* h_hist;        // [K+1, B, C]
    float* act;           // [K, 3, B, C]
    float* dp;            // [K, B, 3C]
    float* hx;            // [2][n_btiles][16 cp], zero at launch: h_t by step parity, each sample
                          // tile's channel tiles' [16 samples][16 channels] blocks in turn
    float* dpx;           // [2][n_btiles][16][64][16], zero at launch: dp_t by step parity, the backward
                          // step's LDS layout
    int* flags;           // [(n_btiles * n_ctiles + 1) * kResFlagStride], zero at launch: steps done per
                          // workgroup, then an error word, each at the start of its own 128-byte line
    int B, C, n_x, K, n_ctiles;
    MfmaLayout L;
    int spin_limit;       // polls of a wait before it gives up and sets the error word
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

// [persistent kernel source: begin]
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
    // n_proj > 0: the launch also forms X.  Workgroups 0 .. n_proj - 1 each
    // form one 64 x 64 tile of X from u (xproj_kernel's tiles and bits)
    // and then set flags[their index] = call; the sample workgroups
    // n_proj .. n_proj + B - 1 wait for every flag (at most spin_limit
    // polls; flags[n_proj] = call marks a wait that gave up) before their
    // first read of X.  n_proj == 0: X comes from an earlier launch.
    const float* u;       // [K, B, n_x]
    int* flags;           // [n_proj + 1 + B ceil(K / 16)]
    int n_proj;
    unsigned call;        // nonzero, distinct between launches that share flags
    int spin_limit;
    // n_fill > 0 (with n_proj > 0 only): the launch also forms the per-sample
    // scratch of scratch_fill_kernel, with its bits.  Workgroups 0 ..
    // max(n_proj, n_fill) - 1 come ahead of the sample workgroups; after its
    // projection tile (if any), such a workgroup takes fill unit f < n_fill:
    // sample f / n_rt, dp rows 64 (f % n_rt) .. + 63, every column of z, one
    // pass of 16 steps per backward chunk c (steps K - 16 c down to
    // max(1, K - 16 c - 15)), each after flags[n_proj + 1 + b ceil(K / 16) + c]
    // holds call: sample b sets it once its dp of that chunk (and every h_t
    // before it) is performed at device scope.  Every workgroup of the launch
    // must be resident at once (the host checks the CU count).
    float* gW_s;          // [B, 3C, n_in]
    float* gb_s;          // [B, 3C]
    int n_fill;           // 0 or B ceil(3C / 64)
};
// Rows of the LDS (floats) that a fill unit stages per pass: dp [16][80] and
// z [16][zp], zp = n_in rounded up to 64, plus 16 (a read's 4 k-slots hit
// distinct banks); the partial buffers of the sample role hold them.
__host__ __device__ inline int persist_fill_zpitch(int n_in) { return ((n_in + 63) / 64) * 64 + 16; }
__host__ __device__ inline int persist_fill_lds_floats(int n_in) { return 16 * (80 + persist_fill_zpitch(n_in)); }
// [persistent kernel source: end]

constexpr int kMaxAdamwSegs = 4;

struct AdamwSeg {
    float* p;             // parameters, updated in place
    const float* g;       // gradients
    float* m;             // first moments, updated in place
    float* v;             // second moments, updated in place
    int64_t n;
    int vec;              // 1: all four arrays 16-byte aligned (float4 moves)
};

struct AdamwArgs {
    AdamwSeg seg[kMaxAdamwSegs];
    int64_t qstart[kMaxAdamwSegs + 1];  // prefix sums of ceil(n / 4): chunks of 4 elements
    int nseg;
    float decay;          // 1 - lr * weight_decay
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float step_size;      // lr / (1 - beta1^step)
    float inv_sqrt_bc2;   // 1 / sqrt(1 - beta2^step)
    float eps;
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
    const float* xin;     // nullable: one more sum, xout[0] = sum of xin[0 .. xn) in fp64 (lane l of the
                          // first workgroup adds l, l + 256, .. in order, then a fixed pairwise tree)
    float* xout;
    int64_t xn;
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
int persist_proj_blocks(int B, int C, int K);   // -1 when too many
// Whether a launch with the projection can also form the scratch (n_fill =
// B ceil(3C / 64) units) for these sizes: z rows of at most 256 floats in
// whole float4, the unit's LDS within the partial buffers, and every
// workgroup resident at once on a device of n_cus CUs (one per CU).
bool persist_fill_fits(int B, int C, int n_x, int K, int n_cus);

hipError_t launch_fwd(const FwdArgs& a, const StepPlan& p, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, const StepPlan& p, hipStream_t s);
hipError_t launch_fill(const FillArgs& a, hipStream_t s);
hipError_t launch_xproj(const XprojArgs& a, hipStream_t s);
hipError_t launch_persist(const PersistArgs& a, hipStream_t s);
hipError_t launch_reduce(const ReduceSeg* segs, int nseg, int64_t B, int V, hipStream_t s);
// The same launch with one more fp64 sum (xn floats at xin, fixed order) into
// xout[0], done by the first workgroup.
hipError_t launch_reduce_with_sum(const ReduceSeg* segs, int nseg, int64_t B, int V, const float* xin, int64_t xn,
                                  float* xout, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_adamw(const AdamwArgs& a, hipStream_t s);

// MFMA step path: layout for (C, n_x) (valid iff pg <= 4, i.e. C <= 320),
// workspace floats of the two re-laid copies of W, and the launches.
MfmaLayout mfma_layout(int C, int n_x);
int64_t mfma_w_floats(int C, int n_x);
bool mfma_fits(int C, int n_x);   // both MFMA step kernels can take this shape
hipError_t launch_permute_w(const PermuteArgs& a, hipStream_t s);
// Workgroups of the resident kernel that can run at once on the current
// device for this layout (0 without cooperative launch); its grid is
// ceil(B / 16) * ceil(C / 16).
int64_t resident_capacity(const MfmaLayout& L);
// Floats of the resident kernel's exchange blocks (hx, then dpx) for B, C.
int64_t resident_exchange_floats(int B, int C);
hipError_t launch_resident(const ResidentArgs& a, hipStream_t s);
hipError_t launch_fwd_mfma(const FwdMfmaArgs& a, hipStream_t s);
hipError_t launch_bwd_mfma(const BwdMfmaArgs& a, hipStream_t s);

}  // namespace cfc
