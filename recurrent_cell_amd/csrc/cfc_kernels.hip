// gfx950 kernels of the CfC K-loop: the input projection of all steps
// (MFMA), forward and backward (BPTT) step kernels on VALU and on MFMA, the
// persistent per-sample K-loop kernel, the deferred fill of the per-sample
// gradient scratch (MFMA), the batch-axis reduction and AdamW.
//
// Parallel structure ("K-loop Parallelization -- Block-per-Batch Kernel
// Refactor", section Architecture Choice): samples are independent, so no
// workgroup waits for another -- except inside the resident MFMA kernel,
// where the channel tiles of one sample tile hand each step's h_t and dp_t
// to one another under bounded waits.
//  * Step kernels: a workgroup owns (a tile of samples) x (16 channels).  A
//    sample is split over ceil(C / 16) workgroups so that B = 32 samples
//    still fill the chip.  Channel tile j is the fastest-varying part of the
//    workgroup id, so it always runs on XCD (j mod 8) and its W rows and
//    scratch rows stay in that XCD's L2 from one K-step to the next.
//  * Resident MFMA kernel (wide shapes): all 2K steps of the MFMA step
//    kernels' arithmetic in one cooperative launch, W operands held in
//    registers; the channel tiles of a sample tile sit on one XCD, and each
//    step's input projection is formed while the tile waits for the others.
//  * Persistent kernel: one 512-lane workgroup (8 wave64) per sample runs all
//    K forward and all K backward steps of the recurrence with the recurrent
//    columns of W (3C x C, C <= 128) held in registers, 96 values per lane at
//    C = 128; the input part of every step comes from the input projection.
// Every (sample, channel) scratch row has exactly one writer.  No atomic
// read-modify-write.
//
// Determinism: every output follows the canonical order of cfc_math.h, which
// depends only on the sizes, so repeated runs, the step-kernel graph, the
// persistent kernel and a B = 1 run of any single sample all produce the
// same bits.
#include "cfc_kernels.h"
#include <climits>
#include "cfc_math.h"

namespace cfc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroups are dispatched round-robin over the 8 XCDs (block i to XCD
// i mod 8), and each XCD has its own L2.  This maps block i to a logical
// index such that each XCD receives one contiguous run of logical indices,
// so tiles that share operands (consecutive logical indices) share an L2.
// A bijection of [0, n); no arithmetic depends on it.
__device__ __forceinline__ int64_t xcd_local_order(int64_t i, int64_t n)
{
    const int64_t q = n / 8, r = n % 8;
    const int64_t x = i % 8, j = i / 8;
    return x * q + min(x, r) + j;
}

// 16-byte load from an address the caller has clamped into bounds, issued
// unconditionally; zero where !valid.  Branch-free, so a run of such loads
// stays in flight together (a load under a branch is waited for where the
// branch joins).
__device__ __forceinline__ f32x4 load4_or_zero(const float* clamped, bool valid)
{
    const f32x4 v = *reinterpret_cast<const f32x4*>(clamped);
    return valid ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// [persistent kernel source: begin]
// 4-byte store at device scope (sc1): written through to memory, so that a
// workgroup on another XCD of the same launch reads it.
__device__ __forceinline__ void st_agent(float* p, float v)
{
    __hip_atomic_store(reinterpret_cast<int*>(p), __float_as_int(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-scope (write-through) store through a raw buffer resource
// over [base, base + bytes); offsets at or past `bytes` write nothing.
__device__ __forceinline__ void st4_dev(float* base, int bytes, int byte_off, f32x4 v)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                           byte_off, 0, 16 /* sc1 */);
}
// [persistent kernel source: end]

// z_s = [u_t[b0+s] ; h_prev[b0+s]] for the tile's samples into LDS rows of
// pitch ldz (zero padded past n_in and for absent samples).
template <int BT>
__device__ __forceinline__ void stage_z(float* zs, int ldz, const float* __restrict__ u_t,
                                        const float* __restrict__ h_prev, int b0, int nb,
                                        int C, int n_x)
{
    const int n_in = n_x + C;
    for (int i = threadIdx.x; i < BT * ldz; i += kThreads) {
        const int s = i / ldz;
        const int k = i - s * ldz;
        float v = 0.0f;
        if (s < nb && k < n_in) {
            const int64_t b = (int64_t)b0 + s;
            v = (k < n_x) ? u_t[b * n_x + k] : h_prev[b * C + (k - n_x)];
        }
        zs[i] = v;
    }
}

// ---------------------------------------------------------------------------
// Forward step.  Workgroup = (sample tile of BT, channel tile of CT).
// Rows of the tile: r = q * nc + cl  (head q, channel c0 + cl), 3 * nc rows.
// An 8-lane group (half a DPP row) owns one W row at a time, for all BT
// samples: lane j runs the recurrent chain P_j over the columns
// n_x + 32 i + 4 j + e, and lanes 0..3 the input chains x_0 .. x_3 (input
// columns k = j mod 4); sum8 and quad_sum4 combine them in the canonical
// order.  u and h are staged in separate LDS rows so the recurrent columns
// start 16-byte aligned whatever n_x is.  V = 4 reads W with float4 (only
// the load width differs).
// ---------------------------------------------------------------------------
template <int BT, int V>
__global__ __launch_bounds__(kThreads) void fwd_step_kernel(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int n_x = a.n_x;
    const int C = a.C;
    const int n_in = n_x + C;
    const int ctile = blockIdx.x % a.n_ctiles;
    const int btile = blockIdx.x / a.n_ctiles;
    const int b0 = btile * BT;
    const int c0 = ctile * a.CT;
    const int nb = min(BT, a.B - b0);
    const int nc = min(a.CT, C - c0);
    const int ldu = a.ldu;
    const int ldh = a.ldh;
    float* us = smem;                  // [BT][ldu]  u_t rows
    float* hs = us + BT * ldu;         // [BT][ldh]  h_prev rows, zero past C
    float* as = hs + BT * ldh;         // [BT][3][CT] pre-activations

    for (int i = threadIdx.x; i < BT * ldu; i += kThreads) {
        const int s = i / ldu;
        const int k = i - s * ldu;
        us[i] = (s < nb && k < n_x) ? a.u_t[((int64_t)b0 + s) * n_x + k] : 0.0f;
    }
    for (int i = threadIdx.x; i < BT * ldh; i += kThreads) {
        const int s = i / ldh;
        const int m = i - s * ldh;
        hs[i] = (s < nb && m < C) ? a.h_prev[((int64_t)b0 + s) * C + m] : 0.0f;
    }
    if (a.h_prev_copy != nullptr && ctile == 0) {
        for (int i = threadIdx.x; i < nb * C; i += kThreads) {
            const int64_t idx = (int64_t)b0 * C + i;
            a.h_prev_copy[idx] = a.h_prev[idx];
        }
    }
    __syncthreads();

    const int grp = threadIdx.x / kHLanes;
    const int j = threadIdx.x % kHLanes;
    constexpr int kRowGroups = kThreads / kHLanes;
    const int rows = 3 * nc;
    for (int r = grp; r < rows; r += kRowGroups) {
        // r is uniform over the 8 lanes of the group.
        const int q = r / nc;
        const int cl = r - q * nc;
        const int wr = q * C + c0 + cl;
        const float* __restrict__ wrow = a.W + (int64_t)wr * n_in;
        float hacc[BT], xacc[BT];
#pragma unroll
        for (int s = 0; s < BT; ++s) hacc[s] = xacc[s] = 0.0f;
        for (int m0 = 4 * j; m0 < C; m0 += 4 * kHLanes) {
            if constexpr (V == 4) {
                const float4 w = *reinterpret_cast<const float4*>(wrow + n_x + m0);
#pragma unroll
                for (int s = 0; s < BT; ++s) {
                    const float4 z = *reinterpret_cast<const float4*>(hs + s * ldh + m0);
                    hacc[s] = fmaf(w.x, z.x, hacc[s]);
                    hacc[s] = fmaf(w.y, z.y, hacc[s]);
                    hacc[s] = fmaf(w.z, z.z, hacc[s]);
                    hacc[s] = fmaf(w.w, z.w, hacc[s]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (m0 + e < C) {
                        const float w = wrow[n_x + m0 + e];
#pragma unroll
                        for (int s = 0; s < BT; ++s) hacc[s] = fmaf(w, hs[s * ldh + m0 + e], hacc[s]);
                    }
                }
            }
        }
        if (j < 4) {
            for (int k = j; k < n_x; k += 4) {
                const float w = wrow[k];
#pragma unroll
                for (int s = 0; s < BT; ++s) xacc[s] = fmaf(w, us[s * ldu + k], xacc[s]);
            }
        }
        const float bq = a.bias[wr];
#pragma unroll
        for (int s = 0; s < BT; ++s) {
            const float hsum = sum8(hacc[s]);
            const float xsum = bq + quad_sum4(xacc[s]);
            if (j == 0) as[(s * 3 + q) * a.CT + cl] = xsum + hsum;
        }
    }
    __syncthreads();

    const int64_t BC = (int64_t)a.B * C;
    for (int i = threadIdx.x; i < nb * nc; i += kThreads) {
        const int s = i / nc;
        const int cl = i - s * nc;
        const int64_t bc = ((int64_t)b0 + s) * C + c0 + cl;
        const CellOut o = cell_forward(as[(s * 3 + 0) * a.CT + cl], as[(s * 3 + 1) * a.CT + cl],
                                       as[(s * 3 + 2) * a.CT + cl]);
        a.h_t[bc] = o.h;
        a.act_t[bc] = o.gate;
        a.act_t[BC + bc] = o.g;
        a.act_t[2 * BC + bc] = o.hh;
    }
}

// ---------------------------------------------------------------------------
// Input projection of the K-loop, all steps at once (fp32 MFMA):
//   X[row, r] = bias[r] + ((x_0 + x_1) + (x_2 + x_3)),
//   x_c = fma chain of W[r, k] u[row, k] over k = c, c + 4, .. (< n_x),
// rows (t, b) of u [K B, n_x], outputs r < 3C.  v_mfma_f32_16x16x4f32
// accumulates its four k in order as an fma chain, so chain c takes the
// columns 16 p + 4 kk + c in k-slot kk of its p-th instruction: every lane
// loads the float4 u[row, 16 p + 4 kk ..] and W[r, 16 p + 4 kk ..] once and
// feeds component c to chain c.  Operand layout (16 x 16 x 4): lane l holds
// A[l % 16][l / 16] and B[l / 16][l % 16]; D[i][j] sits in lane
// j + 16 (i / 4), register i % 4.  Workgroup: 64 rows x 64 outputs, four
// waves of 32 x 32 (2 x 2 MFMA tiles, 4 chains each).  The chains start
// from +0 and zero padding past n_x leaves them unchanged.
// ---------------------------------------------------------------------------
// [persistent kernel source: begin]
// (the tile code is also run by the persistent launch that forms X)
// One 64 x 64 tile (mtile, ntile) of X; wave (0..3) forms its 32 x 32
// block.  The MFMAs take W as their first operand and u as their second,
// so that a lane ends with 4 adjacent outputs of one row (16-byte stores);
// each product and each chain's order are those of the layout above.
// DEV: X stored at device scope (written through to memory), for readers
// in the same launch.
template <bool VEC, bool DEV = false>
__device__ __forceinline__ void xproj_tile(const XprojArgs& a, int64_t mtile, int ntile, int wave)
{
    const int lane = threadIdx.x & 63;
    const int64_t m0 = mtile * 64 + (wave >> 1) * 32;
    const int n0 = ntile * 64 + (wave & 1) * 32;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int n_x = a.n_x;
    const int64_t M = a.M;
    const int N = a.N;

    // the bias first: its load overlaps the operand loads instead of
    // following the MFMAs with a round trip of its own
    float bias[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[nt][e] = a.bias[min(n0 + 16 * nt + 4 * lk + e, N - 1)];

    f32x4 acc[2][2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[mt][nt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Groups of XB blocks of 16 columns: all of a group's operands are loaded
    // before its MFMAs, so their latencies overlap.
    constexpr int XB = 4;
    for (int kg = 0; kg < n_x; kg += 16 * XB) {
        f32x4 av[XB][2], bv[XB][2];
#pragma unroll
        for (int kb = 0; kb < XB; ++kb) {
            const int k = kg + 16 * kb + 4 * lk;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int64_t row = m0 + 16 * mt + li;
                const float* src = a.u + min(row, M - 1) * n_x;
                if (VEC) {
                    av[kb][mt] = load4_or_zero(src + min(k, n_x - 4), row < M && k < n_x);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = src[min(k + e, n_x - 1)];
                        av[kb][mt][e] = (row < M && k + e < n_x) ? x : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int r = n0 + 16 * nt + li;
                const float* src = a.W + (int64_t)min(r, N - 1) * a.n_in;
                if (VEC) {
                    bv[kb][nt] = load4_or_zero(src + min(k, n_x - 4), r < N && k < n_x);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = src[min(k + e, n_x - 1)];
                        bv[kb][nt][e] = (r < N && k + e < n_x) ? x : 0.0f;
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the whole group's loads ahead of its MFMAs
#pragma unroll
        for (int kb = 0; kb < XB; ++kb)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
                        acc[mt][nt][c] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(bv[kb][nt][c], av[kb][mt][c], acc[mt][nt][c], 0, 0, 0);
    }

    wait_vmem_all();   // so that no store below waits behind another
    // lane (li, lk): row m0 + 16 mt + li, outputs n0 + 16 nt + 4 lk .. + 3
    const bool vec_out = (N % 4 == 0) && ((((uintptr_t)a.X) & 15u) == 0);
    const bool dev16 = DEV && vec_out && M * N < (int64_t)(1 << 29);   // byte offsets fit the buffer store's
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int r0 = n0 + 16 * nt + 4 * lk;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int64_t row = m0 + 16 * mt + li;
            if (row >= M) continue;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = xproj_combine(bias[nt][e], acc[mt][nt][0][e], acc[mt][nt][1][e], acc[mt][nt][2][e],
                                     acc[mt][nt][3][e]);
            float* dst = a.X + row * N + r0;
            if (vec_out && r0 + 4 <= N) {
                if (dev16)
                    st4_dev(a.X, (int)(4 * M * N), (int)(4 * (row * N + r0)), v);
                else if (DEV) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) st_agent(dst + e, v[e]);
                } else {
                    *reinterpret_cast<f32x4*>(dst) = v;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (r0 + e < N) {
                        if (DEV)
                            st_agent(dst + e, v[e]);
                        else
                            dst[e] = v[e];
                    }
            }
        }
    }
}

// [persistent kernel source: end]

template <bool VEC>
__global__ __launch_bounds__(kThreads) void xproj_kernel(XprojArgs a)
{
    // the column tiles of a row tile share its u rows: keep them on one XCD
    const int64_t blk = xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
    xproj_tile<VEC>(a, blk / a.n_ntiles, (int)(blk % a.n_ntiles), threadIdx.x >> 6);
}

// ---------------------------------------------------------------------------
// Backward step.  Workgroup = (sample tile, channel tile j).
//  1. dp_q[s, c] for ALL C channels of its samples into LDS (the carry needs
//     every channel; 6 loads per channel, served from L2).
//  2. Either (dp_out != null, K-loop) store the dp of its own channel tile,
//     or (ABI step) update its own scratch rows: gW_s[b, q, c0:c0+nc, :] is
//     one contiguous block of nc * n_in floats per (b, q), streamed with
//     V-wide read-modify-writes; this workgroup is their only writer.
//  3. dz = W^T dp for its share of the columns, in the canonical order:
//     16 slices x 16 columns; slice s forms the channel-group partials P_g of
//     groups g = 4 s .. 4 s + 3 into LDS; then one lane per column takes
//     tree_sum64.
//     Columns [n_x, n_in) give the carry dh_out; [0, n_x) give du_t when
//     requested.  Columns are split evenly over the sample's workgroups.
// ---------------------------------------------------------------------------
template <int BT, int V>
__global__ __launch_bounds__(kThreads) void bwd_step_kernel(BwdArgs a)
{
    extern __shared__ float smem[];
    const int n_in = a.n_x + a.C;
    const int C3 = 3 * a.C;
    const int ctile = blockIdx.x % a.n_ctiles;
    const int btile = blockIdx.x / a.n_ctiles;
    const int b0 = btile * BT;
    const int c0 = ctile * a.CT;
    const int nb = min(BT, a.B - b0);
    const int nc = min(a.CT, a.C - c0);
    const int64_t BC = (int64_t)a.B * a.C;
    float* zs = smem;                    // [BT][ldz]
    float* dps = zs + BT * a.ldz;        // [BT][3C]
    float* red = dps + BT * C3;          // [kDzGroups][BT][kCols]

    if (a.dp_out == nullptr) stage_z<BT>(zs, a.ldz, a.u_t, a.h_prev, b0, nb, a.C, a.n_x);
    for (int i = threadIdx.x; i < BT * a.C; i += kThreads) {
        const int s = i / a.C;
        const int c = i - s * a.C;
        float df = 0.0f, dg = 0.0f, dhh = 0.0f;
        if (s < nb) {
            const int64_t bc = ((int64_t)b0 + s) * a.C + c;
            float dh = a.h_t[bc] - a.y_t[bc];
            if (a.dh_in != nullptr) dh += a.dh_in[bc];
            cell_backward(dh, a.act_t[bc], a.act_t[BC + bc], a.act_t[2 * BC + bc], df, dg, dhh);
        }
        dps[s * C3 + c] = df;
        dps[s * C3 + a.C + c] = dg;
        dps[s * C3 + 2 * a.C + c] = dhh;
    }
    __syncthreads();

    if (a.dp_out != nullptr) {
        for (int i = threadIdx.x; i < nb * 3 * nc; i += kThreads) {
            const int s = i / (3 * nc);
            const int rem = i - s * 3 * nc;
            const int q = rem / nc;
            const int r = q * a.C + c0 + (rem - q * nc);
            a.dp_out[((int64_t)b0 + s) * C3 + r] = dps[s * C3 + r];
        }
    } else {
        const int blk = nc * n_in;
        for (int s = 0; s < nb; ++s) {
            const int64_t b = (int64_t)b0 + s;
            const float* zb = zs + s * a.ldz;
            for (int q = 0; q < 3; ++q) {
                float* __restrict__ dst = a.gW_s + ((b * 3 + q) * a.C + c0) * (int64_t)n_in;
                const float* dq = dps + s * C3 + q * a.C + c0;
                if constexpr (V == 4) {
                    for (int e = threadIdx.x * 4; e < blk; e += kThreads * 4) {
                        const int cl = e / n_in;
                        const int k = e - cl * n_in;
                        const float d = dq[cl];
                        const float4 z = *reinterpret_cast<const float4*>(zb + k);
                        float4 o = *reinterpret_cast<const float4*>(dst + e);
                        o.x = fmaf(d, z.x, o.x);
                        o.y = fmaf(d, z.y, o.y);
                        o.z = fmaf(d, z.z, o.z);
                        o.w = fmaf(d, z.w, o.w);
                        *reinterpret_cast<float4*>(dst + e) = o;
                    }
                } else {
                    for (int e = threadIdx.x; e < blk; e += kThreads) {
                        const int cl = e / n_in;
                        const int k = e - cl * n_in;
                        dst[e] = fmaf(dq[cl], zb[k], dst[e]);
                    }
                }
            }
        }
        for (int i = threadIdx.x; i < nb * 3 * nc; i += kThreads) {
            const int s = i / (3 * nc);
            const int rem = i - s * 3 * nc;
            const int q = rem / nc;
            const int r = q * a.C + c0 + (rem - q * nc);
            const int64_t idx = ((int64_t)b0 + s) * C3 + r;
            a.gb_s[idx] = a.gb_s[idx] + dps[s * C3 + r];
        }
    }

    const int cpg = dz_group_channels(a.C);
    const int klo = (a.du_t != nullptr) ? 0 : a.n_x;
    const int span = n_in - klo;
    const int kw = (span + a.n_ctiles - 1) / a.n_ctiles;
    const int kbeg = klo + ctile * kw;
    const int kend = min(kbeg + kw, n_in);
    const int slice = threadIdx.x / kCols;
    const int col = threadIdx.x % kCols;
    for (int kb = kbeg; kb < kend; kb += kCols) {   // trip count uniform over the workgroup
        const int k = kb + col;
#pragma unroll
        for (int gg = 0; gg < kDzGroups / kSlices; ++gg) {
            const int g = slice * (kDzGroups / kSlices) + gg;
            float P[BT];
#pragma unroll
            for (int s = 0; s < BT; ++s) P[s] = 0.0f;
            if (k < kend) {
                const int c_end = min((g + 1) * cpg, a.C);
                for (int c = g * cpg; c < c_end; ++c) {
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        const int r = q * a.C + c;
                        const float w = a.W[(int64_t)r * n_in + k];
#pragma unroll
                        for (int s = 0; s < BT; ++s) P[s] = fmaf(w, dps[s * C3 + r], P[s]);
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < BT; ++s) red[(g * BT + s) * kCols + col] = P[s];
        }
        __syncthreads();
        if (threadIdx.x < BT * kCols) {
            const int s = threadIdx.x / kCols;
            const int cc = threadIdx.x - s * kCols;
            const int k2 = kb + cc;
            if (s < nb && k2 < kend) {
                const float v = tree_sum64(red + s * kCols + cc, BT * kCols);
                const int64_t b = (int64_t)b0 + s;
                if (k2 >= a.n_x)
                    a.dh_out[b * a.C + (k2 - a.n_x)] = v;
                else
                    a.du_t[b * a.n_x + k2] = v;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// MFMA step path.  Same canonical arithmetic as fwd_step_kernel /
// bwd_step_kernel (fp32 MFMA accumulates its k-slots in order as an fma
// chain), with the operands laid out so that every MFMA operand is a float4.
// ---------------------------------------------------------------------------

// Re-lays W into the forward (Wf) and backward (Wb) operand layouts (see
// MfmaLayout); zeros wherever the canonical chains have no term.
__global__ __launch_bounds__(kThreads) void permute_w_kernel(PermuteArgs a)
{
    const int C = a.C;
    const int n_x = a.n_x;
    const int64_t n_in = (int64_t)n_x + C;
    const MfmaLayout L = a.L;
    const int cpg = dz_group_channels(C);
    const int64_t nf = (int64_t)3 * C * L.ldf;
    const int64_t nb = (int64_t)C * kDzGroups * 16;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nf + nb; i += (int64_t)gridDim.x * kThreads) {
        if (i < nf) {
            const int64_t r = i / L.ldf;
            const int col = (int)(i - r * L.ldf);
            float v = 0.0f;
            if (col < L.nxp) {
                if (col < n_x) v = a.W[r * n_in + col];
            } else {
                const int m = col - L.nxp;   // 32 blk + 8 e + j  <-  recurrent column 32 blk + 4 j + e
                const int src = 32 * (m >> 5) + 4 * (m & 7) + ((m >> 3) & 3);
                if (src < C) v = a.W[r * n_in + n_x + src];
            }
            a.Wf[i] = v;
        } else {
            const int64_t o = i - nf;
            const int k = (int)(o >> 10);            // carry column
            const int g = (int)((o >> 4) & 63);
            const int kk = (int)((o >> 2) & 3);
            const int p = (int)(o & 3);
            const int m = 4 * p + kk;                // element of group g's chain
            float v = 0.0f;
            if (m < 3 * cpg) {
                const int c = g * cpg + m / 3;
                const int q = m - 3 * (m / 3);
                if (c < C) v = a.W[((int64_t)q * C + c) * n_in + n_x + k];
            }
            a.Wb[o] = v;
        }
    }
}

// Moves of the resident kernel (kloop_resident_kernel): its workgroups hand
// h_t, dp_t and the step-K activations to one another through memory while
// they run, so those moves are made at device scope (sc1): write-through
// stores, and loads that the vector L1 does not serve; the step kernels,
// whose launches are ordered by the stream, and the resident kernel's moves
// of a workgroup's own data use plain moves.  (st_agent, above, is the
// 4-byte store.)
//
// [persistent kernel source: begin]
// 16-byte device-scope load through a raw buffer resource over [base, base
// + bytes): one request per 16 bytes, where two 8-byte agent-scope atomic
// loads make two.  Offsets at or past `bytes` read zero.
__device__ __forceinline__ f32x4 ld4_dev(const float* base, int bytes, int byte_off)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */));
}
// [persistent kernel source: end]
// RES: a 16-byte device-scope load (two 8-byte agent-scope loads).
template <bool RES>
__device__ __forceinline__ f32x4 ld4(const float* p)
{
    if constexpr (RES) {
        unsigned long long* q = reinterpret_cast<unsigned long long*>(const_cast<float*>(p));
        const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return f32x4{__int_as_float((int)(unsigned)lo), __int_as_float((int)(unsigned)(lo >> 32)),
                     __int_as_float((int)(unsigned)hi), __int_as_float((int)(unsigned)(hi >> 32))};
    } else {
        return *reinterpret_cast<const f32x4*>(p);
    }
}
// Forward step on MFMA.  Workgroup = 16 samples x 16 channels; three waves
// per head q: part 0 forms the four input chains (x_r: k-slot kk of block p
// is column 16 p + 4 kk + r) and X = bias + ((x0+x1)+(x2+x3)); part 1 the
// recurrent partitions P_0..P_3 and part 2 P_4..P_7 (P_j: k-slot e of block
// i is column n_x + 32 i + 4 j + e), each with its half of sum8.  The cell
// then takes X + (half 1 + half 2): the canonical order.  The lanes' W
// operands come straight from the forward layout into registers; z (u as
// is, h permuted like Wf) is staged in LDS, every load in flight before the
// first LDS store.  Needs n_x, C multiples of 4 and 16-byte aligned rows.  Operand layout (16 x 16 x 4): A[sample l % 16][k-slot l /
// 16], B[k-slot l / 16][channel l % 16]; D[sample i][channel j] in lane
// j + 16 (i / 4), register i % 4.
constexpr int kFwdMfmaThreads = 576;   // three waves per head
constexpr int kMfmaMaxNxb = 8;         // input column blocks of 16: n_x <= 128
constexpr int kMfmaMaxNhb = 10;        // recurrent column blocks of 32: C <= 320
constexpr int kMfmaMaxLdf = 16 * kMfmaMaxNxb + 32 * kMfmaMaxNhb;
constexpr int kFwdMfmaZs = 16 * (kMfmaMaxLdf + 4);   // staged z rows (floats)

// This lane's W operands straight from the forward layout into registers
// (each W value feeds exactly one lane's MFMAs, so it needs no LDS): row
// (head q, channel c0 + li), the four k-slots of every block of the wave's
// part.  Blocks past nxb / nhb load a clamped block, never used.  The bias
// first, in flight with the operand loads (loaded after the MFMAs it was a
// round trip of its own before the epilogue).
__device__ __forceinline__ void fwd_mfma_operands(const FwdMfmaArgs& a, int c0, f32x4 (&wv)[kMfmaMaxNhb],
                                                  float& bias)
{
    const MfmaLayout L = a.L;
    const int C = a.C;
    const int nxb = L.nxp / 16;
    const int nhb = L.cp / 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int q = (tid >> 6) / 3;
    const int part = (tid >> 6) % 3;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const float* wrow = a.Wf + ((int64_t)q * C + min(c0 + li, C - 1)) * L.ldf;
    bias = a.bias[q * C + min(c0 + li, C - 1)];
    static_assert(kMfmaMaxNxb <= kMfmaMaxNhb, "one register block array serves both parts");
#pragma unroll
    for (int i = 0; i < kMfmaMaxNhb; ++i) {
        const int o = (part == 0) ? 16 * max(min(i, nxb - 1), 0) + 4 * lk
                                  : L.nxp + 32 * min(i, nhb - 1) + 8 * lk + 4 * (part - 1);
        wv[i] = *reinterpret_cast<const f32x4*>(wrow + o);
    }
}

// One forward step of the workgroup's tile (btile, ctile) given its W
// operands; zs and as are the step's LDS (kFwdMfmaZs and 3 x 3 x 256 floats).
__device__ __forceinline__ void fwd_mfma_step(const FwdMfmaArgs& a, int btile, int ctile,
                                              const f32x4 (&wv)[kMfmaMaxNhb], float bias, float* zs,
                                              float (*as)[3][16 * 16])
{
    const MfmaLayout L = a.L;
    const int C = a.C;
    const int n_x = a.n_x;
    const int nxb = L.nxp / 16;
    const int nhb = L.cp / 32;
    const int s0 = btile * 16;
    const int c0 = ctile * 16;
    const int ldp = L.ldf + 4;              // row pitch: 4 banks between rows
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int q = (tid >> 6) / 3;       // head
    const int part = (tid >> 6) % 3;    // 0: input chains, 1: P_0..P_3, 2: P_4..P_7 (uniform per wave)
    const int li = lane & 15;
    const int lk = lane >> 4;

    // z rows in float4 units: unit u of row s covers columns 4 u .. 4 u + 3
    // of [u ; h] in their natural order (zero past n_x, past C and for
    // absent samples); h goes to its permuted LDS place.
    {
        const int w4 = L.ldf / 4;
        constexpr int kZSlots = (16 * kMfmaMaxLdf / 4 + kFwdMfmaThreads - 1) / kFwdMfmaThreads;
        f32x4 v[kZSlots];
#pragma unroll
        for (int m = 0; m < kZSlots; ++m) {
            const int i = min(tid + m * kFwdMfmaThreads, 16 * w4 - 1);
            const int s = i / w4;
            const int u4 = i - s * w4;
            const int64_t b = min(s0 + s, a.B - 1);
            const float* src = (4 * u4 < L.nxp) ? a.u_t + b * n_x + min(4 * u4, max(n_x - 4, 0))
                                                : a.h_prev + b * C + min(4 * u4 - L.nxp, C - 4);
            v[m] = *reinterpret_cast<const f32x4*>(src);
        }
#pragma unroll
        for (int m = 0; m < kZSlots; ++m) {
            const int i = tid + m * kFwdMfmaThreads;
            if (i < 16 * w4) {
                const int s = i / w4;
                const int u4 = i - s * w4;
                const bool live = s0 + s < a.B;
                float* row = zs + s * ldp;
                if (4 * u4 < L.nxp) {
                    const bool ok = live && 4 * u4 < n_x;
                    *reinterpret_cast<f32x4*>(row + 4 * u4) = ok ? v[m] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                } else {
                    const int m0 = 4 * u4 - L.nxp;              // recurrent columns m0 .. m0 + 3
                    const bool ok = live && m0 < C;
                    const int base = L.nxp + 32 * (m0 >> 5) + ((m0 & 31) >> 2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) row[base + 8 * e] = ok ? v[m][e] : 0.0f;
                }
            }
        }
    }
    if (a.h_prev_copy != nullptr && ctile == 0) {
        const int nb = min(16, a.B - s0);
        for (int i = tid; i < nb * C; i += kFwdMfmaThreads) {
            const int64_t idx = (int64_t)s0 * C + i;
            a.h_prev_copy[idx] = a.h_prev[idx];
        }
    }
    __syncthreads();

    const float* zr = zs + li * ldp;                 // sample li
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Unrolled over the register-held W blocks; the trip counts are uniform
    // and the blocks past nxb / nhb are never used.
    if (part == 0) {
#pragma unroll
        for (int p = 0; p < kMfmaMaxNxb; ++p) {
            if (p < nxb) {
                const f32x4 zv = *reinterpret_cast<const f32x4*>(zr + 16 * p + 4 * lk);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[c], wv[p][c], acc[c], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMfmaMaxNhb; ++i) {
            if (i < nhb) {
                const f32x4 zv = *reinterpret_cast<const f32x4*>(zr + L.nxp + 32 * i + 8 * lk + 4 * (part - 1));
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[j], wv[i][j], acc[j], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // part 0: X = bias + ((x0 + x1) + (x2 + x3)); parts 1, 2: their half
        // of sum8, (P0 + P1) + (P2 + P3) and (P4 + P5) + (P6 + P7)
        const float v = (part == 0) ? xproj_combine(bias, acc[0][e], acc[1][e], acc[2][e], acc[3][e])
                                    : (acc[0][e] + acc[1][e]) + (acc[2][e] + acc[3][e]);
        as[q][part][(4 * lk + e) * 16 + li] = v;
    }
    __syncthreads();

    const int64_t BC = (int64_t)a.B * C;
    for (int i = tid; i < 256; i += kFwdMfmaThreads) {
        const int s = i >> 4;
        const int cl = i & 15;
        const int b = s0 + s;
        const int c = c0 + cl;
        if (b < a.B && c < C) {
            float pre[3];
#pragma unroll
            for (int h = 0; h < 3; ++h) pre[h] = as[h][0][i] + (as[h][1][i] + as[h][2][i]);   // X + H
            const CellOut o = cell_forward(pre[0], pre[1], pre[2]);
            const int64_t bc = (int64_t)b * C + c;
            a.h_t[bc] = o.h;
            a.act_t[bc] = o.gate;
            a.act_t[BC + bc] = o.g;
            a.act_t[2 * BC + bc] = o.hh;
        }
    }
}

__global__ __launch_bounds__(kFwdMfmaThreads) void fwd_mfma_kernel(FwdMfmaArgs a)
{
    __shared__ __attribute__((aligned(16))) float zs[kFwdMfmaZs];
    __shared__ float as[3][3][16 * 16];   // [head][X, half 1, half 2][sample, channel]
    const int ctile = blockIdx.x % a.n_ctiles;
    const int btile = blockIdx.x / a.n_ctiles;
    f32x4 wv[kMfmaMaxNhb];
    float bias;
    fwd_mfma_operands(a, ctile * 16, wv, bias);
    fwd_mfma_step(a, btile, ctile, wv, bias, zs, as);
}

// Backward step (K-loop: dp out, carry) on MFMA.  Workgroup = 16 samples x
// 16 carry columns.  dp of the tile's samples for every channel goes to LDS
// in the MFMA layout dps[s][g][kk][p] (element 4 p + kk of group g's chain);
// the workgroup stores dp of its own 16 channels.  The canonical subtree T_w
// of dz over groups g = w + 4 m (m = 0..15) is formed by two waves, one per
// half m = 0..7 and m = 8..15: P_g is a chain of PG MFMAs from +0 (the 8
// chains of a wave independent, so their instructions interleave), then
// the first three levels of the pairwise tree of tree_sum16; its last level
// adds the halves.  Then dz = (T0 + T1) + (T2 + T3).
constexpr int kBwdMfmaThreads = 512;   // 4 subtrees x 2 halves of their 16 groups
constexpr int kBwdMfmaDps = 16 * kDzGroups * 16;   // dp of a sample tile in the staged layout
// In LDS a sample's staged dp starts 4 banks after the previous one's, so
// that the 16 samples of a 16-byte operand read fall on distinct banks.
constexpr int kDpsStride = kDzGroups * 16 + 4;
constexpr int kBwdMfmaDpsLds = 16 * kDpsStride;
// The subtree partials [half][subtree][sample][column] at row pitch 20: the
// MFMA tile's stores (samples 4 lk + e, lanes lk = 0..3) fall on distinct
// banks.
constexpr int kTsP = 20;

// This lane's W operands of the carry: the 8 groups g = w + 4 (8 hf + m)
// of its half of subtree w, carry column k0 + li.  Lanes past the 512 that
// form the carry (the resident kernel runs 576) load half 1's, never used.
__device__ __forceinline__ void bwd_mfma_operands(const BwdMfmaArgs& a, int k0, f32x4 (&bv)[8])
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = (tid >> 6) & 3;           // subtree
    const int hf = min(tid >> 8, 1);        // half of the subtree's 16 groups: m = 8 hf .. 8 hf + 7
    const int li = lane & 15;
    const int lk = lane >> 4;
    const float* wb = a.Wb + ((int64_t)min(k0 + li, a.C - 1) * kDzGroups) * 16 + 4 * lk;   // + 16 g
#pragma unroll
    for (int m = 0; m < 8; ++m) bv[m] = *reinterpret_cast<const f32x4*>(wb + 16 * (w + 4 * (8 * hf + m)));
}

// One backward step of the workgroup's tile (btile, ctile); dps and ts are
// its LDS (kBwdMfmaDpsLds and 2 x 4 x 16 x kTsP floats).  The step kernel loads
// the W operands after the dp staging (bv is its own); the resident kernel
// (RES) holds them for every step and reads h, act and dp written by other
// workgroups at agent scope, and also writes dp_{t-1} of its channels to
// the sample tile's exchange block dpx_out in the staged layout, at agent
// scope.  DP: where the step's dp comes from -- kDpRuntime: from dp_in when
// it is not null, else formed from h_t, y_t and act_t (the step kernel);
// kDpIn: the resident kernel's exchange block dpx, copied as it is (the
// positions no channel writes stay zero from the launch); kDpFormed: formed
// (the resident kernel's step K).
constexpr int kDpRuntime = 0, kDpIn = 1, kDpFormed = 2;
template <int PG, bool RES, int DP>
__device__ __forceinline__ void bwd_mfma_step(const BwdMfmaArgs& a, int btile, int ctile, f32x4 (&bv)[8],
                                              float* dps, float (*ts)[4][16][kTsP], float* wstage = nullptr)
{
    const int C = a.C;
    const int cpg = dz_group_channels(C);
    const int s0 = btile * 16;
    const int k0 = ctile * 16;
    int tid = threadIdx.x;
    // the resident kernel runs this body once per step: the per-lane index
    // arithmetic is recomputed each time rather than held in registers
    // across the K steps
    if constexpr (RES) asm volatile("" : "+v"(tid));
    const bool active = !RES || tid < kBwdMfmaThreads;   // uniform per wave
    const int64_t BC = (int64_t)a.B * C;

    // inputs of the epilogue (dp of step t - 1 for (sample tid / 16, channel
    // k0 + tid % 16)), loaded now so that their latency is hidden
    float ep_h = 0.0f, ep_y = 0.0f, ep_g0 = 0.0f, ep_g1 = 0.0f, ep_g2 = 0.0f;
    {
        const int s = (tid >> 4) & 31;
        const int col = tid & 15;
        const int64_t bk = (int64_t)min(s0 + s, a.B - 1) * C + min(k0 + col, C - 1);
        // unconditional loads (a load under a branch is waited for where the
        // branch joins); this step's arrays stand in when there is no step t - 1
        const bool prev = a.dp_prev_out != nullptr;
        const float* hp = prev ? a.h_prev : a.h_t;
        const float* yp = prev ? a.y_prev : a.y_t;
        const float* gp = prev ? a.act_prev : a.act_t;
        // (sample, channel) of this workgroup's own tile: in the resident
        // kernel its own forward wrote them, so plain loads see them
        ep_h = hp[bk];
        ep_y = yp[bk];
        ep_g0 = gp[bk];
        ep_g1 = gp[BC + bk];
        ep_g2 = gp[2 * BC + bk];
    }
    if (DP != kDpIn && active)
        for (int i = tid; i < kBwdMfmaDpsLds; i += kBwdMfmaThreads) dps[i] = 0.0f;
    const int c4n = C / 4;
    if constexpr (DP == kDpIn) {
        constexpr int kXSlots = kBwdMfmaDps / 4 / kBwdMfmaThreads;
        static_assert(kXSlots * 4 * kBwdMfmaThreads == kBwdMfmaDps, "whole passes");
        f32x4 vx[kXSlots];
        if (active) {
#pragma unroll
            for (int m = 0; m < kXSlots; ++m)
                vx[m] = ld4_dev(a.dpx, 4 * kBwdMfmaDps, 16 * (tid + m * kBwdMfmaThreads));
#pragma unroll
            for (int m = 0; m < kXSlots; ++m) {
                const int i = tid + m * kBwdMfmaThreads;   // float4 i of the block: sample i / 256
                *reinterpret_cast<f32x4*>(dps + (i >> 8) * kDpsStride + 4 * (i & 255)) = vx[m];
            }
        }
    } else if (DP == kDpRuntime && a.dp_in != nullptr) {
        // dp of this step, formed at the end of the launch of step t + 1: the
        // tile's samples, all heads and channels (float4 over 4 channels of
        // one head), every load in flight before the LDS stores.
        constexpr int kPSlots = (16 * 3 * 320 / 4 + kBwdMfmaThreads - 1) / kBwdMfmaThreads;
        const int n4 = 16 * 3 * c4n;
        f32x4 vp[kPSlots];
#pragma unroll
        for (int m = 0; m < kPSlots; ++m) {
            const int i = min(tid + m * kBwdMfmaThreads, n4 - 1);
            const int s = i / (3 * c4n);
            const int r4 = i - s * 3 * c4n;   // float4 index within the sample's 3C
            vp[m] = ld4<RES>(a.dp_in + (int64_t)min(s0 + s, a.B - 1) * 3 * C + 4 * r4);
        }
        __syncthreads();   // zeros of dps in place before the dp stores
#pragma unroll
        for (int m = 0; m < kPSlots; ++m) {
            const int i = tid + m * kBwdMfmaThreads;
            const int s = i / (3 * c4n);
            if (active && i < n4 && s0 + s < a.B) {
                const int r4 = i - s * 3 * c4n;
                const int qq = r4 / c4n;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (r4 - qq * c4n) + e;
                    const int g = c / cpg;
                    const int el = 3 * (c - g * cpg) + qq;
                    dps[s * kDpsStride + g * 16 + 4 * (el & 3) + (el >> 2)] = vp[m][e];
                }
            }
        }
    } else {
    // dp of (sample s, channels 4 c4 .. 4 c4 + 3) for the tile's samples and
    // every channel: every load of the pass in flight before the arithmetic.
    constexpr int kDSlots = (16 * 320 / 4 + kBwdMfmaThreads - 1) / kBwdMfmaThreads;
    f32x4 vh[kDSlots], vy[kDSlots], vd[kDSlots], vg0[kDSlots], vg1[kDSlots], vg2[kDSlots];
#pragma unroll
    for (int m = 0; m < kDSlots; ++m) {
        const int i = min(tid + m * kBwdMfmaThreads, 16 * c4n - 1);
        const int s = i / c4n;
        const int64_t bc = (int64_t)min(s0 + s, a.B - 1) * C + 4 * (i - s * c4n);
        vh[m] = ld4<RES>(a.h_t + bc);
        vy[m] = *reinterpret_cast<const f32x4*>(a.y_t + bc);
        vd[m] = (a.dh_in != nullptr) ? *reinterpret_cast<const f32x4*>(a.dh_in + bc) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        vg0[m] = ld4<RES>(a.act_t + bc);
        vg1[m] = ld4<RES>(a.act_t + BC + bc);
        vg2[m] = ld4<RES>(a.act_t + 2 * BC + bc);
    }
    __syncthreads();   // zeros of dps in place before the dp stores
#pragma unroll
    for (int m = 0; m < kDSlots; ++m) {
        const int i = tid + m * kBwdMfmaThreads;
        const int s = i / c4n;
        if (active && i < 16 * c4n && s0 + s < a.B) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 4 * (i - s * c4n) + e;
                float dh = vh[m][e] - vy[m][e];
                if (a.dh_in != nullptr) dh += vd[m][e];
                float d[3];
                cell_backward(dh, vg0[m][e], vg1[m][e], vg2[m][e], d[0], d[1], d[2]);
                const int g = c / cpg;
                const int cl = c - g * cpg;
#pragma unroll
                for (int qq = 0; qq < 3; ++qq) {
                    const int el = 3 * cl + qq;
                    dps[s * kDpsStride + g * 16 + 4 * (el & 3) + (el >> 2)] = d[qq];
                }
                if (c >= k0 && c < k0 + 16) {
                    const int64_t row = (int64_t)(s0 + s) * 3 * C;
#pragma unroll
                    for (int qq = 0; qq < 3; ++qq) a.dp_out[row + qq * C + c] = d[qq];
                }
            }
        }
    }
    }
    __syncthreads();

    if (active) {
        const int lane = tid & 63;
        const int w = (tid >> 6) & 3;   // subtree
        const int hf = (tid >> 8) & 1;  // half of the subtree's 16 groups: m = 8 hf .. 8 hf + 7
        const int li = lane & 15;
        const int lk = lane >> 4;
        if constexpr (!RES || DP == kDpFormed) {
            bwd_mfma_operands(a, k0, bv);
            __builtin_amdgcn_sched_barrier(0);   // the 8 loads ahead of the MFMAs
        }
        const float* da = dps + li * kDpsStride + 4 * lk;   // + 16 g
        // The half's 8 group partials as independent MFMA chains (so that their
        // instructions interleave), then the first three levels of the pairwise
        // tree of tree_sum16; its last level adds the two halves below.
        f32x4 av[8], P[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) av[m] = *reinterpret_cast<const f32x4*>(da + 16 * (w + 4 * (8 * hf + m)));
#pragma unroll
        for (int m = 0; m < 8; ++m) P[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < PG; ++p)
#pragma unroll
            for (int m = 0; m < 8; ++m) P[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m][p], bv[m][p], P[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) P[m] = P[2 * m] + P[2 * m + 1];
#pragma unroll
        for (int m = 0; m < 2; ++m) P[m] = P[2 * m] + P[2 * m + 1];
        const f32x4 T = P[0] + P[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) ts[hf][w][4 * lk + e][li] = T[e];
    }
    __syncthreads();
    if (tid < 256) {
        const int s = tid >> 4;
        const int col = tid & 15;
        const int b = s0 + s;
        const int k = k0 + col;
        if (b < a.B && k < C) {
            float T4[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) T4[v] = ts[0][v][s][col] + ts[1][v][s][col];   // tree_sum16's last level
            const float carry = (T4[0] + T4[1]) + (T4[2] + T4[3]);
            const int64_t bk = (int64_t)b * C + k;
            if (a.dh_out != nullptr) a.dh_out[bk] = carry;
            if (a.dp_prev_out != nullptr) {
                // dp of step t - 1 for channel k, from the carry just formed
                float dh = ep_h - ep_y;
                dh += carry;
                float d[3];
                cell_backward(dh, ep_g0, ep_g1, ep_g2, d[0], d[1], d[2]);
                const int64_t row = (int64_t)b * 3 * C;
#pragma unroll
                for (int qq = 0; qq < 3; ++qq) a.dp_prev_out[row + qq * C + k] = d[qq];
                if constexpr (RES) {
                    const int g = k / cpg;
#pragma unroll
                    for (int qq = 0; qq < 3; ++qq) {
                        const int el = 3 * (k - g * cpg) + qq;
                        const int pos = 4 * (el & 3) + (el >> 2);
                        if (wstage != nullptr)
                            wstage[(s & 3) * 256 + (g - k0 / cpg) * 16 + pos] = d[qq];
                        else
                            st_agent(a.dpx_out + (s * kDzGroups + g) * 16 + pos, d[qq]);
                    }
                }
            }
        }
        if constexpr (RES) {
            if (wstage != nullptr && a.dp_prev_out != nullptr) {
                // this wave's 4 samples of the tile's whole dz groups, read
                // back from its own staging (the wave's LDS moves are ordered)
                // and stored as 16-byte device-scope stores
                const int ng4 = 4 * (16 / cpg);   // float4 per sample
                const int lane = tid & 63;
                for (int i = lane; i < 4 * ng4; i += 64) {
                    const int sl = i / ng4;
                    const int f = i - sl * ng4;
                    const int sg = (tid >> 6) * 4 + sl;   // the sample of the tile
                    st4_dev(a.dpx_out, 4 * kBwdMfmaDps, 4 * ((sg * kDzGroups + k0 / cpg) * 16 + 4 * f),
                            *reinterpret_cast<const f32x4*>(wstage + sl * 256 + 4 * f));
                }
            }
        }
    }
}

template <int PG>
__global__ __launch_bounds__(kBwdMfmaThreads) void bwd_mfma_kernel(BwdMfmaArgs a)
{
    __shared__ __attribute__((aligned(16))) float dps[kBwdMfmaDpsLds];
    __shared__ __attribute__((aligned(16))) float ts[2][4][16][kTsP];   // [half][subtree][sample][column]
    f32x4 bv[8];
    bwd_mfma_step<PG, false, kDpRuntime>(a, blockIdx.x / a.n_ctiles, blockIdx.x % a.n_ctiles, bv, dps, ts);
}

// ---------------------------------------------------------------------------
// Resident MFMA K-loop: each workgroup runs all 2K steps of its (sample
// tile, channel tile) in one cooperative launch with its W operands in
// registers.  Step t of a tile needs h_{t-1} (forward) or dp_t (backward) of
// every channel tile of its samples, so the workgroups of a sample tile
// count their finished steps in `flags` (forward step t: t; backward step t:
// 2K - t + 1) and a step waits until all of them have reached the one it
// needs.  The exchanged arrays move at device scope (see st_agent), and a
// counter is written only after every wave's stores of the step are
// performed, so a workgroup that sees a counter also sees the data behind
// it; no atomics, no cache maintenance.  The backward steps are the
// backward step kernel's body; the forward steps take the input projection
// X (bias included) from xproj_kernel's output and form only the recurrent
// part, one wave per partition (below).  Every sum is the step kernels'
// canonical one, so the bits are theirs.  The launch is cooperative: every
// workgroup is resident, so every wait ends; a wait also gives up after
// spin_limit polls (or once another workgroup has given up), setting the
// error word, so that no failure can keep the kernel running.
// ---------------------------------------------------------------------------
constexpr int kResThreads = kBwdMfmaThreads;   // eight waves
// Forward LDS: h_{t-1} rows [16][cp + 4], u rows [16][nxp + 4], the
// recurrent partials [3][8][16][kResAsP] and X [3][16][kResAsP];
// backward LDS: the step kernel's.  At least 81 KB, so that one workgroup
// sits on each CU (two would share one CU's matrix cores and leave another
// idle).
constexpr int kResHp = 32 * kMfmaMaxNhb + 4;
constexpr int kResUp = 16 * kMfmaMaxNxb + 4;
// partial rows of 16 channels at pitch 20: the MFMA tile's stores (samples
// 4 lk + e, lanes lk = 0..3) fall on distinct banks
constexpr int kResAsP = 20;
constexpr int kResZh = 0, kResZu = 16 * kResHp, kResAs = kResZu + 16 * kResUp,
              kResXs = kResAs + 3 * 8 * 16 * kResAsP;
constexpr int kResFwdLds = kResXs + 3 * 16 * kResAsP;
// + per-wave staging of the dp hand-over: 4 epilogue waves x 4 samples x
// 256 slots
constexpr int kResWs = kBwdMfmaDpsLds + 2 * 4 * 16 * kTsP;
constexpr int kResBwdLds = kResWs + 4 * 4 * 256;
constexpr int kResLdsMin = 81 * 1024 / 4;
constexpr int kResLds = kResFwdLds > kResBwdLds ? (kResFwdLds > kResLdsMin ? kResFwdLds : kResLdsMin)
                                                : (kResBwdLds > kResLdsMin ? kResBwdLds : kResLdsMin);

// The LDS copy of h_{t-1}: recurrent column c = 32 i + 4 m + e of a sample
// sits at 4 (m nhb + i) + e, so that partition m's k-slot e at block i, for
// the 16 samples, is one conflict-free LDS read (row pitch cp + 4) and 4
// consecutive channels (c % 4 = 0..3) land in one float4.
__device__ __forceinline__ int res_hx_pos(int c, int nhb) { return 4 * (((c & 31) >> 2) * nhb + (c >> 5)) + (c & 3); }

// The lane's W operands of the resident forward.  Wave m (0..7) holds, for
// each head q, the B operand of recurrent partition P_m at every block i
// (k-slot lk of block i is recurrent column 32 i + 4 m + lk of channel
// c0 + li, found in the forward layout at the n_x padding + 32 i + 8 lk + m).
// Waves 4..6 form head m - 4's input chains and hold the forward step
// kernel's part-0 operands of that head (wx) and its bias.  Blocks past nhb
// / nxb load a clamped block, never used.
__device__ __forceinline__ void fwd_res_operands(const ResidentArgs& a, int c0, float (&wq)[3][kMfmaMaxNhb],
                                                 f32x4 (&wx)[kMfmaMaxNxb], float& xbias)
{
    const MfmaLayout L = a.L;
    const int C = a.C;
    const int nhb = L.cp / 32;
    const int nxb = L.nxp / 16;
    const int lane = threadIdx.x & 63;
    const int m = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int cl = min(c0 + li, C - 1);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const float* wrow = a.Wf + ((int64_t)q * C + cl) * L.ldf;
#pragma unroll
        for (int i = 0; i < kMfmaMaxNhb; ++i) wq[q][i] = wrow[L.nxp + 32 * min(i, nhb - 1) + 8 * lk + m];
    }
    const int qx = min(max(m - 4, 0), 2);
    const float* xrow = a.Wf + ((int64_t)qx * C + cl) * L.ldf;
#pragma unroll
    for (int p = 0; p < kMfmaMaxNxb; ++p)
        wx[p] = *reinterpret_cast<const f32x4*>(xrow + 16 * max(min(p, nxb - 1), 0) + 4 * lk);
    xbias = a.bias[qx * C + cl];
}

// u_t rows of the tile's samples, one float4 per lane (zero past n_x and
// for absent samples), loaded unconditionally from a clamped address.
// With n_x = 0 nothing is read (u may hold no element).
__device__ __forceinline__ f32x4 res_load_u(const ResidentArgs& a, int t, int s0)
{
    const int w4 = a.L.nxp / 4;
    if (w4 == 0) return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int i = min((int)threadIdx.x, 16 * w4 - 1);
    const int s = i / w4;
    const int k = 4 * (i - s * w4);
    const int b = s0 + s;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.u + ((int64_t)(t - 1) * a.B + min(b, a.B - 1)) * a.n_x +
                                                    min(k, a.n_x - 4));
    return ((int)threadIdx.x < 16 * w4 && b < a.B && k < a.n_x) ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

__device__ __forceinline__ void res_store_u(const ResidentArgs& a, f32x4 v, float* zu)
{
    const int w4 = a.L.nxp / 4;
    if ((int)threadIdx.x < 16 * w4) {
        const int s = threadIdx.x / w4;
        *reinterpret_cast<f32x4*>(zu + s * kResUp + 4 * (threadIdx.x - s * w4)) = v;
    }
}

// Input projection of one step, wave 4 + q for head q (q < 3): the forward
// step kernel's part-0 chains x_r (k-slot kk of block p is input column 16 p
// + 4 kk + r) from the u rows in LDS, then X = bias + ((x0 + x1) + (x2 + x3))
// into xs[q].
__device__ __forceinline__ void res_xproj(const f32x4 (&wx)[kMfmaMaxNxb], float xbias, int nxb, const float* zu,
                                          float (*xs)[16 * kResAsP])
{
    const int lane = threadIdx.x & 63;
    const int q = (threadIdx.x >> 6) - 4;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const float* ur = zu + li * kResUp + 4 * lk;
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < kMfmaMaxNxb; ++p) {
        if (p < nxb) {
            const f32x4 uv = *reinterpret_cast<const f32x4*>(ur + 16 * p);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(uv[c], wx[p][c], acc[c], 0, 0, 0);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        xs[q][(4 * lk + e) * kResAsP + li] = xproj_combine(xbias, acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
}

// One resident forward step t of tile (btile, ctile); X_t is in LDS on
// entry (formed by waves 4..6 from u_t's rows while the workgroup waited for
// the other tiles, or before step 1) and u_{t+1}'s rows on return; uq holds
// this lane's part of u_{t+1} on entry (loaded a step ago) and of u_{t+2} on
// return.  h_{t-1} is copied into LDS from the exchange rows hx (HX) or, at
// t = 1, from h0, its loads issued before u_{t+2}'s.  Wave m forms recurrent
// partition P_m of the three heads (the forward step kernel's chains, with
// their A and B operands) into as[q][m].  Then waves 0..3 run the epilogue,
// pre_q = X_q + (((P0 + P1) + (P2 + P3)) + ((P4 + P5) + (P6 + P7))), the step
// kernel's order, writing h_t to the exchange rows hx_out at device scope and
// h_t, act_t to h_hist and act (at device scope at step K, whose values
// every channel tile reads; plainly before, read again only by this
// workgroup); every lane stores its part of u_{t+1}'s rows.
template <bool HX>
__device__ __forceinline__ void fwd_res_step(const ResidentArgs& a, int t, int btile, int ctile,
                                             const float (&wq)[3][kMfmaMaxNhb], f32x4& uq, float* lds,
                                             const float* hx, float* hx_out)
{
    const int C = a.C;
    const int B = a.B;
    const int cp = a.L.cp;
    const int nhb = cp / 32;
    const int hp = cp + 4;
    const int s0 = btile * 16;
    const int c0 = ctile * 16;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));   // per-step index arithmetic, not held across steps
    const int lane = tid & 63;
    const int m = tid >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int64_t BC = (int64_t)B * C;
    float* zh = lds + kResZh;
    float* zu = lds + kResZu;
    float (*as)[8][16 * kResAsP] = reinterpret_cast<float (*)[8][16 * kResAsP]>(lds + kResAs);
    float (*xs)[16 * kResAsP] = reinterpret_cast<float (*)[16 * kResAsP]>(lds + kResXs);

    // h_{t-1} rows into LDS, every load in flight before the LDS stores.  The
    // exchange rows hold each channel tile's [16 samples][16 channels] block
    // in turn; h0 rows are natural.  Either way float4 idx goes to its
    // partition-major place (res_hx_pos), 4 channels at once.
    const int c4 = cp / 4;
    const int n4 = HX ? 64 * a.n_ctiles : 16 * c4;
    constexpr int kHSlots = (16 * 32 * kMfmaMaxNhb / 4 + kResThreads - 1) / kResThreads;
    static_assert(64 * ((32 * kMfmaMaxNhb + 15) / 16) <= kHSlots * kResThreads, "one pass of slots");
    f32x4 hv4[kHSlots];
#pragma unroll
    for (int k = 0; k < kHSlots; ++k) {
        const int idx = min(tid + k * kResThreads, n4 - 1);
        const int s = idx / c4;
        const int g = idx - s * c4;
        if constexpr (HX) {
            hv4[k] = ld4_dev(hx, 4 * 16 * cp, 16 * idx);
        } else {
            const int b = s0 + s;
            const f32x4 v = *reinterpret_cast<const f32x4*>(a.h0 + (int64_t)min(b, B - 1) * C + min(4 * g, C - 4));
            hv4[k] = (b < B && 4 * g < C) ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    // u_{t+2}'s load, issued after the h loads so that their wait does not
    // include it
    __builtin_amdgcn_sched_barrier(0);
    const f32x4 uq_next = res_load_u(a, min(t + 2, a.K), s0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kHSlots; ++k) {
        const int idx = tid + k * kResThreads;
        if (idx < n4) {
            int s, c;
            if constexpr (HX) {
                s = (idx >> 2) & 15;                    // block idx / 64: channels 16 (idx / 64) ..
                c = 16 * (idx >> 6) + 4 * (idx & 3);
            } else {
                s = idx / c4;
                c = 4 * (idx - s * c4);
            }
            *reinterpret_cast<f32x4*>(zh + s * hp + res_hx_pos(c, nhb)) = hv4[k];
        }
    }
    if (!HX && ctile == 0) {
        const int nb = min(16, B - s0);
        for (int i = tid; i < nb * C; i += kResThreads) {
            const int64_t idx = (int64_t)s0 * C + i;
            st_agent(a.h_hist + idx, a.h0[idx]);
        }
    }
    __syncthreads();

    f32x4 acc[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* zr = zh + li * hp + 4 * (m * nhb) + lk;
#pragma unroll
    for (int i = 0; i < kMfmaMaxNhb; ++i) {
        if (i < nhb) {
            const float hv = zr[4 * i];
#pragma unroll
            for (int q = 0; q < 3; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(hv, wq[q][i], acc[q], 0, 0, 0);
        }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) as[q][m][(4 * lk + e) * kResAsP + li] = acc[q][e];
    __syncthreads();

    if (tid < 256) {
        const int es = tid >> 4;
        const int b = s0 + es;
        const int c = c0 + (tid & 15);
        if (b < B && c < C) {
            float pre[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const float* P = &as[q][0][es * kResAsP + (tid & 15)];
                constexpr int M = 16 * kResAsP;   // one partition's rows
                const float h1 = (P[0 * M] + P[1 * M]) + (P[2 * M] + P[3 * M]);
                const float h2 = (P[4 * M] + P[5 * M]) + (P[6 * M] + P[7 * M]);
                pre[q] = xs[q][es * kResAsP + (tid & 15)] + (h1 + h2);
            }
            const CellOut o = cell_forward(pre[0], pre[1], pre[2]);
            const int64_t bc = (int64_t)b * C + c;
            float* h_t = a.h_hist + (int64_t)t * BC;
            float* act_t = a.act + (int64_t)(t - 1) * 3 * BC;
            st_agent(hx_out + ctile * 256 + tid, o.h);   // the tile's block: sample es, channel c
            if (t < a.K) {
                // read again only by this workgroup (its backward epilogue)
                h_t[bc] = o.h;
                act_t[bc] = o.gate;
                act_t[BC + bc] = o.g;
                act_t[2 * BC + bc] = o.hh;
            } else {
                // step K: every channel tile of the sample tile forms dp_K from them
                st_agent(h_t + bc, o.h);
                st_agent(act_t + bc, o.gate);
                st_agent(act_t + BC + bc, o.g);
                st_agent(act_t + 2 * BC + bc, o.hh);
            }
        }
    }
    res_store_u(a, uq, zu);   // X_t's reads of u_t ended before this step began
    uq = uq_next;
}

// Wave 0 polls the counters of the sample tile's nct workgroups (one lane
// each; the other lanes read the error word, in the same round trip) until
// all reach `need`, or a workgroup has given up; the other waves wait at the
// barrier.  Each counter has a cache line of its own (kResFlagStride ints
// apart), so that the tile's writers do not contend for one line; one poll
// in flight at a time (more slowed the counters' stores).
__device__ __forceinline__ void resident_wait(int* flags, int base, int nct, int err, int need, int spin_limit)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const bool counter = lane < nct;
        int* p = flags + kResFlagStride * (counter ? base + lane : err);
        for (int it = 0;; ++it) {
            const int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__all(!counter || v >= need) || __any(!counter && v != 0)) break;
            if (it >= spin_limit) {
                if (lane == 0) __hip_atomic_store(flags + kResFlagStride * err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    lds_barrier();
}

// Every wave's stores of the step performed, then the workgroup's counter.
__device__ __forceinline__ void resident_report(int* flags, int pos, int steps)
{
    wait_vmem_all();
    lds_barrier();
    if (threadIdx.x == 0) __hip_atomic_store(flags + kResFlagStride * pos, steps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int PG>
__global__ __launch_bounds__(kResThreads) void kloop_resident_kernel(ResidentArgs a)
{
    // the forward's and the backward's LDS share one buffer (the wait before
    // the first backward step orders the last forward reads before it)
    __shared__ __attribute__((aligned(16))) float lds[kResLds];
    const int nct = a.n_ctiles;
    // the channel tiles of a sample tile hand one another h_t and dp_t: keep
    // them on one XCD where the grid allows
    const int v = (int)xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
    const int ctile = v % nct;
    const int btile = v / nct;
    const int base = btile * nct;
    const int err = gridDim.x;
    const int K = a.K;
    const int64_t BC = (int64_t)a.B * a.C;
    {
        float wq[3][kMfmaMaxNhb];
        f32x4 wx[kMfmaMaxNxb];
        float xbias;
        fwd_res_operands(a, ctile * 16, wq, wx, xbias);
        float (*xs)[16 * kResAsP] = reinterpret_cast<float (*)[16 * kResAsP]>(lds + kResXs);
        const bool xw = threadIdx.x >= 256 && threadIdx.x < 448;   // waves 4..6
        // X_1 (the barriers of step 1 order it before its reads)
        res_store_u(a, res_load_u(a, 1, btile * 16), lds + kResZu);
        f32x4 uq = res_load_u(a, min(2, K), btile * 16);
        __syncthreads();
        if (xw) res_xproj(wx, xbias, a.L.nxp / 16, lds + kResZu, xs);
        // h_t of the sample tile in the exchange rows, by the parity of t
        const int64_t hx_tile = (int64_t)16 * a.L.cp;
        const int64_t hx_par = (int64_t)gridDim.x / nct * hx_tile;
        float* hx = a.hx + btile * hx_tile;
        fwd_res_step<false>(a, 1, btile, ctile, wq, uq, lds, nullptr, hx + hx_par);
        for (int t = 2; t <= K; ++t) {
            resident_report(a.flags, base + ctile, t - 1);
            // X_t from the u rows step t - 1 stored, while wave 0 waits
            if (xw) res_xproj(wx, xbias, a.L.nxp / 16, lds + kResZu, xs);
            resident_wait(a.flags, base, nct, err, t - 1, a.spin_limit);
            fwd_res_step<true>(a, t, btile, ctile, wq, uq, lds, hx + ((t - 1) & 1) * hx_par,
                               hx + (t & 1) * hx_par);
        }
        resident_report(a.flags, base + ctile, K);
    }
    {
        float* dps = lds;
        float (*ts)[4][16][kTsP] = reinterpret_cast<float (*)[4][16][kTsP]>(lds + kBwdMfmaDpsLds);
        BwdMfmaArgs g{};
        g.Wb = a.Wb;
        g.B = a.B;
        g.C = a.C;
        g.n_ctiles = nct;
        g.L = a.L;
        // dp_t of the sample tile in the staged layout, by the parity of t
        const int64_t dpx_par = (int64_t)gridDim.x / nct * kBwdMfmaDps;
        float* dpx = a.dpx + btile * (int64_t)kBwdMfmaDps;
        auto set_step = [&](int t) {
            g.dpx = dpx + (t & 1) * dpx_par;
            g.dpx_out = dpx + ((t - 1) & 1) * dpx_par;
            g.h_t = a.h_hist + (int64_t)t * BC;
            g.y_t = a.y + (int64_t)(t - 1) * BC;
            g.act_t = a.act + (int64_t)(t - 1) * 3 * BC;
            g.dp_out = a.dp + (int64_t)(t - 1) * 3 * BC;
            g.dp_in = (t == K) ? nullptr : a.dp + (int64_t)(t - 1) * 3 * BC;
            g.h_prev = (t > 1) ? a.h_hist + (int64_t)(t - 1) * BC : nullptr;
            g.y_prev = (t > 1) ? a.y + (int64_t)(t - 2) * BC : nullptr;
            g.act_prev = (t > 1) ? a.act + (int64_t)(t - 2) * 3 * BC : nullptr;
            g.dp_prev_out = (t > 1) ? a.dp + (int64_t)(t - 2) * 3 * BC : nullptr;
        };
        // t = K: every forward step done; dp formed from h, y and act, the W
        // operands loaded after that staging (as the step kernel does) and
        // then kept for the steps that read dp_t of every channel tile
        f32x4 bv[8];
        // the dp hand-over goes through per-wave LDS staging and 16-byte
        // stores when every dz group lies in one channel tile (its channel
        // count divides 16); staging slots that no channel writes stay zero
        const int cpg = dz_group_channels(a.C);
        float* wstage = nullptr;
        if (16 % cpg == 0) {
            for (int i = threadIdx.x; i < 4 * 4 * 256; i += kResThreads) lds[kResWs + i] = 0.0f;
            wstage = lds + kResWs + (threadIdx.x >> 6) * 4 * 256;   // used by waves 0..3
        }
        resident_wait(a.flags, base, nct, err, K, a.spin_limit);
        set_step(K);
        bwd_mfma_step<PG, true, kDpFormed>(g, btile, ctile, bv, dps, ts, wstage);
        for (int t = K - 1; t >= 1; --t) {
            resident_report(a.flags, base + ctile, 2 * K - t);   // step t + 1 done
            resident_wait(a.flags, base, nct, err, 2 * K - t, a.spin_limit);
            set_step(t);
            bwd_mfma_step<PG, true, kDpIn>(g, btile, ctile, bv, dps, ts, wstage);
        }
    }
}

// ---------------------------------------------------------------------------
// Deferred scratch fill (K-loop): S[b, r, k] = fma chain over t = K .. 1 of
// dp_t[b, r] * z_t[b, k] from +0 -- the same bits as K per-step "+=" updates
// of a zeroed scratch -- and Sb[b, r] = add chain of dp_t[b, r].  Per sample
// this is the product dp_b^T z_b over the K steps, written once in 64 x 64
// tiles.  A workgroup takes one sample's row tile (64 rows of dp) and
// kt_per of its column tiles (64 columns of z each), one after the other.
// Steps are staged in LDS kFillSteps at a time, t descending.  The next
// pass's operands are loaded into registers while the current pass's
// MFMAs run, so a tile's load latency hides behind the previous tile's
// work.  Each wave accumulates a 32 x 32 block with v_mfma_f32_16x16x4f32,
// whose four k-slots are taken in order as an fma chain: slot kk of the
// instruction at staged step tt is step t0 - tt - kk.  Steps past the last multiple of 4 go through VALU fma on
// the same accumulators.  Operand layout (16 x 16 x 4): lane l holds
// A[l % 16][l / 16] and B[l / 16][l % 16]; D[i][j] sits in lane
// j + 16 (i / 4), register i % 4.  The tile leaves through LDS (the z
// buffer) as coalesced rows.
// ---------------------------------------------------------------------------
constexpr int kFillPitch = kFillTile + 16;   // staged row pitch: the 4 k-slots of a read hit distinct banks
constexpr int kFillSeg = kFillSteps * 32 / kThreads;   // 16-byte dp and z segments per thread and pass
static_assert(kFillSteps * 32 % kThreads == 0, "whole staging passes");

__global__ __launch_bounds__(kThreads, 4) void scratch_fill_kernel(FillArgs a)
{
    __shared__ __attribute__((aligned(16))) float dps[kFillSteps][kFillPitch];
    __shared__ __attribute__((aligned(16))) float zs[kFillSteps][kFillPitch];
    const int n_in = a.n_x + a.C;
    const int R3 = 3 * a.C;
    const int n_kg = (a.n_kt + a.kt_per - 1) / a.kt_per;   // column-tile groups per row tile
    const int groups = a.n_rt * n_kg;
    // a sample's tiles share its dp rows and z columns: keep them on one XCD
    const int blk = (int)xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
    const int b = blk / groups;
    const int rem = blk - b * groups;
    const int rt = rem / n_kg;
    const int kt0 = (rem - rt * n_kg) * a.kt_per;
    const int npass = (a.K + kFillSteps - 1) / kFillSteps;
    const int items = min(a.kt_per, a.n_kt - kt0) * npass;   // (column tile, pass) pairs in order
    const int r0 = rt * kFillTile;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int wr = 32 * (wave >> 1);   // the wave's 32 x 32 block of the tile
    const int wc = 32 * (wave & 1);
    // 16-byte staging needs every 4-float segment to lie inside one row of one tensor
    const bool vec = (R3 % 4 == 0) && (a.n_x % 4 == 0) && (a.C % 4 == 0) &&
                     ((((uintptr_t)a.dp) | ((uintptr_t)a.u) | ((uintptr_t)a.h_hist)) & 15u) == 0;

    // Item it's dp rows and z columns, kFillSeg 16-byte segments per thread
    // (32 per staged step: 16 of dp, 16 of z), all in flight at once,
    // clamped into bounds; vok[m] false outside the tile's rows, columns
    // and steps.  The zero select waits until the values go to LDS, so the
    // loads of the next item stay in flight through the current MFMAs.
    f32x4 v[kFillSeg];
    bool vok[kFillSeg];
    // A thread's segments share their column (sgi = threadIdx.x % 32) and
    // differ in the staged step only: one base address per item, one
    // step stride.
    const int sgi = threadIdx.x & 31;
    const bool is_dp = sgi < 16;
    const int x = 4 * (sgi & 15);
    auto issue = [&](int it) __attribute__((always_inline)) {
        const int k0 = (kt0 + it / npass) * kFillTile;
        const int t0 = a.K - (it % npass) * kFillSteps;
        const int nst = min(kFillSteps, t0);
        // base, row length and column picked by selects, not branches: the
        // loads issue back to back
        const int r = r0 + x;
        const int k = min(k0 + x, n_in - 4);
        const bool is_u = k < a.n_x;
        const float* base = is_dp ? a.dp : (is_u ? a.u : a.h_hist);
        const int len = is_dp ? R3 : (is_u ? a.n_x : a.C);
        const int col = is_dp ? min(r, R3 - 4) : (is_u ? k : k - a.n_x);
        const bool inside = is_dp ? r < R3 : k0 + x < n_in;
        const float* p0 = base + (int64_t)b * len + col;
        const int64_t step = (int64_t)a.B * len;   // floats from step t to t + 1
#pragma unroll
        for (int m = 0; m < kFillSeg; ++m) {
            const int tt = (threadIdx.x >> 5) + m * (kThreads / 32);
            const int t = t0 - min(tt, nst - 1) - 1;   // clamped into bounds
            v[m] = *reinterpret_cast<const f32x4*>(p0 + t * step);
            vok[m] = tt < nst && inside;
        }
    };
    auto place = [&]() __attribute__((always_inline)) {
        float* row0 = is_dp ? &dps[threadIdx.x >> 5][x] : &zs[threadIdx.x >> 5][x];
#pragma unroll
        for (int m = 0; m < kFillSeg; ++m)
            *reinterpret_cast<f32x4*>(row0 + m * (kThreads / 32) * kFillPitch) =
                vok[m] ? v[m] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };

    const bool vec_out = (n_in % 4 == 0) && ((((uintptr_t)a.gW_s) & 15u) == 0);

    f32x4 acc[2][2];
    float sb = 0.0f;
    if (vec) issue(0);
    for (int it = 0; it < items; ++it) {
        const int j = it / npass;
        const int p = it - j * npass;
        const int k0 = (kt0 + j) * kFillTile;
        const int t0 = a.K - p * kFillSteps;
        const int nst = min(kFillSteps, t0);   // steps t0, t0 - 1, .., t0 - nst + 1
        const bool do_bias = (kt0 + j == 0) && (threadIdx.x < kFillTile);
        if (vec) {
            place();
        } else {
            for (int i = threadIdx.x; i < kFillSteps * kFillTile; i += kThreads) {
                const int tt = i / kFillTile;
                const int x = i - tt * kFillTile;
                float dv = 0.0f, zv = 0.0f;
                if (tt < nst) {
                    const int64_t tb = (int64_t)(t0 - tt - 1) * a.B + b;
                    const int r = r0 + x;
                    if (r < R3) dv = a.dp[tb * R3 + r];
                    const int k = k0 + x;
                    if (k < n_in)
                        zv = (k < a.n_x) ? a.u[tb * a.n_x + k] : a.h_hist[tb * a.C + (k - a.n_x)];
                }
                dps[tt][x] = dv;
                zs[tt][x] = zv;
            }
        }
        __syncthreads();
        if (vec && it + 1 < items) issue(it + 1);   // in flight during this pass's MFMAs
        if (p == 0) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            sb = 0.0f;
        }
        const int nst4 = nst & ~3;
        // operands of the next 4 steps read while the current MFMAs run
        // (two operand sets in turn, so that no copy waits for a read)
        float a0[2], b0[2], a1[2], b1[2];
        auto rd = [&](int tt, float (&av)[2], float (&bv)[2]) __attribute__((always_inline)) {
            const int r = min(tt, kFillSteps - 4) + lk;   // in bounds; unused past nst4
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) av[mt] = dps[r][wr + 16 * mt + li];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) bv[nt] = zs[r][wc + 16 * nt + li];
        };
        auto mma = [&](const float (&av)[2], const float (&bv)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
        };
        rd(0, a0, b0);
        int tt = 0;
        for (; tt + 8 <= nst4; tt += 8) {
            rd(tt + 4, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mma(a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            rd(tt + 8, a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            mma(a1, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (tt < nst4) mma(a0, b0);   // nst4 % 8 == 4
        for (int tt = nst4; tt < nst; ++tt) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[mt][nt][e] = fmaf(dps[tt][wr + 16 * mt + 4 * lk + e], zs[tt][wc + 16 * nt + li], acc[mt][nt][e]);
        }
        if (do_bias)
            for (int tt = 0; tt < nst; ++tt) sb = sb + dps[tt][threadIdx.x];
        if (p == npass - 1) {
            // The tile through LDS (zs reused as [64][kFillPitch]) for row-wise
            // stores: 16 lanes write one 256-byte row segment, whole cache
            // lines (stores from the accumulators' layout, 64 bytes per row,
            // wrote 1.43 times the scratch's bytes to HBM).
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) zs[wr + 16 * mt + 4 * lk + e][wc + 16 * nt + li] = acc[mt][nt][e];
            __syncthreads();
            // every LDS read of the tile first, then the stores (one LDS wait, not one per store)
            constexpr int kOut = kFillTile * (kFillTile / 4) / kThreads;
            static_assert(kFillTile * (kFillTile / 4) % kThreads == 0, "whole output passes");
            f32x4 ov[kOut];
#pragma unroll
            for (int m = 0; m < kOut; ++m) {
                const int u = threadIdx.x + m * kThreads;
                const int row = u / (kFillTile / 4);
                ov[m] = *reinterpret_cast<const f32x4*>(&zs[row][4 * (u - row * (kFillTile / 4))]);
            }
#pragma unroll
            for (int m = 0; m < kOut; ++m) {
                const int u = threadIdx.x + m * kThreads;
                const int row = u / (kFillTile / 4);
                const int c4 = 4 * (u - row * (kFillTile / 4));
                const int r = r0 + row;
                const int k = k0 + c4;
                if (r < R3 && k < n_in) {
                    float* dst = a.gW_s + ((int64_t)b * R3 + r) * n_in + k;
                    if (vec_out && k + 4 <= n_in) {
                        __builtin_nontemporal_store(ov[m], reinterpret_cast<f32x4*>(dst));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k + e < n_in) dst[e] = ov[m][e];
                    }
                }
            }
            if (do_bias && r0 + (int)threadIdx.x < R3) a.gb_s[(int64_t)b * R3 + r0 + threadIdx.x] = sb;
        }
        __syncthreads();   // LDS free for the next item's operands
    }
}

// [persistent kernel source: begin]
// ---------------------------------------------------------------------------
// Persistent K-loop kernel: workgroup b runs sample b's whole step; the input
// projection X = W_x u + bias of every step comes precomputed (xproj_kernel),
// so the recurrence only carries the recurrent columns.
// 512 lanes = 64 groups of 8 (half a DPP row).  Group g is canonical dz group
// g: channels g CPG .. g CPG + CPG - 1, all three heads.  Their recurrent W
// columns sit in registers as lane j's canonical columns 32 i + 4 j + e.
// Quad jq of the group looks after channel g CPG + jq; lane fn of the quad
// evaluates the channel's nonlinearity fn (gate, g, hh) in the forward and
// sums the interleaved dz subtree fn of its column in the backward.
// The step loops touch no global memory.  Steps run in chunks; at each chunk
// boundary the workgroup
//   - moves the chunk's inputs into LDS from registers, where they were
//     loaded during the previous chunk (X rows for the forward; gate, g, hh,
//     h_t, y_t for the backward),
//   - writes the previous chunk's outputs from LDS to memory with coalesced
//     16-byte stores (h_t and (gate, g, hh); dp_t),
//   - issues the loads of the next chunk's inputs,
// so every wait on memory at a boundary is for operations a whole chunk old.
// Inside a chunk a step is LDS traffic, DPP, arithmetic and one LDS-only
// barrier.
//  forward, per t : 3 CPG recurrent chains per lane; sum8 leaves every lane
//                   of the group with every H; lane fn of quad jq forms
//                   a = X + H of (head fn, its channel) and the nonlinearity;
//                   the quad exchanges the three by DPP and forms h_t, which
//                   goes into the next z buffer and, with (gate, g, hh), into
//                   the chunk's output buffer.
//  backward, per t: quad jq computes dp of its channel from the carry it
//                   summed itself; the group reads both channels' dp back
//                   with ds_swizzle; the group's partial P_g over the carry
//                   columns goes to a double-buffered LDS block; after the
//                   barrier lane fn of quad jq sums subtree fn of its
//                   channel's column (groups fn, fn + 4, ..) and quad_sum4
//                   completes the carry.
// ---------------------------------------------------------------------------
constexpr int kFwdChunk = 16;
constexpr int kBwdChunk = 16;

// 16-byte global load and store at a byte address (global address space:
// a plain pointer made from an integer would be a flat access, which also
// counts on the LDS wait counter).
typedef __attribute__((address_space(1))) f32x4 global_f32x4;
__device__ __forceinline__ f32x4 gload4(uint64_t addr) { return *(const global_f32x4*)addr; }
__device__ __forceinline__ void gstore4(uint64_t addr, f32x4 v) { *(global_f32x4*)addr = v; }
// The same store at device scope (write-through, as st4_dev) at a byte
// address inside [base, base + bytes), for rows that workgroups on other
// XCDs of the same launch read.
__device__ __forceinline__ void gstore4_dev(const float* base, int bytes, uint64_t addr, f32x4 v)
{
    st4_dev(const_cast<float*>(base), bytes, (int)(addr - (uint64_t)base), v);
}

template <int CPG, int NH>
struct PersistLds {
    static constexpr int HW = 32 * NH;           // recurrent columns held (>= C)
    static constexpr int HWP = HW + 8;           // partial row pitch: 8 banks between group rows
    static constexpr int STAGE = (5 * HW * kBwdChunk > 3 * HW * kFwdChunk) ? 5 * HW * kBwdChunk : 3 * HW * kFwdChunk;
    static constexpr int DBUF = kBwdChunk * 3 * HW;
    static constexpr size_t BYTES = sizeof(float) * (2 * HW + 2 * kDzGroups * HWP + STAGE + DBUF);
    static_assert(4 * HW * kFwdChunk <= 2 * kDzGroups * HWP, "forward output buffer fits in the partials");
    static_assert(HW <= 64 * CPG, "every channel belongs to a group");
};

// Coalesced move of `rows` rows of `len` floats between LDS (row pitch
// `pitch` >= len) and global memory (row rr at gptr(rr)); 16-byte moves when
// vec.
template <int THREADS, bool TO_GLOBAL, typename Ptr>
__device__ __forceinline__ void move_rows(float* lds, int rows, int len, int pitch, bool vec, Ptr gptr)
{
    if (vec) {
        const int w = len / 4;
        for (int i = threadIdx.x; i < rows * w; i += THREADS) {
            const int rr = i / w;
            const int x = 4 * (i - rr * w);
            float* g = gptr(rr) + x;
            if (TO_GLOBAL)
                *reinterpret_cast<f32x4*>(g) = *reinterpret_cast<const f32x4*>(lds + rr * pitch + x);
            else
                *reinterpret_cast<f32x4*>(lds + rr * pitch + x) = *reinterpret_cast<const f32x4*>(g);
        }
    } else {
        for (int i = threadIdx.x; i < rows * len; i += THREADS) {
            const int rr = i / len;
            const int x = i - rr * len;
            if (TO_GLOBAL)
                gptr(rr)[x] = lds[rr * pitch + x];
            else
                lds[rr * pitch + x] = gptr(rr)[x];
        }
    }
}

// Lane SRC (0..7) of this lane's aligned 8-lane group (ds_swizzle bit mode:
// and_mask 0x18 keeps the group within the 32-lane half, or_mask picks SRC).
template <int SRC>
__device__ __forceinline__ float group_bcast(float v)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x18 | (SRC << 5)));
}

// The last three levels of tree_sum16 over p[0], p[s], .., p[7 s] (the level-1
// pair sums of the canonical dz subtree), with all 8 LDS reads issued before
// the first add (the empty asm takes every value as an operand, so no read
// can sink below it): ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)).
__device__ __forceinline__ float tree_sum8_loads_first(const float* p, int s)
{
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = p[i * s];
    asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                 "+v"(r[7]));
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = r[2 * i] + r[2 * i + 1];
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// The backward cell's factors that do not depend on the carry, for one
// channel at one staged step (rows gate, g, hh, h_t, y_t at pitch HW):
// cell_backward's operations, split so that only
//   dh = r + carry;  df = (dh A) Bf;  dg = (dh G) Fg;  dhh = (dh H) Fh
// remain once the carry is known (the same operations in the same order,
// hence the same bits).
struct BwdFactors {
    float r, A, Bf, G, Fg, H, Fh;
};

template <int HW>
__device__ __forceinline__ BwdFactors bwd_factors(const float* st, int c)
{
    const float gate = st[c], g = st[HW + c], hh = st[2 * HW + c];
    BwdFactors f;
    f.r = st[3 * HW + c] - st[4 * HW + c];
    f.A = g - hh;
    f.Bf = -gate * (1.0f - gate);
    f.G = gate;
    f.Fg = fmaf(-g, g, 1.0f);
    f.H = 1.0f - gate;
    f.Fh = fmaf(-hh, hh, 1.0f);
    return f;
}

// The projection workgroups of a launch that also forms X (n_proj > 0):
// workgroup p forms tile (p / n_nt, p % n_nt) of X (64 rows (t, b) x 64
// outputs) with xproj_kernel's code and device-scope stores, on waves 0-3
// (one wave per SIMD, as in xproj_kernel: two would share each SIMD's
// matrix core), then, once every wave's stores are performed, sets
// flags[p] = call.
__device__ __forceinline__ void persist_projection(const PersistArgs& a)
{
    const int N = 3 * a.C;
    const int n_nt = (N + 63) / 64;
    const XprojArgs x{a.u, a.W, a.bias, const_cast<float*>(a.X), (int64_t)a.K * a.B, N, a.n_x, a.n_x + a.C, n_nt};
    // the column tiles of a row tile share its u rows: keep them on one XCD
    const int p = (int)xcd_local_order(blockIdx.x, (int64_t)a.n_proj);
    const bool vec = (a.n_x % 4 == 0) && ((a.n_x + a.C) % 4 == 0) &&
                     ((((uintptr_t)a.u) | ((uintptr_t)a.W)) & 15u) == 0;
    if (threadIdx.x < 256) {
        if (vec)
            xproj_tile<true, true>(x, p / n_nt, p % n_nt, threadIdx.x >> 6);
        else
            xproj_tile<false, true>(x, p / n_nt, p % n_nt, threadIdx.x >> 6);
    }
    wait_vmem_all();
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(a.flags + blockIdx.x, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A sample workgroup of such a launch, before its first read of X: wave 0
// polls the n_proj flags and the error word after them until every flag
// holds this launch's call number, or a wait has given up (error word ==
// call); after spin_limit polls it gives up itself and marks the error
// word.  A poll's loads (64 words each, up to kPollLoads of them) are in
// flight together, and two polls are in flight at once, the second issued
// half a round trip after the first, so that flags set between two polls
// are seen about half a round trip sooner.  The other waves wait at the
// barrier.  X is then read with plain loads: it was written through to
// memory, and no cache on this workgroup's CU or XCD holds a line of it
// (they start each launch empty of it, and nothing here reads X before
// this wait).
constexpr int kPollLoads = 4;
__device__ __forceinline__ void persist_poll(const PersistArgs& a, int base, int (&v)[kPollLoads])
{
#pragma unroll
    for (int m = 0; m < kPollLoads; ++m)
        v[m] = __hip_atomic_load(a.flags + min(base + 64 * m + (int)threadIdx.x, a.n_proj), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
}
// 1: every flag of the words [base, base + 64 kPollLoads) holds call; 2: the
// error word among them does; 0: neither
__device__ __forceinline__ int persist_poll_state(const PersistArgs& a, int base, const int (&v)[kPollLoads])
{
    const int call = (int)a.call;
    int ok = 1, gave_up = 0;
#pragma unroll
    for (int m = 0; m < kPollLoads; ++m) {
        const int i = base + 64 * m + (int)threadIdx.x;
        ok &= __all(i >= a.n_proj || v[m] == call) ? 1 : 0;
        gave_up |= __any(i == a.n_proj && v[m] == call) ? 1 : 0;
    }
    return gave_up ? 2 : ok;
}
__device__ __forceinline__ void persist_wait_projection(const PersistArgs& a)
{
    if (threadIdx.x < 64) {
        // groups of 64 kPollLoads words, one after another; within a group
        // two polls in flight (A, B)
        for (int base = 0; base <= a.n_proj; base += 64 * kPollLoads) {
            int va[kPollLoads], vb[kPollLoads];
            persist_poll(a, base, va);
            __builtin_amdgcn_s_sleep(16);   // about 1k cycles: half a round trip
            int st = 0;
            // one poll (A) in flight at the top of every pass, so that each
            // check waits for its own poll only
            for (int it = 0;; it += 2) {
                persist_poll(a, base, vb);
                st = persist_poll_state(a, base, va);
                if (st) break;
                persist_poll(a, base, va);
                st = persist_poll_state(a, base, vb);
                if (st) break;
                if (it >= a.spin_limit) {
                    if (threadIdx.x == 0)
                        __hip_atomic_store(a.flags + a.n_proj, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    st = 2;
                    break;
                }
            }
            if (st == 2) break;   // this wait or another gave up: no further group is waited for
        }
    }
    __syncthreads();
}

// A fill unit's wait for one chunk flag: wave 0 polls the flag (lane 0)
// and the error word (lane 1) until either holds this launch's call number;
// after spin_limit polls it gives up itself and marks the error word.  Two
// polls in flight, the second issued about half a round trip after the
// first, each check waiting for its own poll only (as in the projection
// wait).  The other waves wait at the barrier.
__device__ __forceinline__ int persist_fill_poll(const PersistArgs& a, int word)
{
    return __hip_atomic_load(a.flags + (threadIdx.x == 0 ? word : a.n_proj), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void persist_fill_wait(const PersistArgs& a, int word)
{
    if (threadIdx.x < 64) {
        const int call = (int)a.call;
        auto seen = [&](int v) __attribute__((always_inline)) {
            return __builtin_amdgcn_readlane(v, 0) == call || __builtin_amdgcn_readlane(v, 1) == call;
        };
        int va = persist_fill_poll(a, word);
        __builtin_amdgcn_s_sleep(16);
        for (int it = 0;; it += 2) {
            const int vb = persist_fill_poll(a, word);
            if (seen(va)) break;
            va = persist_fill_poll(a, word);
            if (seen(vb)) break;
            if (it >= a.spin_limit) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(a.flags + a.n_proj, call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Fill unit f of a launch that also forms the scratch: sample b = f / n_rt,
// dp rows r0 = 64 (f % n_rt) .. r0 + 63 against every column of z, i.e.
// the tiles (b, r0 / 64, *) of scratch_fill_kernel with its arithmetic:
// per output an fma chain over t = K .. 1 from +0, the steps in k-slot
// groups of 4 from t = K through v_mfma_f32_16x16x4f32 (slot kk of the
// group at staged step tt is step t0 - tt - kk) and the last K mod 4 steps
// through VALU fma, and the bias sums as an add chain over t descending.
// A pass stages one backward chunk (16 steps): the groups and the order are
// those of the fill's 64-step passes, hence the same bits.  Wave w holds
// rows 32 (w & 1) .. + 31 and 16-column blocks npw (w >> 1) .. + npw - 1.
// dp and h_hist come from the sample workgroups of this launch and are read
// with device-scope loads after the chunk's flag; u is an input.
__device__ __forceinline__ void persist_fill(const PersistArgs& a, int f, float* lds)
{
    const int C = a.C, n_x = a.n_x, n_in = n_x + C, R3 = 3 * C, B = a.B, K = a.K;
    const bool vec = (C % 4 == 0) && (n_x % 4 == 0) && n_in <= 256 &&
                     ((((uintptr_t)a.dp) | ((uintptr_t)a.h_hist) | ((uintptr_t)a.u) | ((uintptr_t)a.gW_s)) & 15u) == 0;
    if (!vec) {   // the host does not fuse such shapes
        if (threadIdx.x == 0)
            __hip_atomic_store(a.flags + a.n_proj, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int n_rt = (R3 + 63) / 64;
    const int b = f / n_rt;
    const int r0 = (f - b * n_rt) * 64;
    const int nc = (K + kBwdChunk - 1) / kBwdChunk;
    const int zp = persist_fill_zpitch(n_in);
    constexpr int DPP = 80;            // dp row pitch
    float* dps = lds;                  // [16][DPP]
    float* zs = lds + 16 * DPP;        // [16][zp]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int rw = 32 * (wave & 1);
    const int npw = ((n_in + 15) / 16 + 3) / 4;
    const int cb0 = 16 * npw * (wave >> 1);
    const int nb = min(npw, max(0, (n_in - cb0 + 15) / 16));   // uniform per wave
    const int w4 = n_in / 4;
    const int dp_bytes = (int)((int64_t)K * B * R3 * 4);       // below 2^31 (host)
    const int h_bytes = (int)((int64_t)(K + 1) * B * C * 4);
    f32x4 acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float sb = 0.0f;
    for (int c = 0; c < nc; ++c) {
        const int t0 = K - kBwdChunk * c;
        const int nst = min(kBwdChunk, t0);   // steps t0, t0 - 1, .., t0 - nst + 1
        persist_fill_wait(a, a.n_proj + 1 + b * nc + c);
        // dp: threads < 256, one float4 each; z: two float4 per thread.
        // Addresses clamped into bounds; LDS rows past nst are never read.
        f32x4 dv;
        {
            const int t = t0 - min(tid >> 4, nst - 1);
            const int r = min(r0 + 4 * (tid & 15), R3 - 4);
            dv = ld4_dev(a.dp, dp_bytes, (int)((((int64_t)(t - 1) * B + b) * R3 + r) * 4));
        }
        f32x4 zv[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = tid + m * kPersistThreads;
            const int tq = i / w4;
            const int k = 4 * (i - tq * w4);
            const int t = t0 - min(tq, nst - 1);
            const int64_t row = (int64_t)(t - 1) * B + b;
            const f32x4 hv = ld4_dev(a.h_hist, h_bytes, (int)((row * C + max(k - n_x, 0)) * 4));
            f32x4 uv = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (n_x > 0) uv = *reinterpret_cast<const f32x4*>(a.u + row * n_x + min(k, n_x - 4));
            zv[m] = (k < n_x) ? uv : hv;
        }
        wait_vmem_all();
        if (tid < 256) *reinterpret_cast<f32x4*>(dps + (tid >> 4) * DPP + 4 * (tid & 15)) = dv;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = tid + m * kPersistThreads;
            if (i < 16 * w4) {
                const int tq = i / w4;
                *reinterpret_cast<f32x4*>(zs + tq * zp + 4 * (i - tq * w4)) = zv[m];
            }
        }
        __syncthreads();
        const int nst4 = nst & ~3;
        for (int tt = 0; tt < nst4; tt += 4) {
            float av[2], bv[4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) av[mt] = dps[(tt + lk) * DPP + rw + 16 * mt + li];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) bv[nt] = zs[(tt + lk) * zp + min(cb0 + 16 * nt, zp - 16) + li];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    if (nt < nb) acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
        }
        for (int tt = nst4; tt < nst; ++tt) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    if (nt < nb) {
                        const float zval = zs[tt * zp + cb0 + 16 * nt + li];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[mt][nt][e] = fmaf(dps[tt * DPP + rw + 16 * mt + 4 * lk + e], zval, acc[mt][nt][e]);
                    }
        }
        if (tid < 64)
            for (int tt = 0; tt < nst; ++tt) sb = sb + dps[tt * DPP + tid];
        __syncthreads();   // LDS free for the next pass
    }
    // The unit through LDS in four rounds of 16 rows, each stored row-wise
    // (16 lanes per 256 bytes: whole cache lines).  Row pitch: the wave's
    // whole 16-column blocks, plus 4 (a round's writes hit distinct banks).
    const int op = ((n_in + 15) & ~15) + 4;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        if ((wave & 1) == (rb >> 1)) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                if (nt < nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) lds[(4 * lk + e) * op + cb0 + 16 * nt + li] = acc[rb & 1][nt][e];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int i = tid + m * kPersistThreads;
            const int row = i / w4;
            const int k = 4 * (i - row * w4);
            const int r = r0 + 16 * rb + row;
            if (i < 16 * w4 && r < R3) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(lds + row * op + k);
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(a.gW_s + ((int64_t)b * R3 + r) * n_in + k));
            }
        }
        __syncthreads();
    }
    if (tid < 64 && r0 + tid < R3) a.gb_s[(int64_t)b * R3 + r0 + tid] = sb;
}

template <int CPG, int NH>
__global__ __launch_bounds__(kPersistThreads) void kloop_persist_kernel(PersistArgs a)
{
    using L = PersistLds<CPG, NH>;
    constexpr int THREADS = kPersistThreads;
    constexpr int HW = L::HW;
    constexpr int HWP = L::HWP;
    static_assert(THREADS == kDzGroups * kHLanes, "one 8-lane group per canonical dz group");
    __shared__ __attribute__((aligned(16))) float zs[2][HW];
    __shared__ __attribute__((aligned(16))) float part[2][kDzGroups][HWP];
    __shared__ __attribute__((aligned(16))) float stage[L::STAGE];
    __shared__ __attribute__((aligned(16))) float dbuf[L::DBUF];
    float* obuf = &part[0][0][0];   // forward output buffer [kFwdChunk][4][C] (partials unused then)
    const int n_help = max(a.n_proj, a.n_fill);
    if ((int)blockIdx.x < n_help) {
        if ((int)blockIdx.x < a.n_proj) persist_projection(a);
        // a sample's fill units on one XCD, where they share its u rows
        const int f = (int)xcd_local_order(blockIdx.x, (int64_t)n_help);
        if (f < a.n_fill) persist_fill(a, f, &part[0][0][0]);
        return;
    }
    const int b = (int)blockIdx.x - n_help;
    const int tid = threadIdx.x;
    const int g = tid >> 3;          // canonical dz group
    const int j = tid & 7;           // lane of the group: recurrent columns 32 i + 4 j + e
    const int jq = j >> 2;           // quad of the group
    const int fn = j & 3;            // lane of the quad
    const int C = a.C;
    const int n_x = a.n_x;
    const int n_in = n_x + C;
    const int B = a.B;
    const int K = a.K;
    const int R3 = 3 * C;
    const int cq = g * CPG + jq;                 // the quad's channel
    const bool q_ok = (jq < CPG) && (cq < C);
    const int cqc = min(cq, C - 1);              // clamped for addressing
    const int64_t BC = (int64_t)B * C;
    const bool wvec = (n_x % 4 == 0) && (n_in % 4 == 0) && ((((uintptr_t)a.W) & 15u) == 0);
    // 16-byte moves need rows of a multiple of 4 floats on 16-byte aligned arrays
    const bool c_vec = (C % 4 == 0) && ((((uintptr_t)a.act) | ((uintptr_t)a.h_hist) | ((uintptr_t)a.y) |
                                          ((uintptr_t)a.dp) | ((uintptr_t)a.X)) & 15u) == 0;
    // fill units in this launch read h_t and dp: device-scope stores, and a
    // flag per backward chunk (the host fuses 16-byte shapes only)
    const bool fuse = a.n_fill > 0 && c_vec;
    const int h_bytes = (int)((int64_t)(K + 1) * BC * 4);   // below 2^31 when fused (host)
    const int dp_bytes = (int)((int64_t)K * BC * 12);
    if (a.n_fill > 0 && !c_vec && tid == 0)
        __hip_atomic_store(a.flags + a.n_proj, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // w[s]: the recurrent columns of channel g CPG + s; in the forward, with
    // CPG == 2, quad 1 holds them swapped (w[s] of channel g CPG + (s ^ jq))
    // so that the last level of sum8 can leave each quad its own channel.
    float w[CPG][3][NH][4];
    if (wvec) {
        // clamped addresses, zero selected: no branch between the loads,
        // so all of them are in flight together (under a per-load branch
        // each was waited for before the next was issued)
#pragma unroll
        for (int cl = 0; cl < CPG; ++cl)
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int c = g * CPG + (CPG == 2 ? (cl ^ jq) : cl);
                const float* wrow = a.W + (int64_t)(q * C + min(c, C - 1)) * n_in + n_x;
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const int m = 32 * i + 4 * j;   // C % 4 == 0 here: m < C covers m + 3
                    const f32x4 v = load4_or_zero(wrow + min(m, C - 4), c < C && m < C);
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[cl][q][i][e] = v[e];
                }
            }
    } else {
#pragma unroll
        for (int cl = 0; cl < CPG; ++cl)
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int c = g * CPG + (CPG == 2 ? (cl ^ jq) : cl);
                const bool ok = c < C;
                const float* wrow = a.W + (int64_t)(q * C + min(c, C - 1)) * n_in + n_x;
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const int m = 32 * i + 4 * j;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[cl][q][i][e] = (ok && m + e < C) ? wrow[min(m + e, C - 1)] : 0.0f;
                }
            }
    }
    // Backward: staged rows per step tt of a chunk: 5 tt + v, v = gate, g, hh (act), h_t,
    // y_t, each C floats at row pitch HW (so that, in a whole chunk, every
    // step's LDS offsets are constants); register prefetch on the 16-byte path.
    const int c_w = C / 4;
    const int c_col = c_w > 0 ? tid % c_w : 0;
    const int c_row0 = c_w > 0 ? tid / c_w : 5 * kBwdChunk;
    const int c_rstep = c_w > 0 ? THREADS / c_w : 1;
    constexpr int CRS_MIN = THREADS / (HW / 4);
    constexpr int BPF = (5 * kBwdChunk + CRS_MIN - 1) / CRS_MIN;
    f32x4 bpf[BPF];
    auto in_row = [&](int t1) {
        return [=](int rr) {
            const int tt = rr / 5;
            const int v = rr - 5 * tt;
            const int t = t1 - tt;
            const float* src = (v < 3) ? a.act + (int64_t)(t - 1) * 3 * BC + v * BC
                             : (v == 3) ? a.h_hist + (int64_t)t * BC : a.y + (int64_t)(t - 1) * BC;
            return const_cast<float*>(src) + (int64_t)b * C;
        };
    };
    auto dp_row = [&](int t1) {
        return [=](int tt) { return a.dp + ((int64_t)(t1 - tt - 1) * B + b) * R3; };
    };
    // Per-thread addresses of the backward boundary moves (16-byte path),
    // computed once as in the forward: the input rows of a whole chunk (row
    // rr clamped to the chunk's last; act for v < 3, else h_hist or y;
    // without the term of step t1), and dp, where float4 move m of this
    // thread is element i = tid + m THREADS of the chunk's [nt][3C / 4] block.
    constexpr int DM = (kBwdChunk * 3 * HW / 4 + THREADS - 1) / THREADS;
    uint64_t i_addr[BPF];
    int i_act[BPF];
    uint64_t d_addr[DM];
    int d_tt[DM], d_lds[DM];
    if (c_vec) {
#pragma unroll
        for (int m = 0; m < BPF; ++m) {
            const int rr = min(c_row0 + m * c_rstep, 5 * kBwdChunk - 1);
            const int tt = rr / 5;
            const int v = rr - 5 * tt;
            i_act[m] = v < 3;
            const int64_t off = (v < 3 ? (int64_t)(-tt - 1) * 3 * BC + (int64_t)v * BC
                                       : v == 3 ? (int64_t)(-tt) * BC : (int64_t)(-tt - 1) * BC) +
                                (int64_t)b * C + 4 * c_col;
            i_addr[m] = (uint64_t)(v < 3 ? a.act : v == 3 ? a.h_hist : a.y) + 4 * (uint64_t)off;
        }
        const int w4 = R3 / 4;
#pragma unroll
        for (int m = 0; m < DM; ++m) {
            const int i = tid + m * THREADS;
            const int tt = i / w4;
            const int xq = i - tt * w4;
            d_tt[m] = tt;
            d_lds[m] = min(tt, kBwdChunk - 1) * R3 + 4 * xq;
            d_addr[m] = (uint64_t)a.dp + 4 * (uint64_t)((int64_t)b * R3 + 4 * xq - (int64_t)(tt + 1) * B * R3);
        }
    }
    // the backward's per-thread map is computed here, while W is in flight
    // (it is integer work the step loops never repeat), and pinned so that
    // it is not moved to the backward
    if (c_vec) {
#pragma unroll
        for (int m = 0; m < BPF; ++m) asm volatile("" : "+v"(i_addr[m]), "+v"(i_act[m]));
#pragma unroll
        for (int m = 0; m < DM; ++m) asm volatile("" : "+v"(d_addr[m]), "+v"(d_tt[m]), "+v"(d_lds[m]));
    }
    for (int i = tid; i < 2 * HW; i += THREADS) (&zs[0][0])[i] = 0.0f;
    __syncthreads();
    for (int c = tid; c < C; c += THREADS) {
        const float h = a.h0[(int64_t)b * C + c];
        zs[0][c] = h;
        st_agent(a.h_hist + (int64_t)b * C + c, h);   // read by fill units of a fused launch
    }
    wait_vmem_all();   // W is in registers before any step loop reads it

    // ---------------- forward ----------------
    // X prefetch into registers: a lane moves one float4 of one staged row
    // of 3C floats per pass, on a map computed once (16-byte path only).
    // A row is x_w <= 3 HW / 4 float4; the lanes cover x_rstep rows per pass.
    // In LDS a row is staged per head at pitch HW ([tt][head][HW]), so that,
    // in a whole chunk, every step's LDS offsets are constants.
    const int x_w = R3 / 4;
    const int x_col = x_w > 0 ? tid % x_w : 0;
    const int x_lds = ((4 * x_col) / C) * HW + (4 * x_col) % C;   // C % 4 == 0 on this path
    const int x_row0 = x_w > 0 ? tid / x_w : kFwdChunk;
    const int x_rstep = x_w > 0 ? THREADS / x_w : 1;
    constexpr int XRS_MIN = THREADS / (3 * HW / 4);
    constexpr int XPF = (kFwdChunk + XRS_MIN - 1) / XRS_MIN;
    f32x4 xpf[XPF];
    auto x_row = [&](int t0) {
        return [=](int rr) { return const_cast<float*>(a.X) + ((int64_t)(t0 - 1 + rr) * B + b) * R3; };
    };
    // Chunk-boundary moves on the 16-byte path use per-thread addresses
    // computed once here, so that each move at a boundary is one 64-bit
    // add of a uniform multiple of the chunk's first step (no division, no
    // per-row choice of array; a per-lane choice between two pointer
    // arguments made the compiler reload the pointer and wait for it at
    // every move).  Unsigned byte addresses: the per-thread part may point
    // before the array; the step's term brings it back in bounds.
    //  - X rows of a whole chunk (row clamped as in load_x's general case);
    //  - the forward outputs: float4 move m of this thread is element
    //    i = tid + m THREADS of the chunk's [4 nt][C / 4] block, whose row
    //    rr = 4 tt + v holds h_t (v = 0) or gate, g, hh (v = 1..3) of step
    //    t0 + tt; its LDS offset is clamped into the block for rows past it.
    constexpr int OM = (kFwdChunk * HW + THREADS - 1) / THREADS;
    uint64_t x_addr[XPF];
    uint64_t o_addr[OM];
    int o_rr[OM], o_lds[OM];
    bool o_act[OM];
    if (c_vec) {
#pragma unroll
        for (int m = 0; m < XPF; ++m) {
            const int rr = min(x_row0 + m * x_rstep, kFwdChunk - 1);
            x_addr[m] = (uint64_t)a.X + 4 * (uint64_t)(((int64_t)(rr - 1) * B + b) * R3 + 4 * x_col);
        }
        const int w4 = C / 4;   // C % 4 == 0 on this path
#pragma unroll
        for (int m = 0; m < OM; ++m) {
            const int i = tid + m * THREADS;
            const int rr = i / w4;
            const int xq = i - rr * w4;
            const int v = rr & 3;
            const int tq = rr >> 2;
            o_rr[m] = rr;
            o_lds[m] = min(rr, 4 * kFwdChunk - 1) * HW + 4 * xq;
            o_act[m] = v != 0;
            const int64_t off = (v == 0 ? (int64_t)tq * BC : (int64_t)(tq - 1) * 3 * BC + (int64_t)(v - 1) * BC) +
                                (int64_t)b * C + 4 * xq;
            o_addr[m] = (uint64_t)(v == 0 ? a.h_hist : a.act) + 4 * (uint64_t)off;
        }
    }
    auto load_x = [&](int t0, int nt) {
        if (nt == kFwdChunk) {
            const uint64_t t0o = 4 * (uint64_t)((int64_t)t0 * B * R3);
#pragma unroll
            for (int m = 0; m < XPF; ++m) xpf[m] = gload4(x_addr[m] + t0o);
            return;
        }
        const auto src = x_row(t0);
#pragma unroll
        for (int m = 0; m < XPF; ++m) {
            const int rr = x_row0 + m * x_rstep;
            // clamped into bounds; rows past the chunk are loaded but never staged
            xpf[m] = *reinterpret_cast<const f32x4*>(src(min(rr, nt - 1)) + 4 * x_col);
        }
    };
    // the chunk's outputs from LDS to h_hist and act (16-byte path): every
    // LDS read first, then the stores of the rows inside the chunk
    auto store_out = [&](int t0, int nt) {
        const uint64_t sh = 4 * (uint64_t)((int64_t)t0 * BC);
        const uint64_t sa = 3 * sh;
        f32x4 v[OM];
#pragma unroll
        for (int m = 0; m < OM; ++m) v[m] = *reinterpret_cast<const f32x4*>(obuf + o_lds[m]);
        if (fuse) {   // h_t rows at device scope (fill units read them); act rows stay local
#pragma unroll
            for (int m = 0; m < OM; ++m)
                if (o_rr[m] < 4 * nt) {
                    if (o_act[m]) gstore4(o_addr[m] + sa, v[m]);
                    else gstore4_dev(a.h_hist, h_bytes, o_addr[m] + sh, v[m]);
                }
        } else {
#pragma unroll
            for (int m = 0; m < OM; ++m)
                if (o_rr[m] < 4 * nt) gstore4(o_addr[m] + (o_act[m] ? sa : sh), v[m]);
        }
    };
    auto out_row = [&](int t0) {
        return [=](int rr) {
            const int t = t0 + (rr >> 2);
            const int v = rr & 3;   // h_t, gate, g, hh
            return (v == 0 ? a.h_hist + (int64_t)t * BC : a.act + (int64_t)(t - 1) * 3 * BC + (v - 1) * BC) +
                   (int64_t)b * C;
        };
    };
    if (a.n_proj > 0) persist_wait_projection(a);   // X is formed by this launch
    if (c_vec && K >= 1) load_x(1, min(kFwdChunk, K));
    int prev_t0 = 0, prev_nt = 0;
    // With K a whole number of chunks the backward's first chunk (steps K ..
    // K - 15) is the forward's last: it is handed over in LDS from the
    // forward's output buffer, with y_t loaded during that chunk, instead of
    // being stored and loaded back after the forward.
    static_assert(kBwdChunk == kFwdChunk, "the last forward chunk is the first backward chunk");
    const bool first_from_lds = (K >= kBwdChunk) && (K % kBwdChunk == 0);
    f32x4 ypf = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int t0 = 1; t0 <= K; t0 += kFwdChunk) {
        const int nt = min(kFwdChunk, K - t0 + 1);
        wait_vmem_all();   // loads and stores issued a whole chunk ago; none waits below
        if (c_vec) {
#pragma unroll
            for (int m = 0; m < XPF; ++m) {
                const int rr = x_row0 + m * x_rstep;
                if (x_row0 < x_rstep && rr < nt)
                    *reinterpret_cast<f32x4*>(stage + rr * 3 * HW + x_lds) = xpf[m];
            }
        } else {
            const auto src = x_row(t0);
            for (int i = tid; i < nt * R3; i += THREADS) {
                const int rr = i / R3;
                const int x = i - rr * R3;
                const int hd = x / C;
                stage[rr * 3 * HW + hd * HW + (x - hd * C)] = src(rr)[x];
            }
        }
        if (prev_nt > 0) {
            if (c_vec) store_out(prev_t0, prev_nt);
            else move_rows<THREADS, true>(obuf, 4 * prev_nt, C, HW, false, out_row(prev_t0));
        }
        if (c_vec && t0 + kFwdChunk <= K) load_x(t0 + kFwdChunk, min(kFwdChunk, K - t0 - kFwdChunk + 1));
        // y of backward row c_row0 (step K - c_row0) during the last chunk
        if (c_vec && first_from_lds && t0 + kFwdChunk > K && c_row0 < kBwdChunk)
            ypf = *reinterpret_cast<const f32x4*>(a.y + ((int64_t)(K - c_row0 - 1) * B + b) * C + 4 * c_col);
        lds_barrier();
        // One step; t0 - 1 is even, so h_{t-1} sits in zs[tt & 1].
        static_assert(kFwdChunk % 2 == 0, "chunks start on odd t");
        auto fstep = [&](int tt) __attribute__((always_inline)) {
            const float* zc = zs[tt & 1];
            float* zn = zs[(tt + 1) & 1];
            const float xv = stage[tt * 3 * HW + min(fn, 2) * HW + cqc];
            f32x4 zv[NH];
#pragma unroll
            for (int i = 0; i < NH; ++i) zv[i] = *reinterpret_cast<const f32x4*>(zc + 32 * i + 4 * j);
            float hs[CPG][3];
#pragma unroll
            for (int cl = 0; cl < CPG; ++cl)
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    float p = 0.0f;
#pragma unroll
                    for (int i = 0; i < NH; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) p = fmaf(w[cl][q][i][e], zv[i][e], p);
                    hs[cl][q] = (CPG == 2) ? quad_sum4(p) : sum8(p);
                }
            float hsel;
            if constexpr (CPG == 2) {
                // sum8's last level, kept by the quad that owns the channel:
                // slot 0 is the quad's own channel, and the mirrored lane of
                // the other quad holds the same channel in its slot 1, so
                // own + mirror(other) is sum8's own + partner, bit for bit.
                float hq[3];
#pragma unroll
                for (int q = 0; q < 3; ++q) hq[q] = hs[0][q] + dpp_get<kDppRowHalfMirror>(hs[1][q]);
                hsel = (fn == 0) ? hq[0] : (fn == 1) ? hq[1] : hq[2];
            } else {
                hsel = (fn == 0) ? hs[0][0] : (fn == 1) ? hs[0][1] : hs[0][2];
            }
            const float v = cell_fn(fn, xv + hsel);
            // lane 0 of the quad (the only one that uses h) holds the gate itself
            const float h = cell_h(v, quad_bcast<1>(v), quad_bcast<2>(v));
            if (q_ok) {
                float* ob = obuf + (tt * 4) * HW + cq;
                if (fn == 0) {
                    zn[cq] = h;
                    ob[0] = h;
                }
                if (fn < 3) ob[(1 + fn) * HW] = v;
            }
            lds_barrier();
        };
#pragma unroll
        for (int tt = 0; tt < kFwdChunk; ++tt)
            if (tt < nt) fstep(tt);
        prev_t0 = t0;
        prev_nt = nt;
    }
    // the stores of the chunks before the last (issued a chunk ago) have
    // landed: after the barrier below the backward may load those rows
    wait_vmem_all();
    if (first_from_lds) {
        // backward row tt (step K - tt): gate, g, hh, h_t from forward row
        // 15 - tt of the output buffer (h_t, gate, g, hh), y_t from ypf
        if (c_vec) {
            if (c_row0 < kBwdChunk) {
                const float* o = obuf + (kBwdChunk - 1 - c_row0) * 4 * HW + 4 * c_col;
                float* st = stage + c_row0 * 5 * HW + 4 * c_col;
                const f32x4 oh = *reinterpret_cast<const f32x4*>(o);
                const f32x4 og = *reinterpret_cast<const f32x4*>(o + HW);
                const f32x4 o2 = *reinterpret_cast<const f32x4*>(o + 2 * HW);
                const f32x4 o3 = *reinterpret_cast<const f32x4*>(o + 3 * HW);
                *reinterpret_cast<f32x4*>(st) = og;
                *reinterpret_cast<f32x4*>(st + HW) = o2;
                *reinterpret_cast<f32x4*>(st + 2 * HW) = o3;
                *reinterpret_cast<f32x4*>(st + 3 * HW) = oh;
                *reinterpret_cast<f32x4*>(st + 4 * HW) = ypf;
            }
        } else {
            for (int tt = 0; tt < kBwdChunk; ++tt)
                for (int c = tid; c < C; c += THREADS) {
                    const float* o = obuf + (kBwdChunk - 1 - tt) * 4 * HW + c;
                    float* st = stage + tt * 5 * HW + c;
                    st[0] = o[HW];
                    st[HW] = o[2 * HW];
                    st[2 * HW] = o[3 * HW];
                    st[3 * HW] = o[0];
                    st[4 * HW] = a.y[((int64_t)(K - tt - 1) * B + b) * C + c];
                }
        }
    }
    if (prev_nt > 0) {
        if (c_vec) store_out(prev_t0, prev_nt);
        else move_rows<THREADS, true>(obuf, 4 * prev_nt, C, HW, false, out_row(prev_t0));
    }
    // otherwise the backward's first loads read the rows just stored, some
    // by other waves: each wave's stores land before the barrier
    if (!first_from_lds) wait_vmem_all();
    __syncthreads();   // the handed-over chunk is visible; obuf is free

    if constexpr (CPG == 2) {
        // back to the canonical slots: w[s] of channel g CPG + s in every quad
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int i = 0; i < NH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a0 = w[0][q][i][e], a1 = w[1][q][i][e];
                    w[0][q][i][e] = jq ? a1 : a0;
                    w[1][q][i][e] = jq ? a0 : a1;
                }
    }

    // ---------------- backward ----------------
    // the chunk's dp from LDS to memory (16-byte path): LDS reads first
    auto store_dp = [&](int t1, int nt) {
        const uint64_t t1o = 4 * (uint64_t)((int64_t)t1 * B * R3);
        f32x4 v[DM];
#pragma unroll
        for (int m = 0; m < DM; ++m) v[m] = *reinterpret_cast<const f32x4*>(dbuf + d_lds[m]);
        if (fuse) {
#pragma unroll
            for (int m = 0; m < DM; ++m)
                if (d_tt[m] < nt) gstore4_dev(a.dp, dp_bytes, d_addr[m] + t1o, v[m]);
        } else {
#pragma unroll
            for (int m = 0; m < DM; ++m)
                if (d_tt[m] < nt) gstore4(d_addr[m] + t1o, v[m]);
        }
    };
    auto load_b = [&](int t1, int nt) {
        if (nt == kBwdChunk) {
            const uint64_t sh = 4 * (uint64_t)((int64_t)t1 * BC);
            const uint64_t sa = 3 * sh;
#pragma unroll
            for (int m = 0; m < BPF; ++m) bpf[m] = gload4(i_addr[m] + (i_act[m] ? sa : sh));
            return;
        }
        const auto src = in_row(t1);
#pragma unroll
        for (int m = 0; m < BPF; ++m) {
            const int rr = c_row0 + m * c_rstep;
            // clamped into bounds; rows past the chunk are loaded but never staged
            bpf[m] = *reinterpret_cast<const f32x4*>(src(min(rr, 5 * nt - 1)) + 4 * c_col);
        }
    };
    if (c_vec && K >= 1 && !first_from_lds) load_b(K, min(kBwdChunk, K));
    float carry_mine = 0.0f;   // the carry of the quad's channel
    int prev_t1 = 0;
    prev_nt = 0;
    // chunk flags (fused launch): the wait at the boundary of chunk ci covers
    // the dp stores of chunk ci - 2, which are published after its barrier;
    // in the last chunk, chunk ci - 1 after step kPub, once every wave has
    // waited for its stores (issued kPub steps before: performed by then);
    // chunks not yet published go after the last chunk's stores
    constexpr int kPub = 10;
    const int nchunks = (K + kBwdChunk - 1) / kBwdChunk;
    int* const cflags = a.flags + a.n_proj + 1 + b * nchunks;
    int ci = 0, published = 0;
    for (int t1 = K; t1 >= 1; t1 -= kBwdChunk) {
        const int nt = min(kBwdChunk, t1);   // steps t1, t1 - 1, .., t1 - nt + 1
        if (!first_from_lds || t1 != K) {
            wait_vmem_all();   // loads and stores issued a whole chunk ago; none waits below
            if (c_vec) {
#pragma unroll
                for (int m = 0; m < BPF; ++m) {
                    const int rr = c_row0 + m * c_rstep;
                    if (c_row0 < c_rstep && rr < 5 * nt)
                        *reinterpret_cast<f32x4*>(stage + rr * HW + 4 * c_col) = bpf[m];
                }
            } else {
                move_rows<THREADS, false>(stage, 5 * nt, C, HW, false, in_row(t1));
            }
        }
        if (prev_nt > 0) {
            if (c_vec) store_dp(prev_t1, prev_nt);
            else move_rows<THREADS, true>(dbuf, prev_nt, R3, R3, false, dp_row(prev_t1));
        }
        if (c_vec && t1 - kBwdChunk >= 1) load_b(t1 - kBwdChunk, min(kBwdChunk, t1 - kBwdChunk));
        lds_barrier();
        if (fuse && ci >= 2) {
            if (tid == 0)
                __hip_atomic_store(cflags + ci - 2, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            published = ci - 1;
        }
        // One step.  The partial buffers alternate with tt (the barrier at
        // a chunk boundary orders the last reads of one chunk before the
        // first writes of the next).
        BwdFactors fb = bwd_factors<HW>(stage, cqc);   // step t1 (staged step 0)
        auto bstep = [&](int tt) __attribute__((always_inline)) {
            float* pb = &part[tt & 1][0][0];
            float mdp[3];
            {
                // carry_mine is +0 at t = K, and h_t - y_t is never -0 (h_t
                // is not), so the add is exact there
                const float dh = fb.r + carry_mine;
                mdp[0] = (dh * fb.A) * fb.Bf;
                mdp[1] = (dh * fb.G) * fb.Fg;
                mdp[2] = (dh * fb.H) * fb.Fh;
            }
            float dp[CPG][3];
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                dp[0][q] = group_bcast<0>(mdp[q]);
                if (CPG > 1) dp[CPG - 1][q] = group_bcast<4>(mdp[q]);
            }
            if (q_ok && fn < 3) dbuf[tt * R3 + fn * C + cq] = (fn == 0) ? mdp[0] : (fn == 1) ? mdp[1] : mdp[2];
            // Partial of the group over the carry columns.  An absent
            // channel carries W = 0 and the finite dp of the clamped channel
            // C - 1; 0 * dp is +-0 and P is never -0, so fma(0, dp, P) == P
            // exactly and the chains need no per-channel branches.
            // P[n], n = 4 i + e: column 32 i + 4 j + e.
            float P[4 * NH];
#pragma unroll
            for (int i = 0; i < NH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float acc = 0.0f;
#pragma unroll
                    for (int cl = 0; cl < CPG; ++cl)
#pragma unroll
                        for (int q = 0; q < 3; ++q) acc = fmaf(w[cl][q][i][e], dp[cl][q], acc);
                    P[4 * i + e] = acc;
                }
            // Level 1 of the canonical dz subtrees: group g + group g + 4,
            // which are lanes l and l + 32 of one wavefront.  One swap of
            // the wavefront halves pairs P[n] with P[n + 2 NH]: lanes < 32
            // then hold the level-1 sums of columns n < 2 NH, lanes >= 32
            // those of the rest, each as (lower group) + (upper group).
            // They go to the lower group's row.
            constexpr int HALF = 2 * NH;
            float S1[HALF];
#pragma unroll
            for (int n = 0; n < HALF; ++n) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[n]), __float_as_uint(P[n + HALF]),
                                                                 false, false);
                S1[n] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            const bool upper = (tid & 32) != 0;
            float* prow = pb + (upper ? g - 4 : g) * HWP + 4 * j;
            if constexpr (NH == 1) {
                float2 v2;
                v2.x = S1[0];
                v2.y = S1[1];
                *reinterpret_cast<float2*>(prow + (upper ? 2 : 0)) = v2;
            } else if constexpr (NH == 3) {
#pragma unroll
                for (int n = 0; n < HALF; ++n) {
                    const int nn = n + (upper ? HALF : 0);
                    prow[32 * (nn >> 2) + (nn & 3)] = S1[n];
                }
            } else {
#pragma unroll
                for (int i = 0; i < NH / 2; ++i) {
                    f32x4 v;
                    v.x = S1[4 * i];
                    v.y = S1[4 * i + 1];
                    v.z = S1[4 * i + 2];
                    v.w = S1[4 * i + 3];
                    *reinterpret_cast<f32x4*>(prow + 32 * (i + (upper ? NH / 2 : 0))) = v;
                }
            }
            lds_barrier();
            // the next step's carry-independent factors: their LDS reads go
            // out ahead of the tree's, off the carry's path (unconditionally,
            // from a staged row inside the buffer: after a chunk's last step
            // they are unused, and the next chunk reloads them)
            fb = bwd_factors<HW>(stage + (tt + 1 < kBwdChunk ? tt + 1 : tt) * 5 * HW, cqc);
            if (jq < CPG) {   // uniform over each quad
                const float v = tree_sum8_loads_first(pb + fn * HWP + cqc, 8 * HWP);
                carry_mine = quad_sum4(v);
            }
        };
        const bool pub = fuse && prev_nt > 0 && nt > kPub && ci == nchunks - 1;
#pragma unroll
        for (int tt = 0; tt < kBwdChunk; ++tt)
            if (tt < nt) {
                if (tt == kPub && pub) wait_vmem_all();
                bstep(tt);   // its barrier orders every wave's wait before the flag
                if (tt == kPub && pub && tid == 0)
                    __hip_atomic_store(cflags + ci - 1, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        if (pub) published = ci;
        prev_t1 = t1;
        prev_nt = nt;
        ++ci;
    }
    lds_barrier();
    if (prev_nt > 0) {
        if (c_vec) store_dp(prev_t1, prev_nt);
        else move_rows<THREADS, true>(dbuf, prev_nt, R3, R3, false, dp_row(prev_t1));
    }
    if (fuse) {
        wait_vmem_all();
        __syncthreads();
        if (tid == 0)
            for (int c = published; c < nchunks; ++c)
                __hip_atomic_store(cflags + c, (int)a.call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
// [persistent kernel source: end]

// ---------------------------------------------------------------------------
// Batch-axis reduction out[n] = sum_b in[b, n] ("reduce_axis0").
// Workgroup = R row slices x (256 / R) column lanes; a lane owns V adjacent
// columns.  Slice i sums rows [i*rps, (i+1)*rps) in ascending b, in fp64.
// The R slice partials of a column are then added by a block tree: while the
// partner slice sits in another wavefront, through LDS (stride halving:
// slice i < s adds slice i + s, s = R/2, R/4, ..), and the last levels, once
// both partners are lanes of one wavefront, by a wavefront exchange; so
// R = 4 gives (p0 + p2) + (p1 + p3).  The fp64 total is rounded to fp32
// once.  R and rps depend on B alone, so the bits of a column do not depend
// on N, V, the segment it sits in or the grid.  Up to two tensors (segments)
// with the same B are reduced by one launch.
// ---------------------------------------------------------------------------
template <int V, int G>
__global__ __launch_bounds__(kThreads) void reduce_axis0_kernel(ReduceArgs a)
{
    // G column groups per lane: group j of this lane is (blockIdx.x G + j)
    // lanes + lane, so that every j is one coalesced row segment per slice;
    // the loads of all G groups of a row are in flight together.
    __shared__ double part[V * G][kThreads];   // component-major: lanes read and write consecutive doubles
    const int lanes = kThreads / a.R;
    const int slice = threadIdx.x / lanes;
    const int lane = threadIdx.x - slice * lanes;
    const float* in[G];
    float* out[G];
    int64_t N[G], n0[G];
    bool valid[G], whole[G];
#pragma unroll
    for (int jg = 0; jg < G; ++jg) {
        int64_t gi = ((int64_t)blockIdx.x * G + jg) * lanes + lane;
        const bool second = gi >= a.seg[0].groups;
        if (second) gi -= a.seg[0].groups;
        in[jg] = second ? a.seg[1].in : a.seg[0].in;
        out[jg] = second ? a.seg[1].out : a.seg[0].out;
        N[jg] = second ? a.seg[1].N : a.seg[0].N;
        const int64_t groups = second ? a.seg[1].groups : a.seg[0].groups;
        valid[jg] = (second ? a.nseg > 1 : true) && gi < groups;
        n0[jg] = gi * V;
        whole[jg] = valid[jg] && n0[jg] + V <= N[jg];
    }

    double acc[G][V];
#pragma unroll
    for (int jg = 0; jg < G; ++jg)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[jg][e] = 0.0;
    const int64_t rb = (int64_t)slice * a.rows_per_slice;
    const int64_t re = min(rb + a.rows_per_slice, a.B);
    bool vec_all = true, any = false;
#pragma unroll
    for (int jg = 0; jg < G; ++jg) {
        vec_all = vec_all && (whole[jg] || !valid[jg]);
        any = any || valid[jg];
    }
    if (V == 4 && vec_all) {
        if (any) {
            // every group of the lane is whole or absent: 16-byte loads; an
            // absent group reads column 0 of the first segment's rows (in
            // bounds: there is a valid group, so that segment has B rows of
            // at least 4 columns) and is dropped
            const float* p[G];
            int64_t st[G];
#pragma unroll
            for (int jg = 0; jg < G; ++jg) {
                st[jg] = valid[jg] ? N[jg] : a.seg[0].N;
                p[jg] = valid[jg] ? in[jg] + rb * N[jg] + n0[jg] : a.seg[0].in + rb * a.seg[0].N;
            }
#pragma unroll 8
            for (int64_t b = rb; b < re; ++b) {
                f32x4 v[G];
#pragma unroll
                for (int jg = 0; jg < G; ++jg)
                    v[jg] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p[jg]));
#pragma unroll
                for (int jg = 0; jg < G; ++jg) {
                    acc[jg][0] += (double)v[jg].x;
                    acc[jg][1] += (double)v[jg].y;
                    acc[jg][2] += (double)v[jg].z;
                    acc[jg][3] += (double)v[jg].w;
                    p[jg] += st[jg];
                }
            }
        }
    } else {
#pragma unroll
        for (int jg = 0; jg < G; ++jg) {
            if (!valid[jg]) continue;
            const float* __restrict__ q = in[jg] + rb * N[jg] + n0[jg];
            for (int64_t b = rb; b < re; ++b, q += N[jg]) {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (n0[jg] + e < N[jg]) acc[jg][e] += (double)q[e];
            }
        }
    }
    // Block tree over the R slices, stride halving: slice i < sh adds slice
    // i + sh, sh = R/2, R/4, ..  The levels whose partner slice is in
    // another wavefront go through LDS in one exchange: every slice writes
    // its partial, and after one barrier each lane of the W0 slices of
    // wavefront 0 (W0 = 64 / lanes when a slice is narrower than a
    // wavefront, else slice 0 alone) reads the partials p[i + m W0] of the
    // slices it gathers and adds them in the tree's order.
    const int W0 = lanes < 64 ? 64 / lanes : 1;
    const int M = a.R / W0 > 0 ? a.R / W0 : 1;   // partials per gathering lane
    int sh = a.R / 2;
    if (M > 1) {
#pragma unroll
        for (int jg = 0; jg < G; ++jg)
#pragma unroll
            for (int e = 0; e < V; ++e) part[jg * V + e][threadIdx.x] = acc[jg][e];
        __syncthreads();
        if (slice < W0) {
            // The stride-halving tree over v[0 .. M) is the pairwise tree of
            // adjacent values over v in bit-reversed index order: take
            // u_k = v[bitrev(k)] in turn and fold it into the pending level
            // sums (lv[l] holds the sum of the last 2^l values), left + right.
            const int L = 31 - __clz(M);
#pragma unroll
            for (int jg = 0; jg < G; ++jg)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    double lv[5];
#pragma unroll
                    for (int l = 0; l < 5; ++l) lv[l] = 0.0;
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        if (k >= M) break;
                        const int idx = L > 0 ? (int)(__brev((unsigned)k) >> (32 - L)) : 0;
                        double x = idx == 0 ? acc[jg][e]
                                            : part[jg * V + e][min((int)threadIdx.x + idx * W0 * lanes, kThreads - 1)];
#pragma unroll
                        for (int l = 0; l < 5; ++l) {
                            if ((k >> l) & 1) {
                                x = lv[l] + x;
                            } else {
                                lv[l] = x;
                                break;
                            }
                        }
                    }
                    double r = lv[0];
#pragma unroll
                    for (int l = 1; l < 5; ++l)
                        if (l == L) r = lv[l];
                    acc[jg][e] = r;
                    // one tree at a time: keeps the register count (and the
                    // occupancy of the streaming phase) down
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        sh = W0 / 2;
    }
    if (threadIdx.x < 64 || slice == 0) {
        // Levels left only when a slice is narrower than a wavefront: then
        // wavefront 0 holds slice 0 and every partner of those levels, and
        // lane l adds lane l ^ (sh lanes) (both partners keep the same bits).
        for (; sh > 0; sh >>= 1) {
#pragma unroll
            for (int jg = 0; jg < G; ++jg)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[jg][e] += __shfl_xor(acc[jg][e], sh * lanes);
        }
        if (slice == 0) {
#pragma unroll
            for (int jg = 0; jg < G; ++jg) {
                if (!valid[jg]) continue;
                if (V == 4 && whole[jg]) {
                    f32x4 o;
                    o.x = (float)acc[jg][0];
                    o.y = (float)acc[jg][1];
                    o.z = (float)acc[jg][2];
                    o.w = (float)acc[jg][3];
                    *reinterpret_cast<f32x4*>(out[jg] + n0[jg]) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        if (n0[jg] + e < N[jg]) out[jg][n0[jg] + e] = (float)acc[jg][e];
                }
            }
        }
    }
    if (a.xn > 0 && blockIdx.x == 0) {
        // lane l adds elements l, l + 256, .. in order; then a fixed pairwise tree
        __shared__ double xs[kThreads];
        double t = 0.0;
        for (int64_t i = threadIdx.x; i < a.xn; i += kThreads) t += (double)a.xin[i];
        xs[threadIdx.x] = t;
        __syncthreads();
        for (int h = kThreads / 2; h > 0; h >>= 1) {
            if ((int)threadIdx.x < h) xs[threadIdx.x] += xs[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) a.xout[0] = (float)xs[0];
    }
}

// AdamW over up to four tensors in one launch (flat index space, grid
// stride), decoupled weight decay:
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps).
// fp32 arithmetic with correctly rounded sqrt and divide; every element is
// independent, so the result does not depend on the grid.
__device__ __forceinline__ void adamw_one(const AdamwArgs& a, float& p, float g, float& m, float& v)
{
    m = a.beta1 * m + a.one_minus_beta1 * g;
    v = a.beta2 * v + a.one_minus_beta2 * (g * g);
    const float denom = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
    p = p * a.decay - a.step_size * (m / denom);
}

// One thread per chunk of 4 consecutive elements of a segment (chunks of all
// segments numbered one after another, grid-stride): a float4 move of each
// array when the segment's arrays are 16-byte aligned and the chunk is whole,
// else element by element.
__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamwArgs a)
{
    const int64_t total = a.qstart[a.nseg];
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        int sg = 0;
#pragma unroll
        for (int k = 1; k < kMaxAdamwSegs; ++k)
            if (k < a.nseg && i >= a.qstart[k]) sg = k;
        const AdamwSeg& S = a.seg[sg];
        const int64_t j = 4 * (i - a.qstart[sg]);
        if (S.vec && j + 4 <= S.n) {
            float4 p = *reinterpret_cast<const float4*>(S.p + j);
            const float4 g = *reinterpret_cast<const float4*>(S.g + j);
            float4 m = *reinterpret_cast<const float4*>(S.m + j);
            float4 v = *reinterpret_cast<const float4*>(S.v + j);
            adamw_one(a, p.x, g.x, m.x, v.x);
            adamw_one(a, p.y, g.y, m.y, v.y);
            adamw_one(a, p.z, g.z, m.z, v.z);
            adamw_one(a, p.w, g.w, m.w, v.w);
            *reinterpret_cast<float4*>(S.p + j) = p;
            *reinterpret_cast<float4*>(S.m + j) = m;
            *reinterpret_cast<float4*>(S.v + j) = v;
        } else {
            const int64_t e = min(j + 4, S.n);
            for (int64_t q = j; q < e; ++q) {
                float p = S.p[q], m = S.m[q], v = S.v[q];
                adamw_one(a, p, S.g[q], m, v);
                S.p[q] = p;
                S.m[q] = m;
                S.v[q] = v;
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

template <int BT>
hipError_t launch_fwd_bt(const FwdArgs& a, const StepPlan& p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.n_btiles * p.n_ctiles));
    if (p.Vf == 4)
        hipLaunchKernelGGL((fwd_step_kernel<BT, 4>), grid, dim3(kThreads), p.fwd_smem, s, a);
    else
        hipLaunchKernelGGL((fwd_step_kernel<BT, 1>), grid, dim3(kThreads), p.fwd_smem, s, a);
    return hipGetLastError();
}

template <int BT>
hipError_t launch_bwd_bt(const BwdArgs& a, const StepPlan& p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.n_btiles * p.n_ctiles));
    if (p.Vb == 4)
        hipLaunchKernelGGL((bwd_step_kernel<BT, 4>), grid, dim3(kThreads), p.bwd_smem, s, a);
    else
        hipLaunchKernelGGL((bwd_step_kernel<BT, 1>), grid, dim3(kThreads), p.bwd_smem, s, a);
    return hipGetLastError();
}

// [persistent kernel source: begin]
// Persistent-kernel instantiations: CPG = ceil(C / 64) channels per
// canonical group, NH = ceil(C / 32) recurrent column blocks of 32;
// 12 CPG NH W values per lane.
struct PersistShape {
    int cpg, nh;
};

bool persist_shape(int C, PersistShape& ps)
{
    if (C < 1 || C > 128) return false;
    ps = PersistShape{dz_group_channels(C), (C + 31) / 32};
    return true;
}

template <int CPG, int NH>
hipError_t launch_persist_t(const PersistArgs& a, hipStream_t s)
{
    const int64_t blocks = (int64_t)(a.n_proj > a.n_fill ? a.n_proj : a.n_fill) + a.B;
    if (a.n_proj < 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.n_proj > 0 && (a.flags == nullptr || (a.u == nullptr && a.n_x > 0) || a.call == 0 ||
                         a.n_proj != persist_proj_blocks(a.B, a.C, a.K)))
        return hipErrorInvalidValue;
    if (a.n_fill != 0 && (a.n_proj == 0 || a.gW_s == nullptr || a.gb_s == nullptr ||
                          a.n_fill != a.B * ((3 * a.C + 63) / 64) || !persist_fill_fits(a.B, a.C, a.n_x, a.K, 1 << 30)))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((kloop_persist_kernel<CPG, NH>), dim3((unsigned)blocks), dim3(kPersistThreads), 0, s, a);
    return hipGetLastError();
}
// [persistent kernel source: end]

}  // namespace

// Row slices of the reduction: a power of two in [1, 16] with about 8 rows
// (16 for B >= 256) per slice.  Depends on B only.
int reduce_slices(int64_t B)
{
    int R = 1;
    while (R < 16 && (int64_t)R * 2 * 8 <= B) R *= 2;
    return R;
}

// Projection workgroups of a launch that also forms X: one 64 x 64 tile of
// X each.
int persist_proj_blocks(int B, int C, int K)
{
    const int64_t rows = (int64_t)K * B;
    const int64_t n = ((rows + 63) / 64) * ((3 * C + 63) / 64);
    return n > 0x3fffffffLL ? -1 : (int)n;
}

// [persistent kernel source: begin]
bool persist_fill_fits(int B, int C, int n_x, int K, int n_cus)
{
    PersistShape ps;
    if (!persist_shape(C, ps) || B < 1 || K < 1 || n_x < 0) return false;
    const int n_in = n_x + C;
    if (C % 4 != 0 || n_x % 4 != 0 || n_in > 256) return false;
    // device-scope loads take 32-bit byte offsets into dp and h_hist
    if ((int64_t)K * B * 3 * C * 4 >= (1LL << 31) || (int64_t)(K + 1) * B * C * 4 >= (1LL << 31)) return false;
    const int part_floats = 2 * kDzGroups * (32 * ps.nh + 8);
    if (persist_fill_lds_floats(n_in) > part_floats || 16 * (((n_in + 15) & ~15) + 4) > part_floats) return false;
    const int n_proj = persist_proj_blocks(B, C, K);
    if (n_proj < 1) return false;
    const int n_fill = B * ((3 * C + 63) / 64);
    return (int64_t)(n_proj > n_fill ? n_proj : n_fill) + B <= n_cus;
}
// [persistent kernel source: end]

size_t persist_smem(int C)
{
    PersistShape ps;
    if (!persist_shape(C, ps)) return 0;
#define CFC_PERSIST_LDS(P_, N_) \
    if (ps.cpg == P_ && ps.nh == N_) return PersistLds<P_, N_>::BYTES;
    CFC_PERSIST_LDS(1, 1)
    CFC_PERSIST_LDS(1, 2)
    CFC_PERSIST_LDS(2, 3)
    CFC_PERSIST_LDS(2, 4)
#undef CFC_PERSIST_LDS
    return 0;
}

hipError_t launch_fwd(const FwdArgs& a, const StepPlan& p, hipStream_t s)
{
    switch (p.BT) {
    case 1: return launch_fwd_bt<1>(a, p, s);
    case 2: return launch_fwd_bt<2>(a, p, s);
    case 4: return launch_fwd_bt<4>(a, p, s);
    case 8: return launch_fwd_bt<8>(a, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd(const BwdArgs& a, const StepPlan& p, hipStream_t s)
{
    switch (p.BT) {
    case 1: return launch_bwd_bt<1>(a, p, s);
    case 2: return launch_bwd_bt<2>(a, p, s);
    case 4: return launch_bwd_bt<4>(a, p, s);
    case 8: return launch_bwd_bt<8>(a, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fill(const FillArgs& a, hipStream_t s)
{
    if (a.n_rt <= 0 || a.n_kt <= 0) return hipSuccess;
    if (a.K < 1) return hipErrorInvalidValue;   // K = 0 has no steps to stage: callers zero the scratch
    // A workgroup walks a whole row of column tiles when the row tiles alone
    // fill the device (at least 4 per CU), so that its next tile loads while
    // this one computes; below that the tiles spread one per workgroup.
    // Measured at B = 256, C = 256, n_x = 128, K = 64: 1, 2, 3, 6 tiles per
    // workgroup 134, 125, 122, 120 us.
    FillArgs f = a;
    f.kt_per = ((int64_t)a.B * a.n_rt >= 1024) ? a.n_kt : 1;
    const int64_t blocks = (int64_t)a.B * a.n_rt * ((a.n_kt + f.kt_per - 1) / f.kt_per);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scratch_fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, f);
    return hipGetLastError();
}

MfmaLayout mfma_layout(int C, int n_x)
{
    MfmaLayout L;
    L.nxp = (n_x + 15) & ~15;
    L.cp = (C + 31) & ~31;
    L.ldf = L.nxp + L.cp;
    L.pg = (3 * dz_group_channels(C) + 3) / 4;
    return L;
}

int64_t mfma_w_floats(int C, int n_x)
{
    const MfmaLayout L = mfma_layout(C, n_x);
    return (int64_t)3 * C * L.ldf + (int64_t)C * kDzGroups * 16;
}

bool mfma_fits(int C, int n_x)
{
    const MfmaLayout L = mfma_layout(C, n_x);
    return L.pg <= 4 && n_x % 4 == 0 && C % 4 == 0 && L.nxp <= 16 * kMfmaMaxNxb && L.cp <= 32 * kMfmaMaxNhb;
}

hipError_t launch_permute_w(const PermuteArgs& a, hipStream_t s)
{
    const int64_t total = (int64_t)3 * a.C * a.L.ldf + (int64_t)a.C * kDzGroups * 16;
    const int64_t blocks = min((total + kThreads - 1) / kThreads, (int64_t)4096);
    hipLaunchKernelGGL(permute_w_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fwd_mfma(const FwdMfmaArgs& a, hipStream_t s)
{
    if (!mfma_fits(a.C, a.n_x) || a.n_ctiles != (a.C + 15) / 16) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)((a.B + 15) / 16) * a.n_ctiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fwd_mfma_kernel, dim3((unsigned)blocks), dim3(kFwdMfmaThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_mfma(const BwdMfmaArgs& a, hipStream_t s)
{
    if (a.L.pg > 4 || a.C % 4 != 0 || a.C > 32 * kMfmaMaxNhb || a.n_ctiles != (a.C + 15) / 16)
        return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)((a.B + 15) / 16) * a.n_ctiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (a.L.pg) {
    case 1: hipLaunchKernelGGL((bwd_mfma_kernel<1>), dim3((unsigned)blocks), dim3(kBwdMfmaThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_mfma_kernel<2>), dim3((unsigned)blocks), dim3(kBwdMfmaThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((bwd_mfma_kernel<3>), dim3((unsigned)blocks), dim3(kBwdMfmaThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_mfma_kernel<4>), dim3((unsigned)blocks), dim3(kBwdMfmaThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

namespace {
const void* resident_fn(int pg)
{
    switch (pg) {
    case 1: return (const void*)kloop_resident_kernel<1>;
    case 2: return (const void*)kloop_resident_kernel<2>;
    case 3: return (const void*)kloop_resident_kernel<3>;
    default: return (const void*)kloop_resident_kernel<4>;
    }
}
}  // namespace

int64_t resident_capacity(const MfmaLayout& L)
{
    constexpr int kMaxDev = 64;
    static int64_t cap[kMaxDev][5];
    static bool known[kMaxDev][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev || L.pg < 1 || L.pg > 4) return 0;
    if (!known[dev][L.pg]) {
        int coop = 0, cus = 0, per_cu = 0;
        int64_t c = 0;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess && coop &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_fn(L.pg), kResThreads, 0) == hipSuccess)
            c = (int64_t)cus * per_cu;
        cap[dev][L.pg] = c;
        known[dev][L.pg] = true;
    }
    return cap[dev][L.pg];
}

int64_t resident_exchange_floats(int B, int C)
{
    const int64_t nbt = ((int64_t)B + 15) / 16;
    return 2 * nbt * ((int64_t)16 * ((C + 31) & ~31) + kBwdMfmaDps);
}

hipError_t launch_resident(const ResidentArgs& a, hipStream_t s)
{
    if (a.L.pg < 1 || a.L.pg > 4 || !mfma_fits(a.C, a.n_x) || a.n_ctiles != (a.C + 15) / 16 || a.K < 1)
        return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)((a.B + 15) / 16) * a.n_ctiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > resident_capacity(a.L)) return hipErrorCooperativeLaunchTooLarge;
    ResidentArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchCooperativeKernel(resident_fn(a.L.pg), dim3((unsigned)blocks), dim3(kResThreads), params, 0, s);
}

hipError_t launch_xproj(const XprojArgs& a, hipStream_t s)
{
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    const int64_t mt = (a.M + 63) / 64;
    const int64_t blocks = mt * a.n_ntiles;
    if (blocks > 0x7fffffffLL || a.n_ntiles != (a.N + 63) / 64) return hipErrorInvalidValue;
    const bool vec = (a.n_x % 4 == 0) && (a.n_in % 4 == 0) &&
                     ((((uintptr_t)a.u) | ((uintptr_t)a.W)) & 15u) == 0;
    if (vec)
        hipLaunchKernelGGL((xproj_kernel<true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((xproj_kernel<false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_persist(const PersistArgs& a, hipStream_t s)
{
    PersistShape ps;
    if (!persist_shape(a.C, ps) || a.B <= 0) return hipErrorInvalidValue;
#define CFC_PERSIST_CASE(P_, N_) \
    if (ps.cpg == P_ && ps.nh == N_) return launch_persist_t<P_, N_>(a, s);
    CFC_PERSIST_CASE(1, 1)
    CFC_PERSIST_CASE(1, 2)
    CFC_PERSIST_CASE(2, 3)
    CFC_PERSIST_CASE(2, 4)
#undef CFC_PERSIST_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceSeg* segs, int nseg, int64_t B, int V, hipStream_t s)
{
    return launch_reduce_with_sum(segs, nseg, B, V, nullptr, 0, nullptr, s);
}

hipError_t launch_reduce_with_sum(const ReduceSeg* segs, int nseg, int64_t B, int V, const float* xin, int64_t xn,
                                  float* xout, hipStream_t s)
{
    ReduceArgs a{};
    a.xin = xin;
    a.xout = xout;
    a.xn = xn > 0 ? xn : 0;
    a.nseg = nseg;
    a.B = B;
    a.R = reduce_slices(B);
    a.rows_per_slice = (B + a.R - 1) / a.R;
    int64_t total = 0;
    for (int i = 0; i < nseg; ++i) {
        a.seg[i] = segs[i];
        total += segs[i].groups;
    }
    for (int i = nseg; i < kMaxReduceSegs; ++i) a.seg[i] = ReduceSeg{nullptr, nullptr, 0, 0};
    if (total == 0 && a.xn == 0) return hipSuccess;
    const int lanes = kThreads / a.R;
    // Two column groups per lane where a slice has few rows and the grid
    // would be very large: more loads in flight per lane (measured: B = 32,
    // N = 8M 0.69 -> 0.73 of the HBM datasheet rate; smaller grids lose by it).
    // The bits of a column do not depend on this.
    const int64_t blocks1 = (total + lanes - 1) / lanes;
    const int G = (V == 4 && a.rows_per_slice <= 8 && blocks1 > 16384) ? 2 : 1;
    const int64_t blocks = total > 0 ? (total + (int64_t)lanes * G - 1) / ((int64_t)lanes * G) : 1;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (V == 4 && G == 2)
        hipLaunchKernelGGL((reduce_axis0_kernel<4, 2>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else if (V == 4)
        hipLaunchKernelGGL((reduce_axis0_kernel<4, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((reduce_axis0_kernel<1, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamwArgs& a, hipStream_t s)
{
    const int64_t total = a.qstart[a.nseg];
    if (total == 0) return hipSuccess;
    const int64_t blocks = min((total + kThreads - 1) / kThreads, (int64_t)4096);
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace cfc
