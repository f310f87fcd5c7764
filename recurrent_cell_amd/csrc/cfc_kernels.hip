// gfx950 kernels of the CfC K-loop: forward step, backward (BPTT) step with
// per-sample gradient scratch, and the batch-axis reduction.
//
// Parallel structure ("K-loop Parallelization -- Block-per-Batch Kernel
// Refactor", section Architecture Choice): samples are independent, so every
// workgroup owns a tile of (samples x channels) and no workgroup waits for
// another inside a step.  The pages map one block per sample; on MI355X a
// sample is split over ceil(C / CT) workgroups by channel tile instead, so
// that B = 32 samples still give >= 256 workgroups for 256 CUs.  Channel tile
// j of every sample is dispatched to XCD (j mod 8), because workgroup ids go
// round-robin over the 8 XCDs and the tile index is the fastest-varying part
// of the id; each XCD's L2 therefore keeps the same scratch rows and the same
// W rows from one K-step to the next.
//
// Determinism: no atomics anywhere.  Each output element is produced by one
// lane with a summation order that depends only on the sizes (C, n_in, and B
// for the reduction) -- not on the sample tile BT, the channel tile CT, the
// batch position of a sample or whether du is requested -- so repeated runs
// and a B = 1 run of any single sample reproduce the batched bits exactly.
#include "cfc_kernels.h"

namespace cfc {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Butterfly sum over the 16 lanes of a group.  Every lane of the group ends
// with the same bits: each step adds the same two operands on both partners.
__device__ __forceinline__ float group_sum16(float v)
{
    v += __shfl_xor(v, 8, kGroup);
    v += __shfl_xor(v, 4, kGroup);
    v += __shfl_xor(v, 2, kGroup);
    v += __shfl_xor(v, 1, kGroup);
    return v;
}

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
// A 16-lane group owns one row at a time: lane j multiplies W[row, k] with
// z_s[k] for k = V*j + 16*V*i (+0..V-1), then the group butterfly-sums.  The
// W element is loaded once and used for all BT samples.
// Sum order of a_q[b, c]: per lane, k ascending within its stride; then the
// 16-lane butterfly; then + bias.
// ---------------------------------------------------------------------------
template <int BT, int V>
__global__ __launch_bounds__(kThreads) void fwd_step_kernel(FwdArgs a)
{
    extern __shared__ float smem[];
    const int n_in = a.n_x + a.C;
    const int ctile = blockIdx.x % a.n_ctiles;
    const int btile = blockIdx.x / a.n_ctiles;
    const int b0 = btile * BT;
    const int c0 = ctile * a.CT;
    const int nb = min(BT, a.B - b0);
    const int nc = min(a.CT, a.C - c0);
    float* zs = smem;                  // [BT][ldz]
    float* as = smem + BT * a.ldz;     // [BT][3][CT] pre-activations

    stage_z<BT>(zs, a.ldz, a.u_t, a.h_prev, b0, nb, a.C, a.n_x);
    if (a.h_prev_copy != nullptr && ctile == 0) {
        for (int i = threadIdx.x; i < nb * a.C; i += kThreads) {
            const int64_t idx = (int64_t)b0 * a.C + i;
            a.h_prev_copy[idx] = a.h_prev[idx];
        }
    }
    __syncthreads();

    const int grp = threadIdx.x / kGroup;
    const int ln = threadIdx.x % kGroup;
    const int rows = 3 * nc;
    for (int r = grp; r < rows; r += kGroups) {
        // r is uniform over the 16 lanes of the group; shuffles stay inside it.
        const int q = r / nc;
        const int cl = r - q * nc;
        const float* __restrict__ wrow = a.W + ((int64_t)q * a.C + c0 + cl) * n_in;
        float acc[BT];
#pragma unroll
        for (int s = 0; s < BT; ++s) acc[s] = 0.0f;
        if constexpr (V == 4) {
            for (int k = ln * 4; k < n_in; k += kGroup * 4) {
                const float4 w = *reinterpret_cast<const float4*>(wrow + k);
#pragma unroll
                for (int s = 0; s < BT; ++s) {
                    const float4 z = *reinterpret_cast<const float4*>(zs + s * a.ldz + k);
                    acc[s] = fmaf(w.x, z.x, acc[s]);
                    acc[s] = fmaf(w.y, z.y, acc[s]);
                    acc[s] = fmaf(w.z, z.z, acc[s]);
                    acc[s] = fmaf(w.w, z.w, acc[s]);
                }
            }
        } else {
            for (int k = ln; k < n_in; k += kGroup) {
                const float w = wrow[k];
#pragma unroll
                for (int s = 0; s < BT; ++s) acc[s] = fmaf(w, zs[s * a.ldz + k], acc[s]);
            }
        }
        const float bq = a.bias[q * a.C + c0 + cl];
#pragma unroll
        for (int s = 0; s < BT; ++s) {
            const float v = group_sum16(acc[s]);
            if (ln == 0) as[(s * 3 + q) * a.CT + cl] = v + bq;
        }
    }
    __syncthreads();

    for (int i = threadIdx.x; i < nb * nc; i += kThreads) {
        const int s = i / nc;
        const int cl = i - s * nc;
        const int64_t b = (int64_t)b0 + s;
        const int c = c0 + cl;
        const float af = as[(s * 3 + 0) * a.CT + cl];
        const float ag = as[(s * 3 + 1) * a.CT + cl];
        const float ah = as[(s * 3 + 2) * a.CT + cl];
        const float gate = 1.0f / (1.0f + expf(af));   // sigmoid(-a_f), dt = 1
        const float g = tanhf(ag);
        const float hh = tanhf(ah);
        const float h = fmaf(gate, g, (1.0f - gate) * hh);
        a.h_t[b * a.C + c] = h;
        a.act_t[(0 * (int64_t)a.B + b) * a.C + c] = gate;
        a.act_t[(1 * (int64_t)a.B + b) * a.C + c] = g;
        a.act_t[(2 * (int64_t)a.B + b) * a.C + c] = hh;
    }
}

// ---------------------------------------------------------------------------
// Backward step.  Workgroup = (sample tile, channel tile j).
//  1. dp_q[s, c] for ALL C channels of its samples into LDS (cheap: 6 loads
//     per channel), because the carry needs every channel.
//  2. Scratch rows of its own channel tile: gW_s[b, q, c0:c0+nc, :] is one
//     contiguous block of nc * n_in floats per (b, q); it is streamed with
//     coalesced V-wide read-modify-writes.  This workgroup is the only writer
//     of those rows.
//  3. dz[k] = sum_{q,c} W[q, c, k] dp_q[c] for its slice of columns k:
//     16 row slices x 16 columns; slice j sums rows r = j, j+16, ... in
//     ascending order, then slices are added in ascending order.
//     Columns [n_x, n_in) give the carry dh_out; [0, n_x) give du_t when it
//     is requested.  Columns are split evenly over the n_ctiles workgroups
//     of the sample.
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
    float* zs = smem;                    // [BT][ldz]
    float* dps = zs + BT * a.ldz;        // [BT][3C]
    float* red = dps + BT * C3;          // [kSlices][BT][kCols]

    stage_z<BT>(zs, a.ldz, a.u_t, a.h_prev, b0, nb, a.C, a.n_x);
    for (int i = threadIdx.x; i < BT * a.C; i += kThreads) {
        const int s = i / a.C;
        const int c = i - s * a.C;
        float df = 0.0f, dg = 0.0f, dhh = 0.0f;
        if (s < nb) {
            const int64_t b = (int64_t)b0 + s;
            const int64_t bc = b * a.C + c;
            const float gate = a.act_t[(0 * (int64_t)a.B + b) * a.C + c];
            const float g = a.act_t[(1 * (int64_t)a.B + b) * a.C + c];
            const float hh = a.act_t[(2 * (int64_t)a.B + b) * a.C + c];
            float dh = a.h_t[bc] - a.y_t[bc];
            if (a.dh_in != nullptr) dh += a.dh_in[bc];
            df = dh * (g - hh) * (-gate * (1.0f - gate));
            dg = dh * gate * (1.0f - g * g);
            dhh = dh * (1.0f - gate) * (1.0f - hh * hh);
        }
        dps[s * C3 + c] = df;
        dps[s * C3 + a.C + c] = dg;
        dps[s * C3 + 2 * a.C + c] = dhh;
    }
    __syncthreads();

    // 2. sole-writer scratch update of this workgroup's channel tile
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
                    float4 o = a.accumulate ? *reinterpret_cast<const float4*>(dst + e)
                                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
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
                    const float o = a.accumulate ? dst[e] : 0.0f;
                    dst[e] = fmaf(dq[cl], zb[k], o);
                }
            }
        }
    }
    for (int i = threadIdx.x; i < nb * 3 * nc; i += kThreads) {
        const int s = i / (3 * nc);
        const int rem = i - s * 3 * nc;
        const int q = rem / nc;
        const int cl = rem - q * nc;
        const int64_t idx = (((int64_t)b0 + s) * 3 + q) * a.C + c0 + cl;
        const float o = a.accumulate ? a.gb_s[idx] : 0.0f;
        a.gb_s[idx] = o + dps[s * C3 + q * a.C + c0 + cl];
    }

    // 3. dz = W^T dp over this workgroup's columns
    const int klo = (a.du_t != nullptr) ? 0 : a.n_x;
    const int span = n_in - klo;
    const int kw = (span + a.n_ctiles - 1) / a.n_ctiles;
    const int kbeg = klo + ctile * kw;
    const int kend = min(kbeg + kw, n_in);
    const int slice = threadIdx.x / kCols;
    const int col = threadIdx.x % kCols;
    for (int kb = kbeg; kb < kend; kb += kCols) {   // trip count uniform over the workgroup
        const int k = kb + col;
        float acc[BT];
#pragma unroll
        for (int s = 0; s < BT; ++s) acc[s] = 0.0f;
        if (k < kend) {
            for (int r = slice; r < C3; r += kSlices) {
                const float w = a.W[(int64_t)r * n_in + k];
#pragma unroll
                for (int s = 0; s < BT; ++s) acc[s] = fmaf(w, dps[s * C3 + r], acc[s]);
            }
        }
#pragma unroll
        for (int s = 0; s < BT; ++s) red[(slice * BT + s) * kCols + col] = acc[s];
        __syncthreads();
        if (threadIdx.x < BT * kCols) {
            const int s = threadIdx.x / kCols;
            const int cc = threadIdx.x - s * kCols;
            const int k2 = kb + cc;
            if (s < nb && k2 < kend) {
                float v = red[(0 * BT + s) * kCols + cc];
                for (int j = 1; j < kSlices; ++j) v += red[(j * BT + s) * kCols + cc];
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
// Batch-axis reduction out[n] = sum_b in[b, n] ("reduce_axis0").
// Workgroup = R row slices x (256 / R) column lanes; a lane owns V adjacent
// columns.  Slice i sums rows [i*rps, (i+1)*rps) in ascending b, in fp64;
// slices are then added in ascending order through LDS by slice 0, and the
// fp64 total is rounded to fp32 once.  R and rps depend on B alone, so the
// bits of a column do not depend on N, V, the segment it sits in or the grid.
// Up to two tensors (segments) with the same B are reduced by one launch.
// ---------------------------------------------------------------------------
template <int V>
__global__ __launch_bounds__(kThreads) void reduce_axis0_kernel(ReduceArgs a)
{
    __shared__ double part[kThreads * V];
    const int lanes = kThreads / a.R;
    const int slice = threadIdx.x / lanes;
    const int lane = threadIdx.x - slice * lanes;
    int64_t g = (int64_t)blockIdx.x * lanes + lane;
    const bool second = g >= a.seg[0].groups;
    if (second) g -= a.seg[0].groups;
    const float* in = second ? a.seg[1].in : a.seg[0].in;
    float* out = second ? a.seg[1].out : a.seg[0].out;
    const int64_t N = second ? a.seg[1].N : a.seg[0].N;
    const int64_t groups = second ? a.seg[1].groups : a.seg[0].groups;
    const bool valid = (second ? a.nseg > 1 : true) && g < groups;

    double acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = 0.0;
    const int64_t n0 = g * V;
    if (valid) {
        const int64_t rb = (int64_t)slice * a.rows_per_slice;
        const int64_t re = min(rb + a.rows_per_slice, a.B);
        const float* __restrict__ p = in + rb * N + n0;
        bool done = false;
        if constexpr (V == 4) {
            if (n0 + 4 <= N) {
#pragma unroll 8
                for (int64_t b = rb; b < re; ++b, p += N) {
                    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
                    acc[0] += (double)v.x;
                    acc[1] += (double)v.y;
                    acc[2] += (double)v.z;
                    acc[3] += (double)v.w;
                }
                done = true;
            }
        }
        if (!done) {
            for (int64_t b = rb; b < re; ++b, p += N) {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    if (n0 + j < N) acc[j] += (double)p[j];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) part[(slice * lanes + lane) * V + j] = acc[j];
    __syncthreads();
    if (slice == 0 && valid) {
        double s[V];
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = part[lane * V + j];
        for (int i = 1; i < a.R; ++i) {
#pragma unroll
            for (int j = 0; j < V; ++j) s[j] += part[(i * lanes + lane) * V + j];
        }
        bool done = false;
        if constexpr (V == 4) {
            if (n0 + 4 <= N) {
                f32x4 o;
                o.x = (float)s[0];
                o.y = (float)s[1];
                o.z = (float)s[2];
                o.w = (float)s[3];
                *reinterpret_cast<f32x4*>(out + n0) = o;
                done = true;
            }
        }
        if (!done) {
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (n0 + j < N) out[n0 + j] = (float)s[j];
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

}  // namespace

// Row slices of the reduction: a power of two in [1, 16] with about 8 rows
// (16 for B >= 256) per slice.  Depends on B only.
int reduce_slices(int64_t B)
{
    int R = 1;
    while (R < 16 && (int64_t)R * 2 * 8 <= B) R *= 2;
    return R;
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

hipError_t launch_reduce(const ReduceSeg* segs, int nseg, int64_t B, int V, hipStream_t s)
{
    ReduceArgs a{};
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
    if (total == 0) return hipSuccess;
    const int lanes = kThreads / a.R;
    const int64_t blocks = (total + lanes - 1) / lanes;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (V == 4)
        hipLaunchKernelGGL(reduce_axis0_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(reduce_axis0_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
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
