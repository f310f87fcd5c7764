// Device arithmetic shared by every kernel of the CfC K-loop.
//
// Each output of the library has ONE canonical evaluation order, a function
// of the sizes (C, n_x, K, B) only.  The per-step kernels, the input
// projection, the persistent K-loop kernel and the deferred scratch fill all
// evaluate through the helpers below (fp32 MFMA accumulation is the same
// sequential fma chain in k order), so every path produces the same bits:
//   X_q[c]   = bias_q[c] + ((x_0 + x_1) + (x_2 + x_3)), x_r = fma chain of
//              W[q C + c, k] u[k] over the input columns k = r, r+4, r+8, ..
//              (k < n_x) from +0;
//   H_q[c]   = sum8 of the lane chains P_0 .. P_7, P_j = fma chain from +0 of
//              W[q C + c, n_x + m] h[m] over the recurrent columns
//              m = 32 i + 4 j + e (i ascending, e = 0..3, m < C);
//   a_q[c]   = X_q[c] + H_q[c];
//   dz[k]    = over 64 groups of cpg = ceil(C / 64) consecutive channels:
//              P_g = fma chain of W[q C + c, k] dp_q[c] over the group's
//              channels c ascending and, within a channel, heads q = 0, 1, 2;
//              then tree_sum64 of P_0 .. P_63 (empty groups: +0): subtree T_q
//              (q = 0..3) is the pairwise sum of P_q, P_{q+4}, .., P_{q+60},
//              and dz = (T_0 + T_1) + (T_2 + T_3);
//   S[b,r,k] = fma chain over t = K, K-1, .., 1 of dp_t[r] * z_t[k] from +0;
//   Sb[b,r]  = add chain over t = K .. 1 of dp_t[r] from +0.
#pragma once

#include <hip/hip_runtime.h>

namespace cfc {

constexpr int kDzGroups = 64;  // channel groups of the canonical W^T dp sum
constexpr int kHLanes = 8;     // lanes of one recurrent-column partition (one DPP half row)

__host__ __device__ inline int dz_group_channels(int C) { return (C + kDzGroups - 1) / kDzGroups; }

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads and stores (which __syncthreads also waits for), so
// prefetched global loads stay in flight across it.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until every vector memory load and store of this wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).  Issued
// through the builtin so that the compiler's wait-count tracking sees it: a
// register loaded before a loop and first read inside it would otherwise
// make the compiler wait inside the loop, where gfx9's shared load/store
// counter forces that wait to drain every later store and prefetch as well.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// gfx9 DPP controls used by row_sum16 and quad_sum4.
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15 - i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_get(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over one 16-lane DPP row.  All 16 lanes must be active; every lane
// ends with identical bits (each step adds the same two values on both
// partners, and after each step the lanes being paired hold equal values).
__device__ __forceinline__ float row_sum16(float v)
{
    v += dpp_get<kDppQuadXor1>(v);
    v += dpp_get<kDppQuadXor2>(v);
    v += dpp_get<kDppRowHalfMirror>(v);
    v += dpp_get<kDppRowMirror>(v);
    return v;
}

// (v0 + v1) + (v2 + v3) over the 4 lanes of a quad (lane 0 holds v0).
__device__ __forceinline__ float quad_sum4(float v)
{
    v += dpp_get<kDppQuadXor1>(v);
    v += dpp_get<kDppQuadXor2>(v);
    return v;
}

// ((v0 + v1) + (v2 + v3)) + ((v4 + v5) + (v6 + v7)) over 8 aligned lanes
// (half a DPP row; lane 0 holds v0); every lane ends with the same bits.
__device__ __forceinline__ float sum8(float v)
{
    v += dpp_get<kDppQuadXor1>(v);
    v += dpp_get<kDppQuadXor2>(v);
    v += dpp_get<kDppRowHalfMirror>(v);
    return v;
}

// Value of lane SRC (0..3) of this lane's quad.
template <int SRC>
__device__ __forceinline__ float quad_bcast(float v)
{
    return dpp_get<SRC * 0x55>(v);
}

// Value of lane SRC (0..15) of this lane's 16-lane row (ds_swizzle bit mode:
// and_mask 0x10 keeps the row, or_mask selects the lane).
template <int SRC>
__device__ __forceinline__ float row_bcast(float v)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x10 | (SRC << 5)));
}

// Pairwise sum of p[0], p[s], .., p[15 s]: ((p0+p1)+(p2+p3)) + ... (4 levels).
__device__ __forceinline__ float tree_sum16(const float* p, int s)
{
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = p[(2 * i) * s] + p[(2 * i + 1) * s];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    return a[0] + a[1];
}

// The canonical sum64 of p[0], p[s], .., p[63 s]: subtree T_q is the
// pairwise sum of p[q s], p[(q + 4) s], .., p[(q + 60) s]; then
// (T0 + T1) + (T2 + T3).  (Interleaved subtrees let the four lanes that
// share a column read four different LDS banks in the persistent kernel.)
__device__ __forceinline__ float tree_sum64(const float* p, int s)
{
    const float t0 = tree_sum16(p, 4 * s);
    const float t1 = tree_sum16(p + s, 4 * s);
    const float t2 = tree_sum16(p + 2 * s, 4 * s);
    const float t3 = tree_sum16(p + 3 * s, 4 * s);
    return (t0 + t1) + (t2 + t3);
}

// The input projection from its four chains: bias + ((x0 + x1) + (x2 + x3)).
__device__ __forceinline__ float xproj_combine(float bias, float x0, float x1, float x2, float x3)
{
    return bias + ((x0 + x1) + (x2 + x3));
}

struct CellOut {
    float gate, g, hh, h;
};

// exp(x) as 2^(x log2 e) on the hardware exp2 (v_exp_f32, about 1 ulp);
// 1 / x on the hardware reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// One of the cell's three nonlinearities, selected per lane (fn = 0: gate
// from a_f, 1: g from a_g, 2: hh from a_h), so that a quad can evaluate a
// channel's three in parallel with the operations of cell_forward:
// gate = 1 / (exp(a_f) + 1) and tanh(a) = 1 - 2 / (exp(2a) + 1) (exact
// limits +-1 when exp overflows to inf or underflows to 0; absolute error a
// few 1e-8 around 0).
__device__ __forceinline__ float cell_fn(int fn, float a)
{
    const float x = (fn == 0) ? a : 2.0f * a;
    const float r = fast_rcp(fast_exp(x) + 1.0f);
    return (fn == 0) ? r : fmaf(-2.0f, r, 1.0f);
}

// h from the three nonlinearities.
__device__ __forceinline__ float cell_h(float gate, float g, float hh)
{
    return fmaf(gate, g, (1.0f - gate) * hh);
}

// The cell, dt = 1: gate = sigmoid(-a_f) = 1 / (1 + exp(a_f)),
// g = tanh(a_g), hh = tanh(a_h), h = gate * g + (1 - gate) * hh.
__device__ __forceinline__ CellOut cell_forward(float af, float ag, float ah)
{
    CellOut o;
    o.gate = cell_fn(0, af);
    o.g = cell_fn(1, ag);
    o.hh = cell_fn(2, ah);
    o.h = cell_h(o.gate, o.g, o.hh);
    return o;
}

// Pre-activation gradients of one channel from dh = dL/dh_t.
__device__ __forceinline__ void cell_backward(float dh, float gate, float g, float hh, float& df,
                                              float& dg, float& dhh)
{
    df = (dh * (g - hh)) * (-gate * (1.0f - gate));
    dg = (dh * gate) * fmaf(-g, g, 1.0f);
    dhh = (dh * (1.0f - gate)) * fmaf(-hh, hh, 1.0f);
}

}  // namespace cfc
