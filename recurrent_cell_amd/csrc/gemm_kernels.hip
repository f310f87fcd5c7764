// gfx950 kernels of the batched MLP training step, also used by the
// GEMM-form CfC weight gradient: one fp32 matrix-core GEMM kernel with three
// epilogues (forward + bias + ReLU, upstream gradient + ReLU mask,
// weight-gradient splits + bias column sums) and the mean-squared-error
// kernel.  Page "H100 Epoch Optimization Phase 2: Kernel Occupancy &
// cuBLAS", Implementation Tasks 1 and 2: the per-sample layer products
// become one batched product per layer, and the weight gradient becomes
// dY^T X summed over the batch.
#include "gemm_kernels.h"

namespace gemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

// Workgroups are dispatched round-robin over the 8 XCDs (block i to XCD
// i mod 8), each with its own L2.  Block i takes the logical index that
// gives each XCD one contiguous run of logical indices, so the column tiles
// of a row tile (consecutive indices, the same A rows) share one L2.  A
// bijection of [0, n).
__device__ __forceinline__ int64_t xcd_local_order(int64_t i, int64_t n)
{
    const int64_t q = n / 8, r = n % 8;
    const int64_t x = i % 8, j = i / 8;
    return x * q + min(x, r) + j;
}

// This thread's share of one staged chunk of an operand: rows [r0, r0 + 64)
// of R, reduction indices [k0, k0 + 32) cut at kend; zero outside.  One
// float4 per thread, in two parts: load_chunk issues the loads on clamped
// (in-bounds) addresses, with no branch and no use of the values, and
// mask_chunk zeroes the out-of-range elements where the chunk goes to LDS.
// A select right after the loads made the compiler wait for them there, so
// the prefetch of the next chunk did not overlap the matrix-core work.
//   KC: element (r, k) at p[r * ld + k] (else p[k * ld + r]);
//   VEC: 16-byte loads along the contiguous index; the host sets it only
//        when ld and that index's extent are multiples of 4 and p is
//        16-byte aligned, so a float4 is entirely inside or entirely
//        outside the range.
template <int KC, bool VEC>
__device__ __forceinline__ f32x4 load_chunk(const float* p, int64_t ld, int R, int r0, int k0, int kend)
{
    const int t = threadIdx.x;
    f32x4 v;
    if constexpr (KC) {
        // 64 rows x 8 float4 along k: row t / 8, k0 + 4 (t % 8)
        const int r = r0 + (t >> 3);
        const int k = k0 + 4 * (t & 7);
        const float* src = p + (int64_t)min(r, R - 1) * ld;
        if constexpr (VEC) {
            v = *reinterpret_cast<const f32x4*>(src + min(k, kend - 4));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = src[min(k + e, kend - 1)];
        }
    } else {
        // 32 reduction rows x 16 float4 along r: k0 + t / 16, r0 + 4 (t % 16)
        const int k = k0 + (t >> 4);
        const int r = r0 + 4 * (t & 15);
        const float* src = p + (int64_t)min(k, kend - 1) * ld;
        if constexpr (VEC) {
            v = *reinterpret_cast<const f32x4*>(src + min(r, R - 4));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = src[min(r + e, R - 1)];
        }
    }
    return v;
}

template <int KC, bool VEC>
__device__ __forceinline__ f32x4 mask_chunk(f32x4 v, int R, int r0, int k0, int kend)
{
    const int t = threadIdx.x;
    if constexpr (KC) {
        const int r = r0 + (t >> 3);
        const int k = k0 + 4 * (t & 7);
        const bool rok = r < R;
        if constexpr (VEC) return (rok && k < kend) ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (rok && k + e < kend) ? v[e] : 0.0f;
    } else {
        const int k = k0 + (t >> 4);
        const int r = r0 + 4 * (t & 15);
        const bool kok = k < kend;
        if constexpr (VEC) return (kok && r < R) ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (kok && r + e < R) ? v[e] : 0.0f;
    }
    return v;
}

// Physical float4 column of logical float4 column c4 (k = 4 c4 .. 4 c4 + 3)
// in staged row `row`: XOR-swizzled by bits 2-4 of the row, so that the
// transposing scalar stores of a wave (16 rows 4 apart, 4 k) hit 32
// different banks and the float4 reads stay 16-byte aligned.
__device__ __forceinline__ int swz(int row, int c4) { return c4 ^ ((row >> 2) & 7); }

// The staged chunk in LDS as [row][k] (row pitch kLdsPitch floats, float4
// columns swizzled by swz).
template <int KC>
__device__ __forceinline__ void store_chunk(float (*dst)[kLdsPitch], f32x4 v)
{
    const int t = threadIdx.x;
    if constexpr (KC) {
        const int row = t >> 3;
        *reinterpret_cast<f32x4*>(&dst[row][4 * swz(row, t & 7)]) = v;
    } else {
        const int k = t >> 4;
        const int r = 4 * (t & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[r + e][4 * swz(r + e, k >> 2) + (k & 3)] = v[e];
    }
}

}  // namespace

// Workgroup = one 64 x 64 output tile of one task (and one reduction split
// for weight gradients); several workgroups share a CU, so one's loads and
// barriers overlap another's matrix-core work.  The eight waves each own
// 16 rows x 32 columns: two v_mfma_f32_16x16x4f32 blocks.  The reduction
// runs in chunks of 32 staged in LDS (double buffered: the next chunk's
// global loads are in flight while the matrix cores work on this one).  In
// a chunk, lane (li, lk) reads row li's k = 16 h + 4 lk .. + 3 as one float4
// and feeds component c to instruction c, so instructions c = 0..3 of half h
// cover k = 16 h .. 16 h + 15 once each.
// EPI fixes the operand layouts: forward A = X [m, k], B = W [n, k];
// upstream gradient A = dY [m, k], B = W [k, n]; weight gradient
// A = dY [k, m], B = X [k, n].
template <int EPI, bool VA, bool VB>
__global__ __launch_bounds__(kGemmThreads) void gemm_mfma_kernel(GemmBatch g)
{
    constexpr int AKC = EPI == kEpiDw ? 0 : 1;
    constexpr int BKC = EPI == kEpiFwd ? 1 : 0;
    __shared__ __attribute__((aligned(16))) float As[2][kTile][kLdsPitch];
    __shared__ __attribute__((aligned(16))) float Bs[2][kTile][kLdsPitch];
    const int64_t blk = xcd_local_order(blockIdx.x, (int64_t)gridDim.x);
    int ti = 0;
#pragma unroll
    for (int i = 1; i < kMaxTasks; ++i)
        if (i < g.ntask && blk >= g.start[i]) ti = i;
    const GemmTask T = g.t[ti];
    const int64_t w = blk - g.start[ti];
    const int per_s = T.n_mt * T.n_nt;
    const int s = (int)(w / per_s);
    const int rem = (int)(w - (int64_t)s * per_s);
    const int mt = rem / T.n_nt;
    const int nt = rem - mt * T.n_nt;
    const int m0 = mt * kTile;
    const int n0 = nt * kTile;
    const int kb = s * T.k_split;
    const int ke = min(kb + T.k_split, T.K);
    const int nch = ke > kb ? (ke - kb + kBK - 1) / kBK : 0;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int wm = wave >> 1;   // 16-row block of the tile
    const int wn = wave & 1;    // 32-column half of the tile
    const bool do_colsum = EPI == kEpiDw && T.colsum != nullptr && nt == 0;
    // A's load extent: its reduction end (K-contiguous A, one split) or its rows
    const int a_lim = T.a_ext > 0 ? T.a_ext : (AKC ? ke : T.M);

    f32x4 acc[2];
    acc[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    acc[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float csum = 0.0f;

    // A: rows T.M (or a_lim) and reduction end a_lim (or ke); B: rows T.N, end ke
    const int a_rows = AKC ? T.M : a_lim;
    const int a_end = AKC ? a_lim : ke;
    if (nch > 0) {
        const f32x4 va = load_chunk<AKC, VA>(T.A.p, T.A.ld, a_rows, m0, kb, a_end);
        const f32x4 vb = load_chunk<BKC, VB>(T.B.p, T.B.ld, T.N, n0, kb, ke);
        store_chunk<AKC>(As[0], mask_chunk<AKC, VA>(va, a_rows, m0, kb, a_end));
        store_chunk<BKC>(Bs[0], mask_chunk<BKC, VB>(vb, T.N, n0, kb, ke));
    }
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        // The next chunk's loads, issued before this chunk's MFMAs and first
        // used at the LDS store after them.  The last chunk loads itself
        // again and stores it into the idle buffer, which no wave reads any
        // more (every wave passed the previous barrier after its last read
        // of it): no branch, so nothing forces an early wait.
        const int kn = kb + min(ch + 1, nch - 1) * kBK;
        const f32x4 va = load_chunk<AKC, VA>(T.A.p, T.A.ld, a_rows, m0, kn, a_end);
        const f32x4 vb = load_chunk<BKC, VB>(T.B.p, T.B.ld, T.N, n0, kn, ke);
        __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the MFMAs
#pragma unroll
        for (int h = 0; h < kBK / 16; ++h) {
            const int ra = wm * 16 + li;
            const f32x4 a = *reinterpret_cast<const f32x4*>(&As[buf][ra][4 * swz(ra, 4 * h + lk)]);
            f32x4 b[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rb = wn * 32 + 16 * j + li;
                b[j] = *reinterpret_cast<const f32x4*>(&Bs[buf][rb][4 * swz(rb, 4 * h + lk)]);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], b[j][c], acc[j], 0, 0, 0);
        }
        if (do_colsum && t < kTile) {
#pragma unroll
            for (int q = 0; q < kBK / 4; ++q) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&As[buf][t][4 * swz(t, q)]);
                csum = (((csum + x[0]) + x[1]) + x[2]) + x[3];
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // and their first use after them
        store_chunk<AKC>(As[buf ^ 1], mask_chunk<AKC, VA>(va, a_rows, m0, kn, a_end));
        store_chunk<BKC>(Bs[buf ^ 1], mask_chunk<BKC, VB>(vb, T.N, n0, kn, ke));
        __syncthreads();
    }

    // epilogue: acc[j][r] is C[m0 + 16 wm + 4 lk + r][n0 + 32 wn + 16 j + li]
    if constexpr (EPI == kEpiFwd) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 32 + 16 * j + li;
            const float bias = T.bias != nullptr ? T.bias[min(n, T.N - 1)] : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 16 + 4 * lk + r;
                float y = acc[j][r] + bias;
                if (T.relu) y = fmaxf(y, 0.0f);
                if (m < T.M && n < T.N) T.out[(int64_t)m * T.ldo + n] = y;
            }
        }
    } else if constexpr (EPI == kEpiDx) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 32 + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 16 + 4 * lk + r;
                if (m < T.M && n < T.N) {
                    float d = acc[j][r];
                    if (T.mask != nullptr && !(T.mask[(int64_t)m * T.ldm + n] > 0.0f)) d = 0.0f;
                    T.out[(int64_t)m * T.ldo + n] = d;
                } else if (m < T.M && n < T.ldo) {
                    T.out[(int64_t)m * T.ldo + n] = 0.0f;   // row padding of the output
                }
            }
        }
    } else {
        float* base = T.out + (int64_t)s * T.split_stride;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 32 + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 16 + 4 * lk + r;
                if (m < T.M && n < T.N) base[(int64_t)m * T.ldo + n] = acc[j][r];
            }
        }
        if (do_colsum && t < kTile && m0 + t < T.M) T.colsum[(int64_t)s * T.colsum_stride + m0 + t] = csum;
        if (mt == 0 && nt == 0) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                for (int64_t z = T.zlo[q] + t; z < T.zhi[q]; z += kGemmThreads) base[z] = 0.0f;
        }
    }
}

// Mean squared error over a contiguous range of the M x N outputs per
// workgroup: dY = gscale (Y - T) and the range's sum of (Y - T)^2 in fp64,
// reduced over the workgroup in a fixed tree, scaled by 1 / (M N) and
// stored as the range's partial loss.
__global__ __launch_bounds__(kMseThreads) void mse_kernel(MseArgs a)
{
    __shared__ double red[kMseThreads];
    const int64_t total = a.M * a.N;
    const int64_t e0 = (int64_t)blockIdx.x * a.rows_per * a.N;
    const int64_t e1 = min(e0 + a.rows_per * a.N, total);
    double acc = 0.0;
    for (int64_t i = e0 + threadIdx.x; i < e1; i += kMseThreads) {
        const int64_t row = i / a.N;
        const int64_t col = i - row * a.N;
        const float d = a.Y[i] - a.T[i];
        a.dY[row * a.ldd + col] = a.gscale * d;
        acc += (double)d * (double)d;
    }
    // zero the row padding of dY (columns N .. ldd - 1)
    const int64_t pad = a.ldd - a.N;
    if (pad > 0) {
        const int64_t r0 = e0 / a.N, r1 = e1 / a.N;
        for (int64_t i = threadIdx.x; i < (r1 - r0) * pad; i += kMseThreads) {
            const int64_t row = r0 + i / pad;
            a.dY[row * a.ldd + a.N + (i - (row - r0) * pad)] = 0.0f;
        }
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kMseThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.lossp[blockIdx.x] = (float)(red[0] * a.lscale);
}

void finish_batch(GemmBatch& g)
{
    g.start[0] = 0;
    for (int i = 0; i < g.ntask; ++i) {
        GemmTask& T = g.t[i];
        T.n_mt = (T.M + kTile - 1) / kTile;
        T.n_nt = (T.N + kTile - 1) / kTile;
        T.n_s = T.K > 0 ? (T.K + T.k_split - 1) / T.k_split : 1;
        g.start[i + 1] = g.start[i] + (int64_t)T.n_mt * T.n_nt * T.n_s;
    }
    for (int i = g.ntask + 1; i <= kMaxTasks; ++i) g.start[i] = g.start[g.ntask];
}

template <int EPI>
hipError_t launch_epi(const GemmBatch& g, unsigned blocks, bool va, bool vb, hipStream_t s)
{
    if (va && vb)
        hipLaunchKernelGGL((gemm_mfma_kernel<EPI, true, true>), dim3(blocks), dim3(kGemmThreads), 0, s, g);
    else if (va)
        hipLaunchKernelGGL((gemm_mfma_kernel<EPI, true, false>), dim3(blocks), dim3(kGemmThreads), 0, s, g);
    else if (vb)
        hipLaunchKernelGGL((gemm_mfma_kernel<EPI, false, true>), dim3(blocks), dim3(kGemmThreads), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<EPI, false, false>), dim3(blocks), dim3(kGemmThreads), 0, s, g);
    return hipGetLastError();
}

// One launch for every task of the batch (all of one epilogue); 16-byte
// operand loads only where every task allows them.
hipError_t launch_gemm(const GemmBatch& g, hipStream_t s)
{
    const int64_t blocks = g.start[g.ntask];
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const int epi = g.t[0].epi;
    bool va = true, vb = true;
    for (int i = 0; i < g.ntask; ++i) {
        if (g.t[i].epi != epi) return hipErrorInvalidValue;
        va = va && g.t[i].A.vec;
        vb = vb && g.t[i].B.vec;
    }
    if (epi == kEpiFwd) return launch_epi<kEpiFwd>(g, (unsigned)blocks, va, vb, s);
    if (epi == kEpiDx) return launch_epi<kEpiDx>(g, (unsigned)blocks, va, vb, s);
    return launch_epi<kEpiDw>(g, (unsigned)blocks, va, vb, s);
}

hipError_t launch_mse(const MseArgs& a, hipStream_t s)
{
    if (a.S <= 0) return hipSuccess;
    hipLaunchKernelGGL(mse_kernel, dim3((unsigned)a.S), dim3(kMseThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gemm
