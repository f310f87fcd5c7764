// C ABI of the batched MLP training step (declared in include/mlp.h):
// argument checks, workspace layout and the launch sequence.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/mlp.h"
#include "api_common.h"
#include "cfc_kernels.h"
#include "gemm_kernels.h"

namespace {

using cfc_host::aligned16;
using cfc_host::fail;
using cfc_host::overlap;
using cfc_host::span;
using cfc_host::Span;

constexpr int kSplitRows = 512;   // target rows of one weight-gradient split
constexpr int kMaxSplits = 32;
constexpr int kMseParts = 256;    // at most this many partial losses

int64_t round4(int64_t n) { return (n + 3) & ~int64_t(3); }

// extent: the length of the contiguous index (K when kc, else the rows).
gemm::Operand operand(const float* p, int64_t ld, int kc, int64_t extent)
{
    return gemm::Operand{p, ld, kc, (ld % 4 == 0 && extent % 4 == 0 && extent >= 4 && aligned16(p)) ? 1 : 0};
}

// Reduction length of one weight-gradient split (a multiple of 16); the
// splits are a function of M alone.
int k_split_for(int M)
{
    int S = M / kSplitRows;
    S = S < 1 ? 1 : (S > kMaxSplits ? kMaxSplits : S);
    const int per = (M + S - 1) / S;
    return (per + gemm::kBK - 1) / gemm::kBK * gemm::kBK;
}

int splits_for(int M) { return M > 0 ? (M + k_split_for(M) - 1) / k_split_for(M) : 1; }

int mse_rows_per(int64_t M) { return (int)((M + kMseParts - 1) / kMseParts > 0 ? (M + kMseParts - 1) / kMseParts : 1); }
int mse_parts(int64_t M) { return M > 0 ? (int)((M + mse_rows_per(M) - 1) / mse_rows_per(M)) : 0; }

int check_mnk(int M, int n_in, int n_out, const char* fn)
{
    if (M < 0 || M > MLP_MAX_B) return fail(CFC_EINVAL, "%s: M=%d out of range [0, %d]", fn, M, MLP_MAX_B);
    if (n_in < 1 || n_in > MLP_MAX_DIM || n_out < 1 || n_out > MLP_MAX_DIM)
        return fail(CFC_EINVAL, "%s: n_in=%d, n_out=%d out of range [1, %d]", fn, n_in, n_out, MLP_MAX_DIM);
    return CFC_OK;
}

int check_dims(const int* dims, int L, const char* fn)
{
    if (!dims) return fail(CFC_EINVAL, "%s: dims is NULL", fn);
    if (L < 1 || L > MLP_MAX_LAYERS) return fail(CFC_EINVAL, "%s: n_layers=%d out of range [1, %d]", fn, L,
                                                 MLP_MAX_LAYERS);
    for (int i = 0; i <= L; ++i)
        if (dims[i] < 1 || dims[i] > MLP_MAX_DIM)
            return fail(CFC_EINVAL, "%s: dims[%d]=%d out of range [1, %d]", fn, i, dims[i], MLP_MAX_DIM);
    return CFC_OK;
}

gemm::GemmTask fwd_task(const float* X, const float* W, const float* b, float* Y, int M, int n_in, int n_out,
                       int relu)
{
    gemm::GemmTask t{};
    t.A = operand(X, n_in, 1, n_in);     // A(m, k) = X[m, k]
    t.B = operand(W, n_in, 1, n_in);     // B(n, k) = W[n, k]
    t.M = M;
    t.N = n_out;
    t.K = n_in;
    t.k_split = (n_in + gemm::kBK - 1) / gemm::kBK * gemm::kBK;
    t.epi = gemm::kEpiFwd;
    t.relu = relu ? 1 : 0;
    t.bias = b;
    t.out = Y;
    t.ldo = n_out;
    return t;
}

gemm::GemmTask dx_task(const float* dY, int64_t lddy, const float* W, const float* mask, float* dX, int64_t lddx,
                      int M, int n_in, int n_out)
{
    gemm::GemmTask t{};
    t.A = operand(dY, lddy, 1, n_out);   // A(m, k) = dY[m, k]
    t.B = operand(W, n_in, 0, n_in);     // B(n, k) = W[k, n]
    t.M = M;
    t.N = n_in;
    t.K = n_out;
    t.k_split = (n_out + gemm::kBK - 1) / gemm::kBK * gemm::kBK;
    t.epi = gemm::kEpiDx;
    t.mask = mask;
    t.ldm = n_in;
    t.out = dX;
    t.ldo = lddx;
    return t;
}

// gW = dY^T X split over the M rows: split s of the weight part at
// wpart + s * wstride, of the bias column sums at bpart + s * bstride.
gemm::GemmTask dw_task(const float* dY, int64_t lddy, const float* X, int M, int n_in, int n_out, float* wpart,
                      int64_t wstride, float* bpart, int64_t bstride)
{
    gemm::GemmTask t{};
    t.A = operand(dY, lddy, 0, n_out);   // A(m, k) = dY[k, m]
    t.B = operand(X, n_in, 0, n_in);     // B(n, k) = X[k, n]
    t.M = n_out;
    t.N = n_in;
    t.K = M;
    t.k_split = k_split_for(M);
    t.epi = gemm::kEpiDw;
    t.out = wpart;
    t.ldo = n_in;
    t.split_stride = wstride;
    t.colsum = bpart;
    t.colsum_stride = bstride;
    return t;
}

// The train step's dY buffers have rows padded to ldy (a multiple of 4)
// with zeros (written by the loss kernel and the upstream-gradient
// epilogue), so A = dY may be read up to ldy with 16-byte loads.
void pad_a(gemm::GemmTask& t, int64_t ldy)
{
    t.a_ext = (int)ldy;
    t.A.vec = (ldy % 4 == 0 && aligned16(t.A.p)) ? 1 : 0;
}

int run_batch(gemm::GemmBatch& g, hipStream_t s, const char* what)
{
    gemm::finish_batch(g);
    CFC_HIP(gemm::launch_gemm(g, s), what);
    return CFC_OK;
}

int64_t param_offsets(const int* dims, int L, int64_t* w_off, int64_t* b_off)
{
    int64_t off = 0;
    for (int l = 0; l < L; ++l) {
        if (w_off) w_off[l] = off;
        off = round4(off + (int64_t)dims[l + 1] * dims[l]);
        if (b_off) b_off[l] = off;
        off = round4(off + dims[l + 1]);
    }
    return off;
}

struct StepWs {
    int64_t dy_off[MLP_MAX_LAYERS];
    int64_t ldy[MLP_MAX_LAYERS];
    int64_t part_off, loss_off, total;   // floats
    int S, P;
    int64_t Ptot;
};

StepWs step_ws(int B, const int* dims, int L)
{
    StepWs w{};
    int64_t off = 0;
    for (int l = 0; l < L; ++l) {
        w.ldy[l] = round4(dims[l + 1]);
        w.dy_off[l] = off;
        off += round4((int64_t)B * w.ldy[l]);
    }
    w.Ptot = param_offsets(dims, L, nullptr, nullptr);
    w.S = splits_for(B);
    w.part_off = off;
    off += round4((int64_t)w.S * w.Ptot);
    w.P = mse_parts(B);
    w.loss_off = off;
    off += round4(w.P);
    w.total = off;
    return w;
}

int enqueue_mse(const float* Y, const float* T, float* dY, int64_t lddy, float* loss, float* lossp, int M, int N,
                hipStream_t s)
{
    gemm::MseArgs a{};
    a.Y = Y;
    a.T = T;
    a.dY = dY;
    a.M = M;
    a.N = N;
    a.ldd = lddy;
    const double mn = (double)M * (double)N;
    a.gscale = (float)(2.0 / mn);
    a.lscale = 1.0 / mn;
    a.lossp = lossp;
    a.rows_per = mse_rows_per(M);
    a.S = mse_parts(M);
    CFC_HIP(gemm::launch_mse(a, s), "mse launch");
    CFC_HIP(cfc::launch_reduce_with_sum(nullptr, 0, 1, 1, lossp, a.S, loss, s), "loss sum launch");
    return CFC_OK;
}

}  // namespace

extern "C" {

int64_t mlp_param_offsets(const int* dims, int n_layers, int64_t* w_off, int64_t* b_off)
{
    cfc_host::last_error().clear();
    if (check_dims(dims, n_layers, "mlp_param_offsets")) return -1;
    return param_offsets(dims, n_layers, w_off, b_off);
}

int mlp_weight_grad_splits(int M) { return M < 0 ? 0 : splits_for(M); }

int mlp_linear_fwd(const float* X, const float* W, const float* b, float* Y, int M, int n_in, int n_out, int relu,
                   void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_mnk(M, n_in, n_out, "mlp_linear_fwd")) return rc;
    if (M == 0) return CFC_OK;
    if (!X || !W || !Y) return fail(CFC_EINVAL, "mlp_linear_fwd: null pointer");
    const Span out = span(Y, (int64_t)M * n_out);
    const Span ins[] = {span(X, (int64_t)M * n_in), span(W, (int64_t)n_out * n_in), span(b, b ? n_out : 0)};
    for (const Span& i : ins)
        if (overlap(out, i)) return fail(CFC_EINVAL, "mlp_linear_fwd: the output overlaps an input");
    gemm::GemmBatch g{};
    g.t[0] = fwd_task(X, W, b, Y, M, n_in, n_out, relu);
    g.ntask = 1;
    return run_batch(g, (hipStream_t)stream, "mlp_linear_fwd launch");
}

int mlp_linear_bwd_data(const float* dY, const float* W, const float* mask, float* dX, int M, int n_in, int n_out,
                        void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_mnk(M, n_in, n_out, "mlp_linear_bwd_data")) return rc;
    if (M == 0) return CFC_OK;
    if (!dY || !W || !dX) return fail(CFC_EINVAL, "mlp_linear_bwd_data: null pointer");
    const Span out = span(dX, (int64_t)M * n_in);
    const Span ins[] = {span(dY, (int64_t)M * n_out), span(W, (int64_t)n_out * n_in),
                        span(mask, mask ? (int64_t)M * n_in : 0)};
    for (const Span& i : ins)
        if (overlap(out, i)) return fail(CFC_EINVAL, "mlp_linear_bwd_data: the output overlaps an input");
    gemm::GemmBatch g{};
    g.t[0] = dx_task(dY, n_out, W, mask, dX, n_in, M, n_in, n_out);
    g.ntask = 1;
    return run_batch(g, (hipStream_t)stream, "mlp_linear_bwd_data launch");
}

size_t mlp_linear_bwd_weight_workspace_bytes(int M, int n_in, int n_out)
{
    if (M < 0 || n_in < 1 || n_out < 1 || M > MLP_MAX_B || n_in > MLP_MAX_DIM || n_out > MLP_MAX_DIM) return 0;
    const int64_t S = splits_for(M);
    return sizeof(float) * (size_t)(round4(S * n_out * (int64_t)n_in) + round4(S * n_out));
}

int mlp_linear_bwd_weight(const float* dY, const float* X, float* gW, float* gb, int M, int n_in, int n_out,
                          void* ws, size_t ws_bytes, void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_mnk(M, n_in, n_out, "mlp_linear_bwd_weight")) return rc;
    if (!gW) return fail(CFC_EINVAL, "mlp_linear_bwd_weight: gW is NULL");
    hipStream_t s = (hipStream_t)stream;
    const int64_t NW = (int64_t)n_out * n_in;
    if (M == 0) {
        CFC_HIP(cfc::launch_fill_zero(gW, NW, s), "zero fill launch");
        if (gb) CFC_HIP(cfc::launch_fill_zero(gb, n_out, s), "zero fill launch");
        return CFC_OK;
    }
    if (!dY || !X || !ws) return fail(CFC_EINVAL, "mlp_linear_bwd_weight: null pointer");
    const size_t need = mlp_linear_bwd_weight_workspace_bytes(M, n_in, n_out);
    if (ws_bytes < need)
        return fail(CFC_EINVAL, "mlp_linear_bwd_weight: workspace of %zu bytes, need %zu", ws_bytes, need);
    const Span outs[] = {span(gW, NW), span(gb, gb ? n_out : 0), Span{ws, need}};
    const Span ins[] = {span(dY, (int64_t)M * n_out), span(X, (int64_t)M * n_in)};
    for (int i = 0; i < 3; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return fail(CFC_EINVAL, "mlp_linear_bwd_weight: an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "mlp_linear_bwd_weight: outputs overlap");
    }
    const int S = splits_for(M);
    float* wpart = static_cast<float*>(ws);
    float* bpart = wpart + round4((int64_t)S * NW);
    gemm::GemmBatch g{};
    g.t[0] = dw_task(dY, n_out, X, M, n_in, n_out, wpart, NW, gb ? bpart : nullptr, n_out);
    g.ntask = 1;
    if (int rc = run_batch(g, s, "mlp_linear_bwd_weight launch")) return rc;
    cfc::ReduceSeg segs[2];
    int nseg = 0;
    segs[nseg++] = cfc::ReduceSeg{wpart, gW, NW, 0};
    if (gb) segs[nseg++] = cfc::ReduceSeg{bpart, gb, n_out, 0};
    bool vec = true;
    for (int i = 0; i < nseg; ++i) vec = vec && segs[i].N % 4 == 0 && aligned16(segs[i].in) && aligned16(segs[i].out);
    const int V = vec ? 4 : 1;
    for (int i = 0; i < nseg; ++i) segs[i].groups = (segs[i].N + V - 1) / V;
    CFC_HIP(cfc::launch_reduce(segs, nseg, S, V, s), "weight-gradient reduce launch");
    return CFC_OK;
}

size_t mlp_mse_workspace_bytes(int M) { return M < 0 ? 0 : sizeof(float) * (size_t)round4(mse_parts(M)); }

int mlp_mse_loss_grad(const float* Y, const float* T, float* dY, float* loss, int M, int N, void* ws,
                      size_t ws_bytes, void* stream)
{
    cfc_host::last_error().clear();
    if (M < 1 || M > MLP_MAX_B || N < 1 || N > MLP_MAX_DIM)
        return fail(CFC_EINVAL, "mlp_mse_loss_grad: M=%d, N=%d out of range", M, N);
    if (!Y || !T || !dY || !loss || !ws) return fail(CFC_EINVAL, "mlp_mse_loss_grad: null pointer");
    const size_t need = mlp_mse_workspace_bytes(M);
    if (ws_bytes < need) return fail(CFC_EINVAL, "mlp_mse_loss_grad: workspace of %zu bytes, need %zu", ws_bytes,
                                     need);
    const int64_t n = (int64_t)M * N;
    const Span outs[] = {span(dY, n), span(loss, 1), Span{ws, need}};
    const Span ins[] = {span(Y, n), span(T, n)};
    for (int i = 0; i < 3; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return fail(CFC_EINVAL, "mlp_mse_loss_grad: an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "mlp_mse_loss_grad: outputs overlap");
    }
    return enqueue_mse(Y, T, dY, N, loss, static_cast<float*>(ws), M, N, (hipStream_t)stream);
}

size_t mlp_train_step_workspace_bytes(int B, const int* dims, int n_layers)
{
    if (B < 1 || B > MLP_MAX_B || !dims || n_layers < 1 || n_layers > MLP_MAX_LAYERS) return 0;
    for (int i = 0; i <= n_layers; ++i)
        if (dims[i] < 1 || dims[i] > MLP_MAX_DIM) return 0;
    return sizeof(float) * (size_t)step_ws(B, dims, n_layers).total;
}

int mlp_train_step(const float* X, const float* T, int B, const int* dims, int n_layers, const float* params,
                   float* grads, float* const* act, float* loss, void* ws, size_t ws_bytes, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "mlp_train_step";
    if (int rc = check_dims(dims, n_layers, fn)) return rc;
    const int L = n_layers;
    if (B < 1 || B > MLP_MAX_B) return fail(CFC_EINVAL, "%s: B=%d out of range [1, %d]", fn, B, MLP_MAX_B);
    if (!X || !T || !params || !grads || !act || !loss || !ws) return fail(CFC_EINVAL, "%s: null pointer", fn);
    for (int l = 0; l < L; ++l)
        if (!act[l]) return fail(CFC_EINVAL, "%s: act[%d] is NULL", fn, l);
    const StepWs w = step_ws(B, dims, L);
    if (ws_bytes < sizeof(float) * (size_t)w.total)
        return fail(CFC_EINVAL, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes,
                    sizeof(float) * (size_t)w.total);
    int64_t w_off[MLP_MAX_LAYERS], b_off[MLP_MAX_LAYERS];
    param_offsets(dims, L, w_off, b_off);
    // outputs: grads, loss, every act[l], the workspace; inputs: X, T, params
    Span outs[MLP_MAX_LAYERS + 3];
    int no = 0;
    outs[no++] = span(grads, w.Ptot);
    outs[no++] = span(loss, 1);
    outs[no++] = Span{ws, sizeof(float) * (size_t)w.total};
    for (int l = 0; l < L; ++l) outs[no++] = span(act[l], (int64_t)B * dims[l + 1]);
    const Span ins[] = {span(X, (int64_t)B * dims[0]), span(T, (int64_t)B * dims[L]), span(params, w.Ptot)};
    for (int i = 0; i < no; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return fail(CFC_EINVAL, "%s: an output overlaps an input", fn);
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "%s: outputs overlap", fn);
    }
    hipStream_t s = (hipStream_t)stream;
    float* wsf = static_cast<float*>(ws);
    auto dy = [&](int l) { return wsf + w.dy_off[l]; };
    auto input = [&](int l) { return l == 0 ? X : static_cast<const float*>(act[l - 1]); };

    // forward, one launch per layer
    for (int l = 0; l < L; ++l) {
        gemm::GemmBatch g{};
        g.t[0] = fwd_task(input(l), params + w_off[l], params + b_off[l], act[l], B, dims[l], dims[l + 1], l < L - 1);
        g.ntask = 1;
        if (int rc = run_batch(g, s, "forward launch")) return rc;
    }
    // loss and the output layer's gradient
    {
        gemm::MseArgs a{};
        a.Y = act[L - 1];
        a.T = T;
        a.dY = dy(L - 1);
        a.M = B;
        a.N = dims[L];
        a.ldd = w.ldy[L - 1];
        const double mn = (double)B * (double)dims[L];
        a.gscale = (float)(2.0 / mn);
        a.lscale = 1.0 / mn;
        a.lossp = wsf + w.loss_off;
        a.rows_per = mse_rows_per(B);
        a.S = w.P;
        CFC_HIP(gemm::launch_mse(a, s), "mse launch");
    }
    // upstream gradients through the ReLUs, one launch per layer > 0
    for (int l = L - 1; l >= 1; --l) {
        gemm::GemmBatch g{};
        g.t[0] = dx_task(dy(l), w.ldy[l], params + w_off[l], act[l - 1], dy(l - 1), w.ldy[l - 1], B, dims[l],
                         dims[l + 1]);
        pad_a(g.t[0], w.ldy[l]);
        g.ntask = 1;
        if (int rc = run_batch(g, s, "upstream-gradient launch")) return rc;
    }
    // every layer's weight- and bias-gradient splits: one launch per group of
    // layers whose operands take the same loads (16-byte or not)
    {
        gemm::GemmBatch groups[4] = {};
        float* part = wsf + w.part_off;
        for (int l = 0; l < L; ++l) {
            gemm::GemmTask t = dw_task(dy(l), w.ldy[l], input(l), B, dims[l], dims[l + 1], part + w_off[l], w.Ptot,
                                      part + b_off[l], w.Ptot);
            pad_a(t, w.ldy[l]);
            const int64_t next = l + 1 < L ? w_off[l + 1] : w.Ptot;
            t.zlo[0] = (int64_t)dims[l + 1] * dims[l];
            t.zhi[0] = b_off[l] - w_off[l];
            t.zlo[1] = b_off[l] - w_off[l] + dims[l + 1];
            t.zhi[1] = next - w_off[l];
            gemm::GemmBatch& g = groups[2 * t.A.vec + t.B.vec];
            g.t[g.ntask++] = t;
        }
        for (gemm::GemmBatch& g : groups)
            if (g.ntask > 0)
                if (int rc = run_batch(g, s, "weight-gradient launch")) return rc;
    }
    // the splits and the partial losses, added in a fixed order, one launch
    {
        float* part = wsf + w.part_off;
        cfc::ReduceSeg seg{part, grads, w.Ptot, 0};
        const int V = (aligned16(part) && aligned16(grads)) ? 4 : 1;
        seg.groups = (seg.N + V - 1) / V;
        CFC_HIP(cfc::launch_reduce_with_sum(&seg, 1, w.S, V, wsf + w.loss_off, w.P, loss, s), "reduce launch");
    }
    return CFC_OK;
}

}  // extern "C"
