// C ABI of libcfc.so (declared in include/cfc.h): argument checks, tiling
// plans, the eager step launches and the cached HIP graph of the whole
// K-loop training step.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/cfc.h"
#include "api_common.h"
#include "cfc_kernels.h"
#include "cfc_math.h"
#include "gemm_kernels.h"

namespace {

using cfc_host::fail;
using cfc_host::hip_fail;
using cfc_host::Span;
using cfc_host::overlap;
using cfc_host::span;
using cfc_host::aligned16;

constexpr int64_t kMaxB = int64_t(1) << 24;

int check_dims(int B, int C, int n_x)
{
    if (B < 0 || B > kMaxB) return fail(CFC_EINVAL, "B=%d out of range [0, %lld]", B, (long long)kMaxB);
    if (C < 1 || C > CFC_MAX_C) return fail(CFC_EINVAL, "C=%d out of range [1, %d]", C, CFC_MAX_C);
    if (n_x < 0 || n_x + C > CFC_MAX_N_IN)
        return fail(CFC_EINVAL, "n_x=%d out of range (n_in = n_x + C must be <= %d)", n_x, CFC_MAX_N_IN);
    return CFC_OK;
}

// Tiling of the step kernels: channel tiles of 16 (one XCD per tile index
// mod 8); several samples per workgroup once the batch is large enough that
// W re-reads from L2, not the number of workgroups, limit the step.  None of
// these choices changes the arithmetic of any output.
cfc::StepPlan make_plan(int B, int C, int n_x, const float* W, const float* scratch)
{
    cfc::StepPlan p{};
    const int n_in = n_x + C;
    p.CT = 16;
    p.n_ctiles = (C + p.CT - 1) / p.CT;
    p.BT = B >= 128 ? 4 : 1;
    p.ldz = (n_in + 3) & ~3;
    p.ldu = (n_x + 3) & ~3;
    p.ldh = (C + 3) & ~3;
    auto smem = [&](int bt) {
        const size_t fwd = sizeof(float) * ((size_t)bt * (p.ldu + p.ldh) + (size_t)bt * 3 * p.CT);
        const size_t bwd = sizeof(float) * ((size_t)bt * p.ldz + (size_t)bt * 3 * C +
                                            (size_t)cfc::kDzGroups * bt * cfc::kCols);
        return std::make_pair(fwd, bwd);
    };
    while (p.BT > 1 && smem(p.BT).second > 64 * 1024) p.BT /= 2;
    p.fwd_smem = smem(p.BT).first;
    p.bwd_smem = smem(p.BT).second;
    p.n_btiles = B > 0 ? (B + p.BT - 1) / p.BT : 0;
    // Only the load width depends on these; the arithmetic does not.
    p.Vf = (n_in % 4 == 0 && n_x % 4 == 0 && aligned16(W)) ? 4 : 1;
    p.Vb = (n_in % 4 == 0 && scratch != nullptr && aligned16(scratch)) ? 4 : 1;
    return p;
}

int check_plan(const cfc::StepPlan& p)
{
    if (p.bwd_smem > 64 * 1024 || p.fwd_smem > 64 * 1024)
        return fail(CFC_EINVAL, "sizes need %zu bytes of LDS per workgroup (limit 65536)", p.bwd_smem);
    if ((int64_t)p.n_btiles * p.n_ctiles > 0x7fffffffLL) return fail(CFC_EINVAL, "grid too large");
    return CFC_OK;
}

int enqueue_fwd(const float* u_t, const float* h_prev, const float* W, const float* bias, float* h_t,
                float* act_t, float* h_prev_copy, int B, int C, int n_x, const cfc::StepPlan& p,
                hipStream_t s)
{
    if (B == 0) return CFC_OK;
    cfc::FwdArgs a{u_t, h_prev, W, bias, h_t, act_t, h_prev_copy, B, C, n_x, p.CT, p.n_ctiles, p.ldu, p.ldh};
    CFC_HIP(cfc::launch_fwd(a, p, s), "forward step launch");
    return CFC_OK;
}

int enqueue_bwd(const float* u_t, const float* h_prev, const float* h_t, const float* y_t,
                const float* W, const float* act_t, const float* dh_in, float* dh_out, float* du_t,
                float* gW_s, float* gb_s, float* dp_out, int B, int C, int n_x, const cfc::StepPlan& p,
                hipStream_t s)
{
    if (B == 0) return CFC_OK;
    cfc::BwdArgs a{u_t, h_prev, h_t, y_t, W, act_t, dh_in, dh_out, du_t, gW_s, gb_s, dp_out,
                   B, C, n_x, p.CT, p.n_ctiles, p.ldz};
    CFC_HIP(cfc::launch_bwd(a, p, s), "backward step launch");
    return CFC_OK;
}

int enqueue_reduce(const cfc::ReduceSeg* segs_in, int nseg, int64_t B, hipStream_t s)
{
    cfc::ReduceSeg segs[cfc::kMaxReduceSegs];
    int n = 0;
    bool vec = true;
    for (int i = 0; i < nseg; ++i) {
        if (segs_in[i].N == 0) continue;
        if (B == 0) {
            CFC_HIP(cfc::launch_fill_zero(segs_in[i].out, segs_in[i].N, s), "reduce (zero fill) launch");
            continue;
        }
        segs[n++] = segs_in[i];
        vec = vec && segs_in[i].N % 4 == 0 && aligned16(segs_in[i].in) && aligned16(segs_in[i].out);
    }
    if (n == 0) return CFC_OK;
    const int V = vec ? 4 : 1;
    for (int i = 0; i < n; ++i) segs[i].groups = (segs[i].N + V - 1) / V;
    CFC_HIP(cfc::launch_reduce(segs, n, B, V, s), "reduce_axis0 launch");
    return CFC_OK;
}

// Workspace: dp [K, B, 3C] | X [K, B, 3C] (input projection, persistent
// path) | dh ping-pong [2, B, C] (step path) | padding to 256 bytes | the
// MFMA step path's re-laid W (forward layout, then backward layout).
int64_t kloop_ws_wofs(int B, int C, int K) { return ((int64_t)2 * K * B * 3 * C + (int64_t)2 * B * C + 63) & ~(int64_t)63; }
// After the re-laid W: the resident kernel's exchange blocks, then its step
// counters (one per workgroup) and error word; all zeroed before its launch.
int64_t kloop_ws_flags(int B, int C)
{
    return ((((int64_t)(B + 15) / 16) * ((C + 15) / 16) + 1) * cfc::kResFlagStride + 63) & ~(int64_t)63;
}
int64_t kloop_ws_resident(int B, int C) { return cfc::resident_exchange_floats(B, C) + kloop_ws_flags(B, C); }
// Last: the flags of the persistent launch that also forms X (one per
// projection workgroup, then its error word, then one per sample and
// backward chunk of 16 steps for a launch that also forms the scratch).
int64_t kloop_ws_pofs(int B, int C, int n_x, int K)
{
    return kloop_ws_wofs(B, C, K) + cfc::mfma_w_floats(C, n_x) + kloop_ws_resident(B, C);
}
int64_t kloop_ws_proj(int B, int C, int K)
{
    const int n = cfc::persist_proj_blocks(B, C, K);
    return n < 0 ? 0 : ((int64_t)n + 1 + (int64_t)B * ((K + 15) / 16) + 63) & ~(int64_t)63;
}
int64_t kloop_ws_floats(int B, int C, int n_x, int K)
{
    return kloop_ws_pofs(B, C, n_x, K) + kloop_ws_proj(B, C, K);
}

struct KloopArgs {
    const float *u, *y, *h0, *W, *bias;
    float *h_hist, *act, *ws, *gW_s, *gb_s, *gW, *gb;
    int B, C, n_x, K;
};

// K-loop paths: step kernels on VALU, step kernels on MFMA, persistent,
// resident MFMA.
enum class Path { Steps = 0, StepsMfma = 1, Persistent = 2, Resident = 3 };

// The path mode of the calling thread (cfc_set_kloop_mode): per thread, so
// that one caller forcing a path never changes another thread's calls.
thread_local int g_kloop_mode = CFC_KLOOP_AUTO;

// Smallest batch for which the automatic choice takes the MFMA step kernels
// (a 16-sample MFMA tile wastes most of its rows below this).
constexpr int kMfmaMinB = 64;

// Polls of one wait of the resident kernel before it gives up (each poll is
// one load of the counters and a short sleep, about a microsecond): far
// beyond any step, so that it only ends a wait that cannot end.
constexpr int kResidentSpinLimit = 1 << 20;
// The persistent launch forms X itself (extra workgroups ahead of the sample
// workgroups, which wait for them) when at most this many samples: the
// sample workgroups, one per CU, then leave at least half the CUs to the
// projection, whatever order the workgroups start in.
constexpr int kPersistFuseMaxB = 128;
constexpr int kPersistSpinLimit = 1 << 20;
// Launch numbers for the projection flags: distinct for 2^32 launches, never 0.
std::atomic<unsigned> g_persist_call{0x9e3779b9u};
unsigned next_persist_call()
{
    unsigned c = g_persist_call.fetch_add(1, std::memory_order_relaxed) + 1;
    while (c == 0) c = g_persist_call.fetch_add(1, std::memory_order_relaxed) + 1;
    return c;
}
// CUs of the current device (read once per device); 0 if unknown.
int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cus[dev].store(n, std::memory_order_relaxed);
    return n > 0 ? n : 0;
}
bool stream_capturing(hipStream_t s)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return !(hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusNone);
}

// A cooperative launch cannot be captured into a graph: a stream under
// capture takes the MFMA step kernels instead of the resident kernel.
Path uncaptured(Path path, hipStream_t s)
{
    if (path != Path::Resident) return path;
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusNone) return path;
    return Path::StepsMfma;
}

// The path a K-loop call of these sizes takes in `mode`; false if the mode
// forces a path the sizes cannot take.
// `ptrs` (nullable) are the arrays the step kernels read with 16-byte loads;
// null means: assume them aligned.
bool choose_path(int mode, int B, int C, int n_x, std::initializer_list<const void*> ptrs, Path* out)
{
    const bool pers_ok = cfc::persist_smem(C) != 0;   // the input projection runs outside it: any n_x
    bool aligned = true;
    for (const void* p : ptrs) aligned = aligned && (p == nullptr || aligned16(p));
    const bool mfma_ok = cfc::mfma_fits(C, n_x) && aligned;
    // the resident kernel: the MFMA step kernels' shapes, with every
    // workgroup of its grid resident on the current device at once
    const bool res_ok = mfma_ok && (int64_t)((B + 15) / 16) * ((C + 15) / 16) <=
                                       cfc::resident_capacity(cfc::mfma_layout(C, n_x));
    switch (mode) {
    case CFC_KLOOP_PERSISTENT: *out = Path::Persistent; return pers_ok;
    case CFC_KLOOP_STEPS_VALU: *out = Path::Steps; return true;
    case CFC_KLOOP_STEPS_MFMA: *out = Path::StepsMfma; return mfma_ok;
    case CFC_KLOOP_RESIDENT: *out = Path::Resident; return res_ok;
    case CFC_KLOOP_STEPS: *out = (mfma_ok && B >= kMfmaMinB) ? Path::StepsMfma : Path::Steps; return true;
    default:
        *out = pers_ok ? Path::Persistent
             : (mfma_ok && B >= kMfmaMinB) ? (res_ok ? Path::Resident : Path::StepsMfma) : Path::Steps;
        return true;
    }
}

// Forward t = 1..K and backward t = K..1 of every sample, storing dp_t.
//  persistent path: the input projection of all steps, then one kernel
//                   with one workgroup per sample;
//  step paths:      K forward step launches (the first also copies h0 into
//                   h_hist[0]) and K backward step launches; the MFMA ones
//                   after one launch that re-lays W into their operand
//                   layouts.
// filled (nullable): the scratch of gW_s / gb_s may be formed by the same
// launch; *filled tells whether it was.
int enqueue_fwd_bwd(const KloopArgs& k, Path path, const cfc::StepPlan& p, hipStream_t s, bool* filled = nullptr)
{
    if (filled) *filled = false;
    const int64_t BC = (int64_t)k.B * k.C;
    const int64_t BX = (int64_t)k.B * k.n_x;
    float* dp = k.ws;                                   // [K, B, 3C]
    float* X = k.ws + (int64_t)k.K * 3 * BC;            // [K, B, 3C]
    float* dh_ws = k.ws + (int64_t)2 * k.K * 3 * BC;    // [2, B, C]
    if (path == Path::Persistent) {
        cfc::PersistArgs a{X, k.y, k.h0, k.W, k.bias, k.h_hist, k.act, dp, k.B, k.C, k.n_x, k.K};
        const int n_proj = cfc::persist_proj_blocks(k.B, k.C, k.K);
        // One launch that forms X and runs the recurrence; a stream under
        // capture takes two (a replayed graph would repeat the launch number
        // that the flags are matched against).
        if (k.B <= kPersistFuseMaxB && n_proj > 0 && !stream_capturing(s)) {
            a.u = k.u;
            a.flags = reinterpret_cast<int*>(k.ws + kloop_ws_pofs(k.B, k.C, k.n_x, k.K));
            a.n_proj = n_proj;
            a.call = next_persist_call();
            a.spin_limit = kPersistSpinLimit;
            // the scratch too, by fill units that follow the backward chunk by chunk
            // (16-byte rows on every array they or the samples move)
            if (filled && k.gW_s && k.gb_s && cfc::persist_fill_fits(k.B, k.C, k.n_x, k.K, device_cus()) &&
                aligned16(k.ws) && aligned16(k.h_hist) && aligned16(k.act) && aligned16(k.y) &&
                aligned16(k.gW_s) && (k.n_x == 0 || aligned16(k.u))) {
                a.gW_s = k.gW_s;
                a.gb_s = k.gb_s;
                a.n_fill = k.B * ((3 * k.C + 63) / 64);
                *filled = true;
            }
            CFC_HIP(cfc::launch_persist(a, s), a.n_fill ? "persistent K-loop launch (with the projection and the scratch)"
                                                        : "persistent K-loop launch (with the input projection)");
            return CFC_OK;
        }
        const cfc::XprojArgs x{k.u, k.W, k.bias, X, (int64_t)k.K * k.B, 3 * k.C, k.n_x, k.n_x + k.C,
                               (3 * k.C + 63) / 64};
        CFC_HIP(cfc::launch_xproj(x, s), "input projection launch");
        CFC_HIP(cfc::launch_persist(a, s), "persistent K-loop launch");
        return CFC_OK;
    }
    if (path == Path::Resident) {
        const cfc::MfmaLayout L = cfc::mfma_layout(k.C, k.n_x);
        float* Wf = k.ws + kloop_ws_wofs(k.B, k.C, k.K);
        float* Wb = Wf + (int64_t)3 * k.C * L.ldf;
        float* xch = k.ws + kloop_ws_wofs(k.B, k.C, k.K) + cfc::mfma_w_floats(k.C, k.n_x);
        float* flags = xch + cfc::resident_exchange_floats(k.B, k.C);
        CFC_HIP(cfc::launch_permute_w(cfc::PermuteArgs{k.W, Wf, Wb, k.C, k.n_x, L}, s), "W re-layout launch");
        CFC_HIP(cfc::launch_fill_zero(xch, kloop_ws_resident(k.B, k.C), s), "exchange and counter zero fill");
        cfc::ResidentArgs a{};
        a.u = k.u;
        a.y = k.y;
        a.h0 = k.h0;
        a.Wf = Wf;
        a.Wb = Wb;
        a.bias = k.bias;
        a.h_hist = k.h_hist;
        a.act = k.act;
        a.dp = dp;
        a.hx = xch;
        a.dpx = xch + 2 * (((int64_t)k.B + 15) / 16) * 16 * ((k.C + 31) & ~31);
        a.flags = reinterpret_cast<int*>(flags);
        a.B = k.B;
        a.C = k.C;
        a.n_x = k.n_x;
        a.K = k.K;
        a.n_ctiles = (k.C + 15) / 16;
        a.L = L;
        a.spin_limit = kResidentSpinLimit;
        CFC_HIP(cfc::launch_resident(a, s), "resident K-loop launch");
        return CFC_OK;
    }
    if (path == Path::StepsMfma) {
        const cfc::MfmaLayout L = cfc::mfma_layout(k.C, k.n_x);
        float* Wf = k.ws + kloop_ws_wofs(k.B, k.C, k.K);
        float* Wb = Wf + (int64_t)3 * k.C * L.ldf;
        CFC_HIP(cfc::launch_permute_w(cfc::PermuteArgs{k.W, Wf, Wb, k.C, k.n_x, L}, s), "W re-layout launch");
        const int nct = (k.C + 15) / 16;
        for (int t = 1; t <= k.K; ++t) {
            const float* h_prev = (t == 1) ? k.h0 : k.h_hist + (t - 1) * BC;
            const cfc::FwdMfmaArgs a{k.u + (t - 1) * BX, h_prev, Wf, k.bias, k.h_hist + t * BC,
                                     k.act + (int64_t)(t - 1) * 3 * BC, t == 1 ? k.h_hist : nullptr,
                                     k.B, k.C, k.n_x, nct, L};
            CFC_HIP(cfc::launch_fwd_mfma(a, s), "forward step launch");
        }
        // The launch of step t forms the carry of its channel tile and, from it,
        // dp of step t - 1 for those channels; the launch of step t - 1 then
        // reads dp instead of forming it (only the first launch, t = K with
        // zero carry, forms dp from h, y and act itself).
        for (int t = k.K; t >= 1; --t) {
            cfc::BwdMfmaArgs a{};
            a.h_t = k.h_hist + t * BC;
            a.y_t = k.y + (t - 1) * BC;
            a.act_t = k.act + (int64_t)(t - 1) * 3 * BC;
            a.dh_in = nullptr;
            a.Wb = Wb;
            a.dh_out = nullptr;
            a.dp_out = dp + (int64_t)(t - 1) * 3 * BC;
            a.B = k.B;
            a.C = k.C;
            a.n_ctiles = nct;
            a.L = L;
            a.dp_in = (t == k.K) ? nullptr : dp + (int64_t)(t - 1) * 3 * BC;
            if (t > 1) {
                a.h_prev = k.h_hist + (t - 1) * BC;
                a.y_prev = k.y + (t - 2) * BC;
                a.act_prev = k.act + (int64_t)(t - 2) * 3 * BC;
                a.dp_prev_out = dp + (int64_t)(t - 2) * 3 * BC;
            }
            CFC_HIP(cfc::launch_bwd_mfma(a, s), "backward step launch");
        }
        return CFC_OK;
    }
    for (int t = 1; t <= k.K; ++t) {
        const float* h_prev = (t == 1) ? k.h0 : k.h_hist + (t - 1) * BC;
        const int rc = enqueue_fwd(k.u + (t - 1) * BX, h_prev, k.W, k.bias, k.h_hist + t * BC,
                                   k.act + (int64_t)(t - 1) * 3 * BC, t == 1 ? k.h_hist : nullptr, k.B, k.C,
                                   k.n_x, p, s);
        if (rc) return rc;
    }
    for (int t = k.K; t >= 1; --t) {
        const int step = k.K - t;  // 0 for t = K
        const float* dh_in = (t == k.K) ? nullptr : dh_ws + ((step - 1) % 2) * BC;
        float* dh_out = dh_ws + (step % 2) * BC;
        const int rc = enqueue_bwd(k.u + (t - 1) * BX, k.h_hist + (t - 1) * BC, k.h_hist + t * BC,
                                   k.y + (t - 1) * BC, k.W, k.act + (int64_t)(t - 1) * 3 * BC, dh_in,
                                   dh_out, nullptr, nullptr, nullptr, dp + (int64_t)(t - 1) * 3 * BC, k.B,
                                   k.C, k.n_x, p, s);
        if (rc) return rc;
    }
    return CFC_OK;
}

int enqueue_fill(const float* dp, const float* u, const float* h_hist, float* gW_s, float* gb_s, int B, int C,
                 int n_x, int K, hipStream_t s)
{
    const int n_in = n_x + C;
    const cfc::FillArgs f{dp, u, h_hist, gW_s, gb_s, B, C, n_x, K,
                          (3 * C + cfc::kFillTile - 1) / cfc::kFillTile,
                          (n_in + cfc::kFillTile - 1) / cfc::kFillTile};
    CFC_HIP(cfc::launch_fill(f, s), "scratch fill launch");
    return CFC_OK;
}

// The whole K-loop step: forward and backward, the scratch fill (each
// sample's sums over t, written once) and one reduction launch over both
// scratch tensors.
int enqueue_kloop(const KloopArgs& k, Path path, const cfc::StepPlan& p, hipStream_t s)
{
    const int n_in = k.n_x + k.C;
    bool filled = false;
    if (int rc = enqueue_fwd_bwd(k, path, p, s, &filled)) return rc;
    if (!filled)
        if (int rc = enqueue_fill(k.ws, k.u, k.h_hist, k.gW_s, k.gb_s, k.B, k.C, k.n_x, k.K, s)) return rc;
    cfc::ReduceSeg segs[2] = {
        {k.gW_s, k.gW, (int64_t)3 * k.C * n_in, 0},
        {k.gb_s, k.gb, (int64_t)3 * k.C, 0},
    };
    return enqueue_reduce(segs, 2, k.B, s);
}

// ---------------------------------------------------------------------------
// Graph cache of the K-loop step, keyed on device, path, pointer values and
// sizes.
// ---------------------------------------------------------------------------
using GraphKey = std::tuple<int, int, const void*, const void*, const void*, const void*, const void*,
                            void*, void*, void*, void*, void*, void*, void*, int, int, int, int>;

struct GraphEntry {
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;
    uint64_t last_use = 0;
};

constexpr size_t kMaxGraphs = 64;

std::mutex g_mu;
std::map<GraphKey, GraphEntry> g_graphs;
std::map<int, hipStream_t> g_capture_streams;
uint64_t g_clock = 0;
// Evicted graphs whose last replay may still be running: destroyed by a later
// call once their completion event reports done, so that no call of the
// K-loop ever waits on the device.
std::vector<GraphEntry> g_retired;

void release_entry(GraphEntry& e)
{
    if (e.done) (void)hipEventDestroy(e.done);
    if (e.exec) (void)hipGraphExecDestroy(e.exec);
    e = GraphEntry{};
}

// Blocking destruction, for cfc_clear_graph_cache only.
void destroy_entry(GraphEntry& e)
{
    if (e.done) (void)hipEventSynchronize(e.done);
    release_entry(e);
}

// Destroy the retired graphs whose last replay has completed; the others
// stay retired.  Never blocks (hipEventQuery only asks).
void reap_retired()
{
    size_t keep = 0;
    for (size_t i = 0; i < g_retired.size(); ++i) {
        GraphEntry& e = g_retired[i];
        if (!e.done || hipEventQuery(e.done) == hipSuccess)
            release_entry(e);
        else
            g_retired[keep++] = e;
    }
    g_retired.resize(keep);
}

int build_graph(const KloopArgs& k, Path path, const cfc::StepPlan& p, int dev, GraphEntry& out)
{
    hipStream_t cap;
    auto it = g_capture_streams.find(dev);
    if (it == g_capture_streams.end()) {
        CFC_HIP(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking), "capture stream create");
        g_capture_streams[dev] = cap;
    } else {
        cap = it->second;
    }
    CFC_HIP(hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal), "graph capture begin");
    const int rc = enqueue_kloop(k, path, p, cap);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(cap, &graph);
    if (rc != CFC_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (ec != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return hip_fail(ec, "graph capture end");
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return hip_fail(ei, "graph instantiate");
    hipEvent_t done;
    const hipError_t ee = hipEventCreateWithFlags(&done, hipEventDisableTiming);
    if (ee != hipSuccess) {
        (void)hipGraphExecDestroy(exec);
        return hip_fail(ee, "event create");
    }
    out.exec = exec;
    out.done = done;
    return CFC_OK;
}

}  // namespace

extern "C" {

const char* cfc_last_error(void) { return cfc_host::last_error().c_str(); }

int cfc_fwd_step(const float* u_t, const float* h_prev, const float* W, const float* bias, float* h_t,
                 float* act_t, int B, int C, int n_x, void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (B == 0) return CFC_OK;
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    if (!h_prev || !W || !bias || !h_t || !act_t || (n_x > 0 && !u_t))
        return fail(CFC_EINVAL, "cfc_fwd_step: null pointer");
    const Span outs[] = {span(h_t, BC), span(act_t, 3 * BC)};
    const Span ins[] = {span(u_t, (int64_t)B * n_x), span(h_prev, BC), span(W, 3 * C * n_in),
                        span(bias, 3 * C)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return fail(CFC_EINVAL, "cfc_fwd_step: an output overlaps an input");
    if (overlap(outs[0], outs[1])) return fail(CFC_EINVAL, "cfc_fwd_step: h_t overlaps act_t");
    const cfc::StepPlan p = make_plan(B, C, n_x, W, nullptr);
    if (int rc = check_plan(p)) return rc;
    return enqueue_fwd(u_t, h_prev, W, bias, h_t, act_t, nullptr, B, C, n_x, p, (hipStream_t)stream);
}

int cfc_bwd_step(const float* u_t, const float* h_prev, const float* h_t, const float* y_t,
                 const float* W, const float* act_t, const float* dh_in, float* dh_out, float* du_t,
                 float* gW_scratch, float* gb_scratch, int B, int C, int n_x, void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (B == 0) return CFC_OK;
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    if (!h_prev || !h_t || !y_t || !W || !act_t || !dh_out || !gW_scratch || !gb_scratch ||
        (n_x > 0 && !u_t))
        return fail(CFC_EINVAL, "cfc_bwd_step: null pointer");
    if (n_x == 0) du_t = nullptr;
    const Span outs[] = {span(dh_out, BC), span(du_t, (int64_t)B * n_x),
                         span(gW_scratch, BC * 3 * n_in), span(gb_scratch, 3 * BC)};
    const Span ins[] = {span(u_t, (int64_t)B * n_x), span(h_prev, BC), span(h_t, BC), span(y_t, BC),
                        span(W, 3 * C * n_in), span(act_t, 3 * BC), span(dh_in, BC)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return fail(CFC_EINVAL, "cfc_bwd_step: an output overlaps an input");
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "cfc_bwd_step: outputs overlap");
    const cfc::StepPlan p = make_plan(B, C, n_x, W, gW_scratch);
    if (int rc = check_plan(p)) return rc;
    return enqueue_bwd(u_t, h_prev, h_t, y_t, W, act_t, dh_in, dh_out, du_t, gW_scratch, gb_scratch, nullptr,
                       B, C, n_x, p, (hipStream_t)stream);
}

int reduce_axis0(const float* per_batch, int64_t n_batch, int64_t n_tail, float* out, void* stream)
{
    cfc_host::last_error().clear();
    if (n_batch < 0 || n_tail < 0) return fail(CFC_EINVAL, "reduce_axis0: negative size");
    if (n_tail == 0) return CFC_OK;
    if (!out || (n_batch > 0 && !per_batch)) return fail(CFC_EINVAL, "reduce_axis0: null pointer");
    if (n_batch > 0 && n_tail > INT64_MAX / 4 / n_batch) return fail(CFC_EINVAL, "reduce_axis0: size overflow");
    if (overlap(Span{per_batch, (size_t)(n_batch * n_tail) * 4}, Span{out, (size_t)n_tail * 4}))
        return fail(CFC_EINVAL, "reduce_axis0: out overlaps per_batch");
    const cfc::ReduceSeg seg{per_batch, out, n_tail, 0};
    return enqueue_reduce(&seg, 1, n_batch, (hipStream_t)stream);
}

size_t cfc_train_kloop_workspace_bytes(int B, int C, int n_x, int K)
{
    if (B < 0 || C < 1 || n_x < 0 || K < 0) return 0;
    return (size_t)kloop_ws_floats(B, C, n_x, K) * sizeof(float);
}

int cfc_set_kloop_mode(int mode)
{
    cfc_host::last_error().clear();
    if (mode < CFC_KLOOP_AUTO || mode > CFC_KLOOP_RESIDENT)
        return fail(CFC_EINVAL, "cfc_set_kloop_mode: unknown mode %d", mode);
    g_kloop_mode = mode;
    return CFC_OK;
}

int cfc_kloop_path(int B, int C, int n_x, int K)
{
    if (B < 0 || K < 0 || C < 1 || n_x < 0) return -1;
    Path path;
    if (!choose_path(g_kloop_mode, B, C, n_x, {}, &path)) return -1;
    return path == Path::Persistent ? CFC_KLOOP_PERSISTENT
         : path == Path::Resident   ? CFC_KLOOP_RESIDENT
         : path == Path::StepsMfma  ? CFC_KLOOP_STEPS_MFMA : CFC_KLOOP_STEPS_VALU;
}

int cfc_kloop_status(const float* ws, size_t ws_bytes, int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "cfc_kloop_status";
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "%s: K=%d out of range", fn, K);
    const int64_t ws_floats = kloop_ws_floats(B, C, n_x, K);
    if (ws == nullptr || ws_bytes < (size_t)ws_floats * sizeof(float))
        return fail(CFC_EINVAL, "%s: workspace of %zu bytes, %lld needed", fn, ws_bytes, (long long)(ws_floats * 4));
    if (K == 0 || B == 0) return CFC_OK;   // nothing was launched
    Path path;
    if (!choose_path(g_kloop_mode, B, C, n_x, {}, &path))
        return fail(CFC_EINVAL, "%s: the K-loop mode forces a path these sizes cannot take", fn);
    hipStream_t s = (hipStream_t)stream;
    int words[2] = {0, 0};
    if (path == Path::Resident) {
        // the error word after the step counters (zeroed before every launch)
        const float* flags = ws + kloop_ws_wofs(B, C, K) + cfc::mfma_w_floats(C, n_x) + cfc::resident_exchange_floats(B, C);
        const int64_t n = ((int64_t)(B + 15) / 16) * ((C + 15) / 16);
        CFC_HIP(hipMemcpyAsync(&words[0], flags + n * cfc::kResFlagStride, sizeof(int), hipMemcpyDeviceToHost, s),
                "status read");
        CFC_HIP(hipStreamSynchronize(s), "status wait");
        if (words[0] != 0)
            return fail(CFC_EHIP, "%s: a bounded wait of the resident K-loop launch gave up; its results are undefined",
                        fn);
        return CFC_OK;
    }
    const int n_proj = cfc::persist_proj_blocks(B, C, K);
    if (path == Path::Persistent && B <= kPersistFuseMaxB && n_proj > 0) {
        // flags[0] holds the number of the last launch that formed X here;
        // the error word holds it too if that launch's wait gave up
        const float* f = ws + kloop_ws_pofs(B, C, n_x, K);
        CFC_HIP(hipMemcpyAsync(&words[0], f, sizeof(int), hipMemcpyDeviceToHost, s), "status read");
        CFC_HIP(hipMemcpyAsync(&words[1], f + n_proj, sizeof(int), hipMemcpyDeviceToHost, s), "status read");
        CFC_HIP(hipStreamSynchronize(s), "status wait");
        if (words[0] != 0 && words[1] == words[0])
            return fail(CFC_EHIP,
                        "%s: the persistent launch's wait for its input projection gave up; its results are undefined",
                        fn);
    }
    return CFC_OK;
}

// Checks shared by cfc_train_kloop and cfc_kloop_fwd_bwd; sets *path.
static int check_kloop(const char* fn, const float* u, const float* y, const float* h0, const float* W,
                const float* bias, float* h_hist, float* act, float* ws, size_t ws_bytes, float* gW_scratch,
                float* gb_scratch, float* gW, float* gb, int B, int C, int n_x, int K, bool full,
                Path* path)
{
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "%s: K=%d out of range", fn, K);
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    const int64_t ws_floats = kloop_ws_floats(B, C, n_x, K);
    if (ws_bytes < (size_t)ws_floats * sizeof(float))
        return fail(CFC_EINVAL, "%s: workspace of %zu bytes, %lld needed", fn, ws_bytes,
                    (long long)(ws_floats * 4));
    // a pointer may be null only when its array is empty
    const struct {
        const void* p;
        int64_t n;
    } need[] = {{u, (int64_t)K * B * n_x}, {y, (int64_t)K * BC}, {h0, BC}, {W, 3 * C * n_in},
                {bias, 3 * C}, {h_hist, (K + 1) * BC}, {act, (int64_t)K * 3 * BC}, {ws, ws_floats},
                {gW_scratch, full ? BC * 3 * n_in : 0}, {gb_scratch, full ? 3 * BC : 0},
                {gW, full ? 3 * C * n_in : 0}, {gb, full ? 3 * C : 0}};
    for (const auto& q : need)
        if (q.n > 0 && q.p == nullptr) return fail(CFC_EINVAL, "%s: null pointer", fn);
    const Span outs[] = {span(h_hist, (K + 1) * BC), span(act, (int64_t)K * 3 * BC), span(ws, ws_floats),
                         span(gW_scratch, BC * 3 * n_in), span(gb_scratch, 3 * BC),
                         span(gW, 3 * C * n_in), span(gb, 3 * C)};
    const Span ins[] = {span(u, (int64_t)K * B * n_x), span(y, (int64_t)K * BC), span(h0, BC),
                        span(W, 3 * C * n_in), span(bias, 3 * C)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return fail(CFC_EINVAL, "%s: an output overlaps an input", fn);
    for (int i = 0; i < 7; ++i)
        for (int j = i + 1; j < 7; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "%s: outputs overlap", fn);
    const int mode = g_kloop_mode;
    if (!choose_path(mode, B, C, n_x, {ws, u, y, h0, h_hist, act}, path)) {
        if (mode == CFC_KLOOP_PERSISTENT)
            return fail(CFC_EINVAL, "%s: the persistent kernel holds C <= 128 channels (C=%d)", fn, C);
        if (mode == CFC_KLOOP_RESIDENT && cfc::mfma_fits(C, n_x))
            return fail(CFC_EINVAL, "%s: the resident kernel's %lld workgroups do not fit the device at once, "
                        "or an array is not 16-byte aligned (B=%d C=%d)", fn,
                        (long long)(((int64_t)B + 15) / 16 * ((C + 15) / 16)), B, C);
        return fail(CFC_EINVAL, "%s: the MFMA step kernels take C <= 320 and n_x <= 128, both multiples of 4, "
                    "and 16-byte aligned arrays (C=%d n_x=%d)", fn, C, n_x);
    }
    if (*path == Path::Steps)
        if (int rc = check_plan(make_plan(B, C, n_x, W, gW_scratch))) return rc;
    return CFC_OK;
}

int cfc_train_kloop(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                    float* h_hist, float* act, float* ws, size_t ws_bytes, float* gW_scratch,
                    float* gb_scratch, float* gW, float* gb, int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    Path path = Path::Steps;
    if (int rc = check_kloop("cfc_train_kloop", u, y, h0, W, bias, h_hist, act, ws, ws_bytes, gW_scratch,
                             gb_scratch, gW, gb, B, C, n_x, K, true, &path))
        return rc;
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    const cfc::StepPlan p = make_plan(B, C, n_x, W, gW_scratch);
    hipStream_t s = (hipStream_t)stream;

    if (K == 0 || B == 0) {
        // Nothing to replay: h_hist[0] = h0, scratch and gradients zero.
        if (BC > 0) CFC_HIP(hipMemcpyAsync(h_hist, h0, BC * 4, hipMemcpyDeviceToDevice, s), "h0 copy");
        CFC_HIP(cfc::launch_fill_zero(gW_scratch, BC * 3 * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb_scratch, 3 * BC, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gW, 3 * C * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb, 3 * C, s), "zero fill");
        return CFC_OK;
    }

    const KloopArgs k{u, y, h0, W, bias, h_hist, act, ws, gW_scratch, gb_scratch, gW, gb, B, C, n_x, K};
    // The persistent path is four launches (input projection, K-loop,
    // scratch fill, reduction), enqueued directly: replaying them as a graph
    // measured about 5 us slower per step.  The step path's 2K + 2 launches
    // go through the cached graph.
    path = uncaptured(path, s);
    if (path == Path::Persistent || path == Path::Resident) return enqueue_kloop(k, path, p, s);

    int dev = 0;
    CFC_HIP(hipGetDevice(&dev), "hipGetDevice");
    const GraphKey key{dev, (int)path, u, y, h0, W, bias, h_hist, act, ws, gW_scratch, gb_scratch,
                       gW, gb, B, C, n_x, K};
    std::lock_guard<std::mutex> lock(g_mu);
    reap_retired();
    auto it = g_graphs.find(key);
    if (it == g_graphs.end()) {
        if (g_graphs.size() >= kMaxGraphs) {
            // the least recently used graph leaves the cache; it is destroyed
            // by a later call once its last replay has completed
            auto victim = g_graphs.begin();
            for (auto j = g_graphs.begin(); j != g_graphs.end(); ++j)
                if (j->second.last_use < victim->second.last_use) victim = j;
            g_retired.push_back(victim->second);
            g_graphs.erase(victim);
        }
        GraphEntry e;
        if (int rc = build_graph(k, path, p, dev, e)) return rc;
        it = g_graphs.emplace(key, e).first;
    }
    GraphEntry& e = it->second;
    e.last_use = ++g_clock;
    CFC_HIP(hipGraphLaunch(e.exec, s), "graph launch");
    CFC_HIP(hipEventRecord(e.done, s), "event record");
    return CFC_OK;
}

int cfc_kloop_fwd_bwd(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                      float* h_hist, float* act, float* ws, size_t ws_bytes, int B, int C, int n_x, int K,
                      void* stream)
{
    cfc_host::last_error().clear();
    Path path = Path::Steps;
    if (int rc = check_kloop("cfc_kloop_fwd_bwd", u, y, h0, W, bias, h_hist, act, ws, ws_bytes, nullptr, nullptr,
                             nullptr, nullptr, B, C, n_x, K, false, &path))
        return rc;
    const int64_t BC = (int64_t)B * C;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0 || B == 0) {
        if (BC > 0) CFC_HIP(hipMemcpyAsync(h_hist, h0, BC * 4, hipMemcpyDeviceToDevice, s), "h0 copy");
        return CFC_OK;
    }
    const KloopArgs k{u, y, h0, W, bias, h_hist, act, ws, nullptr, nullptr, nullptr, nullptr, B, C, n_x, K};
    return enqueue_fwd_bwd(k, uncaptured(path, s), make_plan(B, C, n_x, W, nullptr), s);
}

int cfc_kloop_fwd_bwd_fill(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                           float* h_hist, float* act, float* ws, size_t ws_bytes, float* gW_scratch,
                           float* gb_scratch, int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "cfc_kloop_fwd_bwd_fill";
    Path path = Path::Steps;
    if (int rc = check_kloop(fn, u, y, h0, W, bias, h_hist, act, ws, ws_bytes, gW_scratch, gb_scratch, nullptr,
                             nullptr, B, C, n_x, K, false, &path))
        return rc;
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    if ((BC * 3 * n_in > 0 && !gW_scratch) || (BC > 0 && !gb_scratch)) return fail(CFC_EINVAL, "%s: null pointer", fn);
    hipStream_t s = (hipStream_t)stream;
    if (K == 0 || B == 0) {
        if (BC > 0) CFC_HIP(hipMemcpyAsync(h_hist, h0, BC * 4, hipMemcpyDeviceToDevice, s), "h0 copy");
        CFC_HIP(cfc::launch_fill_zero(gW_scratch, BC * 3 * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb_scratch, 3 * BC, s), "zero fill");
        return CFC_OK;
    }
    const KloopArgs k{u, y, h0, W, bias, h_hist, act, ws, gW_scratch, gb_scratch, nullptr, nullptr, B, C, n_x, K};
    bool filled = false;
    if (int rc = enqueue_fwd_bwd(k, uncaptured(path, s), make_plan(B, C, n_x, W, nullptr), s, &filled)) return rc;
    if (!filled) return enqueue_fill(ws, u, h_hist, gW_scratch, gb_scratch, B, C, n_x, K, s);
    return CFC_OK;
}

// ---------------------------------------------------------------------------
// GEMM-form weight gradient: gW_q = sum over the K*B (t, b) rows of
// dp_t[b, q C + c] z_t[b, k], one matrix-core contraction over the rows
// (input columns from u, recurrent columns from h_hist[0 .. K-1]), cut into
// fixed row splits whose partials are added by the batch-axis reducer.
// ---------------------------------------------------------------------------
namespace {

struct WgPlan {
    int k_split;   // rows per split (multiple of the GEMM chunk)
    int S;         // splits
    int64_t part_floats;
};

// Splits: enough for about 512 workgroups over the output tiles; a function
// of the sizes only.
WgPlan wg_plan(int B, int C, int n_x, int K)
{
    WgPlan p{};
    const int64_t rows = (int64_t)K * B;
    const int tiles = ((3 * C + gemm::kTile - 1) / gemm::kTile) *
                      ((n_x + gemm::kTile - 1) / gemm::kTile + (C + gemm::kTile - 1) / gemm::kTile);
    int64_t S = (512 + tiles - 1) / tiles;
    S = S < 1 ? 1 : (S > 32 ? 32 : S);
    int64_t per = rows > 0 ? (rows + S - 1) / S : 1;
    per = (per + gemm::kBK - 1) / gemm::kBK * gemm::kBK;
    p.k_split = (int)per;
    p.S = rows > 0 ? (int)((rows + per - 1) / per) : 1;
    const int64_t n_in = (int64_t)n_x + C;
    p.part_floats = ((int64_t)p.S * 3 * C * n_in + 3) / 4 * 4 + ((int64_t)p.S * 3 * C + 3) / 4 * 4;
    return p;
}

gemm::Operand wg_operand(const float* p, int64_t ld, int64_t extent)
{
    return gemm::Operand{p, ld, 0, (ld % 4 == 0 && extent % 4 == 0 && extent >= 4 && aligned16(p)) ? 1 : 0};
}

int enqueue_weight_grad_gemm(const float* dp, const float* u, const float* h_hist, float* gW, float* gb, int B,
                             int C, int n_x, int K, float* part, hipStream_t s)
{
    const int64_t n_in = (int64_t)n_x + C, R3 = 3 * (int64_t)C;
    const int64_t rows = (int64_t)K * B;
    const WgPlan p = wg_plan(B, C, n_x, K);
    float* wpart = part;
    float* bpart = part + ((int64_t)p.S * R3 * n_in + 3) / 4 * 4;
    gemm::GemmTask t[2] = {};
    int nt = 0;
    for (int half = 0; half < 2; ++half) {
        const int N = half == 0 ? n_x : C;
        if (N == 0) continue;
        gemm::GemmTask& g = t[nt++];
        g.A = wg_operand(dp, R3, R3);                              // A(m, row) = dp[row, m]
        g.B = half == 0 ? wg_operand(u, n_x, n_x) : wg_operand(h_hist, C, C);   // B(n, row) = z[row, n]
        g.M = (int)R3;
        g.N = N;
        g.K = (int)rows;
        g.k_split = p.k_split;
        g.epi = gemm::kEpiDw;
        g.out = wpart + (half == 0 ? 0 : n_x);
        g.ldo = n_in;
        g.split_stride = R3 * n_in;
        if (nt == 1) {   // the bias gradient once, from the first task's dp tiles
            g.colsum = bpart;
            g.colsum_stride = R3;
        }
    }
    // one launch per group of tasks that take the same loads
    for (int va = 0; va < 2; ++va)
        for (int vb = 0; vb < 2; ++vb) {
            gemm::GemmBatch b{};
            for (int i = 0; i < nt; ++i)
                if (t[i].A.vec == va && t[i].B.vec == vb) b.t[b.ntask++] = t[i];
            if (b.ntask == 0) continue;
            gemm::finish_batch(b);
            CFC_HIP(gemm::launch_gemm(b, s), "weight-gradient GEMM launch");
        }
    cfc::ReduceSeg segs[2] = {{wpart, gW, R3 * n_in, 0}, {bpart, gb, R3, 0}};
    bool vec = true;
    for (const auto& g : segs) vec = vec && g.N % 4 == 0 && aligned16(g.in) && aligned16(g.out);
    const int V = vec ? 4 : 1;
    for (auto& g : segs) g.groups = (g.N + V - 1) / V;
    CFC_HIP(cfc::launch_reduce(segs, 2, p.S, V, s), "weight-gradient reduce launch");
    return CFC_OK;
}

}  // namespace

size_t cfc_weight_grad_gemm_workspace_bytes(int B, int C, int n_x, int K)
{
    if (check_dims(B, C, n_x) || K < 0 || K > (1 << 20)) return 0;
    return sizeof(float) * (size_t)wg_plan(B, C, n_x, K).part_floats;
}

int cfc_weight_grad_gemm(const float* dp, const float* u, const float* h_hist, float* gW, float* gb, int B, int C,
                         int n_x, int K, void* ws, size_t ws_bytes, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "cfc_weight_grad_gemm";
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "%s: K=%d out of range", fn, K);
    const int64_t n_in = (int64_t)n_x + C, R3 = 3 * (int64_t)C, rows = (int64_t)K * B;
    if (rows * R3 > ((int64_t)1 << 31) || rows > ((int64_t)1 << 30))
        return fail(CFC_EINVAL, "%s: K*B=%lld rows too many", fn, (long long)rows);
    if (!gW || !gb) return fail(CFC_EINVAL, "%s: null pointer", fn);
    hipStream_t s = (hipStream_t)stream;
    if (rows == 0) {
        CFC_HIP(cfc::launch_fill_zero(gW, R3 * n_in, s), "zero fill launch");
        CFC_HIP(cfc::launch_fill_zero(gb, R3, s), "zero fill launch");
        return CFC_OK;
    }
    const size_t need = cfc_weight_grad_gemm_workspace_bytes(B, C, n_x, K);
    if (!dp || !h_hist || !ws || (n_x > 0 && !u)) return fail(CFC_EINVAL, "%s: null pointer", fn);
    if (ws_bytes < need) return fail(CFC_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    const Span outs[] = {span(gW, R3 * n_in), span(gb, R3), Span{ws, need}};
    const Span ins[] = {span(dp, rows * R3), span(u, rows * n_x), span(h_hist, rows * C)};
    for (int i = 0; i < 3; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return fail(CFC_EINVAL, "%s: an output overlaps an input", fn);
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "%s: outputs overlap", fn);
    }
    return enqueue_weight_grad_gemm(dp, u, h_hist, gW, gb, B, C, n_x, K, static_cast<float*>(ws), s);
}

size_t cfc_train_kloop_gemm_workspace_bytes(int B, int C, int n_x, int K)
{
    if (check_dims(B, C, n_x) || K < 0 || K > (1 << 20)) return 0;
    return sizeof(float) * (size_t)(kloop_ws_floats(B, C, n_x, K) + wg_plan(B, C, n_x, K).part_floats);
}

int cfc_train_kloop_gemm(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                         float* h_hist, float* act, float* gW, float* gb, void* ws, size_t ws_bytes, int B, int C,
                         int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "cfc_train_kloop_gemm";
    const size_t need = cfc_train_kloop_gemm_workspace_bytes(B, C, n_x, K);
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "%s: K=%d out of range", fn, K);
    if (ws_bytes < need) return fail(CFC_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    const int64_t n_in = (int64_t)n_x + C, R3 = 3 * (int64_t)C, rows = (int64_t)K * B;
    if (rows * R3 > ((int64_t)1 << 31) || rows > ((int64_t)1 << 30))
        return fail(CFC_EINVAL, "%s: K*B=%lld rows too many", fn, (long long)rows);
    if (!gW || !gb) return fail(CFC_EINVAL, "%s: null pointer", fn);
    const Span extra[] = {span(gW, R3 * n_in), span(gb, R3)};
    const Span others[] = {span(u, rows * n_x), span(y, rows * C), span(h0, (int64_t)B * C), span(W, R3 * n_in),
                           span(bias, R3), span(h_hist, (K + 1) * (int64_t)B * C), span(act, rows * R3),
                           Span{ws, need}};
    for (int i = 0; i < 2; ++i) {
        for (const Span& o : others)
            if (overlap(extra[i], o)) return fail(CFC_EINVAL, "%s: gW or gb overlaps another array", fn);
    }
    if (overlap(extra[0], extra[1])) return fail(CFC_EINVAL, "%s: outputs overlap", fn);
    const size_t kws = (size_t)kloop_ws_floats(B, C, n_x, K) * sizeof(float);
    float* wsf = static_cast<float*>(ws);
    if (int rc = cfc_kloop_fwd_bwd(u, y, h0, W, bias, h_hist, act, wsf, kws, B, C, n_x, K, stream)) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (rows == 0) {
        CFC_HIP(cfc::launch_fill_zero(gW, R3 * n_in, s), "zero fill launch");
        CFC_HIP(cfc::launch_fill_zero(gb, R3, s), "zero fill launch");
        return CFC_OK;
    }
    return enqueue_weight_grad_gemm(wsf, u, h_hist, gW, gb, B, C, n_x, K, wsf + kloop_ws_floats(B, C, n_x, K), s);
}

int cfc_adamw_step(float* const* params, const float* const* grads, float* const* m, float* const* v,
                   const int64_t* n, int nseg, float lr, float beta1, float beta2, float eps, float weight_decay,
                   int step, void* stream)
{
    cfc_host::last_error().clear();
    if (nseg < 0 || nseg > cfc::kMaxAdamwSegs)
        return fail(CFC_EINVAL, "cfc_adamw_step: nseg=%d out of range [0, %d]", nseg, cfc::kMaxAdamwSegs);
    if (step < 1) return fail(CFC_EINVAL, "cfc_adamw_step: step=%d (the first step is 1)", step);
    if (!(lr >= 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
        !(weight_decay >= 0.0f))
        return fail(CFC_EINVAL, "cfc_adamw_step: hyperparameters out of range");
    if (nseg > 0 && (!params || !grads || !m || !v || !n)) return fail(CFC_EINVAL, "cfc_adamw_step: null array");
    cfc::AdamwArgs a{};
    a.nseg = nseg;
    a.qstart[0] = 0;
    for (int i = 0; i < nseg; ++i) {
        if (n[i] < 0 || n[i] > ((int64_t)1 << 40)) return fail(CFC_EINVAL, "cfc_adamw_step: n[%d] out of range", i);
        if (n[i] > 0 && (!params[i] || !grads[i] || !m[i] || !v[i]))
            return fail(CFC_EINVAL, "cfc_adamw_step: null pointer in segment %d", i);
        const int vec = (aligned16(params[i]) && aligned16(grads[i]) && aligned16(m[i]) && aligned16(v[i])) ? 1 : 0;
        a.seg[i] = cfc::AdamwSeg{params[i], grads[i], m[i], v[i], n[i], vec};
        a.qstart[i + 1] = a.qstart[i] + (n[i] + 3) / 4;
    }
    // every array of every segment must be disjoint from every other one
    for (int i = 0; i < nseg; ++i) {
        const Span si[] = {span(params[i], n[i]), span(grads[i], n[i]), span(m[i], n[i]), span(v[i], n[i])};
        for (int j = i; j < nseg; ++j) {
            const Span sj[] = {span(params[j], n[j]), span(grads[j], n[j]), span(m[j], n[j]), span(v[j], n[j])};
            for (int x = 0; x < 4; ++x)
                for (int y = (i == j ? x + 1 : 0); y < 4; ++y)
                    if (overlap(si[x], sj[y])) return fail(CFC_EINVAL, "cfc_adamw_step: arrays overlap");
        }
    }
    a.decay = 1.0f - lr * weight_decay;
    a.beta1 = beta1;
    a.one_minus_beta1 = 1.0f - beta1;
    a.beta2 = beta2;
    a.one_minus_beta2 = 1.0f - beta2;
    const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
    const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
    a.step_size = (float)((double)lr / bc1);
    a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    a.eps = eps;
    CFC_HIP(cfc::launch_adamw(a, (hipStream_t)stream), "adamw launch");
    return CFC_OK;
}

int cfc_input_projection(const float* u, const float* W, const float* bias, float* X, int64_t M, int C, int n_x,
                         void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_dims(0, C, n_x)) return rc;
    if (M < 0 || M > ((int64_t)1 << 40)) return fail(CFC_EINVAL, "cfc_input_projection: M=%lld out of range",
                                                     (long long)M);
    if (M == 0) return CFC_OK;
    const int64_t n_in = (int64_t)n_x + C;
    if (!W || !bias || !X || (n_x > 0 && !u)) return fail(CFC_EINVAL, "cfc_input_projection: null pointer");
    const Span out = span(X, M * 3 * C);
    const Span ins[] = {span(u, M * n_x), span(W, 3 * C * n_in), span(bias, 3 * C)};
    for (const Span& i : ins)
        if (overlap(out, i)) return fail(CFC_EINVAL, "cfc_input_projection: the output overlaps an input");
    const cfc::XprojArgs x{u, W, bias, X, M, 3 * C, n_x, (int)n_in, (3 * C + 63) / 64};
    CFC_HIP(cfc::launch_xproj(x, (hipStream_t)stream), "input projection launch");
    return CFC_OK;
}

int cfc_kloop_recurrence(const float* X, const float* y, const float* h0, const float* W, float* h_hist,
                         float* act, float* dp, int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "cfc_kloop_recurrence: K=%d out of range", K);
    if (cfc::persist_smem(C) == 0)
        return fail(CFC_EINVAL, "cfc_kloop_recurrence: the persistent kernel holds C <= 128 channels (C=%d)", C);
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    const struct {
        const void* p;
        int64_t n;
    } need[] = {{X, (int64_t)K * 3 * BC}, {y, (int64_t)K * BC}, {h0, BC}, {W, 3 * C * n_in},
                {h_hist, (K + 1) * BC}, {act, (int64_t)K * 3 * BC}, {dp, (int64_t)K * 3 * BC}};
    for (const auto& q : need)
        if (q.n > 0 && q.p == nullptr) return fail(CFC_EINVAL, "cfc_kloop_recurrence: null pointer");
    const Span outs[] = {span(h_hist, (K + 1) * BC), span(act, (int64_t)K * 3 * BC), span(dp, (int64_t)K * 3 * BC)};
    const Span ins[] = {span(X, (int64_t)K * 3 * BC), span(y, (int64_t)K * BC), span(h0, BC), span(W, 3 * C * n_in)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return fail(CFC_EINVAL, "cfc_kloop_recurrence: an output overlaps an input");
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(CFC_EINVAL, "cfc_kloop_recurrence: outputs overlap");
    hipStream_t s = (hipStream_t)stream;
    if (K == 0 || B == 0) {
        if (BC > 0) CFC_HIP(hipMemcpyAsync(h_hist, h0, BC * 4, hipMemcpyDeviceToDevice, s), "h0 copy");
        return CFC_OK;
    }
    const cfc::PersistArgs a{X, y, h0, W, nullptr, h_hist, act, dp, B, C, n_x, K};
    CFC_HIP(cfc::launch_persist(a, s), "persistent K-loop launch");
    return CFC_OK;
}

int cfc_scratch_fill(const float* dp, const float* u, const float* h_hist, float* gW_scratch, float* gb_scratch,
                     int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "cfc_scratch_fill: K=%d out of range", K);
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    const struct {
        const void* p;
        int64_t n;
    } need[] = {{dp, (int64_t)K * 3 * BC}, {u, (int64_t)K * B * n_x}, {h_hist, (int64_t)K * BC},
                {gW_scratch, BC * 3 * n_in}, {gb_scratch, 3 * BC}};
    for (const auto& q : need)
        if (q.n > 0 && q.p == nullptr) return fail(CFC_EINVAL, "cfc_scratch_fill: null pointer");
    const Span outs[] = {span(gW_scratch, BC * 3 * n_in), span(gb_scratch, 3 * BC)};
    const Span ins[] = {span(dp, (int64_t)K * 3 * BC), span(u, (int64_t)K * B * n_x), span(h_hist, (int64_t)K * BC)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return fail(CFC_EINVAL, "cfc_scratch_fill: an output overlaps an input");
    if (overlap(outs[0], outs[1])) return fail(CFC_EINVAL, "cfc_scratch_fill: outputs overlap");
    if (B == 0) return CFC_OK;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) {
        CFC_HIP(cfc::launch_fill_zero(gW_scratch, BC * 3 * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb_scratch, 3 * BC, s), "zero fill");
        return CFC_OK;
    }
    return enqueue_fill(dp, u, h_hist, gW_scratch, gb_scratch, B, C, n_x, K, s);
}

// ---------------------------------------------------------------------------
// The K-loop step without a caller workspace, for callers that cannot
// allocate device memory: its workspace is a fixed array of the library on
// each device, and every launch is enqueued directly (no graph, whose
// instantiation would allocate).
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// The workspace of cfc_train_kloop_noalloc: one copy per device, held until
// the process ends.  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) float scratch[CFC_NOALLOC_MAX_WS_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device dev (the current device),
// looked up on the first call on that device.
int scratch_on_device(int dev, float** out)
{
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        CFC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "workspace symbol address");
        if (p == nullptr) return cfc_host::fail(CFC_EHIP, "workspace symbol address: null");
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return CFC_OK;
}

}  // namespace

extern "C" {

int cfc_train_kloop_noalloc(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                            float* h_hist, float* act, float* gW_scratch, float* gb_scratch, float* gW, float* gb,
                            int B, int C, int n_x, int K, void* stream)
{
    cfc_host::last_error().clear();
    const char* fn = "cfc_train_kloop_noalloc";
    if (int rc = check_dims(B, C, n_x)) return rc;
    if (K < 0 || K > (1 << 20)) return fail(CFC_EINVAL, "%s: K=%d out of range", fn, K);
    const size_t need = (size_t)kloop_ws_floats(B, C, n_x, K) * sizeof(float);
    if (need > (size_t)CFC_NOALLOC_MAX_WS_BYTES)
        return fail(CFC_EINVAL, "%s: these sizes need %zu bytes of workspace; the fixed workspace holds %zu",
                    fn, need, (size_t)CFC_NOALLOC_MAX_WS_BYTES);
    int dev = 0;
    CFC_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CFC_EINVAL, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    float* ws = nullptr;
    if (int rc = scratch_on_device(dev, &ws)) return rc;
    Path path = Path::Steps;
    if (int rc = check_kloop(fn, u, y, h0, W, bias, h_hist, act, ws, need, gW_scratch, gb_scratch, gW, gb, B, C,
                             n_x, K, true, &path))
        return rc;
    const int64_t n_in = (int64_t)n_x + C, BC = (int64_t)B * C;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0 || B == 0) {
        if (BC > 0) CFC_HIP(hipMemcpyAsync(h_hist, h0, BC * 4, hipMemcpyDeviceToDevice, s), "h0 copy");
        CFC_HIP(cfc::launch_fill_zero(gW_scratch, BC * 3 * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb_scratch, 3 * BC, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gW, 3 * C * n_in, s), "zero fill");
        CFC_HIP(cfc::launch_fill_zero(gb, 3 * C, s), "zero fill");
        return CFC_OK;
    }
    // every part of the workspace is written before it is read within the
    // call (dp, X, the carry, the re-laid W, the resident kernel's counters,
    // which it zeroes first), so nothing needs clearing
    const KloopArgs k{u, y, h0, W, bias, h_hist, act, ws, gW_scratch, gb_scratch, gW, gb, B, C, n_x, K};
    return enqueue_kloop(k, uncaptured(path, s), make_plan(B, C, n_x, W, gW_scratch), s);
}

int cfc_clear_graph_cache(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto& kv : g_graphs) destroy_entry(kv.second);
    g_graphs.clear();
    for (auto& e : g_retired) destroy_entry(e);
    g_retired.clear();
    return CFC_OK;
}

}  // extern "C"
