// C-ABI runtime of convtile: argument checking, the tile-config space and its
// legality check, the built-in default config, the tuning search, the
// per-shape cache (append-only JSON lines), split-reduction workspaces and
// dispatch to the HIP kernels.
//
// The search space and its bookkeeping follow the TVM tutorial "Tuning High
// Performance Convolution on NVIDIA GPUs" (Step 1: define_split with all
// ordered factorizations, define_knob option lists; Step 2: LocalRunner with
// repeat=3, min_repeat_ms=100, timeout=4 and a log file of measure records;
// the final part: apply_history_best / query of the best record per
// workload).  Measurement outcome codes keep the meanings printed in the
// tuning log of the gist that reproduces it (0 ok, 1 rejected as an invalid
// kernel before running, 4 runtime error, 6 timeout).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <functional>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <thread>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/convtile.h"
#include "ct_kernels.hpp"
#include "igemm_common.hpp"

namespace ct {

// Half-precision convolution variants with staging waves (igemm_f16v2.hip):
// the descriptors, and per variant the waves it runs beside its
// waves_m x waves_n matrix waves.
const IgemmVariant* igemm_f16v2x_variants(int* count, const int** extra_waves);

namespace {

constexpr int kMaxLds = 163840;       // bytes of LDS per workgroup on gfx950
constexpr int kMaxThreads = 1024;     // workgroup size limit
constexpr int kNumCU = 256;           // compute units of an MI355X
constexpr long long kMaxWorkspace = 1LL << 30;  // split partials, bytes
constexpr const char* kArch = "gfx950";
constexpr int kSpaceVersion = 1;

// ---------------------------------------------------------------- errors --
thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(CT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool log_debug() {
    static int v = -1;
    if (v < 0) {
        const char* s = getenv("CT_LOG");
        v = (s && strcmp(s, "debug") == 0) ? 1 : 0;
    }
    return v == 1;
}

// ---------------------------------------------------------------- shapes --
struct Shape {
    int N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue;
    int OH, OW;
    long long P;
    int T, K;

    std::string key() const {
        char buf[256];
        snprintf(buf, sizeof(buf), "%d,%d,%d,%d,%d,%d,%d,%d,%d,%d,%d,%s,v%d", N, CI, H, W, CO, KH,
                 KW, stride, pad, dtype, epilogue, kArch, kSpaceVersion);
        return buf;
    }
};

int make_shape(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
               int dtype, int epilogue, Shape* s) {
    if (N <= 0 || CI <= 0 || H <= 0 || W <= 0 || CO <= 0 || KH <= 0 || KW <= 0)
        return fail(CT_ERR_INVALID_ARG, "every dimension must be positive");
    if (stride <= 0) return fail(CT_ERR_INVALID_ARG, "stride must be positive");
    if (pad < 0) return fail(CT_ERR_INVALID_ARG, "pad must be non-negative");
    if (dtype != CT_F32 && dtype != CT_F16 && dtype != CT_BF16)
        return fail(CT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (epilogue != CT_EPI_NONE && epilogue != CT_EPI_BIAS && epilogue != CT_EPI_EXP_BIAS_RSQRT)
        return fail(CT_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
    const long long Hp = (long long)H + 2LL * pad, Wp = (long long)W + 2LL * pad;
    if (Hp < KH || Wp < KW) return fail(CT_ERR_INVALID_ARG, "kernel larger than padded input");
    if (Hp > (1 << 24) || Wp > (1 << 24)) return fail(CT_ERR_INVALID_ARG, "input too large");
    s->N = N; s->CI = CI; s->H = H; s->W = W; s->CO = CO; s->KH = KH; s->KW = KW;
    s->stride = stride; s->pad = pad; s->dtype = dtype; s->epilogue = epilogue;
    s->OH = (int)((Hp - KH) / stride + 1);
    s->OW = (int)((Wp - KW) / stride + 1);
    if (s->OH <= 0 || s->OW <= 0) return fail(CT_ERR_INVALID_ARG, "empty output");
    const long long T = (long long)KH * KW;
    const long long K = (long long)CI * T;
    if (K > (1LL << 30)) return fail(CT_ERR_INVALID_ARG, "reduction too long");
    s->T = (int)T;
    s->K = (int)K;
    s->P = (long long)N * s->OH * s->OW;
    if ((long long)s->OH * s->OW > (1LL << 30)) return fail(CT_ERR_INVALID_ARG, "output too large");
    if (s->P * CO > (1LL << 40)) return fail(CT_ERR_INVALID_ARG, "output too large");
    return CT_OK;
}

int check_pointers(const void* x, const void* w, const float* y, int epilogue, const float* bias,
                   const float* var) {
    if (!x || !w || !y) return fail(CT_ERR_INVALID_ARG, "x, w and y must not be NULL");
    if (epilogue != CT_EPI_NONE && !bias)
        return fail(CT_ERR_INVALID_ARG, "the epilogue reads bias, which is NULL");
    if (epilogue == CT_EPI_EXP_BIAS_RSQRT && !var)
        return fail(CT_ERR_INVALID_ARG, "the epilogue reads var, which is NULL");
    return CT_OK;
}

// -------------------------------------------------------------- variants --
struct Variant {
    ct_variant_desc desc;
    const IgemmVariant* ig;  // nullptr for the direct kernel
};

const std::vector<Variant>& variants() {
    static std::vector<Variant> v = [] {
        std::vector<Variant> out;
        const char* dnames[3] = {"direct_f32", "direct_f16", "direct_bf16"};
        for (int dt = 0; dt < 3; ++dt) {
            Variant d{};
            snprintf(d.desc.name, sizeof(d.desc.name), "%s", dnames[dt]);
            d.desc.dtype = dt;
            d.desc.kind = 0;
            d.desc.threads = 256;
            d.ig = nullptr;
            out.push_back(d);
        }
        int n32 = 0, n16 = 0, nsk = 0, nsk16 = 0, nh2 = 0, nskc = 0, nskt = 0, ngm = 0, nhgm = 0, nh2x = 0;
        const IgemmVariant* t32 = igemm_f32_variants(&n32);
        const IgemmVariant* tsk = igemm_f32_sk_variants(&nsk);
        const IgemmVariant* tsk16 = igemm_f32_sk16_variants(&nsk16);
        const IgemmVariant* tskc = igemm_f32_skc_variants(&nskc);
        const IgemmVariant* tskt = igemm_f32_skt_variants(&nskt);
        const IgemmVariant* t16 = igemm_f16_variants(&n16);
        const IgemmVariant* th2 = igemm_f16v2_variants(&nh2);
        const IgemmVariant* tgm = igemm_f32_gemm_variants(&ngm);
        const IgemmVariant* thgm = igemm_f16_gemm_variants(&nhgm);
        const int* h2x_waves = nullptr;
        const IgemmVariant* th2x = igemm_f16v2x_variants(&nh2x, &h2x_waves);
        auto add = [&](const IgemmVariant* t, int n, const int* extra_waves = nullptr) {
            for (int i = 0; i < n; ++i) {
                Variant v{};
                snprintf(v.desc.name, sizeof(v.desc.name), "%s", t[i].name);
                v.desc.dtype = t[i].dtype;
                v.desc.kind = 1;
                v.desc.mfma_m = t[i].mfma_m;
                v.desc.mfma_n = t[i].mfma_n;
                v.desc.mfma_k = t[i].mfma_k;
                v.desc.waves_m = t[i].waves_m;
                v.desc.waves_n = t[i].waves_n;
                v.desc.waves_k = t[i].waves_k;
                v.desc.reps_m = t[i].reps_m;
                v.desc.reps_n = t[i].reps_n;
                v.desc.tile_m = t[i].waves_m * t[i].reps_m * t[i].mfma_m;
                v.desc.tile_n = t[i].tile_n ? t[i].tile_n : t[i].waves_n * t[i].reps_n * t[i].mfma_n;
                v.desc.kc_max = t[i].kc_max;
                v.desc.threads = (t[i].waves_m * t[i].waves_n * t[i].waves_k + (extra_waves ? extra_waves[i] : 0)) * 64;
                v.ig = &t[i];
                out.push_back(v);
            }
        };
        add(t32, n32);
        add(tsk, nsk);
        add(tsk16, nsk16);
        add(tskc, nskc);
        add(tskt, nskt);
        add(t16, n16);
        add(th2, nh2);
        add(tgm, ngm);  // last: the flat indices of the earlier points stay as they were
        add(thgm, nhgm);
        add(th2x, nh2x, h2x_waves);
        return out;
    }();
    return v;
}

int find_variant(const char* name) {
    const auto& vs = variants();
    for (size_t i = 0; i < vs.size(); ++i)
        if (strcmp(vs[i].desc.name, name) == 0) return (int)i;
    return -1;
}

// Tiled variants that accept a dtype, in registry order: the option list of
// the "variant" knob.
std::vector<int> tiled_variants_for(int dtype) {
    std::vector<int> ids;
    const auto& vs = variants();
    for (size_t i = 0; i < vs.size(); ++i)
        if (vs[i].ig && vs[i].desc.dtype == dtype) ids.push_back((int)i);
    return ids;
}

// --------------------------------------------------------------- splits ---
// All ordered k-factorizations of n, ascending by (x_k, ..., x_2) with
// x_1 = n / (x_2 ... x_k): the order of the "policy=all" split in the
// tutorial's ConfigSpace (the flat indices printed in the tuning log follow
// it).
void gen_splits(long long n, int k, const std::vector<long long>& divs, int depth,
                std::vector<long long>& tail_rev, std::vector<std::vector<long long>>& out) {
    // tail_rev holds x_k, x_{k-1}, ... (outermost loop = x_k)
    if (depth == k - 1) {
        long long prod = 1;
        for (long long f : tail_rev) prod *= f;
        if (n % prod) return;
        std::vector<long long> e(k);
        e[0] = n / prod;
        for (int i = 0; i < k - 1; ++i) e[k - 1 - i] = tail_rev[i];
        out.push_back(e);
        return;
    }
    long long prod = 1;
    for (long long f : tail_rev) prod *= f;
    for (long long d : divs) {
        if ((n / prod) % d) continue;  // prefix must still divide n
        tail_rev.push_back(d);
        gen_splits(n, k, divs, depth + 1, tail_rev, out);
        tail_rev.pop_back();
    }
}

const std::vector<std::vector<long long>>& splits(long long n, int k) {
    static std::mutex mu;
    static std::map<std::pair<long long, int>, std::vector<std::vector<long long>>> memo;
    std::lock_guard<std::mutex> lk(mu);
    auto it = memo.find({n, k});
    if (it != memo.end()) return it->second;
    std::vector<long long> divs;
    for (long long d = 1; d * d <= n; ++d)
        if (n % d == 0) {
            divs.push_back(d);
            if (d != n / d) divs.push_back(n / d);
        }
    std::sort(divs.begin(), divs.end());
    std::vector<std::vector<long long>> out;
    std::vector<long long> tail;
    if (k == 1)
        out.push_back({n});
    else
        gen_splits(n, k, divs, 0, tail, out);
    return memo.emplace(std::make_pair(n, k), std::move(out)).first->second;
}

// ---------------------------------------------------------------- space ---
// knobs: tile_ci = split(CI, 3) -> [split_k, stages, kc]; variant = option.
struct Space {
    const std::vector<std::vector<long long>>* ci;
    std::vector<int> var_ids;
    long long size() const { return (long long)ci->size() * (long long)var_ids.size(); }
};

Space space_of(const Shape& s) {
    Space sp;
    sp.ci = &splits(s.CI, 3);
    sp.var_ids = tiled_variants_for(s.dtype);
    return sp;
}

bool decode(const Space& sp, long long index, ct_tile_config* cfg) {
    if (index < 0 || index >= sp.size()) return false;
    const long long nci = (long long)sp.ci->size();
    const auto& e = (*sp.ci)[index % nci];
    cfg->split_k = (int)e[0];
    cfg->stages = (int)e[1];
    cfg->kc = (int)e[2];
    cfg->variant = sp.var_ids[index / nci];
    cfg->index = index;
    cfg->us = 0.0f;
    cfg->error_no = 0;
    return true;
}

long long encode(const Space& sp, const ct_tile_config& c) {
    const long long nci = (long long)sp.ci->size();
    long long ici = -1, iv = -1;
    for (long long i = 0; i < nci; ++i) {
        const auto& e = (*sp.ci)[i];
        if (e[0] == c.split_k && e[1] == c.stages && e[2] == c.kc) {
            ici = i;
            break;
        }
    }
    for (size_t i = 0; i < sp.var_ids.size(); ++i)
        if (sp.var_ids[i] == c.variant) iv = (long long)i;
    if (ici < 0 || iv < 0) return -1;
    return ici + nci * iv;
}

// Largest padded-input window (rows) any column tile of width tile_n needs.
int window_rows(const Shape& s, int tile_n) {
    static std::mutex mu;
    static std::map<std::pair<std::string, int>, int> memo;
    const std::string k = s.key();
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = memo.find({k, tile_n});
        if (it != memo.end()) return it->second;
    }
    const int Hp = s.H + 2 * s.pad;
    const int OHW = s.OH * s.OW;
    long long best = 0;
    for (long long p0 = 0; p0 < s.P; p0 += tile_n) {
        const long long p1 = std::min(s.P, p0 + tile_n);
        best = std::max(best, window_rows_for(p0, p1, OHW, s.OW, Hp, s.stride, s.KH));
    }
    const int r = (int)std::min<long long>(best, 1 << 30);
    std::lock_guard<std::mutex> lk(mu);
    memo[{k, tile_n}] = r;
    return r;
}

struct Resolved {
    const Variant* v;
    int tiles_m, tiles_n, R, lds;
    long long grid, ws_bytes, aux_bytes;
};

// ------------------------------------------------------- device set-up --
// Once per device: the address of the zero page (a device global, so no
// allocation) and the workgroup-placement probe that gates the XCD-local
// variants.  The probe launches and synchronises on a private stream, so it
// cannot run inside stream capture: ct_init(device) does it up front, and a
// first launch on a device that finds its stream capturing is refused.

// 256 zero bytes: the source address of every padded tap in the direct-to-LDS
// loads (never written).
static __device__ __align__(256) float g_zero_page[64];
// The probe's output: the XCD of each of its workgroups.
constexpr int kProbeBlocks = 4096;
static __device__ int g_probe_out[kProbeBlocks];

struct DeviceState {
    bool ready = false;
    bool xcd_rr = false;          // workgroup b runs on XCD b % 8
    const void* zero = nullptr;   // device address of g_zero_page
};

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceState g_dev[kMaxDevices];
std::atomic<bool> g_dev_ready[kMaxDevices];

int noalloc_setup(int dev, hipStream_t setup_stream);  // the no-allocation entry point's scratch

// Set up device `dev` (current).  Not under capture: the caller checks.
int device_setup_locked(int dev) {
    DeviceState& d = g_dev[dev];
    if (d.ready) return CT_OK;
    void* z = nullptr;
    hipError_t e = hipGetSymbolAddress(&z, HIP_SYMBOL(g_zero_page));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(zero page)");
    int* probe = nullptr;
    e = hipGetSymbolAddress((void**)&probe, HIP_SYMBOL(g_probe_out));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(probe buffer)");
    hipStream_t ps = nullptr;
    e = hipStreamCreateWithFlags(&ps, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
    const int st = noalloc_setup(dev, ps);
    if (st != CT_OK) {
        (void)hipStreamDestroy(ps);
        return st;
    }
    std::vector<int> h(kProbeBlocks, -1);
    bool rr = false;
    if (launch_xcc_probe(probe, kProbeBlocks, ps) == hipSuccess &&
        hipMemcpyAsync(h.data(), probe, kProbeBlocks * sizeof(int), hipMemcpyDeviceToHost, ps) == hipSuccess &&
        hipStreamSynchronize(ps) == hipSuccess) {
        rr = true;
        for (int b = 0; b < kProbeBlocks; ++b) rr = rr && h[b] == b % 8;
    }
    (void)hipStreamDestroy(ps);
    (void)hipGetLastError();
    d.zero = z;
    d.xcd_rr = rr;
    d.ready = true;
    g_dev_ready[dev].store(true, std::memory_order_release);
    return CT_OK;
}

// Set up the current device if that has not happened yet.  `stream` is the
// stream of the launch that needs it: if it is capturing, set-up cannot run
// and the launch is refused.
int ensure_device(hipStream_t stream, int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CT_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    *dev_out = dev;
    if (g_dev_ready[dev].load(std::memory_order_acquire)) return CT_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(CT_ERR_UNSUPPORTED,
                    "first launch on device %d during stream capture: call ct_init(%d) (or launch once "
                    "eagerly) before capturing",
                    dev, dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    return device_setup_locked(dev);
}

// Whether workgroup b of a launch runs on XCD b % 8 on the current device
// (false if the probe failed).  On a host with no device nothing can launch,
// and the tuning log's XCD-local records are taken as they were measured;
// any launch happens on a device, where the probe decides.
bool xcd_round_robin() {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        (void)hipGetLastError();
        return true;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return false;
    }
    if (!g_dev_ready[dev].load(std::memory_order_acquire)) {
        // host-side calls (space, query, tune) set the device up on demand
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (device_setup_locked(dev) != CT_OK) return false;
    }
    return g_dev[dev].xcd_rr;
}

// Legality of a tile config for a shape; launches nothing except, once per
// device, the workgroup-placement probe of XCD-local variants.
bool legal(const Shape& s, const ct_tile_config& c, Resolved* out, std::string* why) {
    const auto& vs = variants();
    auto no = [&](const char* m) {
        if (why) *why = m;
        return false;
    };
    if (c.variant < 0 || c.variant >= (int)vs.size()) return no("unknown variant");
    const Variant& v = vs[c.variant];
    if (!v.ig) return no("not a tiled variant");
    if (v.desc.dtype != s.dtype) return no("variant dtype differs");
    if (c.kc < 1 || c.stages < 1 || c.split_k < 1) return no("non-positive split factor");
    if (c.kc > v.desc.kc_max) return no("kc above the variant's limit");
    // every split must own at least one channel
    const long long per_split = (long long)c.stages * c.kc;
    if ((long long)(c.split_k - 1) * per_split >= s.CI) return no("an empty split");
    if ((long long)c.split_k * per_split < s.CI) return no("splits do not cover CI");
    if (v.desc.threads > kMaxThreads) return no("workgroup too large");
    // virtual padded rows are addressed with 32-bit arithmetic
    if ((long long)s.N * (s.H + 2LL * s.pad) >= (1LL << 31)) return no("too many padded rows");
    const int R = window_rows(s, v.desc.tile_n);
    const long long Wp = (long long)s.W + 2 * s.pad;
    if ((long long)c.kc * R * Wp > (1LL << 28)) return no("window too large");
    ConvParams lp{};
    lp.N = s.N; lp.CI = s.CI; lp.H = s.H; lp.W = s.W; lp.CO = s.CO; lp.KH = s.KH; lp.KW = s.KW;
    lp.stride = s.stride; lp.pad = s.pad; lp.OH = s.OH; lp.OW = s.OW; lp.T = s.T; lp.K = s.K;
    lp.P = s.P; lp.OHW = s.OH * s.OW; lp.Hp = s.H + 2 * s.pad; lp.Wp = (int)Wp;
    lp.kc = c.kc; lp.stages = c.stages; lp.S = c.split_k; lp.R = R;
    const int lds = v.ig->lds_bytes(lp);
    // 64 bytes left for the kernels' static LDS
    if (lds + 64 > kMaxLds || lds <= 0) return no("LDS above 160 KiB");
    const long long tiles_m = (s.CO + v.desc.tile_m - 1) / v.desc.tile_m;
    const long long tiles_n = (s.P + v.desc.tile_n - 1) / v.desc.tile_n;
    const long long grid = tiles_m * tiles_n * c.split_k;
    if (tiles_m * tiles_n > (1LL << 30) || grid > 0x7fffffffLL) return no("grid too large");
    // partial tiles: tile_m rows of tile_n floats, rows padded to 16 bytes
    const long long ws = c.split_k > 1 ? grid * v.desc.tile_m * round_up(v.desc.tile_n, 4) * 4LL : 0;
    if (ws > kMaxWorkspace) return no("split workspace too large");
    const long long aux = v.ig->aux_bytes ? v.ig->aux_bytes(lp) : 0;
    if (aux > kMaxWorkspace) return no("reordered filter too large");
    if (v.ig->xcd_local && !xcd_round_robin())
        return no("workgroups are not placed round-robin over 8 XCDs on this device");
    if (out) {
        out->v = &v;
        out->tiles_m = (int)tiles_m;
        out->tiles_n = (int)tiles_n;
        out->R = R;
        out->lds = lds;
        out->grid = grid;
        out->ws_bytes = ws;
        out->aux_bytes = aux;
    }
    return true;
}

// Rough time model used to pick the default config and to order the search.
double predict_us(const Shape& s, const ct_tile_config& c, const Resolved& r) {
    const auto& d = r.v->desc;
    const double clk = 2.4e9;
    const int kpi = d.mfma_k;
    const int ksp = round_up(c.kc * s.T, kpi);
    const double wg_flops = 2.0 * d.tile_m * d.tile_n * (double)ksp * c.stages;
    int occ = std::max(1, std::min(kMaxLds / std::max(r.lds, 1), 2048 / d.threads));
    occ = std::min(occ, 4);
    const double slots = (double)kNumCU * occ;
    const double rounds = std::ceil((double)r.grid / slots);
    // waves per SIMD decide how well MFMA latency is hidden
    const double waves_per_simd = (double)d.threads / 64.0 * occ / 4.0;
    const double eff = std::min(1.0, 0.35 + 0.25 * waves_per_simd) * (s.dtype == CT_F32 ? 1.0 : 0.7);
    const double flop_per_clk_cu = s.dtype == CT_F32 ? 256.0 : 4096.0;
    const double t_mma = rounds * occ * wg_flops / (flop_per_clk_cu * eff * clk);
    const double elem = s.dtype == CT_F32 ? 4.0 : 2.0;
    const double stage_bytes = (d.tile_m * (double)c.kc * s.T + (double)c.kc * r.R * (s.W + 2 * s.pad)) * elem;
    const double t_load = rounds * occ * c.stages * (stage_bytes / (64.0 * clk) + 1.0e-6);
    const double t_fix = c.split_k > 1 ? (1.5e-6 + c.split_k * d.tile_m * (double)d.tile_n * 4.0 / 100e9) : 0.0;
    const double t_out = (double)s.P * s.CO * 4.0 / 5e12;
    return 1e6 * (t_mma + t_load + t_fix + t_out) + 2.0;
}

// --------------------------------------------------------------- cache ----
struct CacheEntry {
    std::string variant_name;
    ct_tile_config cfg;
    std::string line;  // JSON record as written / read
};

std::mutex g_cache_mu;
std::map<std::string, CacheEntry> g_cache;
std::map<std::string, ct_tile_config> g_default_memo;
// bumped by every change to g_cache (the launch plans built on it go stale)
std::atomic<unsigned> g_cache_gen{1};

std::string json_record(const Shape& s, const ct_tile_config& c, const char* vname,
                        const float* costs, int ncost, double all_cost, double ts) {
    std::ostringstream o;
    o << "{\"key\":\"" << s.key() << "\",\"N\":" << s.N << ",\"CI\":" << s.CI << ",\"H\":" << s.H
      << ",\"W\":" << s.W << ",\"CO\":" << s.CO << ",\"KH\":" << s.KH << ",\"KW\":" << s.KW
      << ",\"stride\":" << s.stride << ",\"pad\":" << s.pad << ",\"dtype\":" << s.dtype
      << ",\"epilogue\":" << s.epilogue << ",\"arch\":\"" << kArch << "\",\"variant\":\"" << vname
      << "\",\"split_k\":" << c.split_k << ",\"stages\":" << c.stages << ",\"kc\":" << c.kc
      << ",\"index\":" << c.index << ",\"us\":" << c.us << ",\"error_no\":" << c.error_no
      << ",\"costs_us\":[";
    for (int i = 0; i < ncost; ++i) o << (i ? "," : "") << costs[i];
    o << "],\"all_cost\":" << all_cost << ",\"timestamp\":" << std::fixed << ts << "}";
    return o.str();
}

// Minimal reader for the flat records written above: "name": value pairs
// where a value is a string, a number or a list of numbers.
bool parse_record(const std::string& line, std::map<std::string, std::string>* kv) {
    size_t i = 0;
    auto ws = [&] {
        while (i < line.size() && isspace((unsigned char)line[i])) ++i;
    };
    ws();
    if (i >= line.size() || line[i] != '{') return false;
    ++i;
    while (true) {
        ws();
        if (i < line.size() && line[i] == '}') return true;
        if (i >= line.size() || line[i] != '"') return false;
        size_t e = line.find('"', i + 1);
        if (e == std::string::npos) return false;
        std::string name = line.substr(i + 1, e - i - 1);
        i = e + 1;
        ws();
        if (i >= line.size() || line[i] != ':') return false;
        ++i;
        ws();
        if (i >= line.size()) return false;
        std::string val;
        if (line[i] == '"') {
            size_t q = line.find('"', i + 1);
            if (q == std::string::npos) return false;
            val = line.substr(i + 1, q - i - 1);
            i = q + 1;
        } else if (line[i] == '[') {
            size_t q = line.find(']', i);
            if (q == std::string::npos) return false;
            val = line.substr(i, q - i + 1);
            i = q + 1;
        } else {
            size_t q = i;
            while (q < line.size() && line[q] != ',' && line[q] != '}') ++q;
            val = line.substr(i, q - i);
            while (!val.empty() && isspace((unsigned char)val.back())) val.pop_back();
            if (val.empty()) return false;
            i = q;
        }
        (*kv)[name] = val;
        ws();
        if (i < line.size() && line[i] == ',') {
            ++i;
            continue;
        }
        if (i < line.size() && line[i] == '}') return true;
        return false;
    }
}

bool to_int(const std::string& s, long long* v) {
    char* end = nullptr;
    errno = 0;
    long long r = strtoll(s.c_str(), &end, 10);
    if (errno || end == s.c_str() || *end) return false;
    *v = r;
    return true;
}

// Insert a record if it parses, names a known variant, is legal for its shape
// and is faster than what the cache holds for that key.
bool cache_insert_line(const std::string& line) {
    std::map<std::string, std::string> kv;
    if (!parse_record(line, &kv)) return false;
    const char* need[] = {"N", "CI", "H", "W", "CO", "KH", "KW", "stride", "pad", "dtype",
                          "epilogue", "split_k", "stages", "kc", "error_no"};
    long long v[15];
    for (int i = 0; i < 15; ++i) {
        auto it = kv.find(need[i]);
        if (it == kv.end() || !to_int(it->second, &v[i])) return false;
    }
    if (kv["arch"] != kArch) return false;
    if (v[14] != 0) return false;  // only successful measurements are kept
    Shape s;
    if (make_shape((int)v[0], (int)v[1], (int)v[2], (int)v[3], (int)v[4], (int)v[5], (int)v[6],
                   (int)v[7], (int)v[8], (int)v[9], (int)v[10], &s) != CT_OK)
        return false;
    const int vid = find_variant(kv["variant"].c_str());
    if (vid < 0) return false;
    ct_tile_config c{};
    c.variant = vid;
    c.split_k = (int)v[11];
    c.stages = (int)v[12];
    c.kc = (int)v[13];
    c.us = (float)atof(kv["us"].c_str());
    c.error_no = 0;
    if (!legal(s, c, nullptr, nullptr)) return false;
    c.index = encode(space_of(s), c);
    const std::string key = s.key();
    auto it = g_cache.find(key);
    if (it != g_cache.end() && it->second.cfg.us > 0 && it->second.cfg.us <= c.us) return true;
    g_cache[key] = CacheEntry{kv["variant"], c, line};
    g_cache_gen.fetch_add(1, std::memory_order_acq_rel);
    return true;
}

// --------------------------------------------------------- workspaces -----
struct Workspace {
    float* ws = nullptr;
    long long ws_bytes = 0;
    unsigned* tickets = nullptr;
    long long n_tickets = 0;
    void* aux = nullptr;  // a variant's own scratch (the reordered filter)
    long long aux_bytes = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Buffers a workspace outgrew.  They stay allocated until ct_release(): a
// graph captured earlier on that stream, or a launch still in flight, may use
// them.
std::vector<std::pair<int, void*>> g_retired;

int get_workspace(int dev, hipStream_t stream, long long ws_bytes, long long n_tickets, long long aux_bytes,
                  Workspace* out) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace& w = g_ws[{dev, stream}];
    if (w.ws_bytes < ws_bytes || w.n_tickets < n_tickets || w.aux_bytes < aux_bytes) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone)
            return fail(CT_ERR_UNSUPPORTED,
                        "the workspace of this stream must grow, which cannot happen during "
                        "stream capture: run the same convolution once on the stream first");
    }
    hipError_t e;
    if (w.ws_bytes < ws_bytes) {
        const long long b = std::max<long long>(ws_bytes, 1 << 20);
        float* nw = nullptr;
        e = hipMalloc((void**)&nw, (size_t)b);
        if (e != hipSuccess) return fail(CT_ERR_NO_MEMORY, "split workspace of %lld bytes: %s", b,
                                         hipGetErrorString(e));
        if (w.ws) g_retired.push_back({dev, w.ws});
        w.ws = nw;
        w.ws_bytes = b;
    }
    if (w.n_tickets < n_tickets) {
        const long long n = std::max<long long>(n_tickets, 4096);
        unsigned* nt = nullptr;
        e = hipMalloc((void**)&nt, (size_t)n * sizeof(unsigned));
        if (e != hipSuccess) return fail(CT_ERR_NO_MEMORY, "ticket array: %s", hipGetErrorString(e));
        // zeroed once, in stream order before the launch that needs them;
        // every launch leaves the counters it used at zero again
        e = launch_fill_u32(nt, n, 0u, stream);
        if (e != hipSuccess) {
            (void)hipFree(nt);
            return hip_fail(e, "ticket fill");
        }
        if (w.tickets) g_retired.push_back({dev, w.tickets});
        w.tickets = nt;
        w.n_tickets = n;
    }
    if (w.aux_bytes < aux_bytes) {
        const long long b = std::max<long long>(aux_bytes, 1 << 20);
        void* na = nullptr;
        e = hipMalloc(&na, (size_t)b);
        if (e != hipSuccess) return fail(CT_ERR_NO_MEMORY, "filter scratch of %lld bytes: %s", b,
                                         hipGetErrorString(e));
        if (w.aux) g_retired.push_back({dev, w.aux});
        w.aux = na;
        w.aux_bytes = b;
    }
    *out = w;
    return CT_OK;
}

// Scratch of one launch: the split partials, their arrival counters and a
// variant's own buffer (the reordered filter).
struct LaunchScratch {
    float* ws = nullptr;
    unsigned* tickets = nullptr;
    void* aux = nullptr;
};

// ------------------------------------------------ no-allocation scratch --
// ct_conv2d_nchw_fwd_noalloc keeps a launch's scratch in this array instead
// of a per-stream workspace, for callers that cannot allocate.  Layout: the
// split arrival counters first (16384 of them), then the split partials,
// then a variant's own buffer (the reordered half-precision filter), each
// 256-byte aligned.  Each device that loads the library holds its own copy
// until the process ends.  In host code the array's name is only a host-side
// stand-in: device set-up takes its device address per device with
// hipGetSymbolAddress, and everything else uses that address.
constexpr long long kScratchTicketBytes = 64LL << 10;
constexpr long long kScratchDataBytes = CT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchTicketBytes + kScratchDataBytes];
unsigned char* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// Called once per device from device set-up (device current, under
// g_dev_mu, not during capture).  The counters must start at zero: they are
// cleared here, and every launch leaves the counters it used at zero again.
int noalloc_setup(int dev, hipStream_t setup_stream) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    e = launch_fill_u32(static_cast<unsigned*>(ptr), kScratchTicketBytes / 4, 0u, setup_stream);
    if (e == hipSuccess) e = hipStreamSynchronize(setup_stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the no-allocation scratch");
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
    return CT_OK;
}

// A launch's scratch carved from the array, or CT_ERR_UNSUPPORTED when it
// does not fit.
int array_scratch(int dev, const ct_tile_config& c, const Resolved& r, long long aux_bytes, LaunchScratch* out) {
    *out = LaunchScratch{};
    const long long nt = c.split_k > 1 ? (long long)r.tiles_m * r.tiles_n * kTicketStride : 0;
    const long long ws = c.split_k > 1 ? (r.ws_bytes + 255) / 256 * 256 : 0;
    const long long aux = aux_bytes > 0 ? aux_bytes : 0;
    if (nt * (long long)sizeof(unsigned) > kScratchTicketBytes)
        return fail(CT_ERR_UNSUPPORTED,
                    "%lld split tiles exceed the %lld arrival counters of the no-allocation scratch",
                    nt / kTicketStride, kScratchTicketBytes / (long long)sizeof(unsigned) / kTicketStride);
    if (ws + aux > kScratchDataBytes)
        return fail(CT_ERR_UNSUPPORTED,
                    "this shape's config needs %lld bytes of scratch (partials %lld, filter %lld), above the "
                    "%lld-byte limit of the no-allocation entry point",
                    ws + aux, ws, aux, kScratchDataBytes);
    unsigned char* base = g_scratch_ptr[dev];
    if (!base) return fail(CT_ERR_HIP, "no-allocation scratch of device %d not set up", dev);
    out->tickets = reinterpret_cast<unsigned*>(base);
    out->ws = reinterpret_cast<float*>(base + kScratchTicketBytes);
    out->aux = aux > 0 ? base + kScratchTicketBytes + ws : nullptr;
    return CT_OK;
}

// ------------------------------------------------------------- launches ---
ConvParams base_params(const Shape& s, const void* x, const void* w, float* y, const float* bias,
                       const float* var, float eps) {
    ConvParams p{};
    p.x = x; p.w = w; p.y = y; p.bias = bias; p.var = var; p.eps = eps;
    p.N = s.N; p.CI = s.CI; p.H = s.H; p.W = s.W; p.CO = s.CO; p.KH = s.KH; p.KW = s.KW;
    p.stride = s.stride; p.pad = s.pad; p.OH = s.OH; p.OW = s.OW;
    p.T = s.T; p.K = s.K; p.P = s.P; p.OHW = s.OH * s.OW; p.epilogue = s.epilogue;
    p.Hp = s.H + 2 * s.pad; p.Wp = s.W + 2 * s.pad;
    return p;
}

int launch_direct(const Shape& s, const void* x, const void* w, float* y, const float* bias,
                  const float* var, float eps, hipStream_t stream) {
    ConvParams p = base_params(s, x, w, y, bias, var, eps);
    if ((s.P * s.CO + 255) / 256 > 0x7fffffffLL)
        return fail(CT_ERR_UNSUPPORTED, "output too large for the direct kernel");
    hipError_t e = launch_conv_direct(p, s.dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "direct convolution launch");
    return CT_OK;
}

// Launch config c, already resolved (r) and checked legal for s, on device
// dev (set up) with the given scratch.
int launch_resolved(int dev, const Shape& s, const ct_tile_config& c, const Resolved& r, const LaunchScratch& sc,
                    const void* x, const void* w, float* y, const float* bias, const float* var, float eps,
                    hipStream_t stream, bool prepared = false) {
    ConvParams p = base_params(s, x, w, y, bias, var, eps);
    p.w_prepared = prepared ? 1 : 0;
    p.kc = c.kc;
    p.stages = c.stages;
    p.S = c.split_k;
    p.tiles_m = r.tiles_m;
    p.tiles_n = r.tiles_n;
    p.R = r.R;
    p.zero = g_dev[dev].zero;
    if (c.split_k > 1) {
        p.ws = sc.ws;
        p.tickets = sc.tickets;
    }
    p.aux = sc.aux;
    hipError_t e = r.v->ig->launch(p, stream);
    if (e != hipSuccess) return hip_fail(e, r.v->desc.name);
    return CT_OK;
}

long long tickets_needed(const ct_tile_config& c, const Resolved& r) {
    return c.split_k > 1 ? (long long)r.tiles_m * r.tiles_n * kTicketStride : 0;
}

// Bytes of a variant's own scratch for a launch (none when the caller passes
// a prepared filter).
long long launch_aux_bytes(const Shape& s, const Resolved& r, bool prepared) {
    if (!r.v->ig->aux_bytes) return 0;
    ConvParams p = base_params(s, nullptr, nullptr, nullptr, nullptr, nullptr, 0.0f);
    p.w_prepared = prepared ? 1 : 0;
    return r.v->ig->aux_bytes(p);
}

// The stream's workspace (grown if needed) as a launch's scratch.
int stream_scratch(int dev, const ct_tile_config& c, const Resolved& r, long long aux_bytes, hipStream_t stream,
                   LaunchScratch* out) {
    *out = LaunchScratch{};
    if (c.split_k <= 1 && aux_bytes <= 0) return CT_OK;
    Workspace ws;
    const int st = get_workspace(dev, stream, r.ws_bytes, tickets_needed(c, r), aux_bytes, &ws);
    if (st != CT_OK) return st;
    out->ws = ws.ws;
    out->tickets = ws.tickets;
    out->aux = ws.aux;
    return CT_OK;
}

int launch_tiled(const Shape& s, const ct_tile_config& c, const void* x, const void* w, float* y,
                 const float* bias, const float* var, float eps, hipStream_t stream) {
    int dev = 0;
    int st = ensure_device(stream, &dev);
    if (st != CT_OK) return st;
    Resolved r;
    std::string why;
    if (!legal(s, c, &r, &why))
        return fail(CT_ERR_UNSUPPORTED, "tile config not legal for this shape: %s", why.c_str());
    LaunchScratch sc;
    st = stream_scratch(dev, c, r, launch_aux_bytes(s, r, false), stream, &sc);
    if (st != CT_OK) return st;
    return launch_resolved(dev, s, c, r, sc, x, w, y, bias, var, eps, stream);
}

// Built-in default: the legal point with the smallest predicted time (only
// among variants that accept a prepared filter when `prepared`).
bool accepts(const Shape& s, const ct_tile_config& c, bool prepared) {
    return !prepared || (variants()[c.variant].ig && variants()[c.variant].ig->prepared_filter);
}

bool default_config(const Shape& s, ct_tile_config* out, bool prepared = false) {
    const std::string key = s.key() + (prepared ? ",prepared" : "");
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = g_default_memo.find(key);
        if (it != g_default_memo.end()) {
            *out = it->second;
            return out->variant >= 0;
        }
    }
    Space sp = space_of(s);
    double best = 1e300;
    ct_tile_config bc{};
    bc.variant = -1;
    for (long long i = 0; i < sp.size(); ++i) {
        ct_tile_config c;
        decode(sp, i, &c);
        Resolved r;
        if (!accepts(s, c, prepared) || !legal(s, c, &r, nullptr)) continue;
        const double t = predict_us(s, c, r);
        if (t < best) {
            best = t;
            bc = c;
        }
    }
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_default_memo[key] = bc;
    *out = bc;
    return bc.variant >= 0;
}

// The config fwd uses: cached winner, else default; variant -1 = direct.
// With `prepared`, only configs whose variant accepts a prepared filter (a
// cached winner that does not is passed over), and no direct fallback:
// variant -1 when none is legal.
ct_tile_config choose(const Shape& s, int* from_cache, bool prepared = false) {
    ct_tile_config c_cached{};
    bool have = false;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = g_cache.find(s.key());
        if (it != g_cache.end()) {
            c_cached = it->second.cfg;
            have = true;
        }
    }
    // a cached config may name a variant this device cannot run
    if (have && accepts(s, c_cached, prepared) && legal(s, c_cached, nullptr, nullptr)) {
        if (from_cache) *from_cache = 1;
        return c_cached;
    }
    if (from_cache) *from_cache = 0;
    ct_tile_config c{};
    if (!default_config(s, &c, prepared)) {
        c.variant = prepared ? -1 : (int)s.dtype;  // the direct kernel of this dtype
        c.split_k = c.stages = c.kc = 1;
        c.index = -1;
    }
    return c;
}

}  // namespace
int tune_impl(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, int dtype, int epilogue,
              int max_trials, float min_repeat_ms, void* stream, ct_tile_config* best_out, ct_tune_record* records,
              int max_records, int* n_records);
namespace {

// CT_TUNE=1: a launch of a shape with no tuning record first runs the
// tile-config search on its stream (once per shape in the process; not while
// the stream is capturing).  CT_TUNE_TRIALS bounds the trials (default: every
// legal point), CT_TUNE_MS is the minimum milliseconds per repeat (default 20).
std::mutex g_autotune_mu;
std::map<std::string, bool> g_autotuned;

void maybe_autotune(const Shape& s, hipStream_t stream) {
    static const bool on = [] {
        const char* v = getenv("CT_TUNE");
        return v && strcmp(v, "1") == 0;
    }();
    if (!on) return;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        if (g_cache.count(s.key())) return;
    }
    {
        std::lock_guard<std::mutex> lk(g_autotune_mu);
        if (g_autotuned.count(s.key())) return;
        g_autotuned[s.key()] = true;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return;
    }
    const char* t = getenv("CT_TUNE_TRIALS");
    const char* m = getenv("CT_TUNE_MS");
    const int trials = t ? std::max(0, atoi(t)) : 0;
    const float ms = m && atof(m) > 0 ? (float)atof(m) : 20.0f;
    ct_tile_config best{};
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    if (tune_impl(s.N, s.CI, s.H, s.W, s.CO, s.KH, s.KW, s.stride, s.pad, s.dtype, s.epilogue, trials, ms, stream,
                  &best, nullptr, 0, nullptr) != CT_OK) {
        if (log_debug()) fprintf(stderr, "[convtile tune] automatic search failed: %s\n", g_last_error);
        memcpy(g_last_error, saved, sizeof(saved));  // the launch goes on with the default config
    }
}

// ------------------------------------------------------------ launch plans --
// The resolved launch of fwd per (device, shape): the config it uses, with
// the legality check's resolution (grid, window rows, LDS and scratch
// sizes), so that a repeated fwd skips the string key, the cache lookup and
// the legality check.  Any change to the config cache bumps g_cache_gen,
// which retires every plan.

struct PlanKey {
    int v[13];
    bool operator==(const PlanKey& o) const { return memcmp(v, o.v, sizeof v) == 0; }
};

struct PlanKeyHash {
    size_t operator()(const PlanKey& k) const {
        uint64_t h = 1469598103934665603ULL;  // FNV-1a over the words
        for (int x : k.v) {
            h ^= (uint32_t)x;
            h *= 1099511628211ULL;
        }
        return (size_t)h;
    }
};

struct Plan {
    unsigned gen = 0;
    bool direct = false;
    int from_cache = 0;
    ct_tile_config cfg{};
    Resolved r{};
};

std::mutex g_plan_mu;
std::unordered_map<PlanKey, Plan, PlanKeyHash> g_plans;
std::atomic<long long> g_plan_misses{0};

// The plan of fwd for shape s on device dev (set up); `prepared`: the plan
// of the prepared-filter entry point.  `stream`: the launch's (for CT_TUNE).
int get_plan(int dev, const Shape& s, Plan* out, hipStream_t stream, bool prepared = false) {
    const PlanKey k{{dev, s.N, s.CI, s.H, s.W, s.CO, s.KH, s.KW, s.stride, s.pad, s.dtype, s.epilogue,
                     prepared ? 1 : 0}};
    const unsigned gen = g_cache_gen.load(std::memory_order_acquire);
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        auto it = g_plans.find(k);
        if (it != g_plans.end() && it->second.gen == gen) {
            *out = it->second;
            return CT_OK;
        }
    }
    g_plan_misses.fetch_add(1, std::memory_order_relaxed);
    maybe_autotune(s, stream);
    Plan pl;
    pl.gen = gen;
    pl.cfg = choose(s, &pl.from_cache, prepared);
    if (pl.cfg.variant < 0)
        return fail(CT_ERR_UNSUPPORTED, "no tile config of this shape accepts a prepared filter");
    pl.direct = !variants()[pl.cfg.variant].ig;
    if (!pl.direct) {
        std::string why;
        if (!legal(s, pl.cfg, &pl.r, &why))
            return fail(CT_ERR_UNSUPPORTED, "the chosen tile config is not legal: %s", why.c_str());
    }
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_plans[k] = pl;
    *out = pl;
    return CT_OK;
}

double now_s() {
    return std::chrono::duration<double>(std::chrono::system_clock::now().time_since_epoch())
        .count();
}

}  // namespace
}  // namespace ct

using namespace ct;

// the depthwise kernel (conv_depthwise.hip)
namespace ct {
int depthwise_plan(int NC, int OH, int OW, int KH, int KW, int stride, int* RB, int* RIN, int* WPAD,
                   int* LDSW, int* PPW, int* TAPS);
hipError_t launch_depthwise(const void* x, const void* w, float* y, int N, int C, int H, int W, int KH,
                            int KW, int stride, int pad, int dtype, int epilogue, const float* bias,
                            const float* var, float eps, hipStream_t stream);
// the general broadcast (broadcast_chain.hip)
bool chain_channel_ok(long long outer, int P, long long inner, int out_dtype, const void* out, const void* x);
hipError_t launch_broadcast_chain(const ct_bcast_program* prog, const float* const a[4], const float* x,
                                  void* out, int out_dtype, long long outer, int P, long long inner,
                                  bool channel, hipStream_t stream);
}  // namespace ct

// ===================================================================== ABI ==
extern "C" {

int ct_conv2d_nchw_fwd(const void* x, const void* w, float* y, int N, int CI, int H, int W, int CO,
                       int KH, int KW, int stride, int pad, int dtype, int epilogue,
                       const float* bias, const float* var, float eps, void* stream) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, w, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int dev = 0;
    st = ensure_device(hs, &dev);
    if (st != CT_OK) return st;
    Plan pl;
    st = get_plan(dev, s, &pl, hs);
    if (st != CT_OK) return st;
    if (pl.direct) return launch_direct(s, x, w, y, bias, var, eps, hs);
    LaunchScratch sc;
    st = stream_scratch(dev, pl.cfg, pl.r, launch_aux_bytes(s, pl.r, false), hs, &sc);
    if (st != CT_OK) return st;
    return launch_resolved(dev, s, pl.cfg, pl.r, sc, x, w, y, bias, var, eps, hs);
}

int ct_conv2d_nchw_fwd_noalloc(const void* x, const void* w, float* y, int N, int CI, int H, int W, int CO,
                               int KH, int KW, int stride, int pad, int dtype, int epilogue,
                               const float* bias, const float* var, float eps, void* stream) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, w, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int dev = 0;
    st = ensure_device(hs, &dev);
    if (st != CT_OK) return st;
    Plan pl;
    st = get_plan(dev, s, &pl, hs);
    if (st != CT_OK) return st;
    if (pl.direct) return launch_direct(s, x, w, y, bias, var, eps, hs);
    LaunchScratch sc;
    st = array_scratch(dev, pl.cfg, pl.r, launch_aux_bytes(s, pl.r, false), &sc);
    if (st != CT_OK) return st;
    return launch_resolved(dev, s, pl.cfg, pl.r, sc, x, w, y, bias, var, eps, hs);
}

long long ct_conv2d_filter_prepared_bytes(int CO, int CI, int KH, int KW, int dtype) {
    if (CO <= 0 || CI <= 0 || KH <= 0 || KW <= 0) return fail(CT_ERR_INVALID_ARG, "every dimension must be positive");
    if (dtype != CT_F16 && dtype != CT_BF16)
        return fail(CT_ERR_INVALID_ARG, "prepared filters exist for CT_F16 and CT_BF16 only");
    return 2LL * CO * ((CI + 63) / 64 * 64) * KH * KW;
}

int ct_conv2d_prepare_filter(const void* w, void* wp, int CO, int CI, int KH, int KW, int dtype, void* stream) {
    const long long bytes = ct_conv2d_filter_prepared_bytes(CO, CI, KH, KW, dtype);
    if (bytes < 0) return (int)bytes;
    if (!w || !wp) return fail(CT_ERR_INVALID_ARG, "w and wp must not be NULL");
    if ((long long)KH * KW > 1024) return fail(CT_ERR_INVALID_ARG, "filter too large");
    const hipError_t e = h2_prepare_filter(w, wp, CO, CI, KH * KW, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "filter preparation");
    return CT_OK;
}

int ct_conv2d_nchw_fwd_prepared(const void* x, const void* wp, float* y, int N, int CI, int H, int W, int CO,
                                int KH, int KW, int stride, int pad, int dtype, int epilogue,
                                const float* bias, const float* var, float eps, void* stream) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, wp, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    if (dtype != CT_F16 && dtype != CT_BF16)
        return fail(CT_ERR_INVALID_ARG, "prepared filters exist for CT_F16 and CT_BF16 only");
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int dev = 0;
    st = ensure_device(hs, &dev);
    if (st != CT_OK) return st;
    Plan pl;
    st = get_plan(dev, s, &pl, hs, true);
    if (st != CT_OK) return st;
    LaunchScratch sc;
    st = stream_scratch(dev, pl.cfg, pl.r, launch_aux_bytes(s, pl.r, true), hs, &sc);
    if (st != CT_OK) return st;
    return launch_resolved(dev, s, pl.cfg, pl.r, sc, x, wp, y, bias, var, eps, hs, true);
}

// Matrix product as the batch-1 1x1 convolution: C[M][N] = A[M][K] B[K][N]
// is y with w = A ([CO=M][CI=K][1][1]) and x = B ([1][CI=K][H][W], H*W = N:
// a 1x1 filter sees the pixels only as a flat index, so the layout is the
// same for every split of N).  W is the largest divisor of N not above 256,
// which keeps the kernels' image-row windows small.
static int gemm_args(int M, int N, int K, int* H, int* W) {
    if (M <= 0 || N <= 0 || K <= 0) return fail(CT_ERR_INVALID_ARG, "M, N and K must be positive (got %d, %d, %d)", M, N, K);
    for (int w = std::min(N, 256); w >= 1; --w)
        if (N % w == 0) {
            *W = w;
            *H = N / w;
            break;
        }
    return CT_OK;
}

int ct_gemm_fwd(const void* A, const void* B, float* C, int M, int N, int K, int dtype, int epilogue,
                const float* bias, const float* var, float eps, void* stream) {
    int H = 1, W = N;
    const int st = gemm_args(M, N, K, &H, &W);
    if (st != CT_OK) return st;
    return ct_conv2d_nchw_fwd(B, A, C, 1, K, H, W, M, 1, 1, 1, 0, dtype, epilogue, bias, var, eps, stream);
}

int ct_gemm_tune(int M, int N, int K, int dtype, int epilogue, int max_trials, float min_repeat_ms,
                 void* stream, ct_tile_config* best_out, ct_tune_record* records, int max_records,
                 int* n_records) {
    int H = 1, W = N;
    const int st = gemm_args(M, N, K, &H, &W);
    if (st != CT_OK) return st;
    return ct_conv2d_tune(1, K, H, W, M, 1, 1, 1, 0, dtype, epilogue, max_trials, min_repeat_ms, stream,
                          best_out, records, max_records, n_records);
}

int ct_gemm_query(int M, int N, int K, int dtype, int epilogue, ct_tile_config* cfg_out, int* from_cache) {
    int H = 1, W = N;
    const int st = gemm_args(M, N, K, &H, &W);
    if (st != CT_OK) return st;
    return ct_conv2d_query(1, K, H, W, M, 1, 1, 1, 0, dtype, epilogue, cfg_out, from_cache);
}

int ct_conv2d_nchw_fwd_config(const void* x, const void* w, float* y, int N, int CI, int H, int W,
                              int CO, int KH, int KW, int stride, int pad, int dtype, int epilogue,
                              const float* bias, const float* var, float eps,
                              const ct_tile_config* cfg, void* stream) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, w, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    if (!cfg) return fail(CT_ERR_INVALID_ARG, "cfg must not be NULL");
    if (cfg->variant < 0 || cfg->variant >= (int)variants().size())
        return fail(CT_ERR_INVALID_ARG, "unknown variant %d", cfg->variant);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const Variant& v = variants()[cfg->variant];
    if (!v.ig) {
        if (v.desc.dtype != dtype) return fail(CT_ERR_UNSUPPORTED, "direct variant dtype differs");
        return launch_direct(s, x, w, y, bias, var, eps, hs);
    }
    return launch_tiled(s, *cfg, x, w, y, bias, var, eps, hs);
}

int ct_conv2d_nchw_direct(const void* x, const void* w, float* y, int N, int CI, int H, int W,
                          int CO, int KH, int KW, int stride, int pad, int dtype, int epilogue,
                          const float* bias, const float* var, float eps, void* stream) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, w, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    return launch_direct(s, x, w, y, bias, var, eps, static_cast<hipStream_t>(stream));
}

long long ct_conv2d_space_size(int N, int CI, int H, int W, int CO, int KH, int KW, int stride,
                               int pad, int dtype, int epilogue) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    return space_of(s).size();
}

int ct_conv2d_space_entity(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
                           int dtype, int epilogue, long long index, ct_tile_config* cfg_out,
                           int* is_legal) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    if (!cfg_out) return fail(CT_ERR_INVALID_ARG, "cfg_out must not be NULL");
    Space sp = space_of(s);
    if (!decode(sp, index, cfg_out)) return fail(CT_ERR_INVALID_ARG, "index outside the space");
    if (is_legal) *is_legal = legal(s, *cfg_out, nullptr, nullptr) ? 1 : 0;
    return CT_OK;
}

int ct_conv2d_query(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
                    int dtype, int epilogue, ct_tile_config* cfg_out, int* from_cache) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    if (!cfg_out) return fail(CT_ERR_INVALID_ARG, "cfg_out must not be NULL");
    int fc = 0;
    *cfg_out = choose(s, &fc);
    if (from_cache) *from_cache = fc;
    return CT_OK;
}

int ct_variant_count(void) { return (int)variants().size(); }

int ct_variant_info(int variant, ct_variant_desc* out) {
    if (!out) return fail(CT_ERR_INVALID_ARG, "out must not be NULL");
    if (variant < 0 || variant >= (int)variants().size())
        return fail(CT_ERR_INVALID_ARG, "unknown variant %d", variant);
    *out = variants()[variant].desc;
    return CT_OK;
}

long long ct_split_count(long long n, int k) {
    if (n <= 0 || k < 1 || k > 8) return fail(CT_ERR_INVALID_ARG, "need n > 0 and 1 <= k <= 8");
    if (n > (1LL << 40)) return fail(CT_ERR_INVALID_ARG, "n too large");
    return (long long)splits(n, k).size();
}

int ct_split_entity(long long n, int k, long long i, long long* out) {
    if (!out) return fail(CT_ERR_INVALID_ARG, "out must not be NULL");
    long long cnt = ct_split_count(n, k);
    if (cnt < 0) return (int)cnt;
    if (i < 0 || i >= cnt) return fail(CT_ERR_INVALID_ARG, "index outside the split");
    const auto& e = splits(n, k)[i];
    for (int j = 0; j < k; ++j) out[j] = e[j];
    return CT_OK;
}

// ---- the tutorial template's space and resource check --------------------

namespace {

constexpr int kTvmUnroll[3] = {0, 512, 1500};

// Knob tables of the template for a shape: the six splits (tile_f, tile_y,
// tile_x over CO, OH, OW into 4; tile_rc, tile_ry, tile_rx over CI, KH, KW
// into 3) and the two option lists, with their lengths in declaration order.
struct TvmKnobs {
    const std::vector<std::vector<long long>>* split[6];
    long long len[8];
    long long size;
};

int tvm_knobs(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, TvmKnobs* k) {
    Shape s;
    const int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, CT_F32, CT_EPI_NONE, &s);
    if (st != CT_OK) return st;
    const long long ext[6] = {s.CO, s.OH, s.OW, s.CI, s.KH, s.KW};
    const int parts[6] = {4, 4, 4, 3, 3, 3};
    k->size = 1;
    for (int i = 0; i < 6; ++i) {
        k->split[i] = &splits(ext[i], parts[i]);
        k->len[i] = (long long)k->split[i]->size();
    }
    k->len[6] = 3;
    k->len[7] = 2;
    for (int i = 0; i < 8; ++i) {
        if (k->size > (1LL << 62) / k->len[i]) return fail(CT_ERR_INVALID_ARG, "space too large");
        k->size *= k->len[i];
    }
    return CT_OK;
}

int* tvm_knob_field(ct_tvm_config* c, int i) {
    switch (i) {
        case 0: return c->tile_f;
        case 1: return c->tile_y;
        case 2: return c->tile_x;
        case 3: return c->tile_rc;
        case 4: return c->tile_ry;
        default: return c->tile_rx;
    }
}

}  // namespace

long long ct_tvm_space_size(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad) {
    TvmKnobs k;
    const int st = tvm_knobs(N, CI, H, W, CO, KH, KW, stride, pad, &k);
    return st != CT_OK ? st : k.size;
}

int ct_tvm_space_entity(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
                        long long index, ct_tvm_config* out) {
    if (!out) return fail(CT_ERR_INVALID_ARG, "out must not be NULL");
    TvmKnobs k;
    const int st = tvm_knobs(N, CI, H, W, CO, KH, KW, stride, pad, &k);
    if (st != CT_OK) return st;
    if (index < 0 || index >= k.size) return fail(CT_ERR_INVALID_ARG, "index outside the space");
    long long rest = index;
    for (int i = 0; i < 6; ++i) {
        const auto& e = (*k.split[i])[rest % k.len[i]];
        rest /= k.len[i];
        int* f = tvm_knob_field(out, i);
        for (size_t j = 0; j < e.size(); ++j) f[j] = (int)e[j];
    }
    out->auto_unroll_max_step = kTvmUnroll[rest % 3];
    rest /= 3;
    out->unroll_explicit = (int)(rest % 2);
    return CT_OK;
}

long long ct_tvm_space_index(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
                             const ct_tvm_config* cfg) {
    if (!cfg) return fail(CT_ERR_INVALID_ARG, "cfg must not be NULL");
    TvmKnobs k;
    const int st = tvm_knobs(N, CI, H, W, CO, KH, KW, stride, pad, &k);
    if (st != CT_OK) return st;
    ct_tvm_config c = *cfg;
    long long digit[8];
    for (int i = 0; i < 6; ++i) {
        const int* f = tvm_knob_field(&c, i);
        digit[i] = -1;
        const auto& sp = *k.split[i];
        for (size_t t = 0; t < sp.size() && digit[i] < 0; ++t) {
            bool same = true;
            for (size_t j = 0; j < sp[t].size(); ++j) same = same && sp[t][j] == f[j];
            if (same) digit[i] = (long long)t;
        }
        if (digit[i] < 0) return -1;
    }
    digit[6] = -1;
    for (int t = 0; t < 3; ++t)
        if (kTvmUnroll[t] == cfg->auto_unroll_max_step) digit[6] = t;
    if (digit[6] < 0 || (cfg->unroll_explicit != 0 && cfg->unroll_explicit != 1)) return -1;
    digit[7] = cfg->unroll_explicit;
    long long index = 0, radix = 1;
    for (int i = 0; i < 8; ++i) {
        index += digit[i] * radix;
        radix *= k.len[i];
    }
    return index;
}

int ct_tvm_config_check(const ct_tvm_config* cfg, int stride, int mode, long long* shared_bytes,
                        int* threads) {
    if (!cfg) return fail(CT_ERR_INVALID_ARG, "cfg must not be NULL");
    if (stride < 1) return fail(CT_ERR_INVALID_ARG, "stride must be positive");
    if (mode != CT_TVM_LIMITS_PAGE && mode != CT_TVM_LIMITS_GFX950)
        return fail(CT_ERR_INVALID_ARG, "unknown mode %d", mode);
    const int* four[3] = {cfg->tile_f, cfg->tile_y, cfg->tile_x};
    const int* three[3] = {cfg->tile_rc, cfg->tile_ry, cfg->tile_rx};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 4; ++j)
            if (four[i][j] < 1) return fail(CT_ERR_INVALID_ARG, "split factors must be >= 1");
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            if (three[i][j] < 1) return fail(CT_ERR_INVALID_ARG, "split factors must be >= 1");
    // a block's output extents: vthread x thread x inner factors
    const long long fb = (long long)cfg->tile_f[1] * cfg->tile_f[2] * cfg->tile_f[3];
    const long long yb = (long long)cfg->tile_y[1] * cfg->tile_y[2] * cfg->tile_y[3];
    const long long xb = (long long)cfg->tile_x[1] * cfg->tile_x[2] * cfg->tile_x[3];
    // reduction extents inside the outer rc, ry, rx loops, where the shared
    // stages are computed (ry split by tile_rx's factors and rx by tile_ry's,
    // as the schedule is printed)
    const long long rcs = (long long)cfg->tile_rc[1] * cfg->tile_rc[2];
    const long long rys = (long long)cfg->tile_rx[1] * cfg->tile_rx[2];
    const long long rxs = (long long)cfg->tile_ry[1] * cfg->tile_ry[2];
    const long long aa = rcs * ((yb - 1) * stride + rys) * ((xb - 1) * stride + rxs);
    const long long ww = fb * rcs * rys * rxs;
    const long long bytes = 4 * (aa + ww);
    const long long nthr = (long long)cfg->tile_f[2] * cfg->tile_y[2] * cfg->tile_x[2];
    if (shared_bytes) *shared_bytes = bytes;
    if (threads) *threads = (int)std::min<long long>(nthr, 1LL << 30);
    const long long limit = mode == CT_TVM_LIMITS_PAGE ? 48LL * 1024 : 160LL * 1024;
    return (bytes <= limit && nthr <= 1024) ? 1 : 0;
}

int ct_broadcast_nchw(const float* var, void* out, int N, int C, int H, int W, int out_dtype, int op,
                      int mode, void* stream) {
    if (!var || !out) return fail(CT_ERR_INVALID_ARG, "var and out must not be NULL");
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0)
        return fail(CT_ERR_INVALID_ARG, "every dimension must be positive");
    if (out_dtype != CT_F32 && out_dtype != CT_F16)
        return fail(CT_ERR_INVALID_ARG, "out_dtype must be CT_F32 or CT_F16");
    if (op != CT_BC_EXP) return fail(CT_ERR_INVALID_ARG, "unknown op %d", op);
    if (mode != CT_BC_AUTO && mode != CT_BC_CHANNEL && mode != CT_BC_FLAT)
        return fail(CT_ERR_INVALID_ARG, "unknown mode %d", mode);
    const long long HW = (long long)H * W;
    if (HW > (1LL << 30) || (long long)N * C * HW > (1LL << 46))
        return fail(CT_ERR_INVALID_ARG, "output too large");
    // channel-bound applies to static H*W that is a multiple of 32, with
    // 16-byte aligned rows (the PR's Init checks, as read here)
    const bool aligned = (reinterpret_cast<uintptr_t>(out) % 16) == 0;
    const bool channel_ok = (HW % 32 == 0) && aligned && N <= 0x7fffffff / 1;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mode == CT_BC_CHANNEL && !channel_ok)
        return fail(CT_ERR_UNSUPPORTED, "channel-bound broadcast needs H*W %% 32 == 0 and 16-byte "
                                        "aligned output");
    if (mode == CT_BC_FLAT || !channel_ok)
        e = launch_bcast_flat(var, out, N, C, (int)HW, out_dtype, hs);
    else
        e = launch_bcast_channel(var, out, N, C, (int)HW, out_dtype, hs);
    if (e != hipSuccess) return hip_fail(e, "broadcast launch");
    return CT_OK;
}

int ct_conv2d_nchw_depthwise(const void* x, const void* w, float* y, int N, int C, int H, int W, int KH,
                             int KW, int stride, int pad, int dtype, int epilogue, const float* bias,
                             const float* var, float eps, void* stream) {
    Shape s;  // the shape checks of a convolution with one input channel per group
    int st = make_shape(N, 1, H, W, C, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = check_pointers(x, w, y, epilogue, bias, var);
    if (st != CT_OK) return st;
    if ((long long)KH * KW > 256)
        return fail(CT_ERR_UNSUPPORTED, "depthwise filters hold at most 256 taps (got %dx%d)", KH, KW);
    if ((long long)N * C > 0x7fffffffLL) return fail(CT_ERR_UNSUPPORTED, "N*C above 2^31 - 1");
    if ((long long)H * W > 0x7fffffffLL) return fail(CT_ERR_UNSUPPORTED, "H*W above 2^31 - 1");
    int rb, rin, wpad, ldsw, ppw, taps;
    if (depthwise_plan(N * C, s.OH, s.OW, KH, KW, stride, &rb, &rin, &wpad, &ldsw, &ppw, &taps) < 0)
        return fail(CT_ERR_UNSUPPORTED, "an output row of %d columns (stride %d, %dx%d filter) does not fit "
                    "one workgroup's LDS window", s.OW, stride, KH, KW);
    const hipError_t e = launch_depthwise(x, w, y, N, C, H, W, KH, KW, stride, pad, dtype, epilogue, bias,
                                          var, eps, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "depthwise launch");
    return CT_OK;
}

int ct_broadcast_chain(const ct_bcast_program* prog, const float* a0, const float* a1, const float* a2,
                       const float* a3, const float* x, void* out, int out_dtype, long long outer, int P,
                       long long inner, int mode, void* stream) {
    if (!prog || !out) return fail(CT_ERR_INVALID_ARG, "prog and out must not be NULL");
    if (outer < 1 || P < 1 || inner < 1) return fail(CT_ERR_INVALID_ARG, "outer, P and inner must be positive");
    if ((double)outer * P * inner > (double)(1LL << 46)) return fail(CT_ERR_INVALID_ARG, "output too large");
    if (out_dtype != CT_F32 && out_dtype != CT_F16)
        return fail(CT_ERR_INVALID_ARG, "out_dtype must be CT_F32 or CT_F16");
    if (mode != CT_BC_AUTO && mode != CT_BC_CHANNEL && mode != CT_BC_FLAT)
        return fail(CT_ERR_INVALID_ARG, "unknown mode %d", mode);
    const float* arrays[4] = {a0, a1, a2, a3};
    bool reads_x = false;
    for (int c = 0; c < 3; ++c) {
        const int n = prog->n_ops[c];
        if (n < 0 || n > CT_CHAIN_MAX_OPS)
            return fail(CT_ERR_INVALID_ARG, "chain %d has %d steps (0..%d)", c, n, CT_CHAIN_MAX_OPS);
        for (int k = 0; k < n; ++k) {
            const ct_chain_op& o = prog->ops[c][k];
            if (o.op < CT_OP_SET || o.op > CT_OP_SQRT)
                return fail(CT_ERR_INVALID_ARG, "chain %d step %d: unknown op %d", c, k, o.op);
            if (o.src < CT_SRC_IMM || o.src > CT_SRC_A0 + 3)
                return fail(CT_ERR_INVALID_ARG, "chain %d step %d: unknown source %d", c, k, o.src);
            // the unary steps ignore their operand
            if (o.op == CT_OP_EXP || o.op == CT_OP_RSQRT || o.op == CT_OP_SQRT) continue;
            const bool allowed = o.src == CT_SRC_IMM || o.src >= CT_SRC_A0 || (o.src == CT_SRC_C0 && c >= 1) ||
                                 (c == 2 && (o.src == CT_SRC_C1 || o.src == CT_SRC_X));
            if (!allowed) return fail(CT_ERR_INVALID_ARG, "chain %d step %d may not read source %d", c, k, o.src);
            if (o.src >= CT_SRC_A0 && !arrays[o.src - CT_SRC_A0])
                return fail(CT_ERR_INVALID_ARG, "chain %d step %d reads array a%d, which is NULL", c, k,
                            o.src - CT_SRC_A0);
            if (o.src == CT_SRC_X) reads_x = true;
        }
    }
    if (reads_x && !x) return fail(CT_ERR_INVALID_ARG, "a step reads x, which is NULL");
    const float* xr = reads_x ? x : nullptr;
    if (xr && (const void*)xr == out && out_dtype != CT_F32)
        return fail(CT_ERR_INVALID_ARG, "x == out needs fp32 output");
    const bool ok = chain_channel_ok(outer, P, inner, out_dtype, out, xr);
    if (mode == CT_BC_CHANNEL && !ok)
        return fail(CT_ERR_UNSUPPORTED, "channel-bound broadcast needs inner >= 32, whole 16-byte vectors per "
                                        "row, 16-byte aligned out and x, and a grid that fits");
    const bool channel = mode == CT_BC_CHANNEL || (mode == CT_BC_AUTO && ok);
    const hipError_t e = launch_broadcast_chain(prog, arrays, xr, out, out_dtype, outer, P, inner, channel,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "broadcast chain launch");
    return CT_OK;
}

int ct_cache_load(const char* path) {
    if (!path) return fail(CT_ERR_INVALID_ARG, "path must not be NULL");
    std::ifstream f(path);
    if (!f) return fail(CT_ERR_IO, "cannot open %s", path);
    std::string line;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    while (std::getline(f, line)) {
        if (line.empty()) continue;
        (void)cache_insert_line(line);  // unparsable or stale lines are skipped
    }
    return CT_OK;
}

int ct_cache_save(const char* path) {
    if (!path) return fail(CT_ERR_INVALID_ARG, "path must not be NULL");
    std::ofstream f(path, std::ios::app);
    if (!f) return fail(CT_ERR_IO, "cannot open %s", path);
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (const auto& kv : g_cache) f << kv.second.line << "\n";
    f.flush();
    if (!f) return fail(CT_ERR_IO, "write to %s failed", path);
    return CT_OK;
}

int ct_cache_clear(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache.clear();
    g_cache_gen.fetch_add(1, std::memory_order_acq_rel);
    return CT_OK;
}

int ct_cache_size(void) {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    return (int)g_cache.size();
}

int ct_release(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : g_ws) {
        (void)hipSetDevice(kv.first.first);
        (void)hipStreamSynchronize(kv.first.second);
        if (kv.second.ws) (void)hipFree(kv.second.ws);
        if (kv.second.tickets) (void)hipFree(kv.second.tickets);
        if (kv.second.aux) (void)hipFree(kv.second.aux);
    }
    for (auto& r : g_retired) {
        (void)hipSetDevice(r.first);
        (void)hipFree(r.second);
    }
    if (have_cur) (void)hipSetDevice(cur);
    (void)hipGetLastError();
    g_ws.clear();
    g_retired.clear();
    return have_cur ? CT_OK : CT_ERR_HIP;
}

int ct_init(int device) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= count || device >= kMaxDevices)
        return fail(CT_ERR_INVALID_ARG, "device %d: %d devices visible", device, count);
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    int st;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        st = device_setup_locked(device);
    }
    if (cur != device) (void)hipSetDevice(cur);
    return st;
}

long long ct_plan_misses(void) { return g_plan_misses.load(std::memory_order_relaxed); }

const char* ct_status_string(int status) {
    switch (status) {
        case CT_OK: return "ok";
        case CT_ERR_INVALID_ARG: return "invalid argument";
        case CT_ERR_UNSUPPORTED: return "unsupported";
        case CT_ERR_HIP: return "HIP error";
        case CT_ERR_NO_MEMORY: return "out of device memory";
        case CT_ERR_IO: return "I/O error";
        case CT_ERR_TUNE_FAILED: return "tuning failed";
        default: return "unknown status";
    }
}

const char* ct_last_error(void) { return g_last_error; }

const char* ct_version(void) { return "convtile 0.1 gfx950"; }

}  // extern "C"

// ================================================================ tuner ==
namespace ct {
namespace {

struct Scratch {
    void* x = nullptr;
    void* w = nullptr;
    float* y = nullptr;
    float* y_ref = nullptr;
    float* bias = nullptr;
    float* var = nullptr;
    unsigned* bad = nullptr;
    ~Scratch() {
        for (void* p : {x, w, (void*)y, (void*)y_ref, (void*)bias, (void*)var, (void*)bad})
            if (p) (void)hipFree(p);
    }
};

// "index:error_no,index:error_no" -- a host-side hook that makes the search
// record the given outcome for a candidate instead of running it.
std::map<long long, int> injected_errors() {
    std::map<long long, int> m;
    const char* s = getenv("CT_TUNE_INJECT");
    if (!s) return m;
    std::string str(s);
    std::stringstream ss(str);
    std::string item;
    while (std::getline(ss, item, ',')) {
        size_t c = item.find(':');
        if (c == std::string::npos) continue;
        m[atoll(item.substr(0, c).c_str())] = atoi(item.substr(c + 1).c_str());
    }
    return m;
}

// Device-side state of a search: scratch inputs filled on the device, the
// direct kernel's reference output, events; trial() times one candidate the
// way the TVM tutorial's runner does (a check of the output, then `repeat`
// measurements of at least min_repeat_ms each, a per-trial time limit).
struct TuneBench {
    Shape s;
    Space sp;
    hipStream_t hs = nullptr;
    Scratch sc;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    float atol = 0, rtol = 0, eps = 1e-5f;
    float min_repeat_ms = 0;
    long long ny = 0;
    std::map<long long, int> inject;
    double timeout_s = 4.0;  // per trial, as the tutorial's runner; CT_TUNE_TIMEOUT_S overrides
    static constexpr int kRepeat = 3;

    // Wait for `ev` while the trial stays within its time limit: the limit
    // is checked while the launches run, not only after them.  On a timeout
    // no more launches of the trial are issued and the ones in flight are
    // drained (they cannot be cancelled) before the next trial.
    int wait_event(hipEvent_t ev, std::chrono::steady_clock::time_point t_start) {
        while (true) {
            const hipError_t q = hipEventQuery(ev);
            if (q == hipSuccess) return CT_TRIAL_OK;
            if (q != hipErrorNotReady) {
                (void)hipGetLastError();
                return CT_TRIAL_RUNTIME;
            }
            const double wall = std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
            if (wall > timeout_s) {
                (void)hipStreamSynchronize(hs);
                (void)hipGetLastError();
                return CT_TRIAL_TIMEOUT;
            }
            std::this_thread::sleep_for(std::chrono::microseconds(20));
        }
    }

    ~TuneBench() {
        if (ev0) (void)hipEventDestroy(ev0);
        if (ev1) (void)hipEventDestroy(ev1);
    }

    int init(const Shape& shape, void* stream, float repeat_ms) {
        s = shape;
        sp = space_of(s);
        hs = static_cast<hipStream_t>(stream);
        min_repeat_ms = repeat_ms;
        const size_t esz = s.dtype == CT_F32 ? 4 : 2;
        const long long nx = (long long)s.N * s.CI * s.H * s.W, nw = (long long)s.CO * s.K;
        ny = s.P * s.CO;
        hipError_t e;
        if ((e = hipMalloc(&sc.x, nx * esz)) != hipSuccess || (e = hipMalloc(&sc.w, nw * esz)) != hipSuccess ||
            (e = hipMalloc((void**)&sc.y, ny * 4)) != hipSuccess ||
            (e = hipMalloc((void**)&sc.y_ref, ny * 4)) != hipSuccess ||
            (e = hipMalloc((void**)&sc.bias, s.CO * 4)) != hipSuccess ||
            (e = hipMalloc((void**)&sc.var, s.CO * 4)) != hipSuccess ||
            (e = hipMalloc((void**)&sc.bad, 4)) != hipSuccess)
            return fail(CT_ERR_NO_MEMORY, "tuning scratch: %s", hipGetErrorString(e));
        const float wa = std::sqrt(6.0f / (float)s.K);
        if ((e = launch_fill_uniform(sc.x, nx, s.dtype, -1.0f, 1.0f, 11u, hs)) != hipSuccess ||
            (e = launch_fill_uniform(sc.w, nw, s.dtype, -wa, wa, 12u, hs)) != hipSuccess ||
            (e = launch_fill_uniform(sc.bias, s.CO, CT_F32, -0.2f, 0.2f, 13u, hs)) != hipSuccess ||
            (e = launch_fill_uniform(sc.var, s.CO, CT_F32, 0.5f, 2.0f, 14u, hs)) != hipSuccess)
            return hip_fail(e, "tuning scratch fill");
        const int st = launch_direct(s, sc.x, sc.w, sc.y_ref, sc.bias, sc.var, eps, hs);
        if (st != CT_OK) return st;
        if ((e = hipStreamSynchronize(hs)) != hipSuccess) return hip_fail(e, "reference run");
        // expected sum |x w| is about K * E|x| * E|w| = K * wa / 4; allow 1e-4 of twice that
        atol = 1e-4f * (float)s.K * wa * 0.5f;
        rtol = s.epilogue == CT_EPI_EXP_BIAS_RSQRT ? atol + 1e-5f : 1e-5f;
        if ((e = hipEventCreate(&ev0)) != hipSuccess) return hip_fail(e, "hipEventCreate");
        if ((e = hipEventCreate(&ev1)) != hipSuccess) return hip_fail(e, "hipEventCreate");
        inject = injected_errors();
        if (const char* t = getenv("CT_TUNE_TIMEOUT_S")) {
            const double v = atof(t);
            if (v > 0.0) timeout_s = v;
        }
        return CT_OK;
    }

    // Time candidate idx; fills *rec (cfg, costs, error_no, wall time).
    void trial(long long idx, ct_tune_record* rec) {
        const auto t_start = std::chrono::steady_clock::now();
        ct_tile_config c;
        decode(sp, idx, &c);
        *rec = ct_tune_record{};
        int err = CT_TRIAL_OK;
        int st = CT_OK;
        hipError_t e;
        auto inj = inject.find(idx);
        Resolved r;
        if (inj != inject.end()) {
            err = inj->second;
        } else if (!legal(s, c, &r, nullptr)) {
            err = CT_TRIAL_ILLEGAL;
        } else {
            // poison the output so a kernel that writes nothing cannot pass
            e = hipMemsetAsync(sc.y, 0xff, ny * 4, hs);
            st = (e == hipSuccess) ? launch_tiled(s, c, sc.x, sc.w, sc.y, sc.bias, sc.var, eps, hs) : CT_ERR_HIP;
            if (st == CT_OK) {
                if (hipEventRecord(ev1, hs) != hipSuccess) {
                    st = CT_ERR_HIP;
                } else {
                    const int w = wait_event(ev1, t_start);
                    if (w == CT_TRIAL_TIMEOUT) err = CT_TRIAL_TIMEOUT;
                    if (w != CT_TRIAL_OK) st = CT_ERR_HIP;
                }
            }
            if (st == CT_OK) {
                unsigned bad = 0;
                if (hipMemsetAsync(sc.bad, 0, 4, hs) != hipSuccess ||
                    launch_compare(sc.y, sc.y_ref, ny, atol, rtol, sc.bad, hs) != hipSuccess ||
                    hipMemcpyAsync(&bad, sc.bad, 4, hipMemcpyDeviceToHost, hs) != hipSuccess ||
                    hipStreamSynchronize(hs) != hipSuccess || bad != 0)
                    st = CT_ERR_TUNE_FAILED;
            }
            if (st != CT_OK) {
                if (err == CT_TRIAL_OK) err = CT_TRIAL_RUNTIME;
            } else {
                // calibrate the launch count so a repeat lasts >= min_repeat_ms
                long long number = 1;
                float ms = 0.0f;
                while (true) {
                    (void)hipEventRecord(ev0, hs);
                    for (long long i = 0; i < number && st == CT_OK; ++i)
                        st = launch_tiled(s, c, sc.x, sc.w, sc.y, sc.bias, sc.var, eps, hs);
                    (void)hipEventRecord(ev1, hs);
                    const int wv = st == CT_OK ? wait_event(ev1, t_start) : CT_TRIAL_RUNTIME;
                    if (wv != CT_TRIAL_OK) {
                        err = wv;
                        break;
                    }
                    (void)hipEventElapsedTime(&ms, ev0, ev1);
                    if (ms >= min_repeat_ms || number >= (1LL << 20)) break;
                    const double want = ms > 0.0f ? 1.25 * min_repeat_ms / ms * number : 2.0 * number;
                    number = std::max<long long>(2 * number, (long long)std::ceil(want));
                    number = std::min<long long>(number, 1LL << 20);
                }
                for (int rep = 0; rep < kRepeat && err == CT_TRIAL_OK; ++rep) {
                    (void)hipEventRecord(ev0, hs);
                    for (long long i = 0; i < number && st == CT_OK; ++i)
                        st = launch_tiled(s, c, sc.x, sc.w, sc.y, sc.bias, sc.var, eps, hs);
                    (void)hipEventRecord(ev1, hs);
                    const int wv = st == CT_OK ? wait_event(ev1, t_start) : CT_TRIAL_RUNTIME;
                    if (wv != CT_TRIAL_OK) {
                        err = wv;
                        break;
                    }
                    (void)hipEventElapsedTime(&ms, ev0, ev1);
                    rec->costs_us[rep] = 1000.0f * ms / (float)number;
                    rec->n_costs = rep + 1;
                }
            }
        }
        rec->error_no = err;
        rec->all_cost_s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
        rec->timestamp = now_s();
        c.error_no = err;
        c.us = 0.0f;
        if (err == CT_TRIAL_OK && rec->n_costs == kRepeat) {
            double mean = 0;
            for (int i = 0; i < kRepeat; ++i) mean += rec->costs_us[i];
            c.us = (float)(mean / kRepeat);
        }
        rec->cfg = c;
    }
};

// The tuning log named by CT_CACHE_PATH (the TVM tutorial's Step 2 writes
// every measure record to a log file as it is measured, log_to_file): one
// JSON line per trial, appended and flushed as each trial ends, so that a
// search that stops part way leaves every finished trial in the file.  A
// search of a shape resumes from it: the (variant, split) points already
// logged for the shape's key are not measured again, and their logged
// outcomes take part in choosing the winner.
struct TuneLog {
    std::string path;
    std::ofstream out;
    // logged trials of this shape: (variant name, split_k, stages, kc) -> record
    std::map<std::tuple<std::string, int, int, int>, ct_tune_record> done;

    static std::tuple<std::string, int, int, int> point(const ct_tile_config& c) {
        return std::make_tuple(std::string(variants()[c.variant].desc.name), c.split_k, c.stages, c.kc);
    }

    // Read the log's records of shape s (when CT_CACHE_PATH is set).
    void open(const Shape& s) {
        const char* p = getenv("CT_CACHE_PATH");
        if (!p || !*p) return;
        path = p;
        std::ifstream in(path);
        std::string line;
        const Space sp = space_of(s);
        while (in && std::getline(in, line)) {
            std::map<std::string, std::string> kv;
            if (!parse_record(line, &kv) || kv["key"] != s.key()) continue;
            long long v[4];
            const char* need[] = {"split_k", "stages", "kc", "error_no"};
            bool ok = true;
            for (int i = 0; i < 4 && ok; ++i) ok = kv.count(need[i]) && to_int(kv[need[i]], &v[i]);
            const int vid = ok ? find_variant(kv["variant"].c_str()) : -1;
            if (vid < 0) continue;
            ct_tune_record r{};
            r.cfg.variant = vid;
            r.cfg.split_k = (int)v[0];
            r.cfg.stages = (int)v[1];
            r.cfg.kc = (int)v[2];
            r.cfg.index = encode(sp, r.cfg);
            r.error_no = (int)v[3];
            r.cfg.error_no = r.error_no;
            r.cfg.us = (float)atof(kv["us"].c_str());
            // costs "[a,b,c]"
            const std::string cs = kv["costs_us"];
            size_t i = cs.find('[');
            while (i != std::string::npos && r.n_costs < 3) {
                char* end = nullptr;
                const double c = strtod(cs.c_str() + i + 1, &end);
                if (end == cs.c_str() + i + 1) break;
                r.costs_us[r.n_costs++] = (float)c;
                i = cs.find(',', i + 1);
            }
            r.all_cost_s = atof(kv["all_cost"].c_str());
            r.timestamp = atof(kv["timestamp"].c_str());
            if (r.cfg.index < 0) continue;  // not a point of this shape's space
            done[point(r.cfg)] = r;
        }
        out.open(path, std::ios::app);
    }

    bool logged(const ct_tile_config& c) const { return done.count(point(c)) != 0; }

    int append(const Shape& s, const ct_tune_record& r) {
        if (path.empty()) return CT_OK;
        if (!out) return fail(CT_ERR_IO, "cannot append to %s", path.c_str());
        out << json_record(s, r.cfg, variants()[r.cfg.variant].desc.name, r.costs_us, r.n_costs, r.all_cost_s,
                           r.timestamp)
            << "\n";
        out.flush();
        if (!out) return fail(CT_ERR_IO, "write to %s failed", path.c_str());
        return CT_OK;
    }
};

// Keep the best of the records (this search's and the ones it resumed from
// the log) and store the winner in the in-memory cache.
int tune_finish(const Shape& s, const std::vector<ct_tune_record>& recs, const TuneLog& log,
                ct_tile_config* best_out, ct_tune_record* records, int max_records, int* n_records) {
    ct_tile_config best{};
    best.variant = -1;
    auto consider = [&](const ct_tune_record& r) {
        if (r.error_no != CT_TRIAL_OK || r.n_costs != TuneBench::kRepeat) return;
        if (best.variant < 0 || r.cfg.us < best.us || (r.cfg.us == best.us && r.cfg.index < best.index))
            best = r.cfg;
    };
    for (size_t k = 0; k < recs.size(); ++k) {
        if ((int)k < max_records) records[k] = recs[k];
        consider(recs[k]);
    }
    for (const auto& kv : log.done) consider(kv.second);
    if (n_records) *n_records = std::min((int)recs.size(), max_records);
    if (best.variant < 0) return fail(CT_ERR_TUNE_FAILED, "no candidate ran correctly");
    *best_out = best;
    float costs[1] = {best.us};
    const std::string line = json_record(s, best, variants()[best.variant].desc.name, costs, 1, 0.0, now_s());
    std::lock_guard<std::mutex> lk(g_cache_mu);
    g_cache[s.key()] = CacheEntry{variants()[best.variant].desc.name, best, line};
    g_cache_gen.fetch_add(1, std::memory_order_acq_rel);
    return CT_OK;
}

// The order in which the exhaustive search times a shape's points: legal
// points by predicted time, then the illegal ones (recorded as error 1
// without a launch), leaving out the points the log already holds, at most
// max_trials of them (0 = all).
std::vector<long long> exhaustive_order(const Shape& s, int max_trials, const TuneLog& log) {
    Space sp = space_of(s);
    std::vector<std::pair<double, long long>> order;
    std::vector<long long> illegal;
    for (long long i = 0; i < sp.size(); ++i) {
        ct_tile_config c;
        decode(sp, i, &c);
        if (log.logged(c)) continue;
        Resolved r;
        if (legal(s, c, &r, nullptr))
            order.push_back({predict_us(s, c, r), i});
        else
            illegal.push_back(i);
    }
    std::stable_sort(order.begin(), order.end());
    std::vector<long long> trials;
    for (auto& o : order) trials.push_back(o.second);
    for (long long i : illegal) trials.push_back(i);
    if (max_trials > 0 && (long long)trials.size() > max_trials) trials.resize(max_trials);
    return trials;
}

int tune_args(int max_trials, float min_repeat_ms, ct_tile_config* best_out, ct_tune_record* records,
              int max_records, int* n_records) {
    if (!best_out) return fail(CT_ERR_INVALID_ARG, "best_out must not be NULL");
    if (max_trials < 0) return fail(CT_ERR_INVALID_ARG, "max_trials must be >= 0");
    if (!(min_repeat_ms >= 0.0f)) return fail(CT_ERR_INVALID_ARG, "min_repeat_ms must be >= 0");
    if (max_records < 0 || (max_records > 0 && !records))
        return fail(CT_ERR_INVALID_ARG, "records / max_records mismatch");
    if (n_records) *n_records = 0;
    return CT_OK;
}

void log_trial(int no, const ct_tune_record& rec) {
    if (log_debug())
        fprintf(stderr, "[convtile tune] No: %d index %lld %s S=%d stages=%d kc=%d  %.3f us  error_no=%d all_cost=%.3fs\n",
                no, rec.cfg.index, variants()[rec.cfg.variant].desc.name, rec.cfg.split_k, rec.cfg.stages,
                rec.cfg.kc, (double)rec.cfg.us, rec.error_no, rec.all_cost_s);
}

}  // namespace

int tune_impl(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, int dtype,
              int epilogue, int max_trials, float min_repeat_ms, void* stream,
              ct_tile_config* best_out, ct_tune_record* records, int max_records, int* n_records) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = tune_args(max_trials, min_repeat_ms, best_out, records, max_records, n_records);
    if (st != CT_OK) return st;

    TuneLog log;
    log.open(s);
    const std::vector<long long> trials = exhaustive_order(s, max_trials, log);

    TuneBench tb;
    st = tb.init(s, stream, min_repeat_ms);
    if (st != CT_OK) return st;
    std::vector<ct_tune_record> recs;
    for (long long idx : trials) {
        ct_tune_record rec;
        tb.trial(idx, &rec);
        recs.push_back(rec);
        log_trial((int)recs.size(), rec);
        st = log.append(s, rec);
        if (st != CT_OK) return st;
    }
    return tune_finish(s, recs, log, best_out, records, max_records, n_records);
}

int tune_order_impl(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, int dtype,
                    int epilogue, int max_trials, long long* order_out, int max_out, int* n_out) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    if (max_trials < 0) return fail(CT_ERR_INVALID_ARG, "max_trials must be >= 0");
    if (!n_out || max_out < 0 || (max_out > 0 && !order_out))
        return fail(CT_ERR_INVALID_ARG, "order_out / max_out / n_out mismatch");
    TuneLog log;
    log.open(s);
    const std::vector<long long> trials = exhaustive_order(s, max_trials, log);
    const int n = (int)std::min<size_t>(trials.size(), (size_t)max_out);
    for (int i = 0; i < n; ++i) order_out[i] = trials[i];
    *n_out = (int)trials.size();
    return CT_OK;
}

// ------------------------------------------------------- guided search --
// The TVM tutorial tunes with a cost-model-guided tuner (XGBTuner, Step 2):
// fit a model on the configs measured so far and measure next the ones it
// ranks best.  Here the model is a ridge regression of log(time) on a few
// features of a config, refitted after every batch; each batch is the
// model's lowest predictions among the untimed points plus a few uniform
// draws (exploration); the first batch is all draws.

namespace {

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): the generator's output function on a counter.
uint64_t splitmix64(uint64_t x) {
    x += 0x9e3779b97f4a7c15ULL;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ULL;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebULL;
    return x ^ (x >> 31);
}

// Minimise |X w - y|^2 + lambda |w|^2 (X row-major n x d) by a Cholesky
// factorisation of X^T X + lambda I.  False if that matrix is not positive
// definite (lambda = 0 and X rank-deficient).
bool ridge(const double* X, const double* y, int n, int d, double lambda, double* w) {
    std::vector<double> A((size_t)d * d, 0.0), b(d, 0.0);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < d; ++j) {
            b[j] += X[(size_t)i * d + j] * y[i];
            for (int k = 0; k <= j; ++k) A[(size_t)j * d + k] += X[(size_t)i * d + j] * X[(size_t)i * d + k];
        }
    for (int j = 0; j < d; ++j) A[(size_t)j * d + j] += lambda;
    // A = L L^T, lower triangle in place
    for (int j = 0; j < d; ++j) {
        double v = A[(size_t)j * d + j];
        for (int k = 0; k < j; ++k) v -= A[(size_t)j * d + k] * A[(size_t)j * d + k];
        if (!(v > 1e-300)) return false;
        const double l = std::sqrt(v);
        A[(size_t)j * d + j] = l;
        for (int i = j + 1; i < d; ++i) {
            double u = A[(size_t)i * d + j];
            for (int k = 0; k < j; ++k) u -= A[(size_t)i * d + k] * A[(size_t)j * d + k];
            A[(size_t)i * d + j] = u / l;
        }
    }
    // L z = b, then L^T w = z
    std::vector<double> z(d);
    for (int i = 0; i < d; ++i) {
        double u = b[i];
        for (int k = 0; k < i; ++k) u -= A[(size_t)i * d + k] * z[k];
        z[i] = u / A[(size_t)i * d + i];
    }
    for (int i = d - 1; i >= 0; --i) {
        double u = z[i];
        for (int k = i + 1; k < d; ++k) u -= A[(size_t)k * d + i] * w[k];
        w[i] = u / A[(size_t)i * d + i];
    }
    return true;
}

// The next batch: up to `batch` untimed points, the lowest `batch -
// n_explore` by pred (ties by index; none when pred is null) and the rest
// drawn uniformly from the untimed points left, draw k of round r taking
// splitmix64(seed ^ (r << 32) ^ k) modulo the count.
std::vector<int> guided_select(const double* pred, int n, const std::vector<char>& timed, int batch, int n_explore,
                               uint64_t seed, int round) {
    std::vector<int> out;
    std::vector<char> taken(timed.begin(), timed.end());
    if (pred) {
        std::vector<int> cand;
        for (int i = 0; i < n; ++i)
            if (!taken[i]) cand.push_back(i);
        std::stable_sort(cand.begin(), cand.end(), [&](int a, int b) { return pred[a] < pred[b]; });
        for (int i : cand) {
            if ((int)out.size() >= batch - n_explore) break;
            out.push_back(i);
            taken[i] = 1;
        }
    }
    std::vector<int> rest;
    for (int i = 0; i < n; ++i)
        if (!taken[i]) rest.push_back(i);
    for (uint64_t k = 0; (int)out.size() < batch && !rest.empty(); ++k) {
        const uint64_t r = splitmix64(seed ^ ((uint64_t)round << 32) ^ k);
        const size_t j = (size_t)(r % rest.size());
        out.push_back(rest[j]);
        rest[j] = rest.back();
        rest.pop_back();
    }
    return out;
}

// The search: measure(i) returns the cost of point i (> 0), or <= 0 / not
// finite for a failed trial, which is left out of the fit.  Returns the
// points in the order they were measured (at most max_trials of them).
std::vector<int> guided_search(int n, int d, const double* feats, int max_trials, int batch, int n_explore,
                               uint64_t seed, double lambda, const std::function<double(int)>& measure) {
    std::vector<int> order;
    std::vector<char> timed(n, 0);
    std::vector<double> X, y;
    std::vector<double> w(d), pred(n);
    const int budget = std::min(max_trials, n);
    bool have_model = false;
    for (int round = 0; (int)order.size() < budget; ++round) {
        const int want = std::min(batch, budget - (int)order.size());
        const auto next = guided_select(have_model ? pred.data() : nullptr, n, timed, want,
                                        have_model ? std::min(n_explore, want) : want, seed, round);
        if (next.empty()) break;
        for (int i : next) {
            timed[i] = 1;
            order.push_back(i);
            const double c = measure(i);
            if (c > 0.0 && std::isfinite(c)) {
                X.insert(X.end(), feats + (size_t)i * d, feats + (size_t)(i + 1) * d);
                y.push_back(std::log(c));
            }
        }
        have_model = !y.empty() && ridge(X.data(), y.data(), (int)y.size(), d, lambda, w.data());
        if (have_model)
            for (int i = 0; i < n; ++i) {
                double v = 0.0;
                for (int j = 0; j < d; ++j) v += feats[(size_t)i * d + j] * w[j];
                pred[i] = v;
            }
    }
    return order;
}

constexpr int kFeatures = 11;

// Features of a legal config: an intercept, the analytic time estimate,
// and log sizes of the split, the stages, the channels a stage, the tile,
// the workgroup, the grid, the grid's shortfall from one workgroup per CU,
// and the LDS a workgroup holds.
void config_features(const Shape& s, const ct_tile_config& c, const Resolved& r, double* f) {
    const auto& d = r.v->desc;
    const double lg = std::log2(std::max<double>((double)r.grid, 1.0));
    f[0] = 1.0;
    f[1] = std::log2(std::max(predict_us(s, c, r), 1e-3));
    f[2] = std::log2((double)c.split_k);
    f[3] = std::log2((double)c.stages);
    f[4] = std::log2((double)c.kc);
    f[5] = std::log2((double)std::max(d.tile_m, 1));
    f[6] = std::log2((double)std::max(d.tile_n, 1));
    f[7] = std::log2((double)std::max(d.threads, 1));
    f[8] = lg;
    f[9] = std::max(0.0, std::log2((double)kNumCU) - lg);
    f[10] = std::log2(1.0 + (double)r.lds);
}

}  // namespace

int tune_guided_impl(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, int dtype,
                     int epilogue, int max_trials, int batch, unsigned long long seed, float min_repeat_ms,
                     void* stream, ct_tile_config* best_out, ct_tune_record* records, int max_records,
                     int* n_records) {
    Shape s;
    int st = make_shape(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, &s);
    if (st != CT_OK) return st;
    st = tune_args(max_trials, min_repeat_ms, best_out, records, max_records, n_records);
    if (st != CT_OK) return st;
    if (batch < 1) return fail(CT_ERR_INVALID_ARG, "batch must be >= 1");
    Space sp = space_of(s);
    TuneLog log;
    log.open(s);
    std::vector<long long> idx;
    std::vector<double> feats;
    for (long long i = 0; i < sp.size(); ++i) {
        ct_tile_config c;
        decode(sp, i, &c);
        Resolved r;
        if (log.logged(c) || !legal(s, c, &r, nullptr)) continue;
        idx.push_back(i);
        feats.resize(feats.size() + kFeatures);
        config_features(s, c, r, feats.data() + feats.size() - kFeatures);
    }
    if (idx.empty() && log.done.empty()) return fail(CT_ERR_TUNE_FAILED, "no legal config for this shape");
    TuneBench tb;
    st = tb.init(s, stream, min_repeat_ms);
    if (st != CT_OK) return st;
    std::vector<ct_tune_record> recs;
    const int n = (int)idx.size();
    const int budget = max_trials == 0 ? n : std::min(max_trials, n);
    int log_st = CT_OK;
    if (n > 0)
        (void)guided_search(n, kFeatures, feats.data(), budget, batch, std::max(1, batch / 4), seed, 1e-3,
                            [&](int i) -> double {
                                ct_tune_record rec;
                                tb.trial(idx[i], &rec);
                                recs.push_back(rec);
                                log_trial((int)recs.size(), rec);
                                const int a = log.append(s, rec);
                                if (a != CT_OK) log_st = a;
                                return rec.error_no == CT_TRIAL_OK ? (double)rec.cfg.us : -1.0;
                            });
    if (log_st != CT_OK) return log_st;
    return tune_finish(s, recs, log, best_out, records, max_records, n_records);
}

}  // namespace ct

extern "C" {

int ct_ridge_fit(const double* X, const double* y, int n, int d, double lambda, double* w) {
    if (!X || !y || !w) return fail(CT_ERR_INVALID_ARG, "X, y and w must not be NULL");
    if (n < 1 || d < 1 || d > 64) return fail(CT_ERR_INVALID_ARG, "need n >= 1 and 1 <= d <= 64");
    if (!(lambda >= 0.0)) return fail(CT_ERR_INVALID_ARG, "lambda must be >= 0");
    if (!ct::ridge(X, y, n, d, lambda, w)) return fail(CT_ERR_INVALID_ARG, "X^T X + lambda I is singular");
    return CT_OK;
}

int ct_guided_search_table(const double* feats, const double* costs, int n, int d, int max_trials, int batch,
                           int n_explore, unsigned long long seed, double lambda, int* order_out, int* n_order) {
    if (!feats || !costs || !order_out || !n_order)
        return fail(CT_ERR_INVALID_ARG, "feats, costs, order_out and n_order must not be NULL");
    if (n < 1 || d < 1 || d > 64) return fail(CT_ERR_INVALID_ARG, "need n >= 1 and 1 <= d <= 64");
    if (max_trials < 1 || batch < 1 || n_explore < 0 || n_explore > batch)
        return fail(CT_ERR_INVALID_ARG, "need max_trials >= 1, batch >= 1 and 0 <= n_explore <= batch");
    if (!(lambda >= 0.0)) return fail(CT_ERR_INVALID_ARG, "lambda must be >= 0");
    const auto order = ct::guided_search(n, d, feats, max_trials, batch, n_explore, seed, lambda,
                                         [&](int i) { return costs[i]; });
    for (size_t k = 0; k < order.size(); ++k) order_out[k] = order[k];
    *n_order = (int)order.size();
    return CT_OK;
}

int ct_conv2d_tune_guided(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad, int dtype,
                          int epilogue, int max_trials, int batch, unsigned long long seed, float min_repeat_ms,
                          void* stream, ct_tile_config* best_out, ct_tune_record* records, int max_records,
                          int* n_records) {
    return ct::tune_guided_impl(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials, batch, seed,
                                min_repeat_ms, stream, best_out, records, max_records, n_records);
}

}  // extern "C"

extern "C" int ct_conv2d_tune_order(int N, int CI, int H, int W, int CO, int KH, int KW, int stride, int pad,
                                    int dtype, int epilogue, int max_trials, long long* order_out, int max_out,
                                    int* n_out) {
    return ct::tune_order_impl(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials, order_out,
                               max_out, n_out);
}

extern "C" int ct_conv2d_tune(int N, int CI, int H, int W, int CO, int KH, int KW, int stride,
                              int pad, int dtype, int epilogue, int max_trials, float min_repeat_ms,
                              void* stream, ct_tile_config* best_out, ct_tune_record* records,
                              int max_records, int* n_records) {
    return ct::tune_impl(N, CI, H, W, CO, KH, KW, stride, pad, dtype, epilogue, max_trials,
                         min_repeat_ms, stream, best_out, records, max_records, n_records);
}
