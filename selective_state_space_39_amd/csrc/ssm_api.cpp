// C ABI of libssm_scan.so: argument validation, chunk plan, workspace layout,
// error reporting, launches.  Declared in include/ssm_scan.h.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "s6_common.h"
#include "ssd_common.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return SSM_OK;
}

constexpr int64_t kN = 16;
constexpr int64_t kChunkAlign = 32;
constexpr int64_t kMaxGrid = 65535;              // grid y (chunks) and z (batch rows)
constexpr int64_t kMaxBytes = int64_t(1) << 60;  // any single tensor
constexpr int64_t kMinChunk = kChunkAlign;      // few channels want many short chunks (1 x 2048 x 768: 32 beats 64 by 28 %)

int64_t esize(int io) { return io == SSM_BF16 ? 2 : 4; }

// a*b without overflow beyond kMaxBytes; -1 on overflow
int64_t mul_ck(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a != 0 && b > kMaxBytes / a) return -1;
    return a * b;
}

struct Range {
    const char* name;
    uintptr_t lo;
    uintptr_t hi;   // exclusive
};

bool overlap(const Range& a, const Range& b) {
    if (!a.lo || !b.lo || a.hi == a.lo || b.hi == b.lo) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

Range rng(const char* name, const void* p, int64_t bytes) {
    uintptr_t u = reinterpret_cast<uintptr_t>(p);
    return Range{name, u, u ? u + static_cast<uintptr_t>(bytes) : 0};
}

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Outputs may overlap neither an input nor each other; the workspace may
// overlap neither an input nor an output.  Inputs may share memory (they are
// only read).  Returns SSM_OK or SSM_ERR_ALIAS with the pair named.
int check_disjoint(const Range* ins, size_t nin, const Range* outs, size_t nout, const Range& ws) {
    for (size_t o = 0; o < nout; ++o) {
        for (size_t i = 0; i < nin; ++i)
            if (overlap(outs[o], ins[i])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[o].name, ins[i].name);
        for (size_t j = 0; j < o; ++j)
            if (overlap(outs[o], outs[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[o].name, outs[j].name);
    }
    for (size_t i = 0; i < nin; ++i)
        if (overlap(ws, ins[i])) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", ins[i].name);
    for (size_t o = 0; o < nout; ++o)
        if (overlap(ws, outs[o])) return fail(SSM_ERR_ALIAS, "workspace overlaps %s", outs[o].name);
    return SSM_OK;
}

struct Plan {
    int64_t chunk_len;
    int64_t n_chunks;
    int64_t ws_bytes;
};

int check_shape(int64_t batch, int64_t L, int64_t D, int64_t N, int io) {
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_DTYPE, "unknown io dtype %d (0 = f32, 1 = bf16)", io);
    if (N != kN) return fail(SSM_ERR_N, "N = %lld: this library is built for N = 16", (long long)N);
    if (batch < 1 || L < 1 || D < 1)
        return fail(SSM_ERR_SHAPE, "batch, L and D must be >= 1 (got %lld, %lld, %lld)",
                    (long long)batch, (long long)L, (long long)D);
    if (batch > kMaxGrid) return fail(SSM_ERR_SHAPE, "batch = %lld exceeds %lld", (long long)batch, (long long)kMaxGrid);
    if (D > (int64_t(1) << 30)) return fail(SSM_ERR_SHAPE, "D = %lld is too large", (long long)D);
    if (L > (int64_t(1) << 30)) return fail(SSM_ERR_SHAPE, "L = %lld is too large", (long long)L);
    int64_t e = mul_ck(mul_ck(mul_ck(batch, L), D), 4);
    int64_t s = mul_ck(mul_ck(mul_ck(batch, L), kN), 4);
    if (e < 0 || s < 0) return fail(SSM_ERR_SHAPE, "batch * L * D overflows");
    return SSM_OK;
}

// Cost model of the MI355X (1024 SIMDs) used by the automatic plan, fitted to
// measured kernel times (us, bf16 io, N = 16, steady clocks).  A pass with W
// wavefronts puts w = ceil(W / 1024) on each SIMD, and its makespan is w x
// (tokens per chunk) x (time per wavefront-token at w waves per SIMD): a lone
// wave cannot hide its own latencies, from about four waves per SIMD the VALU
// stays busy, and more rounds still shorten the per-token time a little (the
// last round's tail is a smaller share).  The carry scan costs ~4 us plus a
// per-carry term set by its traffic (or by its latency when there are few
// channels); every extra launch ~4 us.
constexpr int64_t kSimds = 1024;
constexpr int kMaxW = 12;
constexpr double kOutUs[kMaxW + 1] = {0.0,   0.36,  0.241, 0.235, 0.206, 0.200, 0.192,
                                      0.187, 0.187, 0.187, 0.180, 0.180, 0.175};   // by waves per SIMD
constexpr double kCarryUs[kMaxW + 1] = {0.0,   0.30,  0.211, 0.198, 0.169, 0.165, 0.157,
                                        0.151, 0.151, 0.151, 0.143, 0.143, 0.140};

constexpr double kWaveSetupTokens = 6.0;     // per-wavefront prologue, in token equivalents

double est_pass(int64_t waves, int64_t tokens, const double* per_token) {
    if (waves <= 0) return 0.0;
    const int64_t w = (waves + kSimds - 1) / kSimds;
    return static_cast<double>(w) * (static_cast<double>(tokens) + kWaveSetupTokens) * per_token[w < kMaxW ? w : kMaxW];
}

double est_plan(int64_t batch, int64_t D, int64_t L, int64_t len) {
    const int64_t groups = batch * ((D + 63) / 64);      // wavefronts per chunk
    const int64_t n = (L + len - 1) / len;
    double t = est_pass(groups * n, len, kOutUs);
    if (n > 1) {
        const double per_carry = std::max(static_cast<double>(batch * D) * 2.4e-5, 0.12);
        t += est_pass(groups * (n - 1), len, kCarryUs) + 4.0 + per_carry * static_cast<double>(n - 1) + 8.0;
    }
    return t;
}

// The kernels address a chunk's rows of x, delta, z and y (and their
// gradients) with 32-bit byte offsets from the chunk's first row: a chunk may
// hold at most 2 GiB at 4 bytes per element.
int64_t max_chunk_len(int64_t D) { return ((int64_t(1) << 31) - 1) / (D * 4) / kChunkAlign * kChunkAlign; }

int check_chunk_len(int64_t D, int64_t chunk_len) {
    if (chunk_len < 0 || (chunk_len > 0 && chunk_len % kChunkAlign != 0))
        return fail(SSM_ERR_SHAPE, "chunk_len = %lld must be 0 or a positive multiple of %lld",
                    (long long)chunk_len, (long long)kChunkAlign);
    const int64_t cap = max_chunk_len(D);
    if (cap < kChunkAlign)
        return fail(SSM_ERR_SHAPE, "D = %lld: even a %lld-token chunk exceeds 2 GiB", (long long)D,
                    (long long)kChunkAlign);
    if (chunk_len > cap)
        return fail(SSM_ERR_SHAPE, "chunk_len = %lld: a chunk of %lld channels would exceed 2 GiB (at most %lld tokens)",
                    (long long)chunk_len, (long long)D, (long long)cap);
    return SSM_OK;
}

// Forward workspace for n chunks: carry_S (batch, n-1, D) then carry_H
// (batch, n-1, N, D), float32, 256-byte aligned parts; -1 on overflow.
int64_t fwd_ws_bytes(int64_t batch, int64_t n_chunks, int64_t D) {
    if (n_chunks <= 1) return 0;
    const int64_t carries = mul_ck(mul_ck(batch, n_chunks - 1), D);
    if (carries < 0 || mul_ck(carries, kN * 4) < 0) return -1;
    return (carries * 4 + 255) / 256 * 256 + carries * kN * 4;
}

// max_ws >= 0: only plans whose workspace fits max_ws bytes (the automatic
// plan searches among those; an explicit chunk_len beyond it is an error).
int make_plan(int64_t batch, int64_t L, int64_t D, int64_t chunk_len, Plan& p, int64_t max_ws = -1) {
    if (int rc = check_chunk_len(D, chunk_len)) return rc;
    auto fits = [&](int64_t len) {
        const int64_t w = fwd_ws_bytes(batch, (L + len - 1) / len, D);
        return max_ws < 0 || (w >= 0 && w <= max_ws);
    };
    if (chunk_len == 0) {
        const int64_t whole = std::min((L + kChunkAlign - 1) / kChunkAlign * kChunkAlign, max_chunk_len(D));
        int64_t best = whole;
        double best_t = est_plan(batch, D, L, whole);
        bool found = fits(whole);
        for (int64_t len = whole - kChunkAlign; len >= kMinChunk; len -= kChunkAlign) {
            if ((L + len - 1) / len > kMaxGrid) break;
            if (!fits(len)) continue;
            const double t = est_plan(batch, D, L, len);
            if (!found || t < best_t * 0.999) { best_t = t; best = len; found = true; }
        }
        if (!found)
            return fail(SSM_ERR_WORKSPACE, "no chunk plan of this shape keeps its carries within %lld bytes of scratch",
                        (long long)max_ws);
        chunk_len = best;
    }
    p.chunk_len = chunk_len;
    p.n_chunks = (L + chunk_len - 1) / chunk_len;
    if (p.n_chunks > kMaxGrid)
        return fail(SSM_ERR_SHAPE, "%lld chunks exceed %lld; use a longer chunk_len",
                    (long long)p.n_chunks, (long long)kMaxGrid);
    // one workgroup per (256-channel block, batch row, chunk) in a 1-D grid
    if (batch * ((D + 255) / 256) * p.n_chunks > (int64_t(1) << 31) - 1)
        return fail(SSM_ERR_SHAPE, "batch * ceil(D / 256) * chunks exceeds the grid limit");
    p.ws_bytes = fwd_ws_bytes(batch, p.n_chunks, D);
    if (p.ws_bytes < 0) return fail(SSM_ERR_SHAPE, "workspace size overflows");
    if (max_ws >= 0 && p.ws_bytes > max_ws)
        return fail(SSM_ERR_WORKSPACE, "chunk_len = %lld needs %lld bytes of carries; the scratch holds %lld",
                    (long long)p.chunk_len, (long long)p.ws_bytes, (long long)max_ws);
    return SSM_OK;
}

// Backward plan.  The per-chunk backward kernel holds two wavefronts per
// SIMD, so it runs in rounds of 2048 wavefronts; the two carry passes hold
// six.  Measured on the 130M-layer shape (bf16): ~2.2 us per token and round
// for the backward kernel (64-token chunks: 3 rounds, 0.43 ms), and ~2.25 us
// per token for both carry passes together at one round.  The plan takes
// the chunk length (a multiple of 32) with the smallest estimate.
struct BwdPlan {
    int64_t chunk_len, n_chunks;
    int64_t off_carry_S, off_carry_H, off_rcarry_S, off_rcarry_H, off_ckpt, off_bc, off_p;
    int64_t ws_bytes;
};

double est_bwd(int64_t batch, int64_t D, int64_t L, int64_t len) {
    const int64_t groups = batch * ((D + 63) / 64);
    const int64_t n = (L + len - 1) / len;
    const double rounds = static_cast<double>((groups * n + 2 * kSimds - 1) / (2 * kSimds));
    double t = 2.2 * rounds * static_cast<double>(len + 8);
    if (n > 1) {
        const double crounds = static_cast<double>((groups * (n - 1) + 6 * kSimds - 1) / (6 * kSimds));
        t += 2.25 * crounds * static_cast<double>(len + 6) + 2.0 * (4.0 + 2.4e-5 * static_cast<double>(batch * D * (n - 1)));
    }
    return t;
}

int make_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t chunk_len, BwdPlan& p) {
    if (int rc = check_chunk_len(D, chunk_len)) return rc;
    if (chunk_len == 0) {
        const int64_t whole = std::min((L + kChunkAlign - 1) / kChunkAlign * kChunkAlign, max_chunk_len(D));
        int64_t best = whole;
        double best_t = est_bwd(batch, D, L, whole);
        for (int64_t len = whole - kChunkAlign; len >= kChunkAlign; len -= kChunkAlign) {
            if ((L + len - 1) / len > kMaxGrid) break;
            const double t = est_bwd(batch, D, L, len);
            if (t < best_t * 0.999) { best_t = t; best = len; }
        }
        chunk_len = best;
    }
    p.chunk_len = chunk_len;
    p.n_chunks = (L + chunk_len - 1) / chunk_len;
    if (p.n_chunks > kMaxGrid)
        return fail(SSM_ERR_SHAPE, "%lld chunks exceed %lld; use a longer chunk_len",
                    (long long)p.n_chunks, (long long)kMaxGrid);
    if (batch * ((D + 255) / 256) * p.n_chunks > (int64_t(1) << 31) - 1)
        return fail(SSM_ERR_SHAPE, "batch * ceil(D / 256) * chunks exceeds the grid limit");
    auto part = [](int64_t floats) { return floats < 0 ? int64_t(-1) : (floats * 4 + 255) / 256 * 256; };
    const int64_t carries = mul_ck(mul_ck(batch, p.n_chunks - 1), D);
    const int64_t ckpt = mul_ck(mul_ck(mul_ck(mul_ck(batch, p.n_chunks), chunk_len / kBwdSub), kN + 1), D);
    const int64_t bc = mul_ck(mul_ck(mul_ck(batch, L), (D + 63) / 64), 2 * kN);
    const int64_t pp = mul_ck(mul_ck(mul_ck(batch, p.n_chunks), kBwdParams), D);
    const int64_t sizes[7] = {part(carries), part(mul_ck(carries, kN)), part(carries), part(mul_ck(carries, kN)),
                              part(ckpt), part(bc), part(pp)};
    int64_t* offs[7] = {&p.off_carry_S, &p.off_carry_H, &p.off_rcarry_S, &p.off_rcarry_H, &p.off_ckpt,
                        &p.off_bc, &p.off_p};
    int64_t at = 0;
    for (int i = 0; i < 7; ++i) {
        if (sizes[i] < 0 || at > kMaxBytes - sizes[i]) return fail(SSM_ERR_SHAPE, "workspace size overflows");
        *offs[i] = at;
        at += (i < 4 && p.n_chunks == 1) ? 0 : sizes[i];
    }
    p.ws_bytes = at;
    return SSM_OK;
}

// ---------------------------------------------------------------------------
// per-kernel timing
// ---------------------------------------------------------------------------
struct TimingRec {
    const char* kernel;
    hipEvent_t begin, end;
};

std::atomic<bool> g_timing{false};
std::string g_timing_only;               // empty: every kernel
std::mutex g_timing_mu;
std::vector<TimingRec> g_recs;           // completed pairs
std::vector<hipEvent_t> g_pool;          // reusable events
thread_local hipEvent_t t_open = nullptr;
thread_local const char* t_open_name = nullptr;

hipEvent_t take_event() {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

void s6_timing_mark(const char* kernel, hipStream_t stream, bool begin) {
    if (!g_timing.load(std::memory_order_relaxed)) return;
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        if (!g_timing_only.empty() && g_timing_only != kernel) return;
    }
    hipEvent_t e = take_event();
    if (!e) return;
    if (hipEventRecord(e, stream) != hipSuccess) return;
    if (begin) {
        t_open = e;
        t_open_name = kernel;
    } else if (t_open && t_open_name == kernel) {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        g_recs.push_back(TimingRec{kernel, t_open, e});
        t_open = nullptr;
    }
}

extern "C" {

int ssm_timing_enable(int on, const char* kernel) {
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        g_timing_only = (on && kernel) ? kernel : "";
    }
    g_timing.store(on != 0);
    return ok();
}

int ssm_timing_collect(int max_kernels, const char** names, int64_t* launches, double* total_ms) {
    std::vector<TimingRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        recs.swap(g_recs);
    }
    std::vector<const char*> kn;
    std::vector<int64_t> cnt;
    std::vector<double> ms;
    int status = SSM_OK;
    for (auto& r : recs) {
        if (hipEventSynchronize(r.end) != hipSuccess) status = SSM_ERR_HIP;
        float t = 0.0f;
        if (status == SSM_OK && hipEventElapsedTime(&t, r.begin, r.end) != hipSuccess) status = SSM_ERR_HIP;
        size_t i = 0;
        while (i < kn.size() && std::strcmp(kn[i], r.kernel) != 0) ++i;
        if (i == kn.size()) { kn.push_back(r.kernel); cnt.push_back(0); ms.push_back(0.0); }
        cnt[i] += 1;
        ms[i] += t;
    }
    {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        for (auto& r : recs) { g_pool.push_back(r.begin); g_pool.push_back(r.end); }
    }
    if (status != SSM_OK) return fail(status, "timing events failed: %s", hipGetErrorString(hipGetLastError()));
    for (int i = 0; i < static_cast<int>(kn.size()) && i < max_kernels; ++i) {
        if (names) names[i] = kn[i];
        if (launches) launches[i] = cnt[i];
        if (total_ms) total_ms[i] = ms[i];
    }
    ok();
    return static_cast<int>(kn.size());
}


int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_last_error(void) { return g_err.c_str(); }

int64_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                                     int64_t chunk_len) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    Plan p;
    rc = make_plan(batch, L, D, chunk_len, p);
    if (rc) return rc;
    ok();
    return p.ws_bytes;
}

int ssm_scan_fwd_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype, int64_t chunk_len,
                      int64_t* chunk_len_out, int64_t* n_chunks_out) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    Plan p;
    rc = make_plan(batch, L, D, chunk_len, p);
    if (rc) return rc;
    if (chunk_len_out) *chunk_len_out = p.chunk_len;
    if (n_chunks_out) *n_chunks_out = p.n_chunks;
    return ok();
}

}  // extern "C"

namespace {

struct ConvArgs {
    int64_t k = 0;
    const float* w = nullptr;
    const float* b = nullptr;
    const void* init = nullptr;
    void* last = nullptr;
};

// ---------------------------------------------------------------------------
// scratch of the no-allocation entry point
// ---------------------------------------------------------------------------
// The chunk carries of ssm_scan_fwd_noalloc live in this fixed array instead
// of a caller workspace.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to a kernel.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_dev;          // device address of `scratch`, per device ordinal

// The current device's address of `scratch`, looked up on the first call on
// that device; SSM_ERR_HIP if the runtime cannot give it.
int scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) return fail(SSM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (static_cast<size_t>(dev) >= g_scratch_dev.size()) g_scratch_dev.resize(dev + 1, nullptr);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return SSM_OK;
}

// use_scratch: the carries go to the library's scratch array (the workspace
// arguments are ignored) and the plan is restricted to carries that fit it.
int scan_fwd_impl(const void* x, const void* delta, const void* z, const void* B, const void* C,
                  const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                  void* y, float* h_last, const ConvArgs& cv,
                  int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                  int64_t chunk_len, void* workspace, int64_t workspace_bytes, void* stream,
                  bool use_scratch = false) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    Plan p;
    rc = make_plan(batch, L, D, chunk_len, p, use_scratch ? kScratchBytes : -1);
    if (rc) return rc;
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
    }

    struct { const void* p; const char* n; } req[] = {
        {x, cv.k ? "xin" : "x"}, {delta, "delta"}, {B, "B"}, {C, "C"}, {A, "A"}, {Dskip, "Dskip"},
        {dt_bias, "dt_bias"}, {y, "y"}};
    for (auto& r : req)
        if (!r.p) return fail(SSM_ERR_NULL, "%s is NULL", r.n);
    if (cv.k) {
        if (cv.k < 1 || cv.k > 4) return fail(SSM_ERR_SHAPE, "conv_k = %lld: the local convolution has width 1 to 4",
                                              (long long)cv.k);
        if (!cv.w) return fail(SSM_ERR_NULL, "conv_w is NULL");
        if (!cv.b) return fail(SSM_ERR_NULL, "conv_b is NULL");
    }
    if (p.ws_bytes > 0 && !use_scratch) {
        if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL; %lld bytes needed", (long long)p.ws_bytes);
        if (workspace_bytes < p.ws_bytes)
            return fail(SSM_ERR_WORKSPACE, "workspace has %lld bytes; %lld needed",
                        (long long)workspace_bytes, (long long)p.ws_bytes);
    }

    const int64_t es = esize(io_dtype);
    struct { const void* p; int64_t a; const char* n; } al[] = {
        {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {B, 16, "B"}, {C, 16, "C"}, {y, es, "y"},
        {A, 4, "A"}, {Dskip, 4, "Dskip"}, {dt_bias, 4, "dt_bias"}, {h0, 4, "h0"}, {h_last, 4, "h_last"},
        {workspace, 16, "workspace"}, {cv.w, 4, "conv_w"}, {cv.b, 4, "conv_b"}, {cv.init, es, "conv_init"},
        {cv.last, es, "conv_last"}};
    for (auto& r : al)
        if (r.p && !aligned(r.p, r.a))
            return fail(SSM_ERR_ALIGN, "%s is not %lld-byte aligned", r.n, (long long)r.a);

    const int64_t seq = batch * L * D * es, bc = batch * L * kN * es, st = batch * D * kN * 4;
    const int64_t win = cv.k > 1 ? batch * (cv.k - 1) * D * es : 0;
    const Range ins[] = {rng("x", x, seq), rng("delta", delta, seq), rng("z", z, seq), rng("B", B, bc),
                         rng("C", C, bc), rng("A", A, D * kN * 4), rng("Dskip", Dskip, D * 4),
                         rng("dt_bias", dt_bias, D * 4), rng("h0", h0, st),
                         rng("conv_w", cv.w, D * cv.k * 4), rng("conv_b", cv.b, cv.k ? D * 4 : 0),
                         rng("conv_init", cv.init, win)};
    const Range outs[] = {rng("y", y, seq), rng("h_last", h_last, st), rng("conv_last", cv.last, win)};
    // The carry pass writes the workspace while other workgroups still read
    // the inputs, so it may share memory with nothing else.
    const Range wsr = rng("workspace", p.ws_bytes ? workspace : nullptr, p.ws_bytes);
    if (int rc2 = check_disjoint(ins, sizeof ins / sizeof ins[0], outs, sizeof outs / sizeof outs[0], wsr))
        return rc2;
    if (use_scratch && p.ws_bytes > 0) {
        if (int rc2 = scratch_on_current_device(&workspace)) return rc2;
    }

    S6ScanArgs a{};
    a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0;
    a.y = y; a.h_last = h_last;
    if (p.ws_bytes > 0) {
        const int64_t carries = batch * (p.n_chunks - 1) * D;
        a.carry_S = static_cast<float*>(workspace);
        a.carry_H = reinterpret_cast<float*>(static_cast<char*>(workspace) + (carries * 4 + 255) / 256 * 256);
    }
    a.batch = batch; a.L = L; a.D = D;
    a.chunk_len = p.chunk_len; a.n_chunks = p.n_chunks;
    a.bf16 = io_dtype == SSM_BF16;
    a.pair_loads = a.bf16 && D % 2 == 0 && aligned(x, 4) && aligned(delta, 4) && (!z || aligned(z, 4));
    a.conv_k = static_cast<int>(cv.k);
    a.conv_w = cv.w; a.conv_b = cv.b; a.conv_init = cv.init; a.conv_last = cv.last;
    hipError_t e = s6_launch_scan(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* x, const void* delta, const void* z, const void* B, const void* C,
                 const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                 void* y, float* h_last,
                 int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                 int64_t chunk_len, void* workspace, int64_t workspace_bytes, void* stream) {
    return scan_fwd_impl(x, delta, z, B, C, A, Dskip, dt_bias, h0, y, h_last, ConvArgs{}, batch, L, D, N,
                         io_dtype, chunk_len, workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_noalloc(const void* x, const void* delta, const void* z, const void* B, const void* C,
                         const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                         void* y, float* h_last,
                         int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                         int64_t chunk_len, void* stream) {
    return scan_fwd_impl(x, delta, z, B, C, A, Dskip, dt_bias, h0, y, h_last, ConvArgs{}, batch, L, D, N,
                         io_dtype, chunk_len, nullptr, 0, stream, true);
}

int ssm_conv_scan_fwd(const void* xin, const float* conv_w, const float* conv_b, int64_t conv_k,
                      const void* conv_init, const void* delta, const void* z, const void* B, const void* C,
                      const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                      void* y, float* h_last, void* conv_last,
                      int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                      int64_t chunk_len, void* workspace, int64_t workspace_bytes, void* stream) {
    if (conv_k < 1 || conv_k > 4)
        return fail(SSM_ERR_SHAPE, "conv_k = %lld: the local convolution has width 1 to 4", (long long)conv_k);
    ConvArgs cv;
    cv.k = conv_k; cv.w = conv_w; cv.b = conv_b; cv.init = conv_init; cv.last = conv_last;
    return scan_fwd_impl(xin, delta, z, B, C, A, Dskip, dt_bias, h0, y, h_last, cv, batch, L, D, N, io_dtype,
                         chunk_len, workspace, workspace_bytes, stream);
}

static int ssd_check(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype) {
    if (io_dtype != SSM_BF16)
        return fail(SSM_ERR_DTYPE, "the SSD layer takes bf16 io (its products run on bf16 matrix cores)");
    if (N != 64 && N != 128 && N != 256)
        return fail(SSM_ERR_N, "N = %lld: the SSD layer is built for N = 64, 128 or 256", (long long)N);
    if (P != 64) return fail(SSM_ERR_SHAPE, "P = %lld: the SSD layer is built for 64 channels per head", (long long)P);
    if (batch < 1 || L < 1 || H < 1)
        return fail(SSM_ERR_SHAPE, "batch, L and H must be >= 1 (got %lld, %lld, %lld)", (long long)batch,
                    (long long)L, (long long)H);
    if (L > (int64_t(1) << 30) || H > (int64_t(1) << 20) || batch * H > (int64_t(1) << 31) - 1)
        return fail(SSM_ERR_SHAPE, "shape too large");
    const int64_t elems = mul_ck(mul_ck(mul_ck(batch, L), H), P);
    if (elems < 0 || mul_ck(elems, 4) < 0) return fail(SSM_ERR_SHAPE, "batch * L * H * P overflows");
    // one batch row's x (or y, z) and B, C are addressed with 32-bit byte offsets
    if (L * H * P * 2 > (int64_t(1) << 31) - 1 || L * N * 2 > (int64_t(1) << 31) - 1)
        return fail(SSM_ERR_SHAPE, "L * H * 64 * 2 bytes exceed 2 GiB per batch row");
    // one batch row's C . B chunks (L / 64 x 8 KB) are addressed with 32-bit byte offsets too
    const int64_t nch = (L + 63) / 64;
    if (nch * 8192 > (int64_t(1) << 31) - 1 || batch * nch > (int64_t(1) << 31) - 1)
        return fail(SSM_ERR_SHAPE, "L = %lld: the per-chunk C . B workspace of a batch row exceeds 2 GiB",
                    (long long)L);
    return 0;
}

int64_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype) {
    const int rc = ssd_check(batch, L, H, P, N, io_dtype);
    if (rc) return rc;
    ok();
    return ssd_workspace_bytes(batch, L, H, N);
}

int ssm_ssd_fwd_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype, int64_t* n_segments,
                     int64_t* segment_chunks) {
    const int rc = ssd_check(batch, L, H, P, N, io_dtype);
    if (rc) return rc;
    if (!n_segments || !segment_chunks) return fail(SSM_ERR_NULL, "n_segments or segment_chunks is NULL");
    ssd_segments(batch, L, H, N, n_segments, segment_chunks);
    return ok();
}

int ssm_ssd_fwd(const void* x, const void* delta, const void* z, const void* B, const void* C,
                const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                void* y, float* h_last,
                int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int io_dtype,
                void* workspace, int64_t workspace_bytes, void* stream) {
    int rc = ssd_check(batch, L, H, P, N, io_dtype);
    if (rc) return rc;
    const int64_t elems = batch * L * H * P;
    struct { const void* p; const char* n; } req[] = {
        {x, "x"}, {delta, "delta"}, {B, "B"}, {C, "C"}, {A, "A"}, {Dskip, "Dskip"}, {dt_bias, "dt_bias"}, {y, "y"}};
    for (auto& r : req)
        if (!r.p) return fail(SSM_ERR_NULL, "%s is NULL", r.n);
    struct { const void* p; int64_t a; const char* n; } al[] = {
        {x, 16, "x"}, {z, 16, "z"}, {y, 16, "y"}, {delta, 2, "delta"}, {B, 16, "B"}, {C, 16, "C"},
        {A, 4, "A"}, {Dskip, 4, "Dskip"}, {dt_bias, 4, "dt_bias"}, {h0, 16, "h0"}, {h_last, 16, "h_last"},
        {workspace, 16, "workspace"}};
    const int64_t wsb = ssd_workspace_bytes(batch, L, H, N);
    if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL; %lld bytes needed", (long long)wsb);
    if (workspace_bytes < wsb)
        return fail(SSM_ERR_WORKSPACE, "workspace has %lld bytes; %lld needed", (long long)workspace_bytes,
                    (long long)wsb);
    for (auto& r : al)
        if (r.p && !aligned(r.p, r.a))
            return fail(SSM_ERR_ALIGN, "%s is not %lld-byte aligned", r.n, (long long)r.a);
    const int64_t seq = elems * 2, st = batch * H * P * N * 4, bc = batch * L * N * 2;
    const Range ins[] = {rng("x", x, seq), rng("delta", delta, batch * L * H * 2), rng("z", z, seq),
                         rng("B", B, bc), rng("C", C, bc), rng("A", A, H * 4), rng("Dskip", Dskip, H * 4),
                         rng("dt_bias", dt_bias, H * 4), rng("h0", h0, st)};
    const Range outs[] = {rng("y", y, seq), rng("h_last", h_last, st)};
    if (int rc2 = check_disjoint(ins, sizeof ins / sizeof ins[0], outs, 2, rng("workspace", workspace, wsb)))
        return rc2;
    SsdArgs a{};
    a.gram = static_cast<uint16_t*>(workspace);
    ssd_segments(batch, L, H, N, &a.n_seg, &a.seg_chunks);
    if (a.n_seg > 1) {
        char* wsc = static_cast<char*>(workspace);
        a.seg_state = reinterpret_cast<float*>(wsc + ssd_seg_state_offset(batch, L));
        a.seg_decay = reinterpret_cast<float*>(wsc + ssd_seg_decay_offset(batch, L, H, N, a.n_seg));
    }
    a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C; a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias;
    a.h0 = h0; a.y = y; a.h_last = h_last;
    a.batch = batch; a.L = L; a.H = H; a.N = N;
    hipError_t e = ssd_launch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                                     int64_t chunk_len) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    BwdPlan p;
    rc = make_bwd_plan(batch, L, D, chunk_len, p);
    if (rc) return rc;
    ok();
    return p.ws_bytes;
}

int ssm_scan_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype, int64_t chunk_len,
                      int64_t* chunk_len_out, int64_t* n_chunks_out) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    BwdPlan p;
    rc = make_bwd_plan(batch, L, D, chunk_len, p);
    if (rc) return rc;
    if (chunk_len_out) *chunk_len_out = p.chunk_len;
    if (n_chunks_out) *n_chunks_out = p.n_chunks;
    return ok();
}

int ssm_scan_bwd(const void* x, const void* delta, const void* z, const void* B, const void* C,
                 const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                 const void* dout, const float* dh_last,
                 void* dx, void* ddelta, void* dz, float* dB, float* dC,
                 float* dA, float* dDskip, float* ddt_bias, float* dh0,
                 int64_t batch, int64_t L, int64_t D, int64_t N, int io_dtype,
                 int64_t chunk_len, void* workspace, int64_t workspace_bytes, void* stream) {
    int rc = check_shape(batch, L, D, N, io_dtype);
    if (rc) return rc;
    BwdPlan p;
    rc = make_bwd_plan(batch, L, D, chunk_len, p);
    if (rc) return rc;

    struct { const void* p; const char* n; } req[] = {
        {x, "x"}, {delta, "delta"}, {B, "B"}, {C, "C"}, {A, "A"}, {Dskip, "Dskip"}, {dt_bias, "dt_bias"},
        {dout, "dout"}, {dx, "dx"}, {ddelta, "ddelta"}, {dB, "dB"}, {dC, "dC"}, {dA, "dA"},
        {dDskip, "dDskip"}, {ddt_bias, "ddt_bias"}};
    for (auto& r : req)
        if (!r.p) return fail(SSM_ERR_NULL, "%s is NULL", r.n);
    if ((z == nullptr) != (dz == nullptr))
        return fail(SSM_ERR_NULL, "z and dz must both be given (gated) or both be NULL (ungated)");
    if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace is NULL; %lld bytes needed", (long long)p.ws_bytes);
    if (workspace_bytes < p.ws_bytes)
        return fail(SSM_ERR_WORKSPACE, "workspace has %lld bytes; %lld needed", (long long)workspace_bytes,
                    (long long)p.ws_bytes);

    const int64_t es = esize(io_dtype);
    struct { const void* p; int64_t a; const char* n; } al[] = {
        {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {B, 16, "B"}, {C, 16, "C"}, {dout, es, "dout"},
        {dx, es, "dx"}, {ddelta, es, "ddelta"}, {dz, es, "dz"}, {A, 4, "A"}, {Dskip, 4, "Dskip"},
        {dt_bias, 4, "dt_bias"}, {h0, 4, "h0"}, {dh_last, 4, "dh_last"}, {dB, 4, "dB"}, {dC, 4, "dC"},
        {dA, 4, "dA"}, {dDskip, 4, "dDskip"}, {ddt_bias, 4, "ddt_bias"}, {dh0, 4, "dh0"},
        {workspace, 256, "workspace"}};
    for (auto& r : al)
        if (r.p && !aligned(r.p, r.a))
            return fail(SSM_ERR_ALIGN, "%s is not %lld-byte aligned", r.n, (long long)r.a);

    const int64_t seq = batch * L * D * es, bc = batch * L * kN * es, st = batch * D * kN * 4;
    const int64_t bcf = batch * L * kN * 4;
    const Range ins[] = {rng("x", x, seq), rng("delta", delta, seq), rng("z", z, seq), rng("B", B, bc),
                         rng("C", C, bc), rng("A", A, D * kN * 4), rng("Dskip", Dskip, D * 4),
                         rng("dt_bias", dt_bias, D * 4), rng("h0", h0, st), rng("dout", dout, seq),
                         rng("dh_last", dh_last, st)};
    const Range outs[] = {rng("dx", dx, seq), rng("ddelta", ddelta, seq), rng("dz", dz, seq),
                          rng("dB", dB, bcf), rng("dC", dC, bcf), rng("dA", dA, D * kN * 4),
                          rng("dDskip", dDskip, D * 4), rng("ddt_bias", ddt_bias, D * 4), rng("dh0", dh0, st)};
    const Range wsr = rng("workspace", workspace, p.ws_bytes);
    if (int rc2 = check_disjoint(ins, sizeof ins / sizeof ins[0], outs, sizeof outs / sizeof outs[0], wsr))
        return rc2;

    S6BwdArgs a{};
    a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C; a.dout = dout;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.h0 = h0; a.dh_last = dh_last;
    a.dx = dx; a.ddelta = ddelta; a.dz = dz; a.dB = dB; a.dC = dC;
    a.dA = dA; a.dDskip = dDskip; a.ddt_bias = ddt_bias; a.dh0 = dh0;
    char* ws = static_cast<char*>(workspace);
    if (p.n_chunks > 1) {
        a.carry_S = reinterpret_cast<float*>(ws + p.off_carry_S);
        a.carry_H = reinterpret_cast<float*>(ws + p.off_carry_H);
        a.rcarry_S = reinterpret_cast<float*>(ws + p.off_rcarry_S);
        a.rcarry_H = reinterpret_cast<float*>(ws + p.off_rcarry_H);
    }
    a.ckpt = reinterpret_cast<float*>(ws + p.off_ckpt);
    a.part_bc = reinterpret_cast<float*>(ws + p.off_bc);
    a.part_p = reinterpret_cast<float*>(ws + p.off_p);
    a.batch = batch; a.L = L; a.D = D;
    a.chunk_len = p.chunk_len; a.n_chunks = p.n_chunks;
    a.bf16 = io_dtype == SSM_BF16;
    a.pair_loads = a.bf16 && D % 2 == 0 && aligned(x, 4) && aligned(delta, 4) && aligned(dout, 4) &&
                   (!z || aligned(z, 4));
    hipError_t e = s6_launch_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

int state_update_impl(float* h, const void* x, const void* delta, const void* z, const void* B, const void* C,
                      const float* A, const float* Dskip, const float* dt_bias, void* y,
                      int64_t conv_k, const float* conv_w, const float* conv_b, void* conv_state,
                      int64_t batch, int64_t D, int64_t N, int io_dtype, void* stream) {
    int rc = check_shape(batch, 1, D, N, io_dtype);
    if (rc) return rc;
    struct { const void* p; const char* n; } req[] = {
        {h, "h"}, {x, conv_k ? "xin" : "x"}, {delta, "delta"}, {B, "B"}, {C, "C"}, {A, "A"}, {Dskip, "Dskip"},
        {dt_bias, "dt_bias"}, {y, "y"}};
    for (auto& r : req)
        if (!r.p) return fail(SSM_ERR_NULL, "%s is NULL", r.n);
    if (conv_k) {
        if (conv_k < 1 || conv_k > 4)
            return fail(SSM_ERR_SHAPE, "conv_k = %lld: the local convolution has width 1 to 4", (long long)conv_k);
        if (!conv_w) return fail(SSM_ERR_NULL, "conv_w is NULL");
        if (!conv_b) return fail(SSM_ERR_NULL, "conv_b is NULL");
        if (conv_k > 1 && !conv_state) return fail(SSM_ERR_NULL, "conv_state is NULL");
    }
    const int64_t es = esize(io_dtype);
    struct { const void* p; int64_t a; const char* n; } al[] = {
        {h, 16, "h"}, {x, es, "x"}, {delta, es, "delta"}, {z, es, "z"}, {B, es, "B"}, {C, es, "C"},
        {y, es, "y"}, {A, 4, "A"}, {Dskip, 4, "Dskip"}, {dt_bias, 4, "dt_bias"}, {conv_w, 4, "conv_w"},
        {conv_b, 4, "conv_b"}, {conv_state, es, "conv_state"}};
    for (auto& r : al)
        if (r.p && !aligned(r.p, r.a))
            return fail(SSM_ERR_ALIGN, "%s is not %lld-byte aligned", r.n, (long long)r.a);
    const int64_t tok = batch * D * es, bc = batch * kN * es, st = batch * D * kN * 4;
    const int64_t cs = conv_k > 1 ? batch * (conv_k - 1) * D * es : 0;
    const Range ins[] = {rng("x", x, tok), rng("delta", delta, tok), rng("z", z, tok), rng("B", B, bc),
                         rng("C", C, bc), rng("A", A, D * kN * 4), rng("Dskip", Dskip, D * 4),
                         rng("dt_bias", dt_bias, D * 4), rng("conv_w", conv_w, D * conv_k * 4),
                         rng("conv_b", conv_b, conv_k ? D * 4 : 0)};
    const Range outs[] = {rng("h", h, st), rng("y", y, tok), rng("conv_state", conv_state, cs)};
    for (auto& o : outs)
        for (auto& i : ins)
            if (overlap(o, i)) return fail(SSM_ERR_ALIAS, "%s overlaps %s", o.name, i.name);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], outs[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);

    S6StepArgs a{};
    a.h = h; a.x = x; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.y = y;
    a.batch = batch; a.D = D; a.bf16 = io_dtype == SSM_BF16;
    a.conv_k = static_cast<int>(conv_k); a.conv_w = conv_w; a.conv_b = conv_b; a.conv_state = conv_state;
    hipError_t e = s6_launch_step(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int ssm_state_update(float* h, const void* x, const void* delta, const void* z, const void* B, const void* C,
                     const float* A, const float* Dskip, const float* dt_bias, void* y,
                     int64_t batch, int64_t D, int64_t N, int io_dtype, void* stream) {
    return state_update_impl(h, x, delta, z, B, C, A, Dskip, dt_bias, y, 0, nullptr, nullptr, nullptr, batch, D, N,
                             io_dtype, stream);
}

int ssm_conv_state_update(float* h, void* conv_state, const void* xin, const float* conv_w, const float* conv_b,
                          int64_t conv_k, const void* delta, const void* z, const void* B, const void* C,
                          const float* A, const float* Dskip, const float* dt_bias, void* y,
                          int64_t batch, int64_t D, int64_t N, int io_dtype, void* stream) {
    if (conv_k < 1 || conv_k > 4)
        return fail(SSM_ERR_SHAPE, "conv_k = %lld: the local convolution has width 1 to 4", (long long)conv_k);
    return state_update_impl(h, xin, delta, z, B, C, A, Dskip, dt_bias, y, conv_k, conv_w, conv_b, conv_state,
                             batch, D, N, io_dtype, stream);
}

}  // extern "C"
