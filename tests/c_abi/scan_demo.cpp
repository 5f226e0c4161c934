// A consumer of libssm_scan's C ABI with no Python and no torch.
//
//     scan_demo DIR
//
// Device buffers come from hipMalloc.  The program runs one ssm_scan_fwd over a
// small batch of whole sequences (float32 io, gated, from an h0, keeping h_L,
// 64-token chunks with a ragged last one), then one ssm_state_update step
// against the returned h_L, and checks that a bad call (N = 8) is refused with
// SSM_ERR_N and a message.  Inputs and outputs go to DIR as raw little-endian
// float32 files, so a test can recompute every output from the same bits.
// Exit status 0 on success, 1 on any failure (the reason on stderr).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "ssm_scan.h"

namespace {

constexpr int64_t kBatch = 2, kL = 300, kD = 40, kN = 16, kChunk = 64;

bool check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return false;
}

// deterministic pseudo-random values in [lo, hi): a 32-bit LCG per tensor
std::vector<float> fill(size_t n, uint32_t seed, float lo, float hi) {
    std::vector<float> v(n);
    uint32_t s = seed;
    for (auto& x : v) {
        s = s * 1664525u + 1013904223u;
        x = lo + (hi - lo) * static_cast<float>(s >> 8) / 16777216.0f;
    }
    return v;
}

struct Dev {
    float* p = nullptr;
    size_t n = 0;
    bool alloc(size_t count) {
        n = count;
        return check_hip(hipMalloc(&p, count * sizeof(float)), "hipMalloc");
    }
    bool put(const std::vector<float>& h) {
        return check_hip(hipMemcpy(p, h.data(), n * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy H2D");
    }
    bool get(std::vector<float>& h) const {
        h.resize(n);
        return check_hip(hipMemcpy(h.data(), p, n * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy D2H");
    }
    ~Dev() {
        if (p) (void)hipFree(p);
    }
};

bool save(const std::string& dir, const char* name, const std::vector<float>& v) {
    const std::string path = dir + "/" + name + ".f32";
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) {
        std::fprintf(stderr, "cannot write %s\n", path.c_str());
        return false;
    }
    const bool ok = std::fwrite(v.data(), sizeof(float), v.size(), f) == v.size();
    std::fclose(f);
    return ok;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    if (ssm_abi_version() != SSM_ABI_VERSION) {
        std::fprintf(stderr, "library ABI %d, header %d\n", ssm_abi_version(), SSM_ABI_VERSION);
        return 1;
    }
    const size_t seq = kBatch * kL * kD, bc = kBatch * kL * kN, st = kBatch * kD * kN;
    std::vector<float> x = fill(seq, 1, -2.0f, 2.0f), delta = fill(seq, 2, -1.5f, 1.0f), z = fill(seq, 3, -3.0f, 3.0f);
    std::vector<float> B = fill(bc, 4, -1.5f, 1.5f), C = fill(bc, 5, -1.5f, 1.5f);
    std::vector<float> A = fill(kD * kN, 6, -4.0f, -0.05f), Dskip = fill(kD, 7, 0.5f, 1.5f);
    std::vector<float> dt_bias = fill(kD, 8, -5.0f, -2.0f), h0 = fill(st, 9, -1.0f, 1.0f);
    std::vector<float> x1 = fill(kBatch * kD, 10, -2.0f, 2.0f), d1 = fill(kBatch * kD, 11, -1.5f, 1.0f);
    std::vector<float> z1 = fill(kBatch * kD, 12, -3.0f, 3.0f);
    std::vector<float> B1 = fill(kBatch * kN, 13, -1.5f, 1.5f), C1 = fill(kBatch * kN, 14, -1.5f, 1.5f);

    Dev dx, ddelta, dz, dB, dC, dA, dD, dbias, dh0, dy, dh, dx1, dd1, dz1, dB1, dC1, dy1;
    if (!(dx.alloc(seq) && ddelta.alloc(seq) && dz.alloc(seq) && dB.alloc(bc) && dC.alloc(bc) && dA.alloc(kD * kN) &&
          dD.alloc(kD) && dbias.alloc(kD) && dh0.alloc(st) && dy.alloc(seq) && dh.alloc(st) &&
          dx1.alloc(kBatch * kD) && dd1.alloc(kBatch * kD) && dz1.alloc(kBatch * kD) && dB1.alloc(kBatch * kN) &&
          dC1.alloc(kBatch * kN) && dy1.alloc(kBatch * kD)))
        return 1;
    if (!(dx.put(x) && ddelta.put(delta) && dz.put(z) && dB.put(B) && dC.put(C) && dA.put(A) && dD.put(Dskip) &&
          dbias.put(dt_bias) && dh0.put(h0) && dx1.put(x1) && dd1.put(d1) && dz1.put(z1) && dB1.put(B1) &&
          dC1.put(C1)))
        return 1;

    // the scan: workspace from the query, null stream
    const int64_t ws_bytes = ssm_scan_fwd_workspace_bytes(kBatch, kL, kD, kN, SSM_F32, kChunk);
    if (ws_bytes < 0) {
        std::fprintf(stderr, "workspace query: %s\n", ssm_last_error());
        return 1;
    }
    void* ws = nullptr;
    if (ws_bytes > 0 && !check_hip(hipMalloc(&ws, static_cast<size_t>(ws_bytes)), "hipMalloc workspace")) return 1;
    int rc = ssm_scan_fwd(dx.p, ddelta.p, dz.p, dB.p, dC.p, dA.p, dD.p, dbias.p, dh0.p, dy.p, dh.p, kBatch, kL, kD,
                          kN, SSM_F32, kChunk, ws, ws_bytes, nullptr);
    if (rc != SSM_OK) {
        std::fprintf(stderr, "ssm_scan_fwd: %d %s\n", rc, ssm_last_error());
        return 1;
    }
    if (!check_hip(hipDeviceSynchronize(), "scan")) return 1;
    std::vector<float> y, hL;
    if (!(dy.get(y) && dh.get(hL))) return 1;

    // one decode step against h_L, in place
    rc = ssm_state_update(dh.p, dx1.p, dd1.p, dz1.p, dB1.p, dC1.p, dA.p, dD.p, dbias.p, dy1.p, kBatch, kD, kN,
                          SSM_F32, nullptr);
    if (rc != SSM_OK) {
        std::fprintf(stderr, "ssm_state_update: %d %s\n", rc, ssm_last_error());
        return 1;
    }
    if (!check_hip(hipDeviceSynchronize(), "decode")) return 1;
    std::vector<float> y1, h1;
    if (!(dy1.get(y1) && dh.get(h1))) return 1;

    // a refused call: N = 8 enqueues nothing and says why
    rc = ssm_scan_fwd(dx.p, ddelta.p, dz.p, dB.p, dC.p, dA.p, dD.p, dbias.p, dh0.p, dy.p, dh.p, kBatch, kL, kD, 8,
                      SSM_F32, kChunk, ws, ws_bytes, nullptr);
    if (rc != SSM_ERR_N || std::string(ssm_last_error()).empty()) {
        std::fprintf(stderr, "N = 8 should be SSM_ERR_N with a message, got %d\n", rc);
        return 1;
    }
    if (ws) (void)hipFree(ws);

    const bool ok = save(dir, "x", x) && save(dir, "delta", delta) && save(dir, "z", z) && save(dir, "B", B) &&
                    save(dir, "C", C) && save(dir, "A", A) && save(dir, "Dskip", Dskip) &&
                    save(dir, "dt_bias", dt_bias) && save(dir, "h0", h0) && save(dir, "y", y) &&
                    save(dir, "h_last", hL) && save(dir, "x1", x1) && save(dir, "delta1", d1) &&
                    save(dir, "z1", z1) && save(dir, "B1", B1) && save(dir, "C1", C1) && save(dir, "y1", y1) &&
                    save(dir, "h1", h1);
    if (!ok) return 1;
    std::printf("scan_demo ok: batch %lld, L %lld, D %lld, N %lld, chunk %lld\n", (long long)kBatch, (long long)kL,
                (long long)kD, (long long)kN, (long long)kChunk);
    return 0;
}
