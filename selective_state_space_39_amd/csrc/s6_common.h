// Shared device helpers and launcher declarations for the gfx950 selective scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s6 {

constexpr int kN = 16;          // state size (Mamba-1)
constexpr int kWave = 64;       // CDNA wavefront
constexpr int kBlock = 256;     // 4 waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// io element access: float32, or bfloat16 carried as 16-bit patterns
// ---------------------------------------------------------------------------
struct F32 {
    using T = float;
    static __device__ __forceinline__ float load(const float* p, uint32_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, uint32_t i, float v) { p[i] = v; }
};

struct BF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const uint16_t* p, uint32_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);   // exact widening
    }
    static __device__ __forceinline__ void store(uint16_t* p, uint32_t i, float v) {
        __bf16 b = static_cast<__bf16>(v);                            // round to nearest even
        p[i] = __builtin_bit_cast(uint16_t, b);
    }
};

// ---------------------------------------------------------------------------
// elementwise maps
// ---------------------------------------------------------------------------

// softplus(v) = max(v, 0) + log1p(exp(-|v|)).  log1p(e) is taken as
// log(u) + (e - (u - 1)) with u = fl(1 + e): the second term restores the
// part of e that rounding 1 + e dropped, which matters for small steps.
__device__ __forceinline__ float softplus(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
    const float u = 1.0f + e;
    const float lost = e - (u - 1.0f);
    return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, lost);
}

// softplus(v) and its derivative sigmoid(v), sharing exp(-|v|):
// sigmoid(v) = 1 / (1 + e) for v >= 0, e / (1 + e) below.
__device__ __forceinline__ float softplus_sig(float v, float& sig) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
    const float u = 1.0f + e;
    const float lost = e - (u - 1.0f);
    const float r = __builtin_amdgcn_rcpf(u);
    sig = v >= 0.0f ? r : e * r;
    return fmaxf(v, 0.0f) + fmaf(__builtin_amdgcn_logf(u), kLn2, lost);
}

// silu(z) = z / (1 + exp(-z)); exp overflow gives 1/inf = 0 and a signed zero.
__device__ __forceinline__ float silu(float z) {
    const float e = __builtin_amdgcn_exp2f(-z * kLog2e);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace s6

// ---------------------------------------------------------------------------
// launchers (host side, defined in s6_kernels.hip)
// ---------------------------------------------------------------------------
struct S6ScanArgs {
    const void* x; const void* delta; const void* z;
    const void* B; const void* C;
    const float* A; const float* Dskip; const float* dt_bias;
    const float* h0;
    void* y; float* h_last;
    float* carry_S;    // (batch, n_chunks - 1, D)
    float* carry_H;    // (batch, n_chunks - 1, N, D)
    int64_t batch, L, D;
    int64_t chunk_len, n_chunks;
    int bf16;
    int pair_loads;    // bf16 with D even and x, delta, z 4-byte aligned: dword loads
    // local convolution before the scan (conv_k = 0: none; x is then the scan input itself)
    int conv_k;                    // width 1..4
    const float* conv_w;           // (D, conv_k)
    const float* conv_b;           // (D)
    const void* conv_init;         // (batch, conv_k - 1, D) io inputs before the sequence, or NULL (zeros)
    void* conv_last;               // (batch, conv_k - 1, D) io output: the last inputs, or NULL
};

struct S6StepArgs {
    float* h;
    const void* x; const void* delta; const void* z;
    const void* B; const void* C;
    const float* A; const float* Dskip; const float* dt_bias;
    void* y;
    int64_t batch, D;
    int bf16;
    // local convolution before the step (conv_k = 0: none; x is then the step input itself)
    int conv_k;
    const float* conv_w;           // (D, conv_k)
    const float* conv_b;           // (D)
    void* conv_state;              // (batch, conv_k - 1, D) io: the last inputs, shifted in place
};

struct S6BwdArgs {
    const void* x; const void* delta; const void* z;
    const void* B; const void* C; const void* dout;
    const float* A; const float* Dskip; const float* dt_bias;
    const float* h0; const float* dh_last;
    void* dx; void* ddelta; void* dz;
    float* dB; float* dC;            // (batch, L, N)
    float* dA; float* dDskip; float* ddt_bias;
    float* dh0;                      // (batch, D, N) or NULL
    // workspace
    float* carry_S; float* carry_H;      // forward carries / starting states, (batch, n-1, [N,] D)
    float* rcarry_S; float* rcarry_H;    // adjoint carries / incoming adjoints, same shapes
    float* ckpt;                         // (batch, n, chunk_len / sub, N + 1, D) local sub-chunk states and step sums
    float* part_bc;                      // (batch, L, ceil(D / 64), 2N) per-wavefront dB | dC sums
    float* part_p;                       // (batch, n, N + 2, D) per-chunk dA | dDskip | ddt_bias
    int64_t batch, L, D;
    int64_t chunk_len, n_chunks;
    int bf16;
    int pair_loads;
};

// In-order combine of chunk carries (S = sum of Delta, H = state), in place.
struct S6FoldArgs {
    const float* A;
    const float* init;   // (batch, D, N) starting value, NULL = zero
    float* S;            // (batch, ncar, D)
    float* H;            // (batch, ncar, N, D); overwritten with the prefixes
    int64_t batch, D, ncar;
    int reverse;         // fold carries ncar-1 .. 0 instead of 0 .. ncar-1
};

// Optional per-launch timing (ssm_timing_enable): called before and after
// every kernel launch with the launch's stream.
void s6_timing_mark(const char* kernel, hipStream_t stream, bool begin);

hipError_t s6_launch_scan(const S6ScanArgs& a, hipStream_t stream);
void s6_launch_fold(const S6FoldArgs& f, const char* name, hipStream_t stream);
void s6_launch_fold2(const S6FoldArgs& f0, const S6FoldArgs& f1, const char* name, hipStream_t stream);
void s6_launch_chunk_carry(const S6ScanArgs& a, hipStream_t stream);   // chunks 0 .. n-2
hipError_t s6_launch_bwd(const S6BwdArgs& a, hipStream_t stream);
constexpr int kBwdSub = 4;           // tokens per backward sub-chunk (states kept in registers)
constexpr int kBwdParams = 18;       // dA (16), dDskip, ddt_bias partials per lane and chunk
hipError_t s6_launch_step(const S6StepArgs& a, hipStream_t stream);
