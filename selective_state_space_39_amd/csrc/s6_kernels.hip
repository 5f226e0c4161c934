// gfx950 kernels of the selective scan (S6) forward and its decode step.
//
// Work layout of the scans: one lane per channel d, all 16 state values of
// that channel in VGPRs, a wavefront = 64 consecutive channels of one batch
// row, a workgroup = 4 such wavefronts.  B_t and C_t are the same for every
// channel of a batch row ("Mamba", "Selectivity": B and C are functions of
// the token), so a wavefront reads them with scalar loads and the state
// updates take them as SGPR operands: no LDS, no per-lane copies.
//
// Long sequences are cut into chunks ("Mamba", "Scan View": the recurrence
// is an associative scan over the pairs (Abar_t, Bbar_t x_t)):
//   1. s6_chunk_carry: every chunk but the last scans from a zero state and
//      writes its carry (S = sum of Delta, H = end state) per channel.
//   2. s6_chunk_out: every chunk folds the carries of the chunks before it,
//      in order, from h0 -- (S1,H1) then (S2,H2) = (S1+S2, exp(A S2) H1 + H2),
//      where exp(A * sum Delta) is exactly the product of the chunk's Abar --
//      then rescans its tokens from that true starting state, writing the
//      gated output; the last chunk also writes h_L.
// The (batch, L, D, N) states are never written to memory ("DL0170 Mamba
// Selective SSM vs Attention", engineering paragraph after Figure 1).

#include "s6_common.h"

namespace s6 {

// B_t or C_t (16 values) of one token.  The address is wave-uniform and the
// pointer is in the constant address space, so these are scalar loads
// (s_load_dwordx8 / x16) and the values are SGPR operands of the state update.
template <class IO> struct RowBC;

typedef const __attribute__((address_space(4))) uint32_t cu32;

template <> struct RowBC<BF16> {
    uint32_t w[8];    // 16 bf16 values, two per word
    __device__ __forceinline__ void load(const uint16_t* base, int64_t row) {
        cu32* p = (cu32*)(base + row * kN);
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = p[i];
    }
    __device__ __forceinline__ float get(int n) const {
        return (n & 1) ? bf16_hi(w[n >> 1]) : bf16_lo(w[n >> 1]);
    }
};

template <> struct RowBC<F32> {
    uint32_t w[16];
    __device__ __forceinline__ void load(const float* base, int64_t row) {
        cu32* p = (cu32*)(base + row * kN);
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = p[i];
    }
    __device__ __forceinline__ float get(int n) const { return __uint_as_float(w[n]); }
};

// Scalar loads can return out of order, so any wait on them is a wait for all
// of them.  Waiting here, before the next token's B/C loads are issued, keeps
// those loads in flight across the whole token instead of stalling on them.
__device__ __forceinline__ void lgkm_wait_all() {
    __builtin_amdgcn_s_waitcnt(0xC07F);     // vmcnt/expcnt untouched, lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
}

struct Lane {
    uint32_t d;     // channel; lanes past D take D-1 and duplicate its (identical) results
};

// The wavefront index is made wave-uniform explicitly, so the early exit and
// every bound derived after it stay in SGPRs.
__device__ __forceinline__ bool lane_setup(int64_t D, Lane& ln) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kBlock + wave * kWave;
    if (first >= D) return false;                 // whole wavefront past the last channel
    const int64_t d = first + (threadIdx.x & (kWave - 1));
    ln.d = static_cast<uint32_t>(d < D ? d : D - 1);
    return true;
}

// Tokens of x, delta (and z) are prefetched kRing tokens ahead into a ring of
// registers; the token loop is unrolled by kRing so every ring slot is read
// and refilled in place.  Tokens past the chunk end are masked (Delta = 0
// leaves the state unchanged) and not stored.
constexpr int kRing = 8;

// ---------------------------------------------------------------------------
// phase 1: chunk carries
// ---------------------------------------------------------------------------
template <class IO>
__global__ __launch_bounds__(kBlock) void s6_chunk_carry(S6ScanArgs a) {
    using T = typename IO::T;
    Lane ln;
    if (!lane_setup(a.D, ln)) return;
    const int64_t D = a.D, L = a.L;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    const int t0 = static_cast<int>(c * a.chunk_len);
    const int t1 = t0 + static_cast<int>(a.chunk_len);   // never the ragged last chunk
    const T* X = static_cast<const T*>(a.x) + b * L * D;
    const T* DL = static_cast<const T*>(a.delta) + b * L * D;
    const T* Bm = static_cast<const T*>(a.B);

    float A2[kN], h[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) { A2[n] = a.A[ln.d * kN + n] * kLog2e; h[n] = 0.0f; }
    const float bias = a.dt_bias[ln.d];
    float S = 0.0f;

    float rx[kRing], rd[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        const int t = t0 + j < t1 ? t0 + j : t1 - 1;
        rx[j] = IO::load(X + t * D, ln.d);
        rd[j] = IO::load(DL + t * D, ln.d);
    }
    const int64_t brow = b * L;
    RowBC<IO> bc[2];
    bc[0].load(Bm, brow + t0);
    for (int tb = t0; tb < t1; tb += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int t = tb + j;
            const float xv = rx[j], dv = rd[j];
            const int tn = t + kRing < t1 ? t + kRing : t1 - 1;
            rx[j] = IO::load(X + tn * D, ln.d);
            rd[j] = IO::load(DL + tn * D, ln.d);
            const int tb1 = t + 1 < t1 ? t + 1 : t1 - 1;
            lgkm_wait_all();
            bc[(j + 1) & 1].load(Bm, brow + tb1);
            const RowBC<IO>& Bv = bc[j & 1];

            // chunk_len is a multiple of kRing, so every token here is in range
            const float dt = softplus(dv + bias);
            const float dx = dt * xv;
            S += dt;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float dA = __builtin_amdgcn_exp2f(dt * A2[n]);
                h[n] = fmaf(dA, h[n], dx * Bv.get(n));
            }
        }
    }
    const int64_t cs = (b * (a.n_chunks - 1) + c);
    a.carry_S[cs * D + ln.d] = S;
#pragma unroll
    for (int n = 0; n < kN; ++n) a.carry_H[(cs * kN + n) * D + ln.d] = h[n];
}

// ---------------------------------------------------------------------------
// phase 2 + 3: fold carries, rescan, write gated output (and h_L)
// ---------------------------------------------------------------------------
template <class IO, bool GATED>
__global__ __launch_bounds__(kBlock) void s6_chunk_out(S6ScanArgs a) {
    using T = typename IO::T;
    Lane ln;
    if (!lane_setup(a.D, ln)) return;
    const int64_t D = a.D, L = a.L;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    const int t0 = static_cast<int>(c * a.chunk_len);
    const int t1 = static_cast<int>((t0 + a.chunk_len < L) ? t0 + a.chunk_len : L);
    const T* X = static_cast<const T*>(a.x) + b * L * D;
    const T* DL = static_cast<const T*>(a.delta) + b * L * D;
    const T* Z = GATED ? static_cast<const T*>(a.z) + b * L * D : nullptr;
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    T* Y = static_cast<T*>(a.y) + b * L * D;

    float A2[kN], h[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) A2[n] = a.A[ln.d * kN + n] * kLog2e;
    if (a.h0) {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = a.h0[(b * D + ln.d) * kN + n];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    }
    // fold the carries of chunks 0 .. c-1, in order, into the starting state
    for (int64_t cc = 0; cc < c; ++cc) {
        const int64_t cs = b * (a.n_chunks - 1) + cc;
        const float S = a.carry_S[cs * D + ln.d];
#pragma unroll
        for (int n = 0; n < kN; ++n)
            h[n] = fmaf(__builtin_amdgcn_exp2f(A2[n] * S), h[n], a.carry_H[(cs * kN + n) * D + ln.d]);
    }
    const float bias = a.dt_bias[ln.d];
    const float Dd = a.Dskip[ln.d];

    float rx[kRing], rd[kRing], rz[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        const int t = t0 + j < t1 ? t0 + j : t1 - 1;
        rx[j] = IO::load(X + t * D, ln.d);
        rd[j] = IO::load(DL + t * D, ln.d);
        rz[j] = GATED ? IO::load(Z + t * D, ln.d) : 0.0f;
    }
    const int64_t brow = b * L;
    RowBC<IO> bq[2], cq[2];
    bq[0].load(Bm, brow + t0);
    cq[0].load(Cm, brow + t0);
    for (int tb = t0; tb < t1; tb += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int t = tb + j;
            const bool valid = t < t1;                // wave-uniform
            const float xv = rx[j], dv = rd[j], zv = rz[j];
            const int tn = t + kRing < t1 ? t + kRing : t1 - 1;
            rx[j] = IO::load(X + tn * D, ln.d);
            rd[j] = IO::load(DL + tn * D, ln.d);
            if (GATED) rz[j] = IO::load(Z + tn * D, ln.d);
            const int tb1 = t + 1 < t1 ? t + 1 : t1 - 1;
            lgkm_wait_all();
            bq[(j + 1) & 1].load(Bm, brow + tb1);
            cq[(j + 1) & 1].load(Cm, brow + tb1);
            const RowBC<IO>& Bv = bq[j & 1];
            const RowBC<IO>& Cv = cq[j & 1];

            const float dt = valid ? softplus(dv + bias) : 0.0f;
            const float dx = dt * xv;
            float yv = Dd * xv;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float dA = __builtin_amdgcn_exp2f(dt * A2[n]);
                h[n] = fmaf(dA, h[n], dx * Bv.get(n));
                yv = fmaf(Cv.get(n), h[n], yv);
            }
            if (GATED) yv *= silu(zv);
            if (valid) IO::store(Y + t * D, ln.d, yv);
        }
    }
    if (a.h_last && c == a.n_chunks - 1) {
#pragma unroll
        for (int n = 0; n < kN; ++n) a.h_last[(b * D + ln.d) * kN + n] = h[n];
    }
}

// ---------------------------------------------------------------------------
// decode: one token against the cached state, in place
// ---------------------------------------------------------------------------
// Four lanes per channel, four states per lane: the state rows (64 bytes per
// channel) are read and written as whole 16-byte vectors by consecutive lanes.
constexpr int kStepRows = 8;      // batch rows per workgroup (A is loaded once for them)

template <class IO, bool GATED>
__global__ __launch_bounds__(kBlock) void s6_step(S6StepArgs a) {
    using T = typename IO::T;
    const int q = threadIdx.x & 3;
    const int64_t dl = static_cast<int64_t>(blockIdx.x) * (kBlock / 4) + (threadIdx.x >> 2);
    const bool active = dl < a.D;
    const int64_t d = active ? dl : a.D - 1;
    const uint32_t dd = static_cast<uint32_t>(d);
    const T* __restrict__ X = static_cast<const T*>(a.x);
    const T* __restrict__ DL = static_cast<const T*>(a.delta);
    const T* __restrict__ Z = static_cast<const T*>(a.z);
    const T* __restrict__ Bm = static_cast<const T*>(a.B);
    const T* __restrict__ Cm = static_cast<const T*>(a.C);
    T* __restrict__ Y = static_cast<T*>(a.y);

    float A2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) A2[j] = a.A[d * kN + 4 * q + j] * kLog2e;
    const float bias = a.dt_bias[d];
    const float Dd = a.Dskip[d];

    const int64_t b_begin = static_cast<int64_t>(blockIdx.y) * kStepRows;
    const int64_t b_end = (b_begin + kStepRows < a.batch) ? b_begin + kStepRows : a.batch;
    for (int64_t b = b_begin; b < b_end; ++b) {
        const int64_t bd = b * a.D + d;
        const int64_t brow = b * a.D;
        const float xv = IO::load(X + brow, dd);
        const float dt = softplus(IO::load(DL + brow, dd) + bias);
        const float dx = dt * xv;
        float4* hp = reinterpret_cast<float4*>(a.h + bd * kN) + q;
        float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (active) hv = *hp;
        float hs[4] = {hv.x, hv.y, hv.z, hv.w};
        float p = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float dA = __builtin_amdgcn_exp2f(dt * A2[j]);
            hs[j] = fmaf(dA, hs[j], dx * IO::load(Bm + b * kN, 4 * q + j));
            p = fmaf(IO::load(Cm + b * kN, 4 * q + j), hs[j], p);
        }
        if (active) *hp = make_float4(hs[0], hs[1], hs[2], hs[3]);
        p += __shfl_xor(p, 1, 4);
        p += __shfl_xor(p, 2, 4);
        float yv = fmaf(Dd, xv, p);
        if (GATED) yv *= silu(IO::load(Z + brow, dd));
        if (active && q == 0) IO::store(Y + brow, dd, yv);
    }
}

}  // namespace s6

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
using namespace s6;

template <class IO, bool GATED>
static hipError_t launch_scan_t(const S6ScanArgs& a, hipStream_t stream) {
    const unsigned gx = static_cast<unsigned>((a.D + kBlock - 1) / kBlock);
    if (a.n_chunks > 1) {
        dim3 g1(gx, static_cast<unsigned>(a.n_chunks - 1), static_cast<unsigned>(a.batch));
        s6_timing_mark("s6_chunk_carry", stream, true);
        hipLaunchKernelGGL(s6_chunk_carry<IO>, g1, dim3(kBlock), 0, stream, a);
        s6_timing_mark("s6_chunk_carry", stream, false);
    }
    dim3 g3(gx, static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(a.batch));
    s6_timing_mark("s6_chunk_out", stream, true);
    hipLaunchKernelGGL((s6_chunk_out<IO, GATED>), g3, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_chunk_out", stream, false);
    return hipGetLastError();
}

hipError_t s6_launch_scan(const S6ScanArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16) return gated ? launch_scan_t<BF16, true>(a, stream) : launch_scan_t<BF16, false>(a, stream);
    return gated ? launch_scan_t<F32, true>(a, stream) : launch_scan_t<F32, false>(a, stream);
}

template <class IO, bool GATED>
static hipError_t launch_step_t(const S6StepArgs& a, hipStream_t stream) {
    dim3 g(static_cast<unsigned>((a.D + kBlock / 4 - 1) / (kBlock / 4)),
           static_cast<unsigned>((a.batch + kStepRows - 1) / kStepRows));
    s6_timing_mark("s6_step", stream, true);
    hipLaunchKernelGGL((s6_step<IO, GATED>), g, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_step", stream, false);
    return hipGetLastError();
}

hipError_t s6_launch_step(const S6StepArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16) return gated ? launch_step_t<BF16, true>(a, stream) : launch_step_t<BF16, false>(a, stream);
    return gated ? launch_step_t<F32, true>(a, stream) : launch_step_t<F32, false>(a, stream);
}
