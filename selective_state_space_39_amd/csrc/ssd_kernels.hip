// gfx950 kernel of the SSD (Mamba-2 style) layer: scalar decay per head, so
// the causal matrix mixer of "Mamba", "Relation to Mamba-2" becomes, inside a
// chunk, a masked dense product, and across chunks a carried P x N state per
// head ("Mamba & State-Space Sequence Models", "Core mechanics": the duality
// of structured SSMs and a class of linear attention).
//
// One workgroup (4 wavefronts) per (batch row, head) walks its chunks of
// kQ = 64 tokens in order.  With S_t = A_h * (sum of Delta up to t inside the
// chunk):
//   G^T[i][t]  = B_i . C_t                                   (MFMA over N)
//   M[t][i]    = G^T[i][t] exp(S_t - S_i) Delta_i,  i <= t    (mask, VALU)
//   y_t        = sum_i M[t][i] x_i                            (MFMA over i)
//              + exp(S_t) C_t . state_in                      (MFMA over N)
//              + D_h x_t, then * silu(z_t)
//   state_out  = exp(S_end) state_in + sum_i exp(S_end - S_i) Delta_i x_i B_i^T   (MFMA over i)
// The state (P x N fp32) lives in MFMA accumulators for the whole sequence;
// its bf16 copy in LDS feeds the next chunk's state term.  Operands are bf16
// (the io dtype), accumulation fp32.
//
// v_mfma_f32_16x16x32_bf16 operand layout (lane l, r = l % 16, q = l / 16):
// A: A[m = r][k = 8q .. 8q+7]; B: B[k = 8q .. 8q+7][n = r]; D: D[m = 4q + i][n = r].
// Because a contraction does not care about the order of k, the mask's
// accumulator tiles (G^T rows i = 4q .. 4q+3 of two 16-row tiles) are used
// directly as the A operand of the y product, with the x operand read in the
// same permuted k order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "s6_common.h"

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;          // tokens per chunk
constexpr int kP = 64;          // channels per head
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kLdQ = kQ + 8;    // padded LDS row lengths (bf16), against bank conflicts
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));      // round to nearest even
}
__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {           // 16-byte aligned
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 lds4x2(const uint16_t* p0, const uint16_t* p1) {   // two 8-byte halves
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
    uint4 u;
    u.x = to_bf16(v[0]) | (static_cast<uint32_t>(to_bf16(v[1])) << 16);
    u.y = to_bf16(v[2]) | (static_cast<uint32_t>(to_bf16(v[3])) << 16);
    u.z = to_bf16(v[4]) | (static_cast<uint32_t>(to_bf16(v[5])) << 16);
    u.w = to_bf16(v[6]) | (static_cast<uint32_t>(to_bf16(v[7])) << 16);
    return __builtin_bit_cast(bf16x8, u);
}

template <int N>
struct alignas(16) Smem {
    static constexpr int kLdN = N + 8;
    uint16_t Bs[kQ][kLdN];      // B rows of the chunk          [i][n]
    uint16_t Cs[kQ][kLdN];      // C rows of the chunk          [t][n]
    uint16_t Bt[N][kLdQ];       // B transposed                 [n][i]
    uint16_t Xt[kP][kLdQ];      // x transposed                 [p][i]
    uint16_t XWt[kP][kLdQ];     // (exp(S_end - S_i) Delta_i x_i) transposed
    uint16_t St[kP][kLdN];      // incoming state, bf16         [p][n]
    float S2[kQ];               // S_t * log2(e)
    float Dl[kQ];               // Delta_t
};

// Global rows of one chunk, held in registers between chunks (prefetch).
template <int N>
struct ChunkRegs {
    static constexpr int kXSeg = kQ * kP / 8 / kThreads;    // 16-byte pieces of x per thread
    static constexpr int kBSeg = kQ * N / 8 / kThreads;     // of B (and of C)
    uint4 x[kXSeg], b[kBSeg], c[kBSeg];
    uint16_t dl;
};

template <int N>
__device__ __forceinline__ void load_chunk(const SsdArgs& a, int64_t b, int64_t h, int t0, int nt, ChunkRegs<N>& r) {
    const int tid = threadIdx.x;
    const uint16_t* X = static_cast<const uint16_t*>(a.x);
    const uint16_t* Bg = static_cast<const uint16_t*>(a.B);
    const uint16_t* Cg = static_cast<const uint16_t*>(a.C);
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::kXSeg; ++k) {
        const int s = tid + kThreads * k, t = s / (kP / 8), p0 = (s % (kP / 8)) * 8;
        r.x[k] = t < nt ? *reinterpret_cast<const uint4*>(X + ((b * a.L + t0 + t) * a.H + h) * kP + p0) : zero;
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::kBSeg; ++k) {
        const int s = tid + kThreads * k, t = s / (N / 8), n0 = (s % (N / 8)) * 8;
        const int64_t row = (b * a.L + t0 + t) * N + n0;
        r.b[k] = t < nt ? *reinterpret_cast<const uint4*>(Bg + row) : zero;
        r.c[k] = t < nt ? *reinterpret_cast<const uint4*>(Cg + row) : zero;
    }
    r.dl = 0;
    if (tid < kQ && tid < nt) r.dl = static_cast<const uint16_t*>(a.delta)[(b * a.L + t0 + tid) * a.H + h];
}

// Stage one chunk into LDS: step sizes and the running log-decay S (wavefront
// 0, a prefix sum over the 64 tokens), then B, C, x and the weighted x.
template <int N>
__device__ __forceinline__ void stage_chunk(Smem<N>& sm, const ChunkRegs<N>& r, int nt, float A, float bias) {
    const int tid = threadIdx.x;
    if (tid < kQ) {
        const float dt = tid < nt ? s6::softplus(from_bf16(r.dl) + bias) : 0.0f;
        float s = dt * A * kLog2e;
#pragma unroll
        for (int off = 1; off < kQ; off <<= 1) {                   // inclusive scan over the wavefront
            const float o = __shfl_up(s, off);
            if (tid >= off) s += o;
        }
        sm.S2[tid] = s;
        sm.Dl[tid] = dt;
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::kBSeg; ++k) {
        const int s = tid + kThreads * k, t = s / (N / 8), n0 = (s % (N / 8)) * 8;
        *reinterpret_cast<uint4*>(&sm.Bs[t][n0]) = r.b[k];
        *reinterpret_cast<uint4*>(&sm.Cs[t][n0]) = r.c[k];
        const uint32_t w[4] = {r.b[k].x, r.b[k].y, r.b[k].z, r.b[k].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.Bt[n0 + j][t] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
    }
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::kXSeg; ++k) {
        const int s = tid + kThreads * k, t = s / (kP / 8), p0 = (s % (kP / 8)) * 8;
        const uint32_t w[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.Xt[p0 + j][t] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
    }
    __syncthreads();                                 // S2 and Dl ready
    const float s_end = sm.S2[kQ - 1];
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::kXSeg; ++k) {
        const int s = tid + kThreads * k, t = s / (kP / 8), p0 = (s % (kP / 8)) * 8;
        const float wt = __builtin_amdgcn_exp2f(s_end - sm.S2[t]) * sm.Dl[t];
        const uint32_t w[4] = {r.x[k].x, r.x[k].y, r.x[k].z, r.x[k].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xv = from_bf16(static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1))));
            sm.XWt[p0 + j][t] = to_bf16(wt * xv);
        }
    }
}

template <int N, bool GATED>
__global__ __launch_bounds__(kThreads) void ssd_chunked(SsdArgs a) {
    constexpr int NB = N / 16;            // 16-row blocks of the state's n
    constexpr int NBW = NB / 4;           // n-blocks of the state owned by each wavefront
    constexpr int KS = N / 32;            // k-steps of a product over n
    __shared__ Smem<N> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, r = l & 15, q = l >> 4;
    // (batch row, head): the heads of one batch row stay on one XCD (shared B / C rows in its L2)
    const int64_t units = a.batch * a.H;
    int64_t u = blockIdx.x;
    if (units % 8 == 0) u = (u % 8) * (units / 8) + u / 8;
    const int64_t b = u / a.H, h = u % a.H;
    const float A = a.A[h], bias = a.dt_bias[h], Dd = a.Dskip[h];

    // state^T tiles owned by this wavefront: n-blocks w*NBW .. +NBW-1, p-blocks 0..3
    f32x4 st[NBW][4];
    const float* h0 = a.h0 ? a.h0 + (b * a.H + h) * kP * N : nullptr;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const int n = (w * NBW + nb) * 16 + 4 * q, p = pb * 16 + r;
            if (h0) {
                const float4 v = *reinterpret_cast<const float4*>(h0 + p * N + n);
                st[nb][pb] = f32x4{v.x, v.y, v.z, v.w};
            } else {
                st[nb][pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    auto write_state = [&]() {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int n = (w * NBW + nb) * 16 + 4 * q, p = pb * 16 + r;
                uint2 v;
                v.x = to_bf16(st[nb][pb][0]) | (static_cast<uint32_t>(to_bf16(st[nb][pb][1])) << 16);
                v.y = to_bf16(st[nb][pb][2]) | (static_cast<uint32_t>(to_bf16(st[nb][pb][3])) << 16);
                *reinterpret_cast<uint2*>(&sm.St[p][n]) = v;
            }
    };

    const int nchunks = static_cast<int>((a.L + kQ - 1) / kQ);
    ChunkRegs<N> cr;
    load_chunk<N>(a, b, h, 0, static_cast<int>(a.L < kQ ? a.L : kQ), cr);
    write_state();
    const uint16_t* Zg = static_cast<const uint16_t*>(a.z);
    uint16_t* Yg = static_cast<uint16_t*>(a.y);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * kQ;
        const int nt = static_cast<int>(a.L - t0 < kQ ? a.L - t0 : kQ);
        stage_chunk<N>(sm, cr, nt, A, bias);
        __syncthreads();
        if (c + 1 < nchunks) {
            const int t1 = t0 + kQ;
            load_chunk<N>(a, b, h, t1, static_cast<int>(a.L - t1 < kQ ? a.L - t1 : kQ), cr);
        }

        // --- G^T tiles (i-block ib, t-block w) for ib <= w, masked into M^T
        f32x4 g[4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            g[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ib <= w) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    g[ib] = mfma(lds8(&sm.Bs[ib * 16 + r][ks * 32 + 8 * q]), lds8(&sm.Cs[w * 16 + r][ks * 32 + 8 * q]),
                                 g[ib]);
                const int t = w * 16 + r;
                const float st2 = sm.S2[t];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = ib * 16 + 4 * q + j;
                    const float m = __builtin_amdgcn_exp2f(st2 - sm.S2[i]) * sm.Dl[i];
                    g[ib][j] = i <= t ? g[ib][j] * m : 0.0f;
                }
            }
        }
        // --- y for t-block w: masked intra-chunk product plus the incoming state's term
        f32x4 yd[4], yo[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            yd[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
            yo[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (2 * kb <= w) {
                const float mv[8] = {g[2 * kb][0], g[2 * kb][1], g[2 * kb][2], g[2 * kb][3],
                                     g[2 * kb + 1][0], g[2 * kb + 1][1], g[2 * kb + 1][2], g[2 * kb + 1][3]};
                const bf16x8 am = pack8(mv);
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const uint16_t* xr = &sm.Xt[pb * 16 + r][kb * 32 + 4 * q];
                    yd[pb] = mfma(am, lds4x2(xr, xr + 16), yd[pb]);
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ac = lds8(&sm.Cs[w * 16 + r][ks * 32 + 8 * q]);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) yo[pb] = mfma(ac, lds8(&sm.St[pb * 16 + r][ks * 32 + 8 * q]), yo[pb]);
        }
        // --- outputs: rows t = 16w + 4q + j, column p = 16 pb + r
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = w * 16 + 4 * q + j;
            if (t < nt) {
                const float e = __builtin_amdgcn_exp2f(sm.S2[t]);
                const int64_t row = ((b * a.L + t0 + t) * a.H + h) * kP;
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const int p = pb * 16 + r;
                    float yv = yd[pb][j] + e * yo[pb][j] + Dd * from_bf16(sm.Xt[p][t]);
                    if (GATED) yv *= s6::silu(from_bf16(Zg[row + p]));
                    Yg[row + p] = to_bf16(yv);
                }
            }
        }
        // --- state update: state^T = exp(S_end) state^T + B^T (w x)
        const float dec = __builtin_amdgcn_exp2f(sm.S2[kQ - 1]);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                f32x4 s = st[nb][pb] * dec;
#pragma unroll
                for (int ks = 0; ks < kQ / 32; ++ks)
                    s = mfma(lds8(&sm.Bt[(w * NBW + nb) * 16 + r][ks * 32 + 8 * q]),
                             lds8(&sm.XWt[pb * 16 + r][ks * 32 + 8 * q]), s);
                st[nb][pb] = s;
            }
        __syncthreads();                 // every wavefront is done with this chunk's LDS
        write_state();
    }
    if (a.h_last) {
        float* hl = a.h_last + (b * a.H + h) * kP * N;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int n = (w * NBW + nb) * 16 + 4 * q, p = pb * 16 + r;
                *reinterpret_cast<float4*>(hl + p * N + n) =
                    make_float4(st[nb][pb][0], st[nb][pb][1], st[nb][pb][2], st[nb][pb][3]);
            }
    }
}

}  // namespace ssd

using namespace ssd;

template <int N>
static hipError_t launch_ssd_n(const SsdArgs& a, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>(a.batch * a.H));
    s6_timing_mark("ssd_chunked", stream, true);
    if (a.z) hipLaunchKernelGGL((ssd_chunked<N, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((ssd_chunked<N, false>), grid, dim3(kThreads), 0, stream, a);
    s6_timing_mark("ssd_chunked", stream, false);
    return hipGetLastError();
}

hipError_t ssd_launch(const SsdArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 64: return launch_ssd_n<64>(a, stream);
        case 128: return launch_ssd_n<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
