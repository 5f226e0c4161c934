// gfx950 kernels of the SSD (Mamba-2 style) layer: scalar decay per head, so
// the causal matrix mixer of "Mamba", "Relation to Mamba-2" becomes, inside a
// chunk, a masked dense product, and across chunks a carried P x N state per
// head ("Mamba & State-Space Sequence Models", "Core mechanics": the duality
// of structured SSMs and a class of linear attention).
//
// Chunks of kQ = 64 tokens.  With S_t = A_h * (sum of Delta up to t inside the
// chunk):
//   G[t][i]    = C_t . B_i                       (no head in it: ssd_gram, once
//                                                 per batch row and chunk)
//   M[t][i]    = G[t][i] exp(S_t - S_i) Delta_i, i <= t
//   y_t        = sum_i M[t][i] x_i + exp(S_t) state_in C_t + D_h x_t, then * silu(z_t)
//   state_out  = exp(S_end) state_in + sum_i exp(S_end - S_i) Delta_i x_i B_i^T
// ssd_chunked: one workgroup (4 wavefronts) per (batch row, head) walks its
// chunks in order.  Wavefront w computes the outputs of tokens 16w .. 16w+15
// (its C rows come straight from memory into MFMA operand registers, its M
// entries from G in registers) and owns channels 16w .. 16w+15 of the fp32
// state, kept in MFMA accumulators for the whole sequence; a bf16 copy of the
// state in LDS feeds every wavefront's state term.  Operands are bf16 (the io
// dtype), accumulation fp32.
//
// v_mfma_f32_16x16x32_bf16 operand layout (lane l, r = l % 16, q = l / 16):
// A: A[m = r][k = 8q .. 8q+7]; B: B[k = 8q .. 8q+7][n = r]; D: D[m = 4q + i][n = r].
// Outputs are computed transposed (m = channel, n = token), so a lane ends
// with 4 consecutive channels of one token: 8-byte gate loads and stores.
//
// Operands whose contraction index runs along the rows of a row-major LDS
// tile (x in both products, B in the state update) are fetched with gfx950's
// transposing LDS read ds_read_b64_tr_b16: within each 16-lane group, output
// lane j = 4a + c, element s comes from the 8-byte segment addressed by lane
// 4s + a, element c.  Addressing lane 4s + a at row (row0 + s), columns
// col0 + 4a .. 4a+3 therefore hands lane j the column col0 + j of rows
// row0 .. row0+3 -- the k-major operand layout -- so no tile is ever stored
// transposed.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_common.h"

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;          // tokens per chunk
constexpr int kP = 64;          // channels per head
constexpr int kThreads = 256;   // 4 wavefronts
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) in one dword, low half first
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// v rounded to the nearest bf16 value (ties to even), as a float; finite v
__device__ __forceinline__ float round_bf16(float v) {
    const uint32_t u = __float_as_uint(v);
    return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {           // 16-byte aligned
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
    return __builtin_bit_cast(bf16x8, make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]),
                                                 pack2(v[6], v[7])));
}

// LDS of ssd_chunked: 48 KB for N = 128, so three workgroups fit on a CU
// and every (batch row, head) of a 640-sequence launch is resident at once;
// 79 KB for N = 256 (two per CU).
template <int N>
struct alignas(16) Smem {
    // Row strides, in 4-byte banks modulo 64: B rows 12 (N + 24 = 76 or 140
    // dwords) keep the transposing reads conflict-free, state-copy rows 4
    // (N + 8) the 16-byte reads and 8-byte writes.
    static constexpr int kLdB = N + 24;
    static constexpr int kLdS = N + 8;
    static constexpr int kLdX = kP + 16;
    uint16_t Bs[kQ][kLdB];      // B rows of the chunk            [i][n]
    uint16_t Xs[kQ][kLdX];      // x rows                         [i][p]
    uint16_t St[kP][kLdS];      // bf16 copy of the incoming state [p][n]
    float S2[kQ];               // S_t * log2(e)
    float Dl[kQ];               // Delta_t
    float Wt[kQ];               // exp(S_end - S_t) Delta_t
    // Each wavefront's output rows pass through LDS (fp32, 16 rows of 64
    // channels, row stride kLdY floats, 4 banks modulo 64) to be stored row by
    // row.  When a row of St holds 256 bytes the wavefront's own 16 St rows
    // serve, at St's stride (it rewrites them only afterwards); otherwise a
    // separate area.
    static constexpr bool kYinSt = kLdS * 2 >= kP * 4;
    static constexpr int kLdY = kYinSt ? kLdS / 2 : kP + 4;
    float Ys[kYinSt ? 0 : 4][16][kLdY];
};

template <int N>
__device__ __forceinline__ float* ystage(Smem<N>& sm, int w) {
    if constexpr (Smem<N>::kYinSt) {
        return reinterpret_cast<float*>(&sm.St[16 * w][0]);
    } else {
        return &sm.Ys[w][0][0];
    }
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
// Transposing read: lane (group g = l / 16, local m = l % 16) addresses row
// row0 + m / 4, columns col0 + 4 (m % 4); see the header comment.
__device__ __forceinline__ v4s tr4(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}
// k-major operand: lane l gets column col0 + l % 16 of rows row0 .. row0 + 7
// (row0 may depend on the lane group)
__device__ __forceinline__ bf16x8 opnd_rows8(const uint16_t* base, int ld, int row0, int col0) {
    const int m = threadIdx.x & 15;
    const uint16_t* p = base + (row0 + (m >> 2)) * ld + col0 + 4 * (m & 3);
    const v4s lo = tr4(p), hi = tr4(p + 4 * ld);
    return __builtin_bit_cast(bf16x8, static_cast<v8s>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
}

// Every tensor of one (batch row, head) sequence is addressed through a buffer
// resource based at its first element and bounded by its last row: a lane's
// byte offset inside a chunk is fixed (a VGPR), the chunk's row offset is one
// SGPR, and rows past the sequence end read as zero (stores there are
// dropped), so no load or store needs a bounds check.
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---------------------------------------------------------------------------
// ssd_gram: G[t][i] = C_t . B_i for every (batch row, chunk), the part
// of the mixer that no head changes, accumulated in fp32 and stored as bf16
// (it only ever enters a bf16 matrix-core operand).  Workgroup = (batch row, chunk);
// wavefront w computes rows t = 16w .. 16w+15.  Rows past the sequence end
// read B, C as zero, so their G is zero.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(kThreads) void ssd_gram(SsdArgs a) {
    constexpr int KS = N / 32;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
    const int64_t nch = (a.L + kQ - 1) / kQ;
    const int64_t b = blockIdx.x / nch, c = blockIdx.x % nch;
    const __amdgpu_buffer_rsrc_t rB = rsrc(static_cast<const uint16_t*>(a.B) + b * a.L * N, a.L * N * 2);
    const __amdgpu_buffer_rsrc_t rC = rsrc(static_cast<const uint16_t*>(a.C) + b * a.L * N, a.L * N * 2);
    const uint32_t so = static_cast<uint32_t>(c * kQ * N * 2);
    // B operand: C rows t = 16w + r, n = 32ks + 8q .. +7
    bf16x8 cop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        cop[ks] = __builtin_bit_cast(bf16x8, ld16(rC, ((16 * w + r) * N + 32 * ks + 8 * q) * 2, so));
    uint16_t* g = a.gram + ((b * nch + c) * kQ + 16 * w + r) * kQ;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
        // A operand: B rows i = 16ib + r; D[m = i][n = t]: lane slot j = G[t = 16w + r][i = 16ib + 4q + j]
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = mfma(__builtin_bit_cast(bf16x8, ld16(rB, ((16 * ib + r) * N + 32 * ks + 8 * q) * 2, so)), cop[ks], acc);
        *reinterpret_cast<uint2*>(g + 16 * ib + 4 * q) = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
    }
}

// ---------------------------------------------------------------------------
// ssd_chunked
// ---------------------------------------------------------------------------
struct SeqIO {
    __amdgpu_buffer_rsrc_t x, z, y, B, C, dl, G;
    uint32_t xrow, bcrow, dlrow;             // bytes per token row
    uint32_t gchunk;                         // bytes of G per chunk
};

// x and B of one chunk in registers until they are staged in LDS (prefetch).
template <int N>
struct StageRegs {
    static constexpr int kXSeg = kQ * kP / 8 / kThreads;    // 16-byte pieces of x per thread
    static constexpr int kBSeg = kQ * N / 8 / kThreads;     // of B
    uint4 x[kXSeg], b[kBSeg];
    uint16_t dl;               // delta of token (lane), wavefront 0 only
};

template <int N>
__device__ __forceinline__ void load_stage(const SeqIO& io, int t0, int w, StageRegs<N>& r) {
    const int tid = threadIdx.x;
    // piece k of a thread sits kThreads * k / (row length / 8) rows below piece 0:
    // one lane offset per tensor, the row step goes to the scalar offset
    constexpr int kXRows = kThreads / (kP / 8), kBRows = kThreads / (N / 8);
    const uint32_t vx = (tid / (kP / 8)) * io.xrow + (tid % (kP / 8)) * 16;
    const uint32_t vb = (tid / (N / 8)) * io.bcrow + (tid % (N / 8)) * 16;
#pragma unroll
    for (int k = 0; k < StageRegs<N>::kXSeg; ++k)
        r.x[k] = ld16(io.x, vx, static_cast<uint32_t>(t0 + kXRows * k) * io.xrow);
#pragma unroll
    for (int k = 0; k < StageRegs<N>::kBSeg; ++k)
        r.b[k] = ld16(io.B, vb, static_cast<uint32_t>(t0 + kBRows * k) * io.bcrow);
    const uint32_t so = static_cast<uint32_t>(t0);
    if (w == 0)
        r.dl = static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(io.dl, (tid & 63) * io.dlrow,
                                                                          so * io.dlrow, 0));
}

// What wavefront w reads from memory for its own tokens t = 16w + r: C rows
// (the B operand of the state term), G rows (for M), and the gate of its
// output rows in row order (lane l: row 8k + l / 8, channels 8 (l % 8) .. +7).
template <int N>
struct OwnRegs {
    static constexpr int KS = N / 32;
    bf16x8 c[KS];              // C[t][32ks + 8q .. +7]
    uint4 g[2];                // G[t][32ks + 8q .. +7] (bf16), ks < 1 + (w >= 2)
    uint4 z[2];                // z[16w + 8k + l / 8][8 (l % 8) .. +7]
};

template <int N>
__device__ __forceinline__ void load_cg(const SeqIO& io, int c, int t0, int w, OwnRegs<N>& o) {
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4, t = 16 * w + r;
    const uint32_t so = static_cast<uint32_t>(t0);
#pragma unroll
    for (int ks = 0; ks < OwnRegs<N>::KS; ++ks)
        o.c[ks] = __builtin_bit_cast(bf16x8, ld16(io.C, t * io.bcrow + 8 * q * 2, so * io.bcrow + 64 * ks));
    const uint32_t gs = static_cast<uint32_t>(c) * io.gchunk;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        if (ks == 0 || w >= 2) o.g[ks] = ld16(io.G, (t * kQ + 8 * q) * 2, gs + 64 * ks);
}

__device__ __forceinline__ uint32_t row_off(const SeqIO& io, int w) {          // row-order lane offset
    const int l = threadIdx.x & 63;
    return (16 * w + (l >> 3)) * io.xrow + (l & 7) * 16;
}

template <int N>
__device__ __forceinline__ void load_z(const SeqIO& io, int t0, int w, OwnRegs<N>& o) {
    const uint32_t v = row_off(io, w);
#pragma unroll
    for (int k = 0; k < 2; ++k) o.z[k] = ld16(io.z, v, static_cast<uint32_t>(t0 + 8 * k) * io.xrow);
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: four row
// shifts scan each row of 16 lanes, then row_bcast:15 and row_bcast:31 carry
// the row totals forward (the gfx9-family broadcasts).  Lanes a shift or
// broadcast does not reach add 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_src(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float s) {
    s += dpp_src<0x111, 0xf>(s);        // row_shr:1
    s += dpp_src<0x112, 0xf>(s);        // row_shr:2
    s += dpp_src<0x114, 0xf>(s);        // row_shr:4
    s += dpp_src<0x118, 0xf>(s);        // row_shr:8
    s += dpp_src<0x142, 0xa>(s);        // row_bcast:15 into rows 1 and 3
    s += dpp_src<0x143, 0xc>(s);        // row_bcast:31 into rows 2 and 3
    return s;
}

// Stage one chunk: x and B rows into LDS; wavefront 0 scans the step sizes
// (lane = token) and publishes S, Delta and the state-update weights.
template <int N>
__device__ __forceinline__ void stage_chunk(Smem<N>& sm, const StageRegs<N>& r, int nt, float A, float bias, int w) {
    const int tid = threadIdx.x, l = tid & 63;
    if (w == 0) {
        const float dt = l < nt ? s6::softplus(from_bf16(r.dl) + bias) : 0.0f;
        const float s = wave_inclusive_sum(dt * A * kLog2e);
        const float s_end = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), kQ - 1));
        sm.S2[l] = s;
        sm.Dl[l] = dt;
        sm.Wt[l] = __builtin_amdgcn_exp2f(s_end - s) * dt;
    }
#pragma unroll
    for (int k = 0; k < StageRegs<N>::kBSeg; ++k) {
        const int e = tid + kThreads * k, t = e / (N / 8), n0 = (e % (N / 8)) * 8;
        *reinterpret_cast<uint4*>(&sm.Bs[t][n0]) = r.b[k];
    }
#pragma unroll
    for (int k = 0; k < StageRegs<N>::kXSeg; ++k) {
        const int e = tid + kThreads * k, t = e / (kP / 8), p0 = (e % (kP / 8)) * 8;
        *reinterpret_cast<uint4*>(&sm.Xs[t][p0]) = r.x[k];
    }
}

// State update of this wavefront's channels, state^T = dec state^T + B^T (W x)
// with W_i = exp(S_end - S_i) Delta_i.  W x is formed in fp32 and enters the
// matrix cores as two bf16 operands, its rounded value and the rounding
// remainder (x and B are bf16 inputs, exact as operands), so the carried fp32
// state sees W x to ~2^-17 rather than bf16's 2^-9: the state handed to a
// decode step or a following segment keeps fp32-level accuracy.
template <int N>
__device__ __forceinline__ void state_update(const Smem<N>& sm, f32x4 (&st)[N / 16], float dec, int w) {
    const int l = threadIdx.x & 63, q = l >> 4;
    bf16x8 xh[2], xl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int i0 = 32 * ks + 8 * q;
        const bf16x8 xv = opnd_rows8(&sm.Xs[0][0], Smem<N>::kLdX, i0, 16 * w);
        const float4 wa = *reinterpret_cast<const float4*>(&sm.Wt[i0]);
        const float4 wb = *reinterpret_cast<const float4*>(&sm.Wt[i0 + 4]);
        const float wi[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        float v[8], hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] = static_cast<float>(xv[j]) * wi[j];
            hv[j] = round_bf16(v[j]);
            v[j] -= hv[j];
        }
        xh[ks] = pack8(hv);                // exact: hv holds bf16 values
        xl[ks] = pack8(v);
    }
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) {
        const bf16x8 b0 = opnd_rows8(&sm.Bs[0][0], Smem<N>::kLdB, 8 * q, nb * 16);
        const bf16x8 b1 = opnd_rows8(&sm.Bs[0][0], Smem<N>::kLdB, 32 + 8 * q, nb * 16);
        f32x4 sv = st[nb] * dec;
        sv = mfma(b0, xl[0], sv);
        sv = mfma(b1, xl[1], sv);
        sv = mfma(b0, xh[0], sv);
        sv = mfma(b1, xh[1], sv);
        st[nb] = sv;
    }
}

// bf16 copy of this wavefront's state channels into St[p][n]
template <int N>
__device__ __forceinline__ void publish_state(Smem<N>& sm, const f32x4 (&st)[N / 16], int w) {
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb)
        *reinterpret_cast<uint2*>(&sm.St[16 * w + r][16 * nb + 4 * q]) =
            make_uint2(pack2(st[nb][0], st[nb][1]), pack2(st[nb][2], st[nb][3]));
}

// One workgroup walks one segment of one (batch row, head) sequence.
// LOCAL = false (kernel ssd_chunked): the layer itself, from the segment's
// starting state (the caller's h0 for segment 0, the fold's result for the
// others), writing its outputs.  LOCAL = true (kernel ssd_seg_local): the
// first pass of a segmented layer, segment k < n_seg - 1 from a zero state
// with no outputs, leaving its end state and its total decay in the
// workspace.
template <int N, bool GATED, bool LOCAL>
__device__ __forceinline__ void ssd_walk(const SsdArgs& a) {
    constexpr int NB = N / 16;            // 16-row blocks of the state's n
    constexpr int KS = N / 32;            // k-steps of a product over n
    __shared__ Smem<N> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, r = l & 15, q = l >> 4;
    const int tw = 16 * w + r;            // this lane's token inside a chunk
    const int nks = w >= 2 ? 2 : 1;       // k-steps of 32 tokens that reach token 16w + 15
    // (batch row, segment, head), head fastest: the heads of one batch row and
    // segment stay on one XCD (shared B, C, G rows in its L2)
    const int64_t nseg = LOCAL ? a.n_seg - 1 : a.n_seg;
    const int64_t units = a.batch * nseg * a.H;
    int64_t u = blockIdx.x;
    if (units % 8 == 0) u = (u % 8) * (units / 8) + u / 8;
    const int64_t h = u % a.H, seg = (u / a.H) % nseg, b = u / (a.H * nseg);
    const float A = a.A[h], bias = a.dt_bias[h], Dd = a.Dskip[h];
    const int64_t nslot = a.n_seg - 1;    // segment states per sequence in the workspace

    // This wavefront owns channels p = 16 w .. 16 w + 15 of the state: tiles
    // state^T[n-block nb][p-block w], lane slot j = state^T[16 nb + 4q + j][16 w + r].
    f32x4 st[NB];
    const float* h0 = LOCAL ? nullptr
                      : seg == 0 ? (a.h0 ? a.h0 + (b * a.H + h) * kP * N : nullptr)
                                 : a.seg_state + ((b * a.H + h) * nslot + seg - 1) * kP * N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if (h0) {
            const float4 v = *reinterpret_cast<const float4*>(h0 + (16 * w + r) * N + 16 * nb + 4 * q);
            st[nb] = f32x4{v.x, v.y, v.z, v.w};
        } else {
            st[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if constexpr (!LOCAL) publish_state<N>(sm, st, w);

    const int nchunks = static_cast<int>((a.L + kQ - 1) / kQ);
    const int c_begin = static_cast<int>(seg * a.seg_chunks);
    const int c_end = c_begin + a.seg_chunks < nchunks ? static_cast<int>(c_begin + a.seg_chunks) : nchunks;
    float decay = 0.0f;                   // log2 of the segment's total decay (LOCAL)
    SeqIO io;
    {
        const int64_t xoff = (b * a.L * a.H + h) * kP;                       // first element of the sequence
        const int64_t xbytes = ((a.L - 1) * a.H + 1) * kP * 2;
        io.xrow = static_cast<uint32_t>(a.H * kP * 2);
        io.bcrow = N * 2;
        io.dlrow = static_cast<uint32_t>(a.H * 2);
        io.gchunk = kQ * kQ * 2;
        io.x = rsrc(static_cast<const uint16_t*>(a.x) + xoff, xbytes);
        io.z = rsrc(a.z ? static_cast<const uint16_t*>(a.z) + xoff : nullptr, a.z ? xbytes : 0);
        io.y = rsrc(static_cast<uint16_t*>(a.y) + xoff, xbytes);
        io.B = rsrc(static_cast<const uint16_t*>(a.B) + b * a.L * N, a.L * N * 2);
        io.C = rsrc(static_cast<const uint16_t*>(a.C) + b * a.L * N, a.L * N * 2);
        io.dl = rsrc(static_cast<const uint16_t*>(a.delta) + b * a.L * a.H + h, ((a.L - 1) * a.H + 1) * 2);
        io.G = rsrc(a.gram + b * nchunks * kQ * kQ, static_cast<int64_t>(nchunks) * kQ * kQ * 2);
    }
    StageRegs<N> sr;
    OwnRegs<N> own;
    load_stage<N>(io, c_begin * kQ, w, sr);
    if constexpr (!LOCAL) {
        load_cg<N>(io, c_begin, c_begin * kQ, w, own);
        if constexpr (GATED) load_z<N>(io, c_begin * kQ, w, own);
    }
    const uint32_t vrow = row_off(io, w);

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * kQ;
        const int nt = static_cast<int>(a.L - t0 < kQ ? a.L - t0 : kQ);
        stage_chunk<N>(sm, sr, nt, A, bias, w);
        __syncthreads();                               // chunk staged, incoming state published
        // Prefetches are unconditional (the last chunk reloads itself): with no
        // branch around them the compiler waits on each load by its exact
        // position in the in-order memory counter instead of draining it.
        const int cn = c + 1 < c_end ? c + 1 : c, t1 = cn * kQ;
        load_stage<N>(io, t1, w, sr);
        if constexpr (LOCAL) {
            // state update only: state^T = exp(S_end) state^T + B^T (W x)
            const float s_end = sm.S2[kQ - 1];
            decay += s_end;
            state_update<N>(sm, st, __builtin_amdgcn_exp2f(s_end), w);
            __syncthreads();                           // every read of Xs, Bs of this chunk is done
            continue;
        }

        // M^T as the B operand of y^T: lane (r, q) holds M[t = 16w + r][i = 32ks + 8q .. +7]
        const float s2t = sm.S2[tw];
        bf16x8 mop[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks < nks) {
                const int i0 = 32 * ks + 8 * q;
                const float4 sa = *reinterpret_cast<const float4*>(&sm.S2[i0]);
                const float4 sb = *reinterpret_cast<const float4*>(&sm.S2[i0 + 4]);
                const float4 da = *reinterpret_cast<const float4*>(&sm.Dl[i0]);
                const float4 db = *reinterpret_cast<const float4*>(&sm.Dl[i0 + 4]);
                const float si[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
                const float di[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
                const uint4 gw = own.g[ks];
                const float gi[8] = {lo_bf16(gw.x), hi_bf16(gw.x), lo_bf16(gw.y), hi_bf16(gw.y),
                                     lo_bf16(gw.z), hi_bf16(gw.z), lo_bf16(gw.w), hi_bf16(gw.w)};
                float m[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)     // above the diagonal: exp2(-inf) = +0, no branch
                    m[j] = gi[j] * (__builtin_amdgcn_exp2f(i0 + j <= tw ? s2t - si[j] : -__builtin_inff()) * di[j]);
                mop[ks] = pack8(m);
            }
        }
        const float e = __builtin_amdgcn_exp2f(s2t);

        // y^T before the gate for this wavefront's tokens and every channel
        // block: lane slot j = y[t = 16w + r][p = 16pb + 4q + j]
        f32x4 yp[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            f32x4 yi = f32x4{0.f, 0.f, 0.f, 0.f}, ys = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < nks) yi = mfma(opnd_rows8(&sm.Xs[0][0], Smem<N>::kLdX, 32 * ks + 8 * q, 16 * pb), mop[ks], yi);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                ys = mfma(lds8(&sm.St[16 * pb + r][32 * ks + 8 * q]), own.c[ks], ys);
            const uint2 xv = *reinterpret_cast<const uint2*>(&sm.Xs[tw][16 * pb + 4 * q]);
            yp[pb] = f32x4{yi[0] + e * ys[0] + Dd * lo_bf16(xv.x), yi[1] + e * ys[1] + Dd * hi_bf16(xv.x),
                           yi[2] + e * ys[2] + Dd * lo_bf16(xv.y), yi[3] + e * ys[3] + Dd * hi_bf16(xv.y)};
        }
        // C and G of the next chunk (their registers are free now)
        load_cg<N>(io, cn, t1, w, own);

        // --- state update: state^T = exp(S_end) state^T + B^T (W x), W_i = exp(S_end - S_i) Delta_i
        state_update<N>(sm, st, __builtin_amdgcn_exp2f(sm.S2[kQ - 1]), w);
        __syncthreads();                               // every read of St, Xs, Bs of this chunk is done

        // --- outputs in row order through this wavefront's staging rows, gate (when z is given), store
        float* ysm = ystage<N>(sm, w);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
            *reinterpret_cast<float4*>(ysm + r * Smem<N>::kLdY + 16 * pb + 4 * q) =
                make_float4(yp[pb][0], yp[pb][1], yp[pb][2], yp[pb][3]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float* src = ysm + (8 * k + (l >> 3)) * Smem<N>::kLdY + 8 * (l & 7);
            const float4 u0 = *reinterpret_cast<const float4*>(src);
            const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
            float yv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            if (GATED && a.z) {                      // uniform: one kernel serves both (z NULL: its loads read 0)
                const uint32_t zw[4] = {own.z[k].x, own.z[k].y, own.z[k].z, own.z[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    yv[2 * j] *= s6::silu(lo_bf16(zw[j]));
                    yv[2 * j + 1] *= s6::silu(hi_bf16(zw[j]));
                }
            }
            // rows past the sequence end: stored through the bounded buffer, i.e. dropped
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(v4u, make_uint4(pack2(yv[0], yv[1]), pack2(yv[2], yv[3]), pack2(yv[4], yv[5]),
                                                   pack2(yv[6], yv[7]))),
                io.y, vrow, static_cast<uint32_t>(t0 + 8 * k) * io.xrow, 0);
        }
        if constexpr (GATED) load_z<N>(io, t1, w, own);
        publish_state<N>(sm, st, w);                   // after this wavefront's staging reads (same rows)
    }
    if constexpr (LOCAL) {
        float* hs = a.seg_state + ((b * a.H + h) * nslot + seg) * kP * N;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<float4*>(hs + (16 * w + r) * N + 16 * nb + 4 * q) =
                make_float4(st[nb][0], st[nb][1], st[nb][2], st[nb][3]);
        if (tid == 0) a.seg_decay[(b * a.H + h) * nslot + seg] = decay;
        return;
    }
    if (a.h_last && seg == a.n_seg - 1) {
        float* hl = a.h_last + (b * a.H + h) * kP * N;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<float4*>(hl + (16 * w + r) * N + 16 * nb + 4 * q) =
                make_float4(st[nb][0], st[nb][1], st[nb][2], st[nb][3]);
    }
}

// Occupancy is pinned (three workgroups per CU up to N = 128, two at 256), so
// the compiler schedules for the register budget the layout needs instead of
// chasing a higher occupancy it cannot keep.
template <int N, bool GATED>
__global__ __launch_bounds__(kThreads, (N > 128 ? 2 : 3)) __attribute__((amdgpu_waves_per_eu(N > 128 ? 2 : 3, N > 128 ? 2 : 3)))
void ssd_chunked(SsdArgs a) {
    ssd_walk<N, GATED, false>(a);
}

template <int N>
__global__ __launch_bounds__(kThreads, (N > 128 ? 2 : 3)) __attribute__((amdgpu_waves_per_eu(N > 128 ? 2 : 3, N > 128 ? 2 : 3)))
void ssd_seg_local(SsdArgs a) {
    ssd_walk<N, false, true>(a);
}

// ---------------------------------------------------------------------------
// ssd_seg_fold: the starting state of every segment after the first, in
// order: start(k + 1) = 2^decay(k) start(k) + local(k), start(0) = h0 (or
// zero), written over local(k).  One workgroup per (batch row, head); each
// thread carries kPieces float4 of the 64 x N state, and the next segment's
// pieces are loaded before this segment's are stored.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(kThreads) void ssd_seg_fold(SsdArgs a) {
    constexpr int kPieces = kP * N / 4 / kThreads;       // 4, 8 or 16
    const int64_t bh = blockIdx.x, nslot = a.n_seg - 1;
    const int tid = threadIdx.x;
    float4 v[kPieces], nxt[kPieces];
    const float4* h0 = a.h0 ? reinterpret_cast<const float4*>(a.h0 + bh * kP * N) : nullptr;
    float4* base = reinterpret_cast<float4*>(a.seg_state + bh * nslot * kP * N);
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
        v[k] = h0 ? h0[tid + kThreads * k] : make_float4(0.f, 0.f, 0.f, 0.f);
        nxt[k] = base[tid + kThreads * k];
    }
    for (int64_t sl = 0; sl < nslot; ++sl) {
        const float d = __builtin_amdgcn_exp2f(a.seg_decay[bh * nslot + sl]);
        float4* cur = base + sl * (kP * N / 4);
        float4 loc[kPieces];
#pragma unroll
        for (int k = 0; k < kPieces; ++k) loc[k] = nxt[k];
        const int64_t sn = sl + 1 < nslot ? sl + 1 : sl;   // the last slot reloads itself
#pragma unroll
        for (int k = 0; k < kPieces; ++k) nxt[k] = base[sn * (kP * N / 4) + tid + kThreads * k];
#pragma unroll
        for (int k = 0; k < kPieces; ++k) {
            v[k] = make_float4(fmaf(d, v[k].x, loc[k].x), fmaf(d, v[k].y, loc[k].y), fmaf(d, v[k].z, loc[k].z),
                               fmaf(d, v[k].w, loc[k].w));
            cur[tid + kThreads * k] = v[k];
        }
    }
}

}  // namespace ssd

using namespace ssd;

int64_t ssd_gram_bytes(int64_t batch, int64_t L) { return batch * ((L + kQ - 1) / kQ) * kQ * kQ * 2; }

// Workgroups of ssd_chunked resident per CU (LDS and VGPRs): 3 up to N = 128,
// 2 at N = 256.  Sequences (batch rows x heads) are cut into as many segments
// as keep every (sequence, segment) workgroup resident at once, never more:
// a CU's throughput, not one workgroup's chain, bounds the walk from two
// workgroups per CU on.
constexpr int64_t kCUs = 256;
// A segment spans at least this many chunks (1024 tokens): its first pass and
// the fold then add little to the walk itself.
constexpr int64_t kMinSegChunks = 16;

void ssd_segments(int64_t batch, int64_t L, int64_t H, int64_t N, int64_t* n_seg, int64_t* seg_chunks) {
    const int64_t nch = (L + kQ - 1) / kQ, units = batch * H;
    const int64_t resident = kCUs * (N > 128 ? 2 : 3);
    int64_t n = resident / units;
    if (n > nch / kMinSegChunks) n = nch / kMinSegChunks;
    if (n < 2) n = 1;
    const int64_t per = (nch + n - 1) / n;
    *n_seg = (nch + per - 1) / per;
    *seg_chunks = per;
}

int64_t ssd_seg_state_offset(int64_t batch, int64_t L) { return ssd_gram_bytes(batch, L); }

int64_t ssd_seg_decay_offset(int64_t batch, int64_t L, int64_t H, int64_t N, int64_t n_seg) {
    return ssd_gram_bytes(batch, L) + batch * H * (n_seg - 1) * kP * N * 4;
}

int64_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t N) {
    int64_t n_seg, per;
    ssd_segments(batch, L, H, N, &n_seg, &per);
    if (n_seg == 1) return ssd_gram_bytes(batch, L);
    return ssd_seg_decay_offset(batch, L, H, N, n_seg) + batch * H * (n_seg - 1) * 4;
}

template <int N>
static hipError_t launch_ssd_n(const SsdArgs& a, hipStream_t stream) {
    dim3 g0(static_cast<unsigned>(a.batch * ((a.L + kQ - 1) / kQ)));
    s6_timing_mark("ssd_gram", stream, true);
    hipLaunchKernelGGL((ssd_gram<N>), g0, dim3(kThreads), 0, stream, a);
    s6_timing_mark("ssd_gram", stream, false);
    if (a.n_seg > 1) {
        dim3 g1(static_cast<unsigned>(a.batch * (a.n_seg - 1) * a.H));
        s6_timing_mark("ssd_seg_local", stream, true);
        hipLaunchKernelGGL((ssd_seg_local<N>), g1, dim3(kThreads), 0, stream, a);
        s6_timing_mark("ssd_seg_local", stream, false);
        dim3 g2(static_cast<unsigned>(a.batch * a.H));
        s6_timing_mark("ssd_seg_fold", stream, true);
        hipLaunchKernelGGL((ssd_seg_fold<N>), g2, dim3(kThreads), 0, stream, a);
        s6_timing_mark("ssd_seg_fold", stream, false);
    }
    dim3 grid(static_cast<unsigned>(a.batch * a.n_seg * a.H));
    s6_timing_mark("ssd_chunked", stream, true);
    // one instantiation for gated and ungated layers: the gate is a uniform branch on a.z (the
    // ungated instantiation at N = 128 does not fit its registers with the two-part state update)
    hipLaunchKernelGGL((ssd_chunked<N, true>), grid, dim3(kThreads), 0, stream, a);
    s6_timing_mark("ssd_chunked", stream, false);
    return hipGetLastError();
}

hipError_t ssd_launch(const SsdArgs& a, hipStream_t stream) {
    switch (a.N) {
        case 64: return launch_ssd_n<64>(a, stream);
        case 128: return launch_ssd_n<128>(a, stream);
        case 256: return launch_ssd_n<256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
