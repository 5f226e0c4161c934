// gfx950 kernels of the selective scan (S6) backward pass.
//
// The pages' kernel keeps the expanded states on chip and recomputes them for
// the backward pass instead of storing the (batch, L, D, N) tensor ("DL0170
// Mamba Selective SSM vs Attention", point (3) and the paragraph after
// Figure 1).  Here, with the forward's layout (one lane per channel, its 16
// states in VGPRs, B_t / C_t as SGPR operands):
//
//   dy_t   = dout_t * silu(z_t)                     (dout_t when ungated)
//   mu_t   = dJ/dh_t = C_t dy_t + Abar_{t+1} mu_{t+1}, mu_{L-1} also gets dh_last
//   w_tn   = mu_tn Abar_tn h_{t-1,n}                (dJ/d(Delta_t A_n))
//   dx_t   = Delta_t sum_n mu_tn B_tn + Dskip dy_t
//   dDelta = x_t sum_n mu_tn B_tn + sum_n w_tn A_n,  ddelta_t = dDelta sigmoid(v_t)
//   dA_n  += w_tn Delta_t,   dB_tn += mu_tn Delta_t x_t,   dC_tn += dy_t h_tn
//
// The adjoint mu runs backward in time and has the same chunk algebra as the
// state: a chunk scanned backward from mu = 0 leaves (S = sum Delta,
// Lambda = Abar_{t0} mu_{t0}), and the incoming adjoint of chunk c-1 is
// Lambda_c + exp(A S_c) * (incoming adjoint of chunk c).  Launch order:
//   1. s6_bwd_carries, two independent jobs in one grid so that the
//      HBM-bound one overlaps the VALU-bound one:
//      - every chunk scanned from a zero state, storing the local state at
//        each sub-chunk start and leaving the chunk carry;
//      - the adjoint carries of chunks 1..n-1;
//   2. s6_carry_scan2: the forward fold (starting state per chunk) and the
//      reverse fold from dh_last (incoming adjoint per chunk) in one grid;
//   3. s6_chunk_bwd: per chunk, sub-chunk by sub-chunk from the end, the
//      sub-chunk's starting state is rebuilt from its checkpoint, its states are
//      recomputed into registers (their decays set aside in LDS) and the
//      adjoint runs back through them;
//   4. s6_bwd_reduce: deterministic sums of the per-wavefront dB, dC and the
//      per-chunk dA, dDskip, ddt_bias partials, one grid for both.

#include "s6_device.h"

namespace s6 {

// x, delta, dout and z of kBlk tokens in reverse order: block k holds the
// tokens first - j rows (j = 0..kBlk-1); rows before the chunk start are
// clamped to row 0 and masked by the caller.
template <class LD, int NT>
struct StageRev {
    using IO = typename LD::IO;
    typename LD::R r[NT][kBlk];
    float v[NT][kBlk];

    __device__ __forceinline__ void issue(const LD& ld, const ChunkIO<IO> (&src)[NT], uint32_t vo, int first_row,
                                          uint32_t rowb) {
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int row = first_row - j;
            const uint32_t o = static_cast<uint32_t>(row > 0 ? row : 0) * rowb;
#pragma unroll
            for (int k = 0; k < NT; ++k) r[k][j] = ld.load(src[k], vo, o);
        }
    }
    __device__ __forceinline__ void widen(const LD& ld) {
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
            for (int j = 0; j < kBlk; ++j) v[k][j] = ld.widen(r[k][j]);
    }
};

__device__ __forceinline__ float gate_grad(float g, float z, float& dz_per_y) {
    // dy = g silu(z); dJ/dz = g y sigmoid(z) (1 + z (1 - sigmoid(z))), returned per unit y
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
    dz_per_y = g * sg * fmaf(z, 1.0f - sg, 1.0f);
    return g * z * sg;
}

// ---------------------------------------------------------------------------
// adjoint carries of chunks 1..n-1
// ---------------------------------------------------------------------------
template <class LD, bool GATED>
__device__ __forceinline__ void carry_rev_body(const S6BwdArgs& a, int64_t bid) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = GATED ? 3 : 2;          // delta, dout, z
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a.batch, a.L, a.D, a.chunk_len, a.n_chunks - 1, 1, g, bid)) return;
    const uint32_t rowb = static_cast<uint32_t>(a.D) * es;
    const uint32_t bytes = static_cast<uint32_t>(g.nt) * rowb;
    const int64_t e0 = g.row0 * a.D;
    ChunkIO<IO> src[NT];
    src[0].init(static_cast<const T*>(a.delta) + e0, bytes);
    src[1].init(static_cast<const T*>(a.dout) + e0, bytes);
    if (GATED) src[2].init(static_cast<const T*>(a.z) + e0, bytes);
    const T* Cc = static_cast<const T*>(a.C) + g.row0 * kN;
    const uint32_t vo = ld.voff(g.d);

    float A2[kN], rho[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) { A2[n] = a.A[g.d * kN + n] * kLog2e; rho[n] = 0.0f; }
    const float bias = a.dt_bias[g.d];
    float S = 0.0f;

    StageRev<LD, NT> st;
    st.issue(ld, src, vo, g.nt - 1, rowb);
    st.widen(ld);
    RowBC<IO> cq[2];
    cq[0].load(Cc + (g.nt - 1) * kN);
    for (int tb = 0; tb < g.nt; tb += kBlk) {
        st.issue(ld, src, vo, g.nt - 1 - tb - kBlk, rowb);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int tt = g.nt - 1 - (tb + j);
            const bool valid = tt >= 0;                 // wave-uniform
            lgkm_wait_all();
            cq[(j + 1) & 1].load(Cc + max(tt - 1, 0) * kN);
            const RowBC<IO>& Cv = cq[j & 1];
            const float dt = valid ? softplus(st.v[0][j] + bias) : 0.0f;
            float dy = st.v[1][j];
            if (GATED) {
                float unused;
                dy = gate_grad(dy, st.v[2][j], unused);
            }
            dy = valid ? dy : 0.0f;
            S += dt;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float mu = fmaf(Cv.get(n), dy, rho[n]);
                rho[n] = __builtin_amdgcn_exp2f(dt * A2[n]) * mu;
            }
        }
        st.widen(ld);
    }
    const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c - 1;
    a.rcarry_S[cs * a.D + g.d] = S;
#pragma unroll
    for (int n = 0; n < kN; ++n) a.rcarry_H[(cs * kN + n) * a.D + g.d] = rho[n];
}

// ---------------------------------------------------------------------------
// local states at every sub-chunk start (and the chunk carries)
// ---------------------------------------------------------------------------
// Every chunk (the last one too) is scanned from a zero state; before each
// sub-chunk j >= 1 the local state and the step-size sum so far are stored
// (17 values per lane), so that the backward pass gets the true state there
// as local + exp(A * sum Delta) * (chunk starting state) instead of re-running
// the chunk.  Chunks 0..n-2 also leave their carry for the state fold.
template <class LD>
__device__ __forceinline__ void ckpt_body(const S6BwdArgs& a, int64_t bid) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = 2;
    constexpr int SUB = kBwdSub;
    static_assert(SUB % kBlk == 0, "a sub-chunk starts at a load block");
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a.batch, a.L, a.D, a.chunk_len, a.n_chunks, 0, g, bid)) return;
    const uint32_t rowb = static_cast<uint32_t>(a.D) * es;
    const uint32_t last = static_cast<uint32_t>(g.nt - 1) * rowb;
    const int64_t e0 = g.row0 * a.D;
    ChunkIO<IO> src[NT];
    src[0].init(static_cast<const T*>(a.x) + e0, last + rowb);
    src[1].init(static_cast<const T*>(a.delta) + e0, last + rowb);
    const T* Bc = static_cast<const T*>(a.B) + g.row0 * kN;
    const uint32_t vo = ld.voff(g.d);
    const int64_t nsub_max = a.chunk_len / SUB;
    float* ck = a.ckpt + ((static_cast<int64_t>(g.b) * a.n_chunks + g.c) * nsub_max * (kN + 1)) * a.D + g.d;
    Stage<LD, NT> st;

    float A2[kN], h[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) { A2[n] = a.A[g.d * kN + n] * kLog2e; h[n] = 0.0f; }
    const float bias = a.dt_bias[g.d];
    float S = 0.0f;

    st.issue(ld, src, vo, 0, rowb, last);
    st.widen(ld);
    RowBC<IO> bc[2];
    bc[0].load(Bc);
    for (int tb = 0; tb < g.nt; tb += kBlk) {
        st.issue(ld, src, vo, static_cast<uint32_t>(tb + kBlk) * rowb, rowb, last);
        if (tb > 0 && tb % SUB == 0) {                   // wave-uniform
            float* p = ck + static_cast<int64_t>(tb / SUB) * (kN + 1) * a.D;
#pragma unroll
            for (int n = 0; n < kN; ++n) p[n * a.D] = h[n];
            p[kN * a.D] = S;
        }
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int tt = tb + j;
            const bool valid = tt < g.nt;                 // wave-uniform
            lgkm_wait_all();
            bc[(j + 1) & 1].load(Bc + min(tt + 1, g.nt - 1) * kN);
            const RowBC<IO>& Bv = bc[j & 1];
            const float dt = valid ? softplus(st.v[1][j] + bias) : 0.0f;
            const float dx = dt * st.v[0][j];
            S += dt;
#pragma unroll
            for (int n = 0; n < kN; ++n)
                h[n] = fmaf(__builtin_amdgcn_exp2f(dt * A2[n]), h[n], dx * Bv.get(n));
        }
        st.widen(ld);
    }
    if (g.c < a.n_chunks - 1) {
        const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c;
        a.carry_S[cs * a.D + g.d] = S;
#pragma unroll
        for (int n = 0; n < kN; ++n) a.carry_H[(cs * kN + n) * a.D + g.d] = h[n];
    }
}

// The checkpoint pass (HBM-bound: it writes the checkpoints) and the adjoint
// carry pass (VALU-bound) are independent: one launch runs both, so they
// overlap on the chip.  Workgroups are dispatched in index order, so the two
// jobs alternate in runs of kXcds (one workgroup of each per XCD) and are
// resident together; a job's unit u keeps u % kXcds = blockIdx.x % kXcds, the
// XCD its chunk mapping expects.
template <class LD, bool GATED>
__global__ __launch_bounds__(kBlock) void s6_bwd_carries(S6BwdArgs a) {
    const int64_t nblk = (a.D + kBlock - 1) / kBlock * a.batch;
    const int64_t i = blockIdx.x, r = i % (2 * kXcds);
    const int64_t u = i / (2 * kXcds) * kXcds + r % kXcds;
    if (r < kXcds) {
        if (u < nblk * a.n_chunks) ckpt_body<LD>(a, u);
    } else {
        if (u < nblk * (a.n_chunks - 1)) carry_rev_body<LD, GATED>(a, u);
    }
}

// ---------------------------------------------------------------------------
// sums of 16 per-lane values over the wavefront
// ---------------------------------------------------------------------------
// Reduce-scatter by halving: at each level a lane keeps one half of its
// values and adds the same half from a partner lane that differs in one
// lane-index bit, while the partner keeps (and receives) the other half.
// Lane distance 32 and 16 use the gfx950 half-swaps (one instruction moves a
// pair of registers), distance 8 a DPP row rotation, and the last three lane
// bits DPP mirrors and quad permutes inside rows.  Afterwards lane l holds the
// wavefront sum of value l >> 2 (lanes 4i..4i+3 hold the same sum).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor8 = 0x128;         // lane i of a 16-lane row reads lane (i + 8) mod 16
constexpr int kDppRowHalfMirror = 0x141;   // lane i of an 8-lane half row reads lane 7 - i
constexpr int kDppQuadSwap2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadSwap1 = 0xb1;        // quad_perm [1, 0, 3, 2]

__device__ __forceinline__ float wave_sum16(float (&v)[16]) {
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    // distance 32: v[i] (kept by lanes 0-31) and v[i+8] (kept by lanes 32-63)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 8]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // distance 16: rows 0 and 2 keep v[i], rows 1 and 3 keep v[i+4]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 4]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // distance 8 inside a row, then lane bit 2 via the half-row mirror
    const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b3 ? v[i] : v[i + 2];
        const float keep = b3 ? v[i + 2] : v[i];
        v[i] = keep + dpp<kDppRowRor8>(send);
    }
    {
        const float send = b2 ? v[0] : v[1];
        const float keep = b2 ? v[1] : v[0];
        v[0] = keep + dpp<kDppRowHalfMirror>(send);
    }
    const float s = v[0] + dpp<kDppQuadSwap2>(v[0]);
    return s + dpp<kDppQuadSwap1>(s);
}

// A copy of a wave-uniform pointer that the compiler cannot prove equal to
// the original, so scalar loads through it are not merged with earlier loads
// of the same rows (which would keep those rows live in SGPRs in between).
template <class P>
__device__ __forceinline__ P* opaque(P* p) {
    asm volatile("" : "+s"(p));
    return p;
}

// ---------------------------------------------------------------------------
// per-chunk backward
// ---------------------------------------------------------------------------
template <class LD, bool GATED>
__global__ __launch_bounds__(kBlock, 2) void s6_chunk_bwd(S6BwdArgs a) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int SUB = kBwdSub;
    static_assert(SUB % kBlk == 0 || kBlk % SUB == 0, "sub-chunks and load blocks must nest");
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a.batch, a.L, a.D, a.chunk_len, a.n_chunks, 0, g)) return;
    const int64_t D = a.D;
    const uint32_t rowb = static_cast<uint32_t>(D) * es;
    const uint32_t last = static_cast<uint32_t>(g.nt - 1) * rowb;
    const int64_t e0 = g.row0 * D;
    ChunkIO<IO> X, DL, GO, Z, DX, DDL, DZ;
    X.init(static_cast<const T*>(a.x) + e0, last + rowb);
    DL.init(static_cast<const T*>(a.delta) + e0, last + rowb);
    GO.init(static_cast<const T*>(a.dout) + e0, last + rowb);
    DX.init(static_cast<T*>(a.dx) + e0, last + rowb);
    DDL.init(static_cast<T*>(a.ddelta) + e0, last + rowb);
    if (GATED) {
        Z.init(static_cast<const T*>(a.z) + e0, last + rowb);
        DZ.init(static_cast<T*>(a.dz) + e0, last + rowb);
    }
    const T* Bc = static_cast<const T*>(a.B) + g.row0 * kN;
    const T* Cc = static_cast<const T*>(a.C) + g.row0 * kN;
    const uint32_t vo = ld.voff(g.d);
    const uint32_t vs = g.d * es;
    const int nsub = (g.nt + SUB - 1) / SUB;
    const int64_t nsub_max = a.chunk_len / SUB;
    const float* ck = a.ckpt + ((static_cast<int64_t>(g.b) * a.n_chunks + g.c) * nsub_max * (kN + 1)) * D + g.d;

    float A2[kN], hc[kN];      // hc: the chunk's starting state
#pragma unroll
    for (int n = 0; n < kN; ++n) A2[n] = a.A[g.d * kN + n] * kLog2e;
    const float bias = a.dt_bias[g.d];
    const float Dd = a.Dskip[g.d];
    const int64_t bd = static_cast<int64_t>(g.b) * D + g.d;
    if (g.c > 0) {
        const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c - 1;
#pragma unroll
        for (int n = 0; n < kN; ++n) hc[n] = a.carry_H[(cs * kN + n) * D + g.d];
    } else if (a.h0) {
#pragma unroll
        for (int n = 0; n < kN; ++n) hc[n] = a.h0[bd * kN + n];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) hc[n] = 0.0f;
    }

    // The true state at the start of sub-chunk j >= 1 is its local state (from a
    // zero state at the chunk start) plus the chunk's starting state decayed
    // by exp(A * sum Delta) over the sub-chunks before it.  The chunk's starting
    // state waits in LDS (four values per 16-byte slot, lanes contiguous).
    __shared__ float4 hst_lds[kBlock / kWave][kN / 4][kWave];
    // The decays Abar of the sub-chunk's tokens, from the recompute pass to the
    // adjoint pass (registers are full; recomputing them costs 2 VALU per state
    // and token, LDS a write and a read per four states).  64 KB: with the
    // starting states, two workgroups fill a CU's 160 KB.
    __shared__ float4 abar_lds[kBlock / kWave][SUB][kN / 4][kWave];
    const int wv = static_cast<int>(threadIdx.x) >> 6, ln = static_cast<int>(threadIdx.x) & (kWave - 1);
#pragma unroll
    for (int k = 0; k < kN / 4; ++k) hst_lds[wv][k][ln] = make_float4(hc[4 * k], hc[4 * k + 1], hc[4 * k + 2], hc[4 * k + 3]);
    // Checkpoint j's 17 values are loaded one sub-chunk ahead (raw) and combined
    // with the starting state only when needed, so the load latency is hidden.
    auto ck_load = [&](int j, float (&loc)[kN], float& sl) {
        const float* p = ck + static_cast<int64_t>(j) * (kN + 1) * D;
#pragma unroll
        for (int n = 0; n < kN; ++n) loc[n] = p[n * D];
        sl = p[kN * D];
    };
    auto ck_combine = [&](int j, const float (&loc)[kN], float sl, float (&out)[kN]) {
#pragma unroll
        for (int k = 0; k < kN / 4; ++k) {
            const float4 v = hst_lds[wv][k][ln];          // written by this lane: no barrier needed
            const float hs0[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 4 * k + i;
                out[n] = j == 0 ? hs0[i] : fmaf(__builtin_amdgcn_exp2f(sl * A2[n]), hs0[i], loc[n]);
            }
        }
    };
    // the checkpoint of the last sub-chunk; each iteration below combines the
    // pending one into a fresh starting state (no state is carried across
    // iterations in registers, so the recompute needs no copies of it)
    float hn[kN], sn = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) hn[n] = 0.0f;
    if (nsub > 1) ck_load(nsub - 1, hn, sn);

    // 2. sub-chunks from the last to the first
    float rho[kN], dA[kN];
    if (g.c < a.n_chunks - 1) {
        const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c;
#pragma unroll
        for (int n = 0; n < kN; ++n) rho[n] = a.rcarry_H[(cs * kN + n) * D + g.d];
    } else if (a.dh_last) {
#pragma unroll
        for (int n = 0; n < kN; ++n) rho[n] = a.dh_last[bd * kN + n];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) rho[n] = 0.0f;
    }
#pragma unroll
    for (int n = 0; n < kN; ++n) dA[n] = 0.0f;
    float dD = 0.0f, dbias = 0.0f;
    const int64_t G = (D + kWave - 1) / kWave;
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    float* pbc = a.part_bc + (g.row0 * G + g.group) * (2 * kN) + (lane >> 2);

    // Raw loads of a sub-chunk's tokens (rows past the chunk end clamp to its last
    // row).  The next sub-chunk's loads, and its starting state, are issued
    // before the current sub-chunk's adjoint pass, so they land meanwhile.
    typename LD::R rx[SUB], rd[SUB], rg[SUB], rz[SUB];
    auto issue = [&](int t0) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            const uint32_t o = min(static_cast<uint32_t>(t0 + i) * rowb, last);
            rx[i] = ld.load(X, vo, o);
            rd[i] = ld.load(DL, vo, o);
            rg[i] = ld.load(GO, vo, o);
            if (GATED) rz[i] = ld.load(Z, vo, o);
        }
    };
    issue((nsub - 1) * SUB);
    for (int j = nsub - 1; j >= 0; --j) {
        const int t0 = j * SUB;
        float h[kN];
        ck_combine(j, hn, sn, h);
        // recompute: states before each token, step sizes, dy (and dz)
        float hs[SUB][kN];
        float xs[SUB], dts[SUB], sgs[SUB], dys[SUB];
        {
            const T* Bs = opaque(Bc);
            const T* Cs = opaque(Cc);
            RowBC<IO> bq[2], cq[2];
            lgkm_wait_all();
            bq[0].load(Bs + min(t0, g.nt - 1) * kN);
            if (GATED) cq[0].load(Cs + min(t0, g.nt - 1) * kN);
#pragma unroll
            for (int i = 0; i < SUB; ++i) {
                const int tt = t0 + i;
                const bool valid = tt < g.nt;                    // wave-uniform
                lgkm_wait_all();
                if (i + 1 < SUB) {
                    bq[(i + 1) & 1].load(Bs + min(tt + 1, g.nt - 1) * kN);
                    if (GATED) cq[(i + 1) & 1].load(Cs + min(tt + 1, g.nt - 1) * kN);
                }
                const RowBC<IO>& Bv = bq[i & 1];
                const RowBC<IO>& Cv = cq[i & 1];
#pragma unroll
                for (int n = 0; n < kN; ++n) hs[i][n] = h[n];
                const float xv = ld.widen(rx[i]);
                float sg = 0.0f;
                const float dt = valid ? softplus_sig(ld.widen(rd[i]) + bias, sg) : 0.0f;
                const float u = dt * xv;
                xs[i] = xv;
                dts[i] = dt;
                sgs[i] = sg;
                float yv = Dd * xv;
#pragma unroll
                for (int k = 0; k < kN / 4; ++k) {
                    float ab[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int n = 4 * k + m;
                        ab[m] = __builtin_amdgcn_exp2f(dt * A2[n]);
                        h[n] = fmaf(ab[m], h[n], u * Bv.get(n));
                        if (GATED) yv = fmaf(Cv.get(n), h[n], yv);
                    }
                    abar_lds[wv][i][k][ln] = make_float4(ab[0], ab[1], ab[2], ab[3]);
                }
                float gv = ld.widen(rg[i]);
                if (GATED) {
                    float dzy;
                    gv = gate_grad(gv, ld.widen(rz[i]), dzy);
                    if (valid) store_io(DZ, vs, static_cast<uint32_t>(tt) * rowb, dzy * yv);
                }
                dys[i] = gv;
            }
        }
        if (j > 0) {
            issue(t0 - SUB);
            if (j > 1) ck_load(j - 1, hn, sn);
        }
        // adjoint back through the sub-chunk
        {
            const T* Bs = opaque(Bc);
            const T* Cs = opaque(Cc);
            RowBC<IO> bq[2], cq[2];
            const int tl = min(t0 + SUB - 1, g.nt - 1);
            lgkm_wait_all();
            bq[(SUB - 1) & 1].load(Bs + tl * kN);
            cq[(SUB - 1) & 1].load(Cs + tl * kN);
#pragma unroll
            for (int i = SUB - 1; i >= 0; --i) {
                const int tt = t0 + i;
                lgkm_wait_all();
                if (i > 0) {
                    bq[(i - 1) & 1].load(Bs + min(tt - 1, g.nt - 1) * kN);
                    cq[(i - 1) & 1].load(Cs + min(tt - 1, g.nt - 1) * kN);
                }
                if (tt >= g.nt) continue;                         // wave-uniform
                const RowBC<IO>& Bv = bq[i & 1];
                const RowBC<IO>& Cv = cq[i & 1];
                const float dy = dys[i];
                const float dt = dts[i];
                float abar[kN];
#pragma unroll
                for (int k = 0; k < kN / 4; ++k) {
                    const float4 v = abar_lds[wv][i][k][ln];     // written by this lane: no barrier needed
                    abar[4 * k] = v.x; abar[4 * k + 1] = v.y; abar[4 * k + 2] = v.z; abar[4 * k + 3] = v.w;
                }
                const float u = dt * xs[i];
                // the dB / dC terms of lanes that only duplicate channel D-1 must add nothing
                const float uk = g.active ? u : 0.0f;
                const float dyk = g.active ? dy : 0.0f;
                float du = 0.0f, sw = 0.0f;
                float pb[kN], pc[kN];
#pragma unroll
                for (int n = 0; n < kN; ++n) {
                    const float ht = (i == SUB - 1) ? h[n] : hs[i + 1][n];
                    const float mu = fmaf(Cv.get(n), dy, rho[n]);
                    du = fmaf(mu, Bv.get(n), du);
                    pc[n] = dyk * ht;
                    const float q = abar[n] * mu;
                    const float w = q * hs[i][n];
                    sw = fmaf(w, A2[n], sw);
                    dA[n] = fmaf(w, dt, dA[n]);
                    pb[n] = mu * uk;
                    rho[n] = q;
                }
                const float dxv = fmaf(du, dt, dy * Dd);
                const float dv = fmaf(sw, kLn2, du * xs[i]) * sgs[i];
                const uint32_t so = static_cast<uint32_t>(tt) * rowb;
                store_io(DX, vs, so, dxv);
                store_io(DDL, vs, so, dv);
                dD = fmaf(dy, xs[i], dD);
                dbias += dv;
                const float sb = wave_sum16(pb);
                const float sc = wave_sum16(pc);
                if ((lane & 3) == 0) {
                    float* q = pbc + static_cast<int64_t>(tt) * G * (2 * kN);
                    q[0] = sb;
                    q[kN] = sc;
                }
            }
        }
    }
    if (g.c == 0 && a.dh0) {
#pragma unroll
        for (int n = 0; n < kN; ++n) a.dh0[bd * kN + n] = rho[n];
    }
    if (g.active) {
        float* pp = a.part_p + (static_cast<int64_t>(g.b) * a.n_chunks + g.c) * kBwdParams * D + g.d;
#pragma unroll
        for (int n = 0; n < kN; ++n) pp[n * D] = dA[n];
        pp[kN * D] = dD;
        pp[(kN + 1) * D] = dbias;
    }
}

// ---------------------------------------------------------------------------
// deterministic reductions of the partial sums
// ---------------------------------------------------------------------------
// dB, dC: one lane per (b, t, k), k < 2N; sums the ceil(D / 64) wavefront partials.
__device__ __forceinline__ void reduce_bc_body(const S6BwdArgs& a, int64_t bid) {
    const int64_t i = bid * kBlock + threadIdx.x;
    if (i >= a.batch * a.L * 2 * kN) return;
    const int64_t row = i / (2 * kN);
    const int k = static_cast<int>(i % (2 * kN));
    const int64_t G = (a.D + kWave - 1) / kWave;
    const float* p = a.part_bc + row * G * (2 * kN) + k;
    float s = 0.0f;
    for (int64_t gi = 0; gi < G; ++gi) s += p[gi * 2 * kN];
    if (k < kN) a.dB[row * kN + k] = s;
    else a.dC[row * kN + k - kN] = s;
}

// dA, dDskip, ddt_bias: a workgroup per (64 channels, parameter k); its four
// wavefronts sum every fourth (batch row, chunk) partial with eight
// independent accumulators, then wavefront 0 adds the four sums in a fixed
// order.
__device__ __forceinline__ void reduce_params_body(const S6BwdArgs& a, int64_t bid, float (&part)[kBlock / kWave][kWave]) {
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    const int64_t gd = (a.D + kWave - 1) / kWave;
    const int64_t k = bid / gd;
    const int64_t dl = (bid % gd) * kWave + lane;
    const int64_t d = dl < a.D ? dl : a.D - 1;
    const int64_t units = a.batch * a.n_chunks;
    const int64_t stride = kBwdParams * a.D;
    const float* p = a.part_p + k * a.D + d;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    int64_t u = wave;
    for (; u + 7 * 4 < units; u += 8 * 4) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += p[(u + 4 * j) * stride];
    }
    for (int j = 0; u < units; u += 4, ++j) acc[j & 7] += p[u * stride];
    part[wave][lane] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    if (wave == 0 && dl < a.D) {
        const float s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
        if (k < kN) a.dA[d * kN + k] = s;
        else if (k == kN) a.dDskip[d] = s;
        else a.ddt_bias[d] = s;
    }
}

// Both reductions in one launch: workgroups [0, ceil(D / 64) * 18) reduce the
// parameters, the rest dB and dC.
__global__ __launch_bounds__(kBlock) void s6_bwd_reduce(S6BwdArgs a) {
    __shared__ float part[kBlock / kWave][kWave];
    const int64_t first = (a.D + kWave - 1) / kWave * kBwdParams;
    const int64_t i = blockIdx.x;
    if (i < first) reduce_params_body(a, i, part);
    else reduce_bc_body(a, i - first);
}

}  // namespace s6

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
using namespace s6;

template <class LD, bool GATED>
static hipError_t launch_bwd_t(const S6BwdArgs& a, hipStream_t stream) {
    const int64_t nblk = (a.D + kBlock - 1) / kBlock * a.batch;
    dim3 g0(static_cast<unsigned>((nblk * a.n_chunks + kXcds - 1) / kXcds * 2 * kXcds));
    s6_timing_mark("s6_bwd_carries", stream, true);
    hipLaunchKernelGGL((s6_bwd_carries<LD, GATED>), g0, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_bwd_carries", stream, false);
    if (a.n_chunks > 1)
        s6_launch_fold2(S6FoldArgs{a.A, a.h0, a.carry_S, a.carry_H, a.batch, a.D, a.n_chunks - 1, 0},
                        S6FoldArgs{a.A, a.dh_last, a.rcarry_S, a.rcarry_H, a.batch, a.D, a.n_chunks - 1, 1},
                        "s6_carry_scan2", stream);
    dim3 g3(static_cast<unsigned>(nblk * a.n_chunks));
    s6_timing_mark("s6_chunk_bwd", stream, true);
    hipLaunchKernelGGL((s6_chunk_bwd<LD, GATED>), g3, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_chunk_bwd", stream, false);
    const int64_t nbc = a.batch * a.L * 2 * kN;
    const int64_t nred = (a.D + kWave - 1) / kWave * kBwdParams + (nbc + kBlock - 1) / kBlock;
    s6_timing_mark("s6_bwd_reduce", stream, true);
    hipLaunchKernelGGL(s6_bwd_reduce, dim3(static_cast<unsigned>(nred)), dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_bwd_reduce", stream, false);
    return hipGetLastError();
}

hipError_t s6_launch_bwd(const S6BwdArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16 && a.pair_loads)
        return gated ? launch_bwd_t<LdPairBF16, true>(a, stream) : launch_bwd_t<LdPairBF16, false>(a, stream);
    if (a.bf16) return gated ? launch_bwd_t<LdBF16, true>(a, stream) : launch_bwd_t<LdBF16, false>(a, stream);
    return gated ? launch_bwd_t<LdF32, true>(a, stream) : launch_bwd_t<LdF32, false>(a, stream);
}
