// gfx950 kernels of the selective scan (S6) forward and its decode step.
//
// Work layout of the scans: one lane per channel d, all 16 state values of
// that channel in VGPRs, a wavefront = 64 consecutive channels of one batch
// row, a workgroup = 4 such wavefronts (independent: no LDS, no barriers).
// B_t and C_t are the same for every channel of a batch row ("Mamba",
// "Selectivity": B and C are functions of the token), so a wavefront reads
// them with scalar loads and the state updates take them as SGPR operands.
// (An SGPR operand halves an fp32 instruction's issue rate on gfx950; fp32
// copies of the rows staged through LDS for VGPR operands were measured
// slower: 39 more VGPRs cost two of the six wavefronts per SIMD.)
//
// Long sequences are cut into chunks ("Mamba", "Scan View": the recurrence
// is an associative scan over the pairs (Abar_t, Bbar_t x_t)):
//   1. s6_chunk_carry: every chunk but the last scans from a zero state and
//      writes its carry (S = sum of Delta, H = end state) per channel.
//   2. s6_carry_scan: per channel and state, the carries are combined in
//      chunk order from h0 -- (S1,H1) then (S2,H2) = (S1+S2, exp(A S2) H1 + H2),
//      where exp(A * sum Delta) is exactly the product of the chunk's Abar --
//      and each prefix (the true starting state of the next chunk) replaces
//      that chunk's H in place.
//   3. s6_chunk_out: every chunk rescans its tokens from its starting state,
//      writing the gated output; the last chunk also writes h_L.
//
// Workgroup mapping: workgroups are dealt to the 8 XCDs round-robin by their
// linear index, and every XCD has its own L2.  The kernels decode their
// (channel block, chunk, batch row) from the linear index so that each XCD
// owns a contiguous range of channel blocks with all their chunks: B/C rows
// of a batch row are shared in that XCD's L2, and carries stay on one XCD.
// The (batch, L, D, N) states are never written to memory ("DL0170 Mamba
// Selective SSM vs Attention", engineering paragraph after Figure 1).
//
// Addressing: x, delta, z and y of one chunk are read and written through
// buffer resources based at the chunk's first token, with the lane's channel
// as the VGPR offset and the token's row offset as one SGPR offset shared by
// all four tensors, so the token loop does no per-lane address arithmetic.

#include "s6_device.h"

namespace s6 {

// ---------------------------------------------------------------------------
// the local convolution before the scan (K = 0: none)
// ---------------------------------------------------------------------------
// x_t = silu(b_d + sum_k w_dk xin_{t-K+1+k}): a causal depthwise convolution of
// width K along time, then silu.  Each lane keeps its channel's K-1 previous
// inputs in registers, so the convolution reads every input once; a chunk
// starts its window from the K-1 inputs before it (the previous chunk's last
// tokens, or conv_init / zeros before the sequence).
template <class IO, int K>
struct ConvWin {
    float w[K > 0 ? K : 1];
    float bias;
    float win[K > 1 ? K - 1 : 1];

    __device__ __forceinline__ void init(const S6ScanArgs& a, const Geo& g) {
        if constexpr (K > 0) {
            using T = typename IO::T;
#pragma unroll
            for (int k = 0; k < K; ++k) w[k] = a.conv_w[g.d * K + k];
            bias = a.conv_b[g.d];
            const T* X = static_cast<const T*>(a.x);
            const T* I = static_cast<const T*>(a.conv_init);
#pragma unroll
            for (int i = 0; i < K - 1; ++i) {
                const int p = g.t0 - (K - 1) + i;                 // wave-uniform
                if (p >= 0) win[i] = IO::load(X + (static_cast<int64_t>(g.b) * a.L + p) * a.D, g.d);
                else if (I) win[i] = IO::load(I + (static_cast<int64_t>(g.b) * (K - 1) + (K - 1) + p) * a.D, g.d);
                else win[i] = 0.0f;
            }
        }
    }
    // the convolved, activated input of the next token; shifts the window
    __device__ __forceinline__ float apply(float xin) {
        if constexpr (K == 0) {
            return xin;
        } else {
            float v = bias;
#pragma unroll
            for (int k = 0; k < K - 1; ++k) v = fmaf(w[k], win[k], v);
            v = fmaf(w[K - 1], xin, v);
#pragma unroll
            for (int k = 0; k + 1 < K - 1; ++k) win[k] = win[k + 1];
            if constexpr (K > 1) win[K - 2] = xin;
            return silu(v);
        }
    }
    // the last K-1 inputs of the sequence, for a caller that continues the stream
    __device__ __forceinline__ void store_last(const S6ScanArgs& a, const Geo& g) const {
        if constexpr (K > 1) {
            using T = typename IO::T;
            T* O = static_cast<T*>(a.conv_last);
#pragma unroll
            for (int i = 0; i < K - 1; ++i) IO::store(O + (static_cast<int64_t>(g.b) * (K - 1) + i) * a.D, g.d, win[i]);
        }
    }
};

// ---------------------------------------------------------------------------
// phase 1: chunk carries
// ---------------------------------------------------------------------------
template <class LD, int K>
__global__ __launch_bounds__(kBlock) void s6_chunk_carry(S6ScanArgs a) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = 2;
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a.batch, a.L, a.D, a.chunk_len, a.n_chunks - 1, 0, g)) return;
    const uint32_t rowb = static_cast<uint32_t>(a.D) * es;       // bytes per token row
    const uint32_t last = static_cast<uint32_t>(g.nt - 1) * rowb;
    const int64_t e0 = g.row0 * a.D;                             // element offset of the chunk
    ChunkIO<IO> src[NT];
    src[0].init(static_cast<const T*>(a.x) + e0, last + rowb);
    src[1].init(static_cast<const T*>(a.delta) + e0, last + rowb);
    const T* Bc = static_cast<const T*>(a.B) + g.row0 * kN;
    const uint32_t vo = ld.voff(g.d);
    Stage<LD, NT> st;

    float A2[kN], h[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) { A2[n] = a.A[g.d * kN + n] * kLog2e; h[n] = 0.0f; }
    const float bias = a.dt_bias[g.d];
    float S = 0.0f;
    ConvWin<IO, K> cv;
    cv.init(a, g);

    st.issue(ld, src, vo, 0, rowb, last);
    st.widen(ld);
    RowBC<IO> bc[2];
    bc[0].load(Bc);
    // a carry chunk is never the ragged last one, so nt is a multiple of kBlk
    for (int tb = 0; tb < g.nt; tb += kBlk) {
        st.issue(ld, src, vo, static_cast<uint32_t>(tb + kBlk) * rowb, rowb, last);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int tt = tb + j;
            lgkm_wait_all();
            bc[(j + 1) & 1].load(Bc + min(tt + 1, g.nt - 1) * kN);
            const RowBC<IO>& Bv = bc[j & 1];

            const float dt = softplus(st.v[1][j] + bias);
            const float dx = dt * cv.apply(st.v[0][j]);
            S += dt;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float dA = __builtin_amdgcn_exp2f(dt * A2[n]);
                h[n] = fmaf(dA, h[n], dx * Bv.get(n));
            }
        }
        st.widen(ld);
    }
    const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c;
    a.carry_S[cs * a.D + g.d] = S;
#pragma unroll
    for (int n = 0; n < kN; ++n) a.carry_H[(cs * kN + n) * a.D + g.d] = h[n];
}

// ---------------------------------------------------------------------------
// phase 2: combine the chunk carries (reduce, then scan, then re-fold)
// ---------------------------------------------------------------------------
// One workgroup of W wavefronts per (batch row, 64 channels, state n); lanes
// are channels, so every carry read and every prefix write is a coalesced
// 256-byte row.  The combine of two carries, (S1,H1) then (S2,H2) =
// (S1+S2, e2 H1 + H2) with e = exp(A_n S), is associative ("Mamba", "Scan
// View"), so the ncar carries are scanned in three steps per round of up to
// W x kFoldSeg carries:
//   1. wavefront w loads a contiguous segment of carries into registers (all
//      loads in flight at once), turns each S into e, and folds the segment
//      from zero into its aggregate (E = product of e, H);
//   2. the W aggregates of each channel are transposed through LDS so that a
//      channel's segments sit in W consecutive lanes, and scanned with
//      log2(W) DPP row shifts (Hillis-Steele, the left operand first), giving
//      each segment's exclusive prefix and so its starting state from the
//      round's incoming state;
//   3. every wavefront re-folds its segment from that starting state (the e
//      are still in registers) and writes each prefix over its H in place.
// A carry is read once and written once.  The prefix after carry c is the
// true starting state of chunk c+1.  The forward folds the carries in chunk
// order from h0; the backward folds its adjoint carries in reverse order
// from dh_last (the same combine: the adjoint obeys the transposed recurrence).
constexpr int kFoldSeg = 32;          // carries per wavefront and round
// Wavefronts per workgroup, at most 16 (a DPP row is 16 lanes).  Eight: at
// ~114 VGPRs two such workgroups share a CU, so every unit of a 128k-token
// combine is resident at once and takes its 511 carries in two rounds, one
// round's stores overlapping the next one's loads (33.2 us against 35.5 with
// sixteen wavefronts and one round, 37.3 with four and four rounds).
constexpr int kFoldMaxW = 8;

// value of lane (l - s) in the same 16-lane row; lanes with l % 16 < s keep `self`
__device__ __forceinline__ float row_shr(float self, float v, int s) {
    const int iv = __float_as_int(v), is = __float_as_int(self);
    int r;
    switch (s) {
        case 1: r = __builtin_amdgcn_update_dpp(is, iv, 0x111, 0xf, 0xf, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(is, iv, 0x112, 0xf, 0xf, false); break;
        case 4: r = __builtin_amdgcn_update_dpp(is, iv, 0x114, 0xf, 0xf, false); break;
        default: r = __builtin_amdgcn_update_dpp(is, iv, 0x118, 0xf, 0xf, false); break;
    }
    return __int_as_float(r);
}

// Unit (batch row, 64 channels, state n) of the fold: the lane's channel and
// its carry rows.
struct FoldUnit {
    int64_t b, d, ncar, hs;
    bool active;
    float A2;
    const float* S;
    float* H;
    __device__ __forceinline__ FoldUnit(const S6FoldArgs& a, int64_t unit) {
        const int l = threadIdx.x & (kWave - 1);
        const int64_t gx = (a.D + kWave - 1) / kWave;           // 64-channel groups per batch row
        const int n = static_cast<int>(unit % kN);
        const int64_t grp = unit / kN;
        b = grp / gx;
        const int64_t dl = (grp % gx) * kWave + l;
        active = dl < a.D;
        d = active ? dl : a.D - 1;
        ncar = a.ncar;
        A2 = a.A[d * kN + n] * kLog2e;
        S = a.S + b * ncar * a.D + d;
        H = a.H + (b * ncar * kN + n) * a.D + d;
        hs = kN * a.D;                                          // H stride between carries
    }
    __device__ __forceinline__ int64_t slot(const S6FoldArgs& a, int64_t k) const {
        return a.reverse ? ncar - 1 - k : k;
    }
    __device__ __forceinline__ float init(const S6FoldArgs& a, int64_t unit) const {
        return a.init ? a.init[(b * a.D + d) * kN + unit % kN] : 0.0f;
    }
};

// Chains of at most kFoldSeg carries: one wavefront per unit loads every carry
// at once and folds them in order (no cross-wavefront scan, no LDS).
__device__ __forceinline__ void fold_short(const S6FoldArgs& a, int64_t unit) {
    const FoldUnit u(a, unit);
    const int cnt = static_cast<int>(u.ncar);
    float e[kFoldSeg], hv[kFoldSeg];
#pragma unroll
    for (int k = 0; k < kFoldSeg; ++k) {
        if (k < cnt) {                                              // wave-uniform
            const int64_t c = u.slot(a, k);
            e[k] = u.S[c * a.D];
            hv[k] = u.H[c * u.hs];
        }
    }
    float h = u.init(a, unit);
#pragma unroll
    for (int k = 0; k < kFoldSeg; ++k) {
        if (k < cnt) {
            h = fmaf(__builtin_amdgcn_exp2f(u.A2 * e[k]), h, hv[k]);
            if (u.active) u.H[u.slot(a, k) * u.hs] = h;
        }
    }
}

// W wavefronts per unit (blockDim.x = 64 W), LDS: segment aggregates e, h and
// starting states, W rows of 65 floats each (padded: the transposed reads hit
// distinct banks), and the incoming state of the round (64 floats).
__device__ __forceinline__ void fold_scan(const S6FoldArgs& a, int64_t unit, int W, float* lds) {
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int l = threadIdx.x & (kWave - 1);
    const FoldUnit u(a, unit);
    constexpr int kRow = kWave + 1;
    float* se = lds;
    float* sh = se + W * kRow;
    float* sst = sh + W * kRow;
    float* spre = sst + W * kRow;
    const int64_t ncar = u.ncar;
    if (w == 0) spre[l] = u.init(a, unit);
    // the transposed view of step 2: this thread scans segment sg of channel ch
    const int ch = static_cast<int>(threadIdx.x) / W, sg = static_cast<int>(threadIdx.x) % W;

    for (int64_t base = 0; base < ncar; base += static_cast<int64_t>(W) * kFoldSeg) {
        const int64_t rem = min(ncar - base, static_cast<int64_t>(W) * kFoldSeg);
        const int seg = static_cast<int>((rem + W - 1) / W);
        const int64_t k0 = base + static_cast<int64_t>(w) * seg;
        const int cnt = static_cast<int>(max(min(rem - static_cast<int64_t>(w) * seg, static_cast<int64_t>(seg)),
                                             static_cast<int64_t>(0)));
        // 1. load the segment, fold it from zero
        float e[kFoldSeg], hv[kFoldSeg];
#pragma unroll
        for (int k = 0; k < kFoldSeg; ++k) {
            if (k < cnt) {                                          // wave-uniform
                const int64_t c = u.slot(a, k0 + k);
                e[k] = u.S[c * a.D];
                hv[k] = u.H[c * u.hs];
            }
        }
        float ae = 1.0f, ah = 0.0f;
#pragma unroll
        for (int k = 0; k < kFoldSeg; ++k) {
            if (k < cnt) {
                e[k] = __builtin_amdgcn_exp2f(u.A2 * e[k]);
                ah = fmaf(e[k], ah, hv[k]);
                ae *= e[k];
            }
        }
        se[w * kRow + l] = ae;
        sh[w * kRow + l] = ah;
        __syncthreads();
        // 2. scan the W segment aggregates of each channel across lanes
        {
            float ve = se[sg * kRow + ch], vh = sh[sg * kRow + ch];
            for (int s = 1; s < W; s <<= 1) {
                const float pe = row_shr(ve, ve, s), ph = row_shr(vh, vh, s);
                if (sg >= s) {                                      // (pe, ph) then (ve, vh)
                    vh = fmaf(ve, ph, vh);
                    ve *= pe;
                }
            }
            float xe = row_shr(1.0f, ve, 1), xh = row_shr(0.0f, vh, 1);
            if (sg == 0) { xe = 1.0f; xh = 0.0f; }
            const float p = spre[ch];
            sst[sg * kRow + ch] = fmaf(xe, p, xh);
            __syncthreads();                                        // every thread has read the incoming state
            if (sg == W - 1) spre[ch] = fmaf(ve, p, vh);            // incoming state of the next round
        }
        __syncthreads();
        // 3. re-fold the segment from its starting state, prefixes over H
        float h = sst[w * kRow + l];
#pragma unroll
        for (int k = 0; k < kFoldSeg; ++k) {
            if (k < cnt) {
                h = fmaf(e[k], h, hv[k]);
                if (u.active) u.H[u.slot(a, k0 + k) * u.hs] = h;
            }
        }
        __syncthreads();                                            // LDS is reused by the next round
    }
}

// LDS bytes of fold_scan for W wavefronts
static inline size_t fold_lds_bytes(int W) { return (3 * static_cast<size_t>(W) * (kWave + 1) + kWave) * sizeof(float); }

// Workgroup i of a fold launch -> its first unit ((batch row, 64-channel
// group) x kN + state), or -1 past the end; `per` units per workgroup (1 or
// 4).  Workgroups are dealt to the XCDs round-robin (i % 8).  The kN states of
// a group read the same S rows, and a channel block's carries were written on
// the XCD that wg_coords gave it: when the channel blocks spread evenly over
// the XCDs, the fold of a group runs on that same XCD (which also reads its
// prefixes next); otherwise the workgroups of a group still share one XCD.
__device__ __forceinline__ int64_t fold_unit(int64_t i, int64_t batch, int64_t D, int per) {
    const int64_t G = (D + kWave - 1) / kWave;                  // 64-channel groups per batch row
    const int64_t gx = (D + kBlock - 1) / kBlock;               // channel blocks per batch row
    const int64_t nblk = gx * batch, bpg = kN / per;            // workgroups per group
    const int64_t x = i % kXcds, j = i / kXcds;
    int64_t b, c;
    if (nblk % kXcds == 0) {
        const int64_t pb = (kBlock / kWave) * bpg;              // workgroups per channel block
        const int64_t blk = x * (nblk / kXcds) + j / pb;
        b = blk / gx;
        c = (blk % gx) * (kBlock / kWave) + (j % pb) / bpg;
        if (c >= G) return -1;
    } else {
        const int64_t grp = (j / bpg) * kXcds + x;
        if (grp >= batch * G) return -1;
        b = grp / G;
        c = grp % G;
    }
    return (b * G + c) * kN + (j % bpg) * per;
}

// Workgroups of a fold launch (a multiple of kXcds).
static inline int64_t fold_blocks(int64_t batch, int64_t D, int per) {
    const int64_t G = (D + kWave - 1) / kWave, gx = (D + kBlock - 1) / kBlock, bpg = kN / per;
    if (gx * batch % kXcds == 0) return gx * batch * (kBlock / kWave) * bpg;
    return (batch * G + kXcds - 1) / kXcds * kXcds * bpg;
}

// SHORT: four units per workgroup, one wavefront each (fold_short); else one
// unit per workgroup of W wavefronts (fold_scan, dynamic LDS).  A workgroup
// with no unit leaves before any barrier.
template <bool SHORT>
__device__ __forceinline__ void fold_dispatch(const S6FoldArgs& a, int64_t i, int W, float* lds) {
    if constexpr (SHORT) {
        const int64_t u0 = fold_unit(i, a.batch, a.D, kBlock / kWave);
        if (u0 >= 0) fold_short(a, u0 + (threadIdx.x >> 6));
    } else {
        const int64_t unit = fold_unit(i, a.batch, a.D, 1);
        if (unit >= 0) fold_scan(a, unit, W, lds);
    }
}

template <bool SHORT>
__global__ __launch_bounds__(kWave * kFoldMaxW) void s6_carry_scan(S6FoldArgs a, int W) {
    extern __shared__ float fold_lds[];
    fold_dispatch<SHORT>(a, blockIdx.x, W, fold_lds);
}

// two independent folds (the backward's state and adjoint carries) in one
// launch; `first` (the first fold's workgroups) is a multiple of kXcds, so
// both keep their XCD placement
template <bool SHORT>
__global__ __launch_bounds__(kWave * kFoldMaxW) void s6_carry_scan2(S6FoldArgs a, S6FoldArgs b, int64_t first,
                                                                   int W) {
    extern __shared__ float fold_lds[];
    const int64_t i = blockIdx.x;
    if (i < first) fold_dispatch<SHORT>(a, i, W, fold_lds);
    else fold_dispatch<SHORT>(b, i - first, W, fold_lds);
}

// ---------------------------------------------------------------------------
// phase 3: rescan from the starting state, write gated output (and h_L)
// ---------------------------------------------------------------------------
template <class LD, bool GATED, int K>
__global__ __launch_bounds__(kBlock) void s6_chunk_out(S6ScanArgs a) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = GATED ? 3 : 2;
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a.batch, a.L, a.D, a.chunk_len, a.n_chunks, 0, g)) return;
    const int64_t D = a.D;
    const uint32_t rowb = static_cast<uint32_t>(D) * es;
    const uint32_t last = static_cast<uint32_t>(g.nt - 1) * rowb;
    const int64_t e0 = g.row0 * D;
    ChunkIO<IO> src[NT], Y;
    src[0].init(static_cast<const T*>(a.x) + e0, last + rowb);
    src[1].init(static_cast<const T*>(a.delta) + e0, last + rowb);
    if (GATED) src[NT - 1].init(static_cast<const T*>(a.z) + e0, last + rowb);
    Y.init(static_cast<T*>(a.y) + e0, last + rowb);
    const T* Bc = static_cast<const T*>(a.B) + g.row0 * kN;
    const T* Cc = static_cast<const T*>(a.C) + g.row0 * kN;
    const uint32_t vo = ld.voff(g.d);           // load offset (LdPairBF16: the shared dword)
    const uint32_t vs = g.d * es;               // store offset

    float A2[kN], h[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) A2[n] = a.A[g.d * kN + n] * kLog2e;
    if (a.h0) {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = a.h0[(static_cast<int64_t>(g.b) * D + g.d) * kN + n];
    } else {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    }
    // The first block's loads go out first, so they land during the fold.
    Stage<LD, NT> st;
    st.issue(ld, src, vo, 0, rowb, last);
    if (g.c > 0) {
        // starting state of this chunk, left in carry slot c-1 by s6_carry_scan
        const int64_t cs = static_cast<int64_t>(g.b) * (a.n_chunks - 1) + g.c - 1;
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = a.carry_H[(cs * kN + n) * D + g.d];
    }
    const float bias = a.dt_bias[g.d];
    const float Dd = a.Dskip[g.d];
    ConvWin<IO, K> cv;
    cv.init(a, g);

    st.widen(ld);
    uint32_t so = 0;                 // row offset of the current token
    RowBC<IO> bq[2], cq[2];
    bq[0].load(Bc);
    cq[0].load(Cc);
    for (int tb = 0; tb < g.nt; tb += kBlk) {
        st.issue(ld, src, vo, static_cast<uint32_t>(tb + kBlk) * rowb, rowb, last);
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const int tt = tb + j;
            const bool valid = tt < g.nt;             // wave-uniform
            lgkm_wait_all();
            const int tn = min(tt + 1, g.nt - 1);
            bq[(j + 1) & 1].load(Bc + tn * kN);
            cq[(j + 1) & 1].load(Cc + tn * kN);
            const RowBC<IO>& Bv = bq[j & 1];
            const RowBC<IO>& Cv = cq[j & 1];

            float xv = st.v[0][j];
            if constexpr (K > 0) {
                if (valid) xv = cv.apply(xv);                // masked tokens leave the window alone
            }
            const float dt = valid ? softplus(st.v[1][j] + bias) : 0.0f;
            const float dx = dt * xv;
            float yv = Dd * xv;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float dA = __builtin_amdgcn_exp2f(dt * A2[n]);
                h[n] = fmaf(dA, h[n], dx * Bv.get(n));
                yv = fmaf(Cv.get(n), h[n], yv);
            }
            if (GATED) yv *= silu(st.v[NT - 1][j]);
            if (valid) store_io(Y, vs, so, yv);
            so += rowb;
        }
        st.widen(ld);
    }
    if constexpr (K > 1) {
        if (a.conv_last && g.c == a.n_chunks - 1) cv.store_last(a, g);
    }
    if (a.h_last && g.c == a.n_chunks - 1) {
#pragma unroll
        for (int n = 0; n < kN; ++n) a.h_last[(static_cast<int64_t>(g.b) * D + g.d) * kN + n] = h[n];
    }
}

// ---------------------------------------------------------------------------
// decode: one token against the cached state, in place
// ---------------------------------------------------------------------------
// Four lanes per channel, four states per lane: the state rows (64 bytes per
// channel) are read and written as whole 16-byte vectors by consecutive lanes.
// Batch rows per workgroup (A is loaded once for them).  Two beat eight on the
// 256 x 5120 step (27.1 vs 28.2 us hot, 37.7 vs 42.4 us from HBM): many small
// workgroups keep more of the state in flight than long per-wavefront runs.
constexpr int kStepRows = 2;

// Four consecutive io elements (a lane's four B or C entries), loaded as one
// vector when the tensor is aligned for it (VEC), else element by element, and
// widened on use.
template <class IO, bool VEC> struct Quad;
template <bool VEC> struct Quad<F32, VEC> {
    float4 v;
    __device__ __forceinline__ void load(const float* p) {
        if constexpr (VEC) v = *reinterpret_cast<const float4*>(p);
        else v = make_float4(p[0], p[1], p[2], p[3]);
    }
    __device__ __forceinline__ float get(int j) const { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }
};
template <bool VEC> struct Quad<BF16, VEC> {
    uint2 v;
    __device__ __forceinline__ void load(const uint16_t* p) {
        if constexpr (VEC) v = *reinterpret_cast<const uint2*>(p);
        else v = make_uint2(p[0] | (static_cast<uint32_t>(p[1]) << 16), p[2] | (static_cast<uint32_t>(p[3]) << 16));
    }
    __device__ __forceinline__ float get(int j) const {
        const uint32_t w = j < 2 ? v.x : v.y;
        return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// With the local convolution (K > 0) the step input is silu(b + w . [conv
// state, xin]); the four lanes of a channel compute it redundantly and the
// first one shifts the conv state in place.
template <class IO, bool GATED, int K, bool VEC>
__global__ __launch_bounds__(kBlock) void s6_step(S6StepArgs a) {
    using T = typename IO::T;
    const int q = threadIdx.x & 3;
    const int64_t dl = static_cast<int64_t>(blockIdx.x) * (kBlock / 4) + (threadIdx.x >> 2);
    const bool active = dl < a.D;
    const int64_t d = active ? dl : a.D - 1;
    const uint32_t dd = static_cast<uint32_t>(d);
    const T* X = static_cast<const T*>(a.x);
    const T* DL = static_cast<const T*>(a.delta);
    const T* Z = static_cast<const T*>(a.z);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    T* Y = static_cast<T*>(a.y);

    float A2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) A2[j] = a.A[d * kN + 4 * q + j] * kLog2e;
    const float bias = a.dt_bias[d];
    const float Dd = a.Dskip[d];
    float cw[K > 0 ? K : 1], cb = 0.0f;
    if constexpr (K > 0) {
#pragma unroll
        for (int k = 0; k < K; ++k) cw[k] = a.conv_w[d * K + k];
        cb = a.conv_b[d];
    }
    T* CS = static_cast<T*>(a.conv_state);

    // Every load of the workgroup's rows is issued before the first store, so
    // the rows' memory latencies overlap (the compiler would not move a later
    // row's loads above an earlier row's stores: it cannot see that they never
    // alias).  Rows past the batch end load the last row and are not stored.
    const int64_t b_begin = static_cast<int64_t>(blockIdx.y) * kStepRows;
    float4 hv[kStepRows];
    T xr[kStepRows], dr[kStepRows], zr[kStepRows];
    Quad<IO, VEC> br[kStepRows], cr[kStepRows];
    T wr[kStepRows][K > 1 ? K - 1 : 1];
#pragma unroll
    for (int r = 0; r < kStepRows; ++r) {
        const int64_t b = b_begin + r < a.batch ? b_begin + r : a.batch - 1;
        const int64_t brow = b * a.D;
        xr[r] = X[brow + dd];
        dr[r] = DL[brow + dd];
        if (GATED) zr[r] = Z[brow + dd];
        br[r].load(Bm + b * kN + 4 * q);
        cr[r].load(Cm + b * kN + 4 * q);
        hv[r] = reinterpret_cast<const float4*>(a.h + (b * a.D + d) * kN)[q];   // d is clamped: always in bounds
        if constexpr (K > 1) {
#pragma unroll
            for (int i = 0; i < K - 1; ++i) wr[r][i] = CS[(b * (K - 1) + i) * a.D + dd];
        }
    }
#pragma unroll
    for (int r = 0; r < kStepRows; ++r) {
        const int64_t b = b_begin + r;
        if (b >= a.batch) break;                       // uniform over the workgroup
        const int64_t brow = b * a.D;
        float xv = IO::load(&xr[r], 0);
        if constexpr (K > 0) {
            float v = cb;
#pragma unroll
            for (int i = 0; i < K - 1; ++i) v = fmaf(cw[i], IO::load(&wr[r][i], 0), v);
            v = fmaf(cw[K - 1], xv, v);
            if (active && q == 0) {
#pragma unroll
                for (int i = 0; i + 1 < K - 1; ++i) CS[(b * (K - 1) + i) * a.D + dd] = wr[r][i + 1];
                if constexpr (K > 1) CS[(b * (K - 1) + K - 2) * a.D + dd] = xr[r];
            }
            xv = silu(v);
        }
        const float dt = softplus(IO::load(&dr[r], 0) + bias);
        const float dx = dt * xv;
        float hs[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
        float p = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float dA = __builtin_amdgcn_exp2f(dt * A2[j]);
            hs[j] = fmaf(dA, hs[j], dx * br[r].get(j));
            p = fmaf(cr[r].get(j), hs[j], p);
        }
        if (active) reinterpret_cast<float4*>(a.h + (b * a.D + d) * kN)[q] = make_float4(hs[0], hs[1], hs[2], hs[3]);
        p += __shfl_xor(p, 1, 4);
        p += __shfl_xor(p, 2, 4);
        float yv = fmaf(Dd, xv, p);
        if (GATED) yv *= silu(IO::load(&zr[r], 0));
        if (active && q == 0) IO::store(Y + brow, dd, yv);
    }
}

}  // namespace s6

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
using namespace s6;

template <class LD, bool GATED, int K>
static hipError_t launch_scan_t(const S6ScanArgs& a, hipStream_t stream) {
    const int64_t nblk = (a.D + kBlock - 1) / kBlock * a.batch;
    if (a.n_chunks > 1) {
        dim3 g1(static_cast<unsigned>(nblk * (a.n_chunks - 1)));
        s6_timing_mark("s6_chunk_carry", stream, true);
        hipLaunchKernelGGL((s6_chunk_carry<LD, K>), g1, dim3(kBlock), 0, stream, a);
        s6_timing_mark("s6_chunk_carry", stream, false);
        S6FoldArgs f{a.A, a.h0, a.carry_S, a.carry_H, a.batch, a.D, a.n_chunks - 1, 0};
        s6_launch_fold(f, "s6_carry_scan", stream);
    }
    dim3 g3(static_cast<unsigned>(nblk * a.n_chunks));
    s6_timing_mark("s6_chunk_out", stream, true);
    hipLaunchKernelGGL((s6_chunk_out<LD, GATED, K>), g3, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_chunk_out", stream, false);
    return hipGetLastError();
}

// Wavefronts per fold unit: one while a wavefront can hold every carry in one
// round (the short path: no cross-wavefront scan, no LDS), then as many as
// keep each at most kFoldSeg carries per round, at most kFoldMaxW (longer
// chains take several rounds).
static int fold_waves(int64_t ncar) {
    int W = 1;
    while (W < kFoldMaxW && static_cast<int64_t>(W) * kFoldSeg < ncar) W *= 2;
    return W;
}

void s6_launch_fold(const S6FoldArgs& f, const char* name, hipStream_t stream) {
    const int W = fold_waves(f.ncar);
    s6_timing_mark(name, stream, true);
    if (W == 1)
        hipLaunchKernelGGL(s6_carry_scan<true>, dim3(static_cast<unsigned>(fold_blocks(f.batch, f.D, kBlock / kWave))),
                           dim3(kBlock), 0, stream, f, W);
    else
        hipLaunchKernelGGL(s6_carry_scan<false>, dim3(static_cast<unsigned>(fold_blocks(f.batch, f.D, 1))),
                           dim3(kWave * W), fold_lds_bytes(W), stream, f, W);
    s6_timing_mark(name, stream, false);
}

void s6_launch_fold2(const S6FoldArgs& f0, const S6FoldArgs& f1, const char* name, hipStream_t stream) {
    const int W = fold_waves(f0.ncar);
    s6_timing_mark(name, stream, true);
    if (W == 1) {
        const int64_t per = fold_blocks(f0.batch, f0.D, kBlock / kWave);
        hipLaunchKernelGGL(s6_carry_scan2<true>, dim3(static_cast<unsigned>(2 * per)), dim3(kBlock), 0, stream, f0, f1,
                           per, W);
    } else {
        const int64_t per = fold_blocks(f0.batch, f0.D, 1);
        hipLaunchKernelGGL(s6_carry_scan2<false>, dim3(static_cast<unsigned>(2 * per)), dim3(kWave * W),
                           fold_lds_bytes(W), stream, f0, f1, per, W);
    }
    s6_timing_mark(name, stream, false);
}

void s6_launch_chunk_carry(const S6ScanArgs& a, hipStream_t stream) {
    dim3 g1(static_cast<unsigned>((a.D + kBlock - 1) / kBlock * a.batch * (a.n_chunks - 1)));
    s6_timing_mark("s6_chunk_carry", stream, true);
    if (a.bf16 && a.pair_loads) hipLaunchKernelGGL((s6_chunk_carry<LdPairBF16, 0>), g1, dim3(kBlock), 0, stream, a);
    else if (a.bf16) hipLaunchKernelGGL((s6_chunk_carry<LdBF16, 0>), g1, dim3(kBlock), 0, stream, a);
    else hipLaunchKernelGGL((s6_chunk_carry<LdF32, 0>), g1, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_chunk_carry", stream, false);
}

template <int K>
static hipError_t launch_scan_k(const S6ScanArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16 && a.pair_loads)
        return gated ? launch_scan_t<LdPairBF16, true, K>(a, stream) : launch_scan_t<LdPairBF16, false, K>(a, stream);
    if (a.bf16) return gated ? launch_scan_t<LdBF16, true, K>(a, stream) : launch_scan_t<LdBF16, false, K>(a, stream);
    return gated ? launch_scan_t<LdF32, true, K>(a, stream) : launch_scan_t<LdF32, false, K>(a, stream);
}

hipError_t s6_launch_scan(const S6ScanArgs& a, hipStream_t stream) {
    switch (a.conv_k) {
        case 0: return launch_scan_k<0>(a, stream);
        case 1: return launch_scan_k<1>(a, stream);
        case 2: return launch_scan_k<2>(a, stream);
        case 3: return launch_scan_k<3>(a, stream);
        case 4: return launch_scan_k<4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class IO, bool GATED, int K>
static hipError_t launch_step_t(const S6StepArgs& a, hipStream_t stream) {
    dim3 g(static_cast<unsigned>((a.D + kBlock / 4 - 1) / (kBlock / 4)),
           static_cast<unsigned>((a.batch + kStepRows - 1) / kStepRows));
    // B and C rows are 16 elements: with 4-element alignment at the base every lane's quad is aligned
    const uintptr_t qa = 4 * sizeof(typename IO::T) - 1;
    const bool vec = ((reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C)) & qa) == 0;
    s6_timing_mark("s6_step", stream, true);
    if (vec) hipLaunchKernelGGL((s6_step<IO, GATED, K, true>), g, dim3(kBlock), 0, stream, a);
    else hipLaunchKernelGGL((s6_step<IO, GATED, K, false>), g, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_step", stream, false);
    return hipGetLastError();
}

template <int K>
static hipError_t launch_step_k(const S6StepArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16) return gated ? launch_step_t<BF16, true, K>(a, stream) : launch_step_t<BF16, false, K>(a, stream);
    return gated ? launch_step_t<F32, true, K>(a, stream) : launch_step_t<F32, false, K>(a, stream);
}

hipError_t s6_launch_step(const S6StepArgs& a, hipStream_t stream) {
    switch (a.conv_k) {
        case 0: return launch_step_k<0>(a, stream);
        case 1: return launch_step_k<1>(a, stream);
        case 2: return launch_step_k<2>(a, stream);
        case 3: return launch_step_k<3>(a, stream);
        case 4: return launch_step_k<4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
