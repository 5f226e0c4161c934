// gfx950 kernels of the selective scan (S6) forward and its decode step.
//
// Work layout of the scans: one lane per channel d, all 16 state values of
// that channel in VGPRs, a wavefront = 64 consecutive channels of one batch
// row, a workgroup = 4 such wavefronts (independent: no LDS, no barriers).
// B_t and C_t are the same for every channel of a batch row ("Mamba",
// "Selectivity": B and C are functions of the token), so a wavefront reads
// them with scalar loads and the state updates take them as SGPR operands.
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

#include "s6_common.h"

namespace s6 {

// ---------------------------------------------------------------------------
// B_t / C_t rows through the scalar cache
// ---------------------------------------------------------------------------
typedef const __attribute__((address_space(4))) uint32_t cu32;

template <class IO> struct RowBC;

template <> struct RowBC<BF16> {
    uint32_t w[8];    // 16 bf16 values, two per word
    __device__ __forceinline__ void load(const uint16_t* row) {
        cu32* p = (cu32*)row;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = p[i];
    }
    __device__ __forceinline__ float get(int n) const {
        return (n & 1) ? bf16_hi(w[n >> 1]) : bf16_lo(w[n >> 1]);
    }
};

template <> struct RowBC<F32> {
    uint32_t w[16];
    __device__ __forceinline__ void load(const float* row) {
        cu32* p = (cu32*)row;
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

// ---------------------------------------------------------------------------
// one (batch, L, D) io tensor, restricted to a chunk, as a buffer resource
// ---------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data format (gfx9 family)

template <class IO> struct ChunkIO {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ void init(const void* chunk_base, uint32_t bytes) {
        r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(chunk_base), 0, static_cast<int>(bytes),
                                              kRsrcWord3);
    }
};

// Element loaders of x, delta and z.  load() returns raw bits that stay in
// the prefetch ring; widen() turns them into fp32 where they are used.  The
// ring must hold plain 32-bit values: anything the compiler has to do to a
// loaded value before the loop back-edge (zero-extend, pack two 16-bit values
// into one register) makes it wait for the whole ring.
//   LdPairBF16 (bf16, D even, 4-byte aligned io): each lane loads the aligned
//     dword that holds its element (two lanes share it) and picks its half
//     with one byte permute at use.
//   LdBF16: 16-bit loads (any D); the compiler packs the ring, which costs a
//     wait per ring turn.
//   LdF32: 32-bit loads.
struct LdPairBF16 {
    using IO = BF16;
    using R = uint32_t;
    uint32_t sel;                                   // byte-permute selector of this lane's half
    __device__ __forceinline__ uint32_t voff(uint32_t d) {
        sel = (d & 1u) ? 0x03020c0cu : 0x01000c0cu;
        return (d * 2u) & ~3u;
    }
    __device__ __forceinline__ R load(const ChunkIO<BF16>& s, uint32_t vo, uint32_t so) const {
        return __builtin_amdgcn_raw_buffer_load_b32(s.r, vo, so, 0);
    }
    __device__ __forceinline__ float widen(R w) const { return __uint_as_float(__builtin_amdgcn_perm(0u, w, sel)); }
};

struct LdBF16 {
    using IO = BF16;
    using R = uint16_t;
    __device__ __forceinline__ uint32_t voff(uint32_t d) { return d * 2u; }
    __device__ __forceinline__ R load(const ChunkIO<BF16>& s, uint32_t vo, uint32_t so) const {
        return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(s.r, vo, so, 0));
    }
    __device__ __forceinline__ float widen(R u) const { return __uint_as_float(static_cast<uint32_t>(u) << 16); }
};

struct LdF32 {
    using IO = F32;
    using R = uint32_t;
    __device__ __forceinline__ uint32_t voff(uint32_t d) { return d * 4u; }
    __device__ __forceinline__ R load(const ChunkIO<F32>& s, uint32_t vo, uint32_t so) const {
        return __builtin_amdgcn_raw_buffer_load_b32(s.r, vo, so, 0);
    }
    __device__ __forceinline__ float widen(R u) const { return __uint_as_float(u); }
};

__device__ __forceinline__ void store_io(const ChunkIO<BF16>& s, uint32_t voff, uint32_t soff, float v) {
    const __bf16 b = static_cast<__bf16>(v);                  // round to nearest even
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), s.r, voff, soff, 0);
}
__device__ __forceinline__ void store_io(const ChunkIO<F32>& s, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), s.r, voff, soff, 0);
}

// ---------------------------------------------------------------------------
// lane / chunk geometry
// ---------------------------------------------------------------------------
struct Geo {
    uint32_t d;        // channel; lanes past D take D-1 and duplicate its (identical) results
    int b, c;          // batch row, chunk
    int t0, nt;        // first token and token count of the chunk
    int64_t row0;      // b * L + t0: token row of the chunk start
};

// The wavefront index is made wave-uniform explicitly, so the early exit and
// every bound derived after it stay in SGPRs.
constexpr int kXcds = 8;

// Linear workgroup index -> (channel block, chunk, batch row).  The launch is
// a 1-D grid of nblk * nchunks workgroups (nblk = channel blocks x batch
// rows, batch-row major).  When nblk is a multiple of the XCD count,
// workgroup i runs on XCD i % 8 at position i / 8 there; XCD x is given the
// contiguous channel blocks [x * nblk/8, (x+1) * nblk/8) with all their
// chunks, so a batch row's B/C rows are shared in one L2 and every carry is
// read on the XCD that wrote it.  Otherwise the plain row-major order is used.
__device__ __forceinline__ void wg_coords(int64_t nblk, int64_t nchunks, int64_t& blk, int64_t& chunk) {
    const int64_t i = blockIdx.x;
    if (nblk % kXcds == 0) {
        const int64_t xcd = i % kXcds, pos = i / kXcds;
        blk = xcd * (nblk / kXcds) + pos / nchunks;
        chunk = pos % nchunks;
    } else {
        blk = i % nblk;
        chunk = i / nblk;
    }
}

__device__ __forceinline__ bool geo_setup(const S6ScanArgs& a, int64_t nchunks, Geo& g) {
    const int64_t gx = (a.D + kBlock - 1) / kBlock;            // channel blocks per batch row
    int64_t blk, chunk;
    wg_coords(gx * a.batch, nchunks, blk, chunk);
    const int64_t bx = blk % gx;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t first = bx * kBlock + wave * kWave;
    if (first >= a.D) return false;               // whole wavefront past the last channel
    const int64_t d = first + (threadIdx.x & (kWave - 1));
    g.d = static_cast<uint32_t>(d < a.D ? d : a.D - 1);
    g.c = static_cast<int>(chunk);
    g.b = static_cast<int>(blk / gx);
    g.t0 = g.c * static_cast<int>(a.chunk_len);
    const int t1 = g.t0 + static_cast<int>(a.chunk_len);
    g.nt = (t1 < a.L ? t1 : static_cast<int>(a.L)) - g.t0;
    g.row0 = static_cast<int64_t>(g.b) * a.L + g.t0;
    return true;
}

// x, delta (and z) are double-buffered in registers in blocks of kBlk tokens:
// while a wavefront computes block k from fp32 values v, the global loads of
// block k+1 are in flight into raw registers r; after the compute, r is
// widened into v.  No value whose load is still in flight is live across the
// loop back-edge, so the only wait for the loads is that widening, once per
// block, after a whole block of compute.  Load offsets are clamped to the
// chunk's last token; tokens past the chunk end (only in a ragged last chunk)
// are masked: Delta = 0 leaves the state unchanged, and they are not stored.
constexpr int kBlk = 4;

template <class LD, int NT>
struct Stage {
    using IO = typename LD::IO;
    typename LD::R r[NT][kBlk];                    // raw loads of the next block, in flight
    float v[NT][kBlk];                             // fp32 values of the current block

    __device__ __forceinline__ void issue(const LD& ld, const ChunkIO<IO> (&src)[NT], uint32_t vo,
                                          uint32_t first, uint32_t rowb, uint32_t last) {
#pragma unroll
        for (int j = 0; j < kBlk; ++j) {
            const uint32_t o = min(first + static_cast<uint32_t>(j) * rowb, last);
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

// ---------------------------------------------------------------------------
// phase 1: chunk carries
// ---------------------------------------------------------------------------
template <class LD>
__global__ __launch_bounds__(kBlock) void s6_chunk_carry(S6ScanArgs a) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = 2;
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a, a.n_chunks - 1, g)) return;
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
            const float dx = dt * st.v[0][j];
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
// phase 2: combine the chunk carries in order
// ---------------------------------------------------------------------------
// One wavefront per (batch row, 64 channels, state n): lanes are channels, so
// every carry read and every prefix write is one coalesced 256-byte row.  The
// carries of up to kScanBlk chunks are loaded at once, then combined in
// order: h <- exp(A_n S_c) h + H_c, starting from h0.  The combined prefix
// after chunk c is the starting state of chunk c+1 and overwrites H_c.
constexpr int kScanBlk = 16;

__global__ __launch_bounds__(kBlock) void s6_carry_scan(S6ScanArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t gx = (a.D + kWave - 1) / kWave;               // 64-channel groups per batch row
    const int64_t unit = static_cast<int64_t>(blockIdx.x) * (kBlock / kWave) + wave;
    if (unit >= a.batch * gx * kN) return;                      // whole wavefront past the end
    const int n = static_cast<int>(unit % kN);
    const int64_t grp = unit / kN;
    const int64_t b = grp / gx;
    const int64_t first = (grp % gx) * kWave;
    const int64_t dl = first + (threadIdx.x & (kWave - 1));
    const int64_t d = dl < a.D ? dl : a.D - 1;
    const int64_t ncar = a.n_chunks - 1;
    const float A2 = a.A[d * kN + n] * kLog2e;
    float h = a.h0 ? a.h0[(b * a.D + d) * kN + n] : 0.0f;
    const float* S = a.carry_S + b * ncar * a.D + d;
    float* H = a.carry_H + (b * ncar * kN + n) * a.D + d;
    const int64_t hs = kN * a.D;                                // H stride between chunks
    for (int64_t c0 = 0; c0 < ncar; c0 += kScanBlk) {
        float Sv[kScanBlk], Hv[kScanBlk];
#pragma unroll
        for (int k = 0; k < kScanBlk; ++k) {
            const int64_t c = c0 + k < ncar ? c0 + k : ncar - 1;
            Sv[k] = S[c * a.D];
            Hv[k] = H[c * hs];
        }
#pragma unroll
        for (int k = 0; k < kScanBlk; ++k) {
            if (c0 + k < ncar) {                                  // wave-uniform
                h = fmaf(__builtin_amdgcn_exp2f(A2 * Sv[k]), h, Hv[k]);
                H[(c0 + k) * hs] = h;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// phase 3: rescan from the starting state, write gated output (and h_L)
// ---------------------------------------------------------------------------
template <class LD, bool GATED>
__global__ __launch_bounds__(kBlock) void s6_chunk_out(S6ScanArgs a) {
    using IO = typename LD::IO;
    using T = typename IO::T;
    constexpr int NT = GATED ? 3 : 2;
    LD ld;
    constexpr uint32_t es = sizeof(T);
    Geo g;
    if (!geo_setup(a, a.n_chunks, g)) return;
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

            const float xv = st.v[0][j];
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
constexpr int kStepRows = 8;      // batch rows per workgroup (A is loaded once for them)

template <class IO, bool GATED>
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

template <class LD, bool GATED>
static hipError_t launch_scan_t(const S6ScanArgs& a, hipStream_t stream) {
    const int64_t nblk = (a.D + kBlock - 1) / kBlock * a.batch;
    if (a.n_chunks > 1) {
        dim3 g1(static_cast<unsigned>(nblk * (a.n_chunks - 1)));
        s6_timing_mark("s6_chunk_carry", stream, true);
        hipLaunchKernelGGL(s6_chunk_carry<LD>, g1, dim3(kBlock), 0, stream, a);
        s6_timing_mark("s6_chunk_carry", stream, false);
        const int64_t waves = a.batch * ((a.D + kWave - 1) / kWave) * kN;
        dim3 g2(static_cast<unsigned>((waves + kBlock / kWave - 1) / (kBlock / kWave)));
        s6_timing_mark("s6_carry_scan", stream, true);
        hipLaunchKernelGGL(s6_carry_scan, g2, dim3(kBlock), 0, stream, a);
        s6_timing_mark("s6_carry_scan", stream, false);
    }
    dim3 g3(static_cast<unsigned>(nblk * a.n_chunks));
    s6_timing_mark("s6_chunk_out", stream, true);
    hipLaunchKernelGGL((s6_chunk_out<LD, GATED>), g3, dim3(kBlock), 0, stream, a);
    s6_timing_mark("s6_chunk_out", stream, false);
    return hipGetLastError();
}

hipError_t s6_launch_scan(const S6ScanArgs& a, hipStream_t stream) {
    const bool gated = a.z != nullptr;
    if (a.bf16 && a.pair_loads)
        return gated ? launch_scan_t<LdPairBF16, true>(a, stream) : launch_scan_t<LdPairBF16, false>(a, stream);
    if (a.bf16) return gated ? launch_scan_t<LdBF16, true>(a, stream) : launch_scan_t<LdBF16, false>(a, stream);
    return gated ? launch_scan_t<LdF32, true>(a, stream) : launch_scan_t<LdF32, false>(a, stream);
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
