// Device-side building blocks shared by the gfx950 scan kernels: scalar-cache
// B/C rows, buffer-resource chunk addressing, element loaders, the
// register double buffer and the XCD-aware lane geometry.
#pragma once

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
    bool active;       // d is this lane's own channel (false: a duplicate of D-1)
    int group;         // 64-channel group of the wavefront within its batch row
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
__device__ __forceinline__ void wg_coords(int64_t nblk, int64_t nchunks, int64_t& blk, int64_t& chunk,
                                          int64_t i) {
    if (nblk % kXcds == 0) {
        const int64_t xcd = i % kXcds, pos = i / kXcds;
        blk = xcd * (nblk / kXcds) + pos / nchunks;
        chunk = pos % nchunks;
    } else {
        blk = i % nblk;
        chunk = i / nblk;
    }
}

// Geometry of this lane: chunk index space [chunk_first, chunk_first + nchunks)
// of a (batch, L, D) problem cut into chunks of chunk_len tokens.
// bid: the workgroup's index in this job (blockIdx.x unless several jobs share one launch)
__device__ __forceinline__ bool geo_setup(int64_t batch, int64_t L, int64_t D, int64_t chunk_len,
                                          int64_t nchunks, int64_t chunk_first, Geo& g, int64_t bid = -1) {
    const int64_t gx = (D + kBlock - 1) / kBlock;              // channel blocks per batch row
    int64_t blk, chunk;
    wg_coords(gx * batch, nchunks, blk, chunk, bid < 0 ? static_cast<int64_t>(blockIdx.x) : bid);
    const int64_t bx = blk % gx;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t first = bx * kBlock + wave * kWave;
    if (first >= D) return false;                 // whole wavefront past the last channel
    const int64_t d = first + (threadIdx.x & (kWave - 1));
    g.active = d < D;
    g.d = static_cast<uint32_t>(g.active ? d : D - 1);
    g.group = static_cast<int>(first / kWave);
    g.c = static_cast<int>(chunk + chunk_first);
    g.b = static_cast<int>(blk / gx);
    g.t0 = g.c * static_cast<int>(chunk_len);
    const int t1 = g.t0 + static_cast<int>(chunk_len);
    g.nt = (t1 < L ? t1 : static_cast<int>(L)) - g.t0;
    g.row0 = static_cast<int64_t>(g.b) * L + g.t0;
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

}  // namespace s6
