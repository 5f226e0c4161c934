// Launch arguments of the SSD (Mamba-2 style) layer kernel, shared by the
// kernel source and the C ABI.
#pragma once
#include "s6_common.h"

// SSD (Mamba-2 style) layer: scalar decay per head, P = 64 channels per head.
struct SsdArgs {
    const void* x;       // (batch, L, H, 64) bf16
    const void* delta;   // (batch, L, H) bf16
    const void* z;       // (batch, L, H, 64) bf16 or NULL
    const void* B;       // (batch, L, N) bf16
    const void* C;       // (batch, L, N) bf16
    const float* A;      // (H)
    const float* Dskip;  // (H)
    const float* dt_bias;// (H)
    const float* h0;     // (batch, H, 64, N) or NULL
    void* y;             // (batch, L, H, 64) bf16
    float* h_last;       // (batch, H, 64, N) or NULL
    uint16_t* gram;      // workspace: (batch, ceil(L / 64), 64, 64) bf16, C_t . B_i per chunk
    // Sequences too few to fill the GPU are cut into n_seg segments of
    // seg_chunks chunks (the last one may be shorter), walked in parallel:
    float* seg_state;    // workspace: (batch, H, n_seg - 1, 64, N) fp32: segment k's local end state
                         // from zero, then (after the fold) segment k + 1's starting state
    float* seg_decay;    // workspace: (batch, H, n_seg - 1): log2 of segment k's total decay
    int64_t seg_chunks, n_seg;
    int64_t batch, L, H, N;
};
hipError_t ssd_launch(const SsdArgs& a, hipStream_t stream);
// bytes of the gram workspace
int64_t ssd_gram_bytes(int64_t batch, int64_t L);
// segments per sequence and chunks per segment for a shape (1 segment: walked whole)
void ssd_segments(int64_t batch, int64_t L, int64_t H, int64_t N, int64_t* n_seg, int64_t* seg_chunks);
// bytes of the whole workspace (gram blocks, then the segment states and decays when n_seg > 1)
int64_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t N);
// byte offsets of the segment states and decays in the workspace
int64_t ssd_seg_state_offset(int64_t batch, int64_t L);
int64_t ssd_seg_decay_offset(int64_t batch, int64_t L, int64_t H, int64_t N, int64_t n_seg);
