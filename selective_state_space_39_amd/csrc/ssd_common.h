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
    int64_t batch, L, H, N;
};
hipError_t ssd_launch(const SsdArgs& a, hipStream_t stream);
// bytes of the gram workspace
int64_t ssd_gram_bytes(int64_t batch, int64_t L);
