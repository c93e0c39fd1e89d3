// fa_std_launch.h -- host-side launchers of the stored-P standard attention
// (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {

// Standard attention that stores the N x N matrices (the pages' baseline).
// N x N arrays of one slice have std_row_stride(N) elements per row.
inline int std_row_stride(int N) { return (N + 127) / 128 * 128; }

// S fp32 and P (dtype) [B*H, N, ldn], then O and LSE.
hipError_t launch_std_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                          const void *V, float scale, int causal, float *S, void *P, void *O,
                          float *LSE, hipStream_t stream);

// D fp32 [B*H*N] and dS (dtype) [B*H, N, ldn] as scratch, then dQ, dK, dV.
hipError_t launch_std_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                          const void *V, const void *O, const void *dO, const void *P,
                          float scale, void *dS, float *Dv, void *dQ, void *dK, void *dV,
                          hipStream_t stream);

}  // namespace fa
