// fa_launch.h -- host-side launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Element type codes as in fa.h.
enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

hipError_t launch_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                      const void *V, float scale, int causal, void *O, float *LSE,
                      hipStream_t stream);

// D = rowsum(dO o O), fp32 [B*H*N].
hipError_t launch_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                                 const void *dO, float *Dvec, hipStream_t stream);

// dK, dV (key blocks outer).
hipError_t launch_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                           const void *V, const void *dO, const float *LSE, const float *Dvec,
                           float scale, int causal, void *dK, void *dV, hipStream_t stream);

// dQ (query blocks outer).
hipError_t launch_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                         const void *V, const void *dO, const float *LSE, const float *Dvec,
                         float scale, int causal, void *dQ, hipStream_t stream);

}  // namespace fa
