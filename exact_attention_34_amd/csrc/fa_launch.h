// fa_launch.h -- host-side launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Element type codes as in fa.h.
enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

hipError_t launch_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                      const void *V, float scale, int causal, void *O, float *LSE,
                      hipStream_t stream);

hipError_t launch_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                                 const void *dO, float *Dvec, float *dQacc, hipStream_t stream);

hipError_t launch_bwd_main(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                           const void *V, const void *dO, const float *LSE, const float *Dvec,
                           float scale, int causal, float *dQacc, void *dK, void *dV,
                           hipStream_t stream);

hipError_t launch_bwd_dq_convert(int dtype, int B, int H, int N, int d, const float *dQacc,
                                 float scale, void *dQ, hipStream_t stream);

}  // namespace fa
