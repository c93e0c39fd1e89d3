// fa_launch.h -- host-side launchers behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Element type codes as in fa.h.
enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

hipError_t launch_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                      const void *V, float scale, int causal, void *O, float *LSE,
                      hipStream_t stream);

// Workgroup size of the query-block-outer sweeps (forward, dQ). Eight waves
// (256 query rows) share each K and V tile loaded into LDS, half the
// direct-load traffic of four waves per CU (the loads measured about 13% of
// the forward's time); four waves (128 rows) when eight-wave units would not
// give every CU one (few slices or short rows), and under the causal mask
// for N < 4096, where a 256-row block runs more fully masked diagonal tiles
// than the loads save.
// fp32 forward: with fewer 128-row blocks than this (half the CUs of an
// MI355X), each 32-row group runs in one workgroup whose waves split its
// key tiles and merge their parts (fwd_f32_ks_kernel).
constexpr long kF32SplitBelow = 128;

inline bool use_256_row_blocks(int BH, int N, bool causal) {
  const int nqb = (N + 255) / 256;
  const long units = (long)BH * (causal ? (nqb + 1) / 2 : nqb);
  return units >= 256 && (!causal || N >= 4096);
}

// Under the causal mask at d = 64 and N <= 4096 the forward and the dQ sweep
// take one 128-row query block per workgroup, longest first, at three waves
// per SIMD, in place of pairs of blocks: pairs leave too few workgroups to
// keep the chip busy through the tail at these sizes.
inline bool use_single_block_order(int d, int N, bool causal) {
  return causal && d == 64 && N <= 4096;
}
// Slices per group of that order: as many as keep the group's K and V
// within 4 MiB (one XCD's L2), at least one.
inline int single_block_group(int BH, int N, int d) {
  const long per_slice = 4L * N * d;  // K and V, 16-bit
  const long s = (4L << 20) / per_slice;
  return (int)(s < 1 ? 1 : s > BH ? BH : s);
}

// Split-key forward: key tiles (64 keys) are divided into ranges of
// split_key_count(N, nsplit) keys, split_parts(N, nsplit) <= nsplit of them,
// none empty.
inline int split_key_count(int N, int nsplit) {
  const int tiles = (N + 63) / 64;
  return (tiles + nsplit - 1) / nsplit * 64;
}
inline int split_parts(int N, int nsplit) {
  const int per = split_key_count(N, nsplit);
  return (N + per - 1) / per;
}

// Partial results of every range of the Nk keys for Nq queries (query i at
// position Nk - Nq + i under the causal mask): O parts fp32
// [parts, B*H*Nq, d] at Op, LSE parts fp32 [parts, B*H*Nq] at Lp. With a
// single range, O (dtype) and LSE may be given instead: the kernel then
// writes the final result and no merge is needed.
hipError_t launch_fwd_split(int dtype, int B, int H, int Nq, int Nk, int d, const void *Q,
                            const void *K, const void *V, float scale, int causal, int nsplit,
                            float *Op, float *Lp, void *O, float *LSE, hipStream_t stream);

// O [rows, d] (dtype) and LSE [rows] from parts partial results.
hipError_t launch_lse_merge(int dtype, int parts, long rows, int d, const float *Op,
                            const float *Lp, void *O, float *LSE, hipStream_t stream);

// D = rowsum(dO o O), fp32 [B*H*N].
hipError_t launch_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                                 const void *dO, float *Dvec, hipStream_t stream);

// dK, dV (key blocks outer). LSE2, if not null, holds LSE * log2(e) per row
// (as launch_bwd_dq_fused writes it) and is read instead of LSE.
hipError_t launch_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                           const void *V, const void *dO, const float *LSE, const float *LSE2,
                           const float *Dvec, float scale, int causal, void *dK, void *dV,
                           hipStream_t stream);

// dQ (query blocks outer).
hipError_t launch_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                         const void *V, const void *dO, const float *LSE, const float *Dvec,
                         float scale, int causal, void *dQ, hipStream_t stream);

// dQ as launch_bwd_dq, with D formed from O and dO inside the sweep (the
// same values launch_bwd_preprocess computes, bit for bit) and written to
// Dvec for a dK/dV sweep launched after it; if LSE2 is not null, the sweep
// also writes LSE * log2(e) there, the form that sweep's exponentials use.
hipError_t launch_bwd_dq_fused(int dtype, int B, int H, int N, int d, const void *Q,
                               const void *K, const void *V, const void *O, const void *dO,
                               const float *LSE, float *Dvec, float *LSE2, float scale,
                               int causal, void *dQ, hipStream_t stream);

}  // namespace fa
