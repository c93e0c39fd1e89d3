// fa_std.hip -- standard attention that stores the N x N matrices, the
// baseline that the pages set exact tiled attention against.
//
// "Flash Attention" notes, section 1: the plain method forms S = Q K^T, the
// softmax P and O = P V as whole N x N arrays in device memory, and its
// backward reads the stored P (section 3: storing P against recomputing it;
// the backward-derivation page, parts 3-5, for dV, dP, dS, dQ, dK). Here
// every step is its own kernel and every N x N intermediate goes through HBM:
//   forward   S = scale Q K^T (fp32, masked), P = softmax(S) (T), O = P V,
//             LSE = m + log l per row;
//   backward  D = rowsum(dO o O), dV = P^T dO, dS = P o (dO V^T - D) (T),
//             dQ = scale dS K, dK = scale dS^T Q.
// The N x N arrays have rows of ldn = N rounded up to 128 elements; the
// padding columns hold P = 0 and dS = 0.
//
// One batched MFMA GEMM (v_mfma_f32_32x32x16) serves all five products: a
// workgroup of four waves computes a 128 x NC tile of C = A B over K in
// steps of 32, with A and B staged in LDS as they are stored. An operand
// whose contraction index is contiguous in memory is read row-wise
// (ds_read_b128); one whose contraction index is the row index is read with
// transposing reads (ds_read_b64_tr_b16). The row softmax is a separate
// HBM-bound kernel, one workgroup per row.

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_std_launch.h"

namespace fa {

namespace {

// Epilogues.
enum Epi {
  kEpiScores = 0,  // C fp32 = scale * acc; -inf where the key is past N or (causal) after the row
  kEpiStore = 1,   // C (T) = scale * acc
  kEpiDs = 2,      // C (T) = P * (acc - D[row]), the softmax backward
};

// Tile shape: 128 rows x NC columns of C per workgroup, K in steps of 32.
template <int NC>
struct GemmCfg {
  static constexpr int kThreads = 256;
  static constexpr int BM = 128, BK = 32;
  static constexpr int WN = NC / 64;  // 32-column MFMA blocks per wave (waves are 2 x 2)
  // LDS row strides (elements) of the two staging layouts, padded so that
  // the row-wise reads (16 rows x 16 B per quarter-wave) and the transposing
  // reads (4 rows x 32 B per 16 lanes) hit distinct banks.
  static constexpr int SR = BK + 8;  // [128 or NC rows][32 k]
  static constexpr int SC_A = BM + 16, SC_B = NC + 16;  // [32 k][128 or NC]
};

// Batched C = A B. Slice z: A at A + z*sA, B at B + z*sB, C at C + z*sC.
// M rows of C exist (rows past M are neither loaded nor stored), NC columns
// per column tile; Kend (a multiple of 32) contraction steps, of which the
// first Kvalid exist (the rest are zero).
//   TA = 0: A stored [M][K], row stride lda;  TA = 1: A stored [K][M].
//   TB = 0: B stored [K][NCtot], row stride ldb;  TB = 1: B stored [NCtot][K].
// For TA = 1 / TB = 0 the stored rows are contraction rows: rows past Kvalid
// read as zero. For TB = 1 the stored rows are columns of C: rows past
// ncols_valid read as zero.
template <typename T, int NC, int TA, int TB, int EPI>
__global__ __launch_bounds__(256, 2) void std_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ Cout,
    long sA, long sB, long sC, int lda, int ldb, int ldc, int M, int ncols_valid, int Kvalid,
    int Kend, int ntm, int ntn, int total, float scale, int causal,
    const uint16_t *__restrict__ P, const float *__restrict__ Dv, int ldpv) {
  using C = GemmCfg<NC>;
  constexpr int A_ELEMS = TA ? C::BK * C::SC_A : C::BM * C::SR;
  constexpr int B_ELEMS = TB ? NC * C::SR : C::BK * C::SC_B;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][B_ELEMS];

  const int tile = xcd_tile(blockIdx.x, total);
  const int per = ntm * ntn;
  const int z = tile / per;
  const int r = tile - z * per;
  const int tm = r / ntn, tn = r - tm * ntn;
  const int m0 = tm * C::BM, n0 = tn * NC;
  const uint16_t *Az = A + z * sA;
  const uint16_t *Bz = B + z * sB;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // Global -> register staging: A tile 128 x 32 (512 16-byte chunks, two
  // per thread), B tile NC x 32 (NC / 64 per thread).
  constexpr int ACH = 2, BCH = NC / 64;
  u32x4 ra[ACH], rb[BCH];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (TA == 0) {
        const int row = c >> 2, kc = c & 3;
        if (m0 + row < M) v = ld128(Az + (size_t)(m0 + row) * lda + k0 + 8 * kc);
      } else {
        const int krow = c >> 4, mc = c & 15;
        if (k0 + krow < Kvalid) v = ld128(Az + (size_t)(k0 + krow) * lda + m0 + 8 * mc);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + 256 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (TB == 1) {
        const int row = c >> 2, kc = c & 3;
        if (n0 + row < ncols_valid) v = ld128(Bz + (size_t)(n0 + row) * ldb + k0 + 8 * kc);
      } else {
        const int krow = c / (NC / 8), nc = c % (NC / 8);
        if (k0 + krow < Kvalid) v = ld128(Bz + (size_t)(k0 + krow) * ldb + n0 + 8 * nc);
      }
      rb[i] = v;
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int c = tid + 256 * i;
      const int off = TA == 0 ? (c >> 2) * C::SR + 8 * (c & 3) : (c >> 4) * C::SC_A + 8 * (c & 15);
      st128(&As[buf][off], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + 256 * i;
      const int off = TB == 1 ? (c >> 2) * C::SR + 8 * (c & 3)
                              : (c / (NC / 8)) * C::SC_B + 8 * (c % (NC / 8));
      st128(&Bs[buf][off], rb[i]);
    }
  };

  // MFMA operands. Row-wise: lane reads row (block row + l%32), k = 16kk +
  // 8g .. +7. Transposed: two ds_read_b64_tr_b16, rows (k) 16kk + 8g + 4h +
  // (l%16)/4, columns (block column + 16((l/16)%2) + 4(l%4)); lane receives
  // k = 16kk + 8g .. +7 of its column l%32 -- the same k order as the
  // row-wise read.
  auto opnd_row = [&](const uint16_t *S, int row0, int kk) __attribute__((always_inline)) {
    return ld128(S + (row0 + l32) * C::SR + 16 * kk + 8 * g);
  };
  auto opnd_col = [&](const uint16_t *S, int stride, int col0, int kk)
      __attribute__((always_inline)) {
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int k = 16 * kk + 8 * g + (lane & 15) / 4;
    return cat(ld_tr16(S + k * stride + col), ld_tr16(S + (k + 4) * stride + col));
  };

  f32x16 acc[2][C::WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < C::WN; ++j) acc[i][j] = kZero16;

  // The dS epilogue's P values, loaded before the (short, K = d) product so
  // that their latency overlaps it: the same (row, 4-column run) positions
  // the epilogue below writes.
  u32x2 pre[2][C::WN][4];
  if constexpr (EPI == kEpiDs) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = min(m0 + 64 * wm + 32 * i + l32, M - 1);
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + (NC / 2) * wn + 32 * j + 8 * q + 4 * g;
          pre[i][j][q] = *(const u32x2 *)(P + z * sC + (size_t)row * ldpv + col);
        }
    }
  }

  const int nk = Kend / C::BK;
  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * C::BK);
    const uint16_t *Ab = As[buf], *Bb = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[2], b[C::WN];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = TA == 0 ? opnd_row(Ab, 64 * wm + 32 * i, kk)
                       : opnd_col(Ab, C::SC_A, 64 * wm + 32 * i, kk);
#pragma unroll
      for (int j = 0; j < C::WN; ++j)
        b[j] = TB == 1 ? opnd_row(Bb, (NC / 2) * wn + 32 * j, kk)
                       : opnd_col(Bb, C::SC_B, (NC / 2) * wn + 32 * j, kk);
      // The fp32 scores: A as the first operand, so that the result's lane
      // is a column of C (32 lanes store 128 contiguous bytes of a row).
      // The 16-bit outputs: B first, so that the lane is a row of C and
      // its registers are columns (each lane stores runs of 4 columns).
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < C::WN; ++j)
          acc[i][j] = EPI == kEpiScores ? mfma32<T>(a[i], b[j], acc[i][j])
                                        : mfma32<T>(b[j], a[i], acc[i][j]);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  if constexpr (EPI == kEpiScores) {
    // Result block (i, j): lane holds column l%32 of its 32 x 32 block and
    // rows 8(r/4) + 4g + r%4 in register r.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < C::WN; ++j) {
        const int col = n0 + (NC / 2) * wn + 32 * j + l32;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int row = m0 + 64 * wm + 32 * i + 8 * (rr >> 2) + 4 * g + (rr & 3);
          if (row >= M) continue;
          const bool masked = col >= ncols_valid || (causal && col > row);
          ((float *)Cout)[z * sC + (size_t)row * ldc + col] =
              masked ? -INFINITY : acc[i][j][rr] * scale;
        }
      }
    return;
  }
  // Result block (i, j): lane holds row m = l%32 of its 32 x 32 block and
  // columns 8q + 4g + (0..3) in registers 4q .. 4q+3.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = m0 + 64 * wm + 32 * i + l32;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < C::WN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + (NC / 2) * wn + 32 * j + 8 * q + 4 * g;
        const size_t at = z * sC + (size_t)row * ldc + col;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[i][j][4 * q + e];
        if constexpr (EPI == kEpiDs) {
          const u32x2 pv = pre[i][j][q];
          const float dd = Dv[(size_t)z * M + row];
          const float p[4] = {to_f32<T>((uint16_t)(pv[0] & 0xffffu)),
                              to_f32<T>((uint16_t)(pv[0] >> 16)),
                              to_f32<T>((uint16_t)(pv[1] & 0xffffu)),
                              to_f32<T>((uint16_t)(pv[1] >> 16))};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = col + e < ncols_valid ? p[e] * (x[e] - dd) : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= scale;
        }
        u32x2 o;
        o[0] = pack2<T>(x[0], x[1]);
        o[1] = pack2<T>(x[2], x[3]);
        *(u32x2 *)((uint16_t *)Cout + at) = o;
      }
  }
}

// One row of S (fp32, ldn columns of which the first N exist): P = exp(S -
// m) / l rounded to T (0 in the padding columns), LSE = m + log l. The row
// is read from device memory once and kept in registers (4 * kCache
// values per thread, rows up to 8192); longer rows re-read the rest.
template <typename T>
__global__ __launch_bounds__(256) void std_softmax_kernel(const float *__restrict__ S,
                                                          uint16_t *__restrict__ P,
                                                          float *__restrict__ LSE, int N,
                                                          int ldn) {
  constexpr int kCache = 8;
  __shared__ float red[4];
  const long row = blockIdx.x;  // slice-major: row = z * N + i
  const float *s = S + row * ldn;
  uint16_t *p = P + row * ldn;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off, 64);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();  // red[] is free again
    if (lane == 0) red[w] = v;
    __syncthreads();
    const float a = red[0], b = red[1], c = red[2], d = red[3];
    return is_max ? fmaxf(fmaxf(a, b), fmaxf(c, d)) : (a + b) + (c + d);
  };
  // Chunk c of this thread: columns 4 tid + 1024 c .. +3 (ldn is a multiple
  // of 128, so a chunk is inside the row or wholly past it).
  f32x4 v[kCache];
  auto chunk = [&](int c) __attribute__((always_inline)) {
    const int j = 4 * tid + 1024 * c;
    f32x4 x = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (j < ldn) x = *(const f32x4 *)(s + j);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e >= N) x[e] = -INFINITY;
    return x;
  };
  const int nch = (ldn + 1023) / 1024;
#pragma unroll
  for (int c = 0; c < kCache; ++c) v[c] = c < nch ? chunk(c) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < kCache; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, v[c][e]);
  for (int c = kCache; c < nch; ++c) {
    const f32x4 x = chunk(c);
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, x[e]);
  }
  m = block_reduce(m, true);
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < kCache; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) l += __expf(v[c][e] - m);
  for (int c = kCache; c < nch; ++c) {
    const f32x4 x = chunk(c);
#pragma unroll
    for (int e = 0; e < 4; ++e) l += __expf(x[e] - m);
  }
  l = block_reduce(l, false);
  const float inv = 1.f / l;
  auto put = [&](int c, const f32x4 &x) __attribute__((always_inline)) {
    const int j = 4 * tid + 1024 * c;
    if (j >= ldn) return;
    u32x2 o;
    o[0] = pack2<T>(__expf(x[0] - m) * inv, __expf(x[1] - m) * inv);
    o[1] = pack2<T>(__expf(x[2] - m) * inv, __expf(x[3] - m) * inv);
    *(u32x2 *)(p + j) = o;
  };
#pragma unroll
  for (int c = 0; c < kCache; ++c) put(c, v[c]);
  for (int c = kCache; c < nch; ++c) put(c, chunk(c));
  if (tid == 0) LSE[row] = m + __logf(l);
}

template <typename T, int NC, int TA, int TB, int EPI>
hipError_t gemm(const void *A, const void *B, void *Cout, long sA, long sB, long sC, int lda,
                int ldb, int ldc, int BH, int M, int ncols_tot, int ncols_valid, int Kvalid,
                int Kend, float scale, int causal, const void *P, const float *Dv, int ldpv,
                hipStream_t st) {
  const int ntm = (M + 127) / 128, ntn = ncols_tot / NC;
  const long total = (long)BH * ntm * ntn;
  hipLaunchKernelGGL((std_gemm_kernel<T, NC, TA, TB, EPI>), dim3((unsigned)total), dim3(256), 0,
                     st, (const uint16_t *)A, (const uint16_t *)B, Cout, sA, sB, sC, lda, ldb,
                     ldc, M, ncols_valid, Kvalid, Kend, ntm, ntn, (int)total, scale, causal,
                     (const uint16_t *)P, Dv, ldpv);
  return hipGetLastError();
}

inline int round_up_int(int x, int a) { return (x + a - 1) / a * a; }

template <typename T, int D>
hipError_t std_fwd_t(int BH, int N, const void *Q, const void *K, const void *V, float scale,
                     int causal, float *S, void *P, void *O, float *LSE, hipStream_t st) {
  const int ldn = std_row_stride(N);
  const long snd = (long)N * D, snn = (long)N * ldn;
  // S = scale Q K^T: A = Q [N][D], B = K stored [N][D] (columns of C).
  hipError_t e = gemm<T, 128, 0, 1, kEpiScores>(Q, K, S, snd, snd, snn, D, D, ldn, BH, N, ldn, N,
                                                D, D, scale, causal, nullptr, nullptr, 0, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((std_softmax_kernel<T>), dim3((unsigned)((long)BH * N)), dim3(256), 0, st, S,
                     (uint16_t *)P, LSE, N, ldn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // O = P V: A = P [N][ldn], B = V stored [N (k)][D].
  return gemm<T, D, 0, 0, kEpiStore>(P, V, O, snn, snd, snd, ldn, D, D, BH, N, D, D, N,
                                     round_up_int(N, 32), 1.f, 0, nullptr, nullptr, 0, st);
}

template <typename T, int D>
hipError_t std_bwd_t(int BH, int N, const void *Q, const void *K, const void *V, const void *O,
                     const void *dO, const void *P, float scale, void *dS, float *Dv, void *dQ,
                     void *dK, void *dV, hipStream_t st) {
  const int ldn = std_row_stride(N);
  const long snd = (long)N * D, snn = (long)N * ldn;
  const int kq = round_up_int(N, 32);
  hipError_t e = launch_bwd_preprocess(std::is_same<T, BF16>::value ? kBF16 : kF16, BH, 1, N, D,
                                       O, dO, Dv, st);
  if (e != hipSuccess) return e;
  // dV = P^T dO: A = P stored [queries (k)][keys], B = dO stored [queries (k)][D].
  if ((e = gemm<T, D, 1, 0, kEpiStore>(P, dO, dV, snn, snd, snd, ldn, D, D, BH, N, D, D, N, kq,
                                       1.f, 0, nullptr, nullptr, 0, st)) != hipSuccess)
    return e;
  // dS = P o (dO V^T - D): A = dO [N][D], B = V stored [keys][D] (columns of C).
  if ((e = gemm<T, 128, 0, 1, kEpiDs>(dO, V, dS, snd, snd, snn, D, D, ldn, BH, N, ldn, N, D, D,
                                      1.f, 0, P, Dv, ldn, st)) != hipSuccess)
    return e;
  // dQ = scale dS K: A = dS [N][ldn], B = K stored [keys (k)][D].
  if ((e = gemm<T, D, 0, 0, kEpiStore>(dS, K, dQ, snn, snd, snd, ldn, D, D, BH, N, D, D, N, kq,
                                       scale, 0, nullptr, nullptr, 0, st)) != hipSuccess)
    return e;
  // dK = scale dS^T Q: A = dS stored [queries (k)][keys], B = Q stored [queries (k)][D].
  return gemm<T, D, 1, 0, kEpiStore>(dS, Q, dK, snn, snd, snd, ldn, D, D, BH, N, D, D, N, kq,
                                     scale, 0, nullptr, nullptr, 0, st);
}

}  // namespace

hipError_t launch_std_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                          const void *V, float scale, int causal, float *S, void *P, void *O,
                          float *LSE, hipStream_t st) {
  const int BH = B * H;
  if (dtype == kBF16)
    return d == 64 ? std_fwd_t<BF16, 64>(BH, N, Q, K, V, scale, causal, S, P, O, LSE, st)
                   : std_fwd_t<BF16, 128>(BH, N, Q, K, V, scale, causal, S, P, O, LSE, st);
  return d == 64 ? std_fwd_t<F16, 64>(BH, N, Q, K, V, scale, causal, S, P, O, LSE, st)
                 : std_fwd_t<F16, 128>(BH, N, Q, K, V, scale, causal, S, P, O, LSE, st);
}

hipError_t launch_std_bwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                          const void *V, const void *O, const void *dO, const void *P,
                          float scale, void *dS, float *Dv, void *dQ, void *dK, void *dV,
                          hipStream_t st) {
  const int BH = B * H;
  if (dtype == kBF16)
    return d == 64 ? std_bwd_t<BF16, 64>(BH, N, Q, K, V, O, dO, P, scale, dS, Dv, dQ, dK, dV, st)
                   : std_bwd_t<BF16, 128>(BH, N, Q, K, V, O, dO, P, scale, dS, Dv, dQ, dK, dV, st);
  return d == 64 ? std_bwd_t<F16, 64>(BH, N, Q, K, V, O, dO, P, scale, dS, Dv, dQ, dK, dV, st)
                 : std_bwd_t<F16, 128>(BH, N, Q, K, V, O, dO, P, scale, dS, Dv, dQ, dK, dV, st);
}

}  // namespace fa
