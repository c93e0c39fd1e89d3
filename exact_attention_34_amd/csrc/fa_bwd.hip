// fa_bwd.hip -- backward pass of exact attention on gfx950.
//
// Follows the blocked backward of the "Flash Attention" notes (section 3,
// part 4.2, and the backward-derivation page, part 6), with the two loops
// swapped: each workgroup owns a block of KB keys, keeps dK and dV for them in
// registers, and walks the query tiles. For each tile it recomputes
//   S = Q K^T,  P = exp(scale*S - LSE)            (section 3, part 4.1)
// and accumulates
//   dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   dK += dS^T Q,  dQ += dS K                      (derivation, parts 3-4)
// with D = rowsum(dO o O) precomputed by a separate pass (derivation, part 5).
// dQ rows receive contributions from every key block, so they are summed with
// fp32 atomics into a workspace and converted (times scale) at the end; the
// scale of dK is applied in the epilogue (the Ascend recompute article writes
// 1/sqrt(d_k) into both dQ and dK).
//
// Per wave (32 keys): K and V stay in VGPRs as the B operands of S = Q K^T and
// dP = dO V^T. S/P and dP/dS come out of the MFMA with one key per lane
// (column l % 32) and 16 query rows per lane, which is exactly the B-operand
// layout of dV^T = dO^T P and dK^T = Q^T dS, so P and dS never leave
// registers for those two products; the dO^T and Q^T operands are read from
// the row-major tiles with transposing LDS reads (ds_read_b64_tr_b16). dS is
// also written to LDS,
// where each wave reads a 32x32 (query, column) tile of dQ = dS K over all KB
// keys and adds it into the fp32 workspace.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik (fp32), and dQacc = 0.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                      const uint16_t *__restrict__ dO,
                                                      float *__restrict__ Dvec,
                                                      float *__restrict__ dQacc, long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / TPR;
  const int sub = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld128(O + row * D + 8 * sub);
    const u32x4 b = ld128(dO + row * D + 8 * sub);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc += to_f32<T>((uint16_t)(a[h] & 0xffffu)) * to_f32<T>((uint16_t)(b[h] & 0xffffu));
      acc += to_f32<T>((uint16_t)(a[h] >> 16)) * to_f32<T>((uint16_t)(b[h] >> 16));
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4 *)(dQacc + row * D + 8 * sub) = z;
    *(f32x4 *)(dQacc + row * D + 8 * sub + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// dQ = dtype(scale * dQacc)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float *__restrict__ acc,
                                                         uint16_t *__restrict__ dQ, long n8,
                                                         float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4 *)(acc + 8 * i);
  const f32x4 b = *(const f32x4 *)(acc + 8 * i + 4);
  u32x4 v;
  v[0] = pack2<T>(a[0] * scale, a[1] * scale);
  v[1] = pack2<T>(a[2] * scale, a[3] * scale);
  v[2] = pack2<T>(b[0] * scale, b[1] * scale);
  v[3] = pack2<T>(b[2] * scale, b[3] * scale);
  st128(dQ + 8 * i, v);
}

// ---------------------------------------------------------------------------
// Main backward kernel.
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int kThreads = 256;               // 4 waves
  static constexpr int KB = 128;                     // keys per workgroup, 32 per wave
  static constexpr int BR = (D == 128) ? 32 : 64;    // query rows per step
  static constexpr int NQT = BR / 32;                // 32-row query subtiles per step
  static constexpr int NCH = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int TPR = D / 8;
  static constexpr int QS = D + 32;  // Q / dO row stride: an odd multiple of 64 bytes (swizzled)
  static constexpr int SS = KB + 8;  // dS row stride
  static constexpr int KSTG = D + 8; // K staging stride (prologue only)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BR * QS;
  static constexpr int OFF_DS = OFF_DO + BR * QS;
  static constexpr int N16_LOOP = OFF_DS + BR * SS;
  static constexpr int N16 = (N16_LOOP > KB * KSTG) ? N16_LOOP : KB * KSTG;  // 16-bit elements
  static constexpr int CPT = (BR * D / 8) / kThreads;  // 16-byte chunks per thread per tensor
  static_assert(CPT == 2, "each thread loads two chunks per tensor");
  static_assert(NQT * NDT == 4, "one 32x32 dQ tile per wave");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, float *__restrict__ dQacc,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int N, int nkb, int total, float c2,
    float scale) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::N16];
  __shared__ float lse2s[C::BR];
  __shared__ float dvs[C::BR];
  uint16_t *Qs = lds + C::OFF_Q, *dOs = lds + C::OFF_DO, *dSs = lds + C::OFF_DS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nkb;
  const int kb = tile - bh * nkb;
  const int k0 = kb * C::KB;
  const int wk0 = k0 + 32 * w;   // first key of this wave
  const int mykey = wk0 + l32;   // key of this lane's S/P column
  const size_t base = (size_t)bh * N * D;
  const uint16_t *Qh = Q + base, *Kh = K + base, *Vh = V + base, *dOh = dO + base;
  const float *LSEh = LSE + (size_t)bh * N, *Dh = Dvec + (size_t)bh * N;
  float *dQh = dQacc + base;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // K and V of this wave's keys as B operands (k = d).
  u32x4 kreg[C::NCH], vreg[C::NCH];
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    kreg[c] = (mykey < N) ? ld128(Kh + (size_t)mykey * D + 16 * c + 8 * g) : zero4;
    vreg[c] = (mykey < N) ? ld128(Vh + (size_t)mykey * D + 16 * c + 8 * g) : zero4;
  }
  // K of the whole key block, transposed, as the B operand of this wave's dQ
  // tile (query subtile dq_qt, columns 32*dq_dt..+31): staged through LDS.
  const int dq_qt = w / C::NDT, dq_dt = w % C::NDT;
  for (int c = tid; c < C::KB * C::TPR; c += C::kThreads) {
    const int row = c / C::TPR, col = 8 * (c % C::TPR);
    const int key = k0 + row;
    st128(lds + row * C::KSTG + col, (key < N) ? ld128(Kh + (size_t)key * D + col) : zero4);
  }
  __syncthreads();
  u32x4 ktreg[C::KB / 16];
#pragma unroll
  for (int c = 0; c < C::KB / 16; ++c)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int kr = 16 * c + 8 * g + 2 * h;
      const uint32_t lo = lds[kr * C::KSTG + 32 * dq_dt + l32];
      const uint32_t hi = lds[(kr + 1) * C::KSTG + 32 * dq_dt + l32];
      ktreg[c][h] = lo | (hi << 16);
    }
  __syncthreads();

  const int nq = (N + C::BR - 1) / C::BR;
  const int it0 = CAUSAL ? k0 / C::BR : 0;  // earlier queries see none of these keys

  // Query-tile prefetch: chunk c = tid + 256*r of the tile is row c / TPR,
  // 16-byte chunk c % TPR; stored row-major with the chunk swizzle.
  u32x4 qpre[2], dopre[2];
  float lpre = 0.f, dpre = 0.f;
  auto gload = [&](int it) {
    const int q0 = it * C::BR;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + C::kThreads * r;
      const int q = q0 + c / C::TPR, col = 8 * (c % C::TPR);
      qpre[r] = (q < N) ? ld128(Qh + (size_t)q * D + col) : zero4;
      dopre[r] = (q < N) ? ld128(dOh + (size_t)q * D + col) : zero4;
    }
    if (tid < C::BR) {
      const int q = q0 + tid;
      lpre = (q < N) ? LSEh[q] * kLog2e : INFINITY;  // rows past N get P = 0
      dpre = (q < N) ? Dh[q] : 0.f;
    }
  };
  auto swrite = [&]() {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + C::kThreads * r;
      const int row = c / C::TPR, pos = 8 * swz(row, c % C::TPR);
      st128(Qs + row * C::QS + pos, qpre[r]);
      st128(dOs + row * C::QS + pos, dopre[r]);
    }
    if (tid < C::BR) {
      lse2s[tid] = lpre;
      dvs[tid] = dpre;
    }
  };
  // Row-wise operand read (lane = row, 8 consecutive columns 16c + 8g).
  auto rd_row = [&](const uint16_t *tile, int row, int c) {
    return ld128(tile + row * C::QS + 8 * swz(row, 2 * c + g));
  };
  // Transposed operand read: rows q0 + 4g + (l%16)/4 and that + 8, column
  // block 32dt + 16*((l/16)%2) + 4*(l%4) -> lane holds column 32dt + l%32 at
  // rows q0 + 4g + (0..3) and q0 + 8 + 4g + (0..3).
  const int tr_row = 4 * g + (lane & 15) / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto rd_tr = [&](const uint16_t *tile, int q0, int dt) {
    const int r1 = q0 + tr_row, r2 = r1 + 8, col = 32 * dt + tr_col;
    const u32x2 a = ld_tr16(tile + r1 * C::QS + 8 * swz(r1, col >> 3) + (col & 7));
    const u32x2 b = ld_tr16(tile + r2 * C::QS + 8 * swz(r2, col >> 3) + (col & 7));
    return cat(a, b);
  };

  // dK^T and dV^T accumulators: column = key (l % 32), rows = d.
  f32x16 dk[C::NDT], dv[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  if (it0 < nq) {
    gload(it0);
    swrite();
  }
  for (int it = it0; it < nq; ++it) {
    const int q0 = it * C::BR;
    __syncthreads();  // tile `it` in LDS; every wave is past its dQ reads of dS
    const bool need_mask = (wk0 + 32 > N) || (CAUSAL && wk0 + 31 > q0);

    // S = Q K^T and P = 2^(S*scale*log2e - LSE*log2e)
    f32x16 s[C::NQT], dp[C::NQT];
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[qt][r] = 0.f;
        dp[qt][r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
        s[qt] = mfma32<T>(rd_row(Qs, 32 * qt + l32, c), kreg[c], s[qt]);
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
        dp[qt] = mfma32<T>(rd_row(dOs, 32 * qt + l32, c), vreg[c], dp[qt]);
    }
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
        float p = fast_exp2(s[qt][r] * c2 - lse2s[ql]);
        if (need_mask && (mykey >= N || (CAUSAL && mykey > q0 + ql))) p = 0.f;
        s[qt][r] = p;
      }
    // dV^T += dO^T P
    u32x4 pk[C::NQT][2];
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pk[qt][cc][h] = pack2<T>(s[qt][8 * cc + 2 * h], s[qt][8 * cc + 2 * h + 1]);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          dv[dt] = mfma32<T>(rd_tr(dOs, 32 * qt + 16 * cc, dt), pk[qt][cc], dv[dt]);
    // dS = P o (dP - D)
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
        dp[qt][r] = s[qt][r] * (dp[qt][r] - dvs[ql]);
      }
    // dK^T += Q^T dS
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pk[qt][cc][h] = pack2<T>(dp[qt][8 * cc + 2 * h], dp[qt][8 * cc + 2 * h + 1]);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          dk[dt] = mfma32<T>(rd_tr(Qs, 32 * qt + 16 * cc, dt), pk[qt][cc], dk[dt]);
    // dS (16-bit) to LDS, [query][key]
#pragma unroll
    for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int r = 8 * cc + 2 * h;
          const int ql = 32 * qt + 8 * (r >> 2) + 4 * g + (r & 3);
          dSs[ql * C::SS + 32 * w + l32] = (uint16_t)(pk[qt][cc][h] & 0xffffu);
          dSs[(ql + 1) * C::SS + 32 * w + l32] = (uint16_t)(pk[qt][cc][h] >> 16);
        }
    if (it + 1 < nq) gload(it + 1);
    __syncthreads();  // dS complete; Q/dO tiles no longer read

    // dQ tile (queries 32*dq_qt.., columns 32*dq_dt..) over the KB keys
    f32x16 dq;
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[r] = 0.f;
#pragma unroll
    for (int c = 0; c < C::KB / 16; ++c) {
      const u32x4 a = ld128(dSs + (32 * dq_qt + l32) * C::SS + 16 * c + 8 * g);
      dq = mfma32<T>(a, ktreg[c], dq);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = q0 + 32 * dq_qt + 8 * (r >> 2) + 4 * g + (r & 3);
      if (q < N) unsafeAtomicAdd(dQh + (size_t)q * D + 32 * dq_dt + l32, dq[r]);
    }
    if (it + 1 < nq) swrite();
  }

  // Epilogue: dK = scale * dK, dV; lane holds 4 consecutive columns per row.
  if (mykey < N) {
    uint16_t *dKrow = dK + base + (size_t)mykey * D;
    uint16_t *dVrow = dV + base + (size_t)mykey * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 a, b;
        a[0] = pack2<T>(dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale);
        a[1] = pack2<T>(dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale);
        b[0] = pack2<T>(dv[dt][4 * i], dv[dt][4 * i + 1]);
        b[1] = pack2<T>(dv[dt][4 * i + 2], dv[dt][4 * i + 3]);
        *(u32x2 *)(dKrow + 32 * dt + 8 * i + 4 * g) = a;
        *(u32x2 *)(dVrow + 32 * dt + 8 * i + 4 * g) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t pre(long rows, const void *O, const void *dO, float *Dv, float *acc,
                      hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t *)O, (const uint16_t *)dO, Dv, acc, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                                 const void *dO, float *Dvec, float *dQacc, hipStream_t st) {
  const long rows = (long)B * H * N;
  if (dtype == kBF16)
    return d == 64 ? pre<BF16, 64>(rows, O, dO, Dvec, dQacc, st)
                   : pre<BF16, 128>(rows, O, dO, Dvec, dQacc, st);
  return d == 64 ? pre<F16, 64>(rows, O, dO, Dvec, dQacc, st)
                 : pre<F16, 128>(rows, O, dO, Dvec, dQacc, st);
}

template <typename T, int D, bool CAUSAL>
static hipError_t bmain(int BH, int N, const void *Q, const void *K, const void *V,
                        const void *dO, const float *LSE, const float *Dv, float c2, float scale,
                        float *acc, void *dK, void *dV, hipStream_t st) {
  using C = BwdCfg<D>;
  const int nkb = (N + C::KB - 1) / C::KB;
  const int total = nkb * BH;
  hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL>), dim3(total), dim3(C::kThreads), 0, st,
                     (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                     (const uint16_t *)dO, LSE, Dv, acc, (uint16_t *)dK, (uint16_t *)dV, N, nkb,
                     total, c2, scale);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t bmain_c(int causal, int BH, int N, const void *Q, const void *K, const void *V,
                          const void *dO, const float *LSE, const float *Dv, float c2,
                          float scale, float *acc, void *dK, void *dV, hipStream_t st) {
  return causal ? bmain<T, D, true>(BH, N, Q, K, V, dO, LSE, Dv, c2, scale, acc, dK, dV, st)
                : bmain<T, D, false>(BH, N, Q, K, V, dO, LSE, Dv, c2, scale, acc, dK, dV, st);
}

hipError_t launch_bwd_main(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                           const void *V, const void *dO, const float *LSE, const float *Dvec,
                           float scale, int causal, float *dQacc, void *dK, void *dV,
                           hipStream_t st) {
  const int BH = B * H;
  const float c2 = scale * kLog2e;
  if (dtype == kBF16)
    return d == 64 ? bmain_c<BF16, 64>(causal, BH, N, Q, K, V, dO, LSE, Dvec, c2, scale, dQacc,
                                       dK, dV, st)
                   : bmain_c<BF16, 128>(causal, BH, N, Q, K, V, dO, LSE, Dvec, c2, scale,
                                        dQacc, dK, dV, st);
  return d == 64 ? bmain_c<F16, 64>(causal, BH, N, Q, K, V, dO, LSE, Dvec, c2, scale, dQacc, dK,
                                    dV, st)
                 : bmain_c<F16, 128>(causal, BH, N, Q, K, V, dO, LSE, Dvec, c2, scale, dQacc,
                                     dK, dV, st);
}

hipError_t launch_bwd_dq_convert(int dtype, int B, int H, int N, int d, const float *dQacc,
                                 float scale, void *dQ, hipStream_t st) {
  const long n8 = (long)B * H * N * d / 8;
  const long blocks = (n8 + 255) / 256;
  if (dtype == kBF16)
    hipLaunchKernelGGL((dq_convert_kernel<BF16>), dim3((unsigned)blocks), dim3(256), 0, st,
                       dQacc, (uint16_t *)dQ, n8, scale);
  else
    hipLaunchKernelGGL((dq_convert_kernel<F16>), dim3((unsigned)blocks), dim3(256), 0, st,
                       dQacc, (uint16_t *)dQ, n8, scale);
  return hipGetLastError();
}

}  // namespace fa
