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
// also written to LDS, where each wave reads a 32x32 (query, column) tile of
// dQ = dS K over all KB keys and adds it into the fp32 workspace. Query tiles
// (Q, dO, LSE, D) are double-buffered in LDS and filled by direct buffer ->
// LDS loads issued one tile ahead.

#include <type_traits>

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
  static constexpr int kThreads = 512;               // 8 waves, two per SIMD
  static constexpr int KB = 128;                     // keys per workgroup, 32 per wave pair
  static constexpr int BR = (D == 128) ? 64 : 128;   // query rows per step
  static constexpr int NQW = BR / 64;                // 32-row query subtiles per wave
  static constexpr int NCH = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int QTILE = BR * D;               // 16-bit elements per Q or dO tile
  static constexpr int LPW = BR * CPR / kThreads;    // direct loads per wave per tile and tensor
  static constexpr int SS = KB + 8;                  // dS row stride
  static_assert(LPW == 2, "two direct loads per wave per tile");
  static_assert((BR / 32) * NDT == 8, "one 32x32 dQ tile per wave");
};

// Q, dO, K and V tiles are unpadded, row-major at 16-byte-chunk granularity,
// with the chunk index XOR-ed by swz_q(row). They are read two ways: row-wise
// (16 consecutive rows, one chunk each, per quarter-wave) and with
// transposing loads (4 consecutive rows x 4 chunks per half-wave). swz_q maps
// both access groups onto 16 distinct four-bank groups of the 64-bank LDS.
template <int D>
__device__ __forceinline__ int swz_q(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_main_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, float *__restrict__ dQacc,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int N, int nkb, int total, float c2,
    float scale) {
  using C = BwdCfg<D>;
  // Double buffers for the query tiles (named separately so the compiler can
  // tell the direct loads into one from the reads of the other), their fp32
  // LSE and D rows, dS, and the key block's K and V.
  __shared__ __attribute__((aligned(1024))) uint16_t Q0[C::QTILE], O0[C::QTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Q1[C::QTILE], O1[C::QTILE];
  __shared__ __attribute__((aligned(256))) float L0[2 * C::BR], L1[2 * C::BR];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[C::BR * C::SS];
  __shared__ __attribute__((aligned(1024))) uint16_t Kst[C::KB * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vst[C::KB * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int l32 = lane & 31, g = lane >> 5;
  const int ks = w & 3;   // key slice: keys 32 ks .. +31 of the block
  const int qh = w >> 2;  // query half: subtiles qh*NQW .. +NQW-1 of each query tile
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nkb;
  const int kb = tile - bh * nkb;
  const int k0 = kb * C::KB;
  const int wk0 = k0 + 32 * ks;  // first key of this wave
  const int mykey = wk0 + l32;   // key of this lane's S/P column
  const size_t base = (size_t)bh * N * D;
  const uint16_t *Qh = Q + base, *Kh = K + base, *Vh = V + base, *dOh = dO + base;
  float *dQh = dQacc + base;

  // K and V of the key block into LDS; keys past N read row N - 1 (masked).
  for (int c = tid; c < C::KB * C::CPR; c += C::kThreads) {
    const int row = c / C::CPR, ch = c % C::CPR;
    const int key = min(k0 + row, N - 1);
    const int pos = row * D + 8 * (ch ^ swz_q<D>(row));
    st128(Kst + pos, ld128(Kh + (size_t)key * D + 8 * ch));
    st128(Vst + pos, ld128(Vh + (size_t)key * D + 8 * ch));
  }

  const int nq = (N + C::BR - 1) / C::BR;
  const int it0 = CAUSAL ? k0 / C::BR : 0;  // earlier queries see none of these keys

  // Direct buffer -> LDS loads of a query tile: instruction i of wave w fills
  // LDS chunks (w*LPW + i)*64 + lane with the global chunk the swizzle puts
  // there. Waves 0 .. 2*BR/64-1 also load 64 LSE or D values each. Rows
  // past N re-read row N - 1 and are masked.
  const i32x4 qrs = make_rsrc(Qh, (uint32_t)N * D * 2);
  const i32x4 ors = make_rsrc(dOh, (uint32_t)N * D * 2);
  const i32x4 lrs = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4);
  const i32x4 drs = make_rsrc(Dvec + (size_t)bh * N, (uint32_t)N * 4);
  constexpr int kVecParts = C::BR / 64;
  int gq[C::LPW], grow[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int p = (w * C::LPW + i) * 64 + lane;
    const int r = p / C::CPR, sw = p % C::CPR;
    grow[i] = r;
    gq[i] = 2 * (r * D + 8 * (sw ^ swz_q<D>(r)));
  }
  auto issue = [&](uint16_t *Qb, uint16_t *Ob, float *Lb, int it) __attribute__((always_inline)) {
    const int q0 = it * C::BR;
    const int soff = q0 * D * 2;
    if (q0 + C::BR <= N) {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        buffer_load_lds16(qrs, gq[i], soff, Qb + (w * C::LPW + i) * 512);
        buffer_load_lds16(ors, gq[i], soff, Ob + (w * C::LPW + i) * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int shift = 2 * D * (min(q0 + grow[i], N - 1) - q0 - grow[i]);  // <= 0
        buffer_load_lds16(qrs, gq[i] + shift, soff, Qb + (w * C::LPW + i) * 512);
        buffer_load_lds16(ors, gq[i] + shift, soff, Ob + (w * C::LPW + i) * 512);
      }
    }
    if (w < 2 * kVecParts) {
      const int vec = w / kVecParts, part = w % kVecParts;
      const int voff = 4 * (min(q0 + 64 * part + lane, N - 1) - q0);
      raw_buffer_load_lds(vec == 0 ? lrs : drs,
                          (__attribute__((address_space(3))) void *)(Lb + vec * C::BR + 64 * part),
                          4, voff, 4 * q0, 0, 0);
    }
  };

  // Per-lane LDS byte offsets. The swizzle only touches address bits that
  // the row and column terms of one access leave zero, so every access is a
  // per-lane base XOR-ed with a compile-time constant (one v_xor per read):
  //  * row-wise reads (row 32qt + l%32, 16-byte chunk 2c + g):
  //      rb ^ (32 c + 64 D qt);
  //  * transposing reads (rows rowbase + (l%16)/4 of a 16-row block, columns
  //    32dt + 16((l/16)%2) + 4(l%4)): base(rowbase) ^ (64 dt + 2 D * block row),
  //    with one base per half of an operand (the swizzle depends on the row).
  const int jr = (lane & 15) / 4;
  const int cq = 2 * ((lane >> 4) & 1) + (lane & 3) / 2;  // chunk within a 64-byte column group
  auto tr_base = [&](int row) {
    const int f = swz_q<D>(row);
    return row * 2 * D + 16 * (cq ^ (f & 3)) + 8 * (lane & 1) + 64 * (f >> 2);
  };
  int rb;
  {
    const int f = swz_q<D>(l32);
    rb = l32 * 2 * D + 16 * (g ^ (f & 1)) + 32 * (f >> 1);
  }
  // Row-wise reads of this wave's keys 32 ks + l%32 in the K and V tiles.
  const int kb_off = rb ^ (64 * D * ks);
  // Q^T / dO^T operands: rows 16cc + 4g + (0..3) and 16cc + 8 + 4g + (0..3)
  // of a 32-row subtile (the P / dS register layout).
  const int tb1 = tr_base(4 * g + jr), tb2 = tr_base(8 + 4 * g + jr);
  // This wave's dQ tile: query subtile dq_qt, columns 32 dq_dt .. +31. Its K
  // operand: keys 16c + 8g + (0..3) and 16c + 8g + 4 + (0..3).
  const int dq_qt = w / C::NDT, dq_dt = w % C::NDT;
  const int tk1 = tr_base(8 * g + jr) ^ (64 * dq_dt), tk2 = tr_base(8 * g + 4 + jr) ^ (64 * dq_dt);
  // dQ atomics: this lane's element of row 8(r/4) + 4g + r%4 of its tile.
  const int dq_lane = (32 * dq_qt + 4 * g) * D + 32 * dq_dt + l32;
  auto at = [](const uint16_t *tile, int byte_off) {
    return (const uint16_t *)((const char *)tile + byte_off);
  };

  // dK^T and dV^T partial sums (this wave's query half): column = key
  // (l % 32), rows = d.
  f32x16 dk[C::NDT], dv[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  // Scheduling pattern of a product phase of kM MFMAs fed by two transposing
  // reads each: reads two MFMAs ahead, then the phase ends.
  auto tr_pipeline = [&](auto km_tag) __attribute__((always_inline)) {
    constexpr int kM = decltype(km_tag)::value;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < kM - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using KM = std::integral_constant<int, 2 * C::NQW * C::NDT>;

  // This wave's part of one query tile, up to dS in LDS. need_mask: the rows
  // hold rows past N, keys past N, or (causal) keys after some row; masked
  // scores become -inf, so P and dS are exactly 0 there. The mask is a
  // VALU-only branch, so every MFMA accumulation runs on one code path.
  auto part1 = [&](const uint16_t *Qs, const uint16_t *Os, const float *Lb, int q0,
                   bool need_mask) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    // S = Q K^T and dP = dO V^T: column = key, rows 8(r/4) + 4g + r%4.
    f32x16 s[C::NQW], dp[C::NQW];
#pragma unroll
    for (int t = 0; t < C::NQW; ++t) {
      const int qt = qh * C::NQW + t;
      s[t] = mfma32<T>(ld128(at(Qs, rb ^ (64 * D * qt))), ld128(at(Kst, kb_off)), kZero16);
      dp[t] = mfma32<T>(ld128(at(Os, rb ^ (64 * D * qt))), ld128(at(Vst, kb_off)), kZero16);
#pragma unroll
      for (int c = 1; c < C::NCH; ++c) {
        s[t] = mfma32<T>(ld128(at(Qs, rb ^ (32 * c + 64 * D * qt))),
                         ld128(at(Kst, kb_off ^ (32 * c))), s[t]);
        dp[t] = mfma32<T>(ld128(at(Os, rb ^ (32 * c + 64 * D * qt))),
                          ld128(at(Vst, kb_off ^ (32 * c))), dp[t]);
      }
    }
    // Operand reads two MFMAs ahead of their use (bounded register use).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::NQW * C::NCH - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < C::NQW; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * (qh * C::NQW + t) + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q >= N || mykey >= N || (CAUSAL && mykey > q)) s[t][r] = -INFINITY;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // P = 2^(S*scale*log2e - LSE*log2e); rows j = 0..3 of group i are
    // consecutive in LDS, read as one 16-byte word.
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 lse = *(const f32x4 *)(Lb + 32 * (qh * C::NQW + t) + 8 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * i + j;
          s[t][r] = fast_exp2(__builtin_fmaf(s[t][r], c2, -lse[j] * kLog2e));
        }
      }
    // dV^T += dO^T P
    u32x4 pk[C::NQW][2];
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pk[t][cc][h] = pack2<T>(s[t][8 * cc + 2 * h], s[t][8 * cc + 2 * h + 1]);
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
          const int x = 64 * dt + 2 * D * (32 * (qh * C::NQW + t) + 16 * cc);
          dv[dt] = mfma32<T>(cat(ld_tr16(at(Os, tb1 ^ x)), ld_tr16(at(Os, tb2 ^ x))),
                             pk[t][cc], dv[dt]);
        }
    tr_pipeline(KM{});
    // dS = P o (dP - D)
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 dd = *(const f32x4 *)(Lb + C::BR + 32 * (qh * C::NQW + t) + 8 * i + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[t][4 * i + j] = s[t][4 * i + j] * (dp[t][4 * i + j] - dd[j]);
      }
    // dK^T += Q^T dS
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pk[t][cc][h] = pack2<T>(dp[t][8 * cc + 2 * h], dp[t][8 * cc + 2 * h + 1]);
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
          const int x = 64 * dt + 2 * D * (32 * (qh * C::NQW + t) + 16 * cc);
          dk[dt] = mfma32<T>(cat(ld_tr16(at(Qs, tb1 ^ x)), ld_tr16(at(Qs, tb2 ^ x))),
                             pk[t][cc], dk[dt]);
        }
    tr_pipeline(KM{});
    // dS (16-bit) to LDS, [query][key]
#pragma unroll
    for (int t = 0; t < C::NQW; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int r = 8 * cc + 2 * h;
          const int ql = 32 * (qh * C::NQW + t) + 8 * (r >> 2) + 4 * g + (r & 3);
          dSs[ql * C::SS + 32 * ks + l32] = (uint16_t)(pk[t][cc][h] & 0xffffu);
          dSs[(ql + 1) * C::SS + 32 * ks + l32] = (uint16_t)(pk[t][cc][h] >> 16);
        }
    __builtin_amdgcn_sched_barrier(0);
  };
  // This wave's dQ tile over the KB keys, added into the fp32 accumulator.
  auto part2 = [&](int q0) __attribute__((always_inline)) {
    f32x16 dq = kZero16;
#pragma unroll
    for (int c = 0; c < C::KB / 16; ++c) {
      const int x = 2 * D * 16 * c;
      dq = mfma32<T>(ld128(dSs + (32 * dq_qt + l32) * C::SS + 16 * c + 8 * g),
                     cat(ld_tr16(at(Kst, tk1 ^ x)), ld_tr16(at(Kst, tk2 ^ x))),
                     c == 0 ? kZero16 : dq);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < C::KB / 16 - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    float *rowp = dQh + (size_t)q0 * D + dq_lane;
    if (q0 + C::BR <= N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) unsafeAtomicAdd(rowp + (8 * (r >> 2) + (r & 3)) * D, dq[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 32 * dq_qt + 8 * (r >> 2) + 4 * g + (r & 3);
        if (q < N) unsafeAtomicAdd(rowp + (8 * (r >> 2) + (r & 3)) * D, dq[r]);
      }
    }
  };
  auto step = [&](const uint16_t *Qs, const uint16_t *Os, const float *Lb, int it, auto next)
      __attribute__((always_inline)) {
    const int q0 = it * C::BR;
    const int q0w = q0 + 32 * C::NQW * qh;  // first query row of this wave
    part1(Qs, Os, Lb, q0,
          (q0w + 32 * C::NQW > N) || (wk0 + 32 > N) || (CAUSAL && wk0 + 31 > q0w));
    // This wave has read the tile: load the next one into the other buffer
    // (every wave finished reading that buffer before the previous dS
    // barrier); the loads land during the dQ product and the atomics.
    next();
    barrier_lds();  // dS complete (the loads just issued keep flying)
    part2(q0);
  };

  // Double-buffered sweep over the query tiles: wait for this wave's loads,
  // barrier (every wave's loads landed; every wave done reading dS), compute
  // (issuing the next tile's loads once the current tile has been read).
  __syncthreads();  // K and V staged
  if (it0 < nq) issue(Q0, O0, L0, it0);
  for (int it = it0; it < nq; ++it) {
    const bool odd = (it - it0) & 1;
    wait_vmem_all();
    __syncthreads();
    step(odd ? Q1 : Q0, odd ? O1 : O0, odd ? L1 : L0, it,
         [&]() __attribute__((always_inline)) {
           if (it + 1 < nq) {
             if (odd) issue(Q0, O0, L0, it + 1);
             else issue(Q1, O1, L1, it + 1);
           }
         });
  }

  // Sum the two query halves' partial dK, dV (waves ks and ks + 4) through
  // LDS: the second half writes its partials lane-major into free tiles.
  __syncthreads();
  float *xk = ks == 0 ? (float *)Q0 : ks == 1 ? (float *)Q1 : ks == 2 ? (float *)Kst : (float *)Vst;
  float *xv = ks == 0 ? (float *)O0 : ks == 1 ? (float *)O1 : xk + C::NDT * 16 * 64;
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        xk[(dt * 16 + r) * 64 + lane] = dk[dt][r];
        xv[(dt * 16 + r) * 64 + lane] = dv[dt][r];
      }
  }
  __syncthreads();
  if (qh == 0 && mykey < N) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[dt][r] += xk[(dt * 16 + r) * 64 + lane];
        dv[dt][r] += xv[(dt * 16 + r) * 64 + lane];
      }
    // dK = scale * dK, dV; lane holds 4 consecutive columns per row.
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
