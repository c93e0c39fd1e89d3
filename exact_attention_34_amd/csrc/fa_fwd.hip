// fa_fwd.hip -- forward pass of exact attention on gfx950.
//
// One workgroup (4 or 8 waves) computes BR = 32 * waves query rows of one
// (batch, head) slice and sweeps the key/value tiles once ("Flash Attention"
// notes, section 1: Q blocks in the outer loop, K/V blocks in the inner one;
// section 2, part 4.2: the forward loop). It keeps a running reference m and
// normaliser l per row and rescales the unnormalised output O~ by
// exp(m_old - m_new) whenever m moves (section 2, parts 3.1 and 4.1, the
// two-block merges), so no N x N array is formed; the division by l is
// deferred to the end and LSE = m + log l is returned for the backward
// (section 3, part 3).
//
// Work is done in base 2: scores are scaled by scale * log2(e) so that one
// v_exp_f32 (2^x) gives each exponential, and m is kept in those units.
//
// Data flow per wave (32 query rows, 16-bit inputs):
//   * Q rows stay in VGPRs for the whole sweep, as the B operand of
//     S^T = K Q^T (v_mfma_f32_32x32x16_{bf16,f16}); lane l owns query row
//     l % 32, so a row's 64 tile scores sit in two lanes (l and l ^ 32).
//   * The row sum is an in-register reduction plus one v_permlane32_swap
//     between the wave halves (at the end of the sweep). The row max is
//     formed only when the reference m has to move (see below).
//   * P, rounded to the input type, is the B operand of O~^T += V^T P^T
//     straight from registers; the V^T operand is read from the row-major V
//     tile with transposing LDS reads (ds_read_b64_tr_b16).
//   * K and V tiles are double-buffered in LDS (row-major, XOR-swizzled at
//     16-byte granularity) and filled by direct buffer->LDS loads
//     (buffer_load_dwordx4 ... lds), issued between the MFMAs of the step
//     that opens with the barrier: K two tiles ahead, V one step before it is
//     used. The waves of a workgroup share every tile.
// The fp32 variant is the same loop on v_mfma_f32_32x32x2_f32 with P kept in
// fp32.

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int W = 4>
struct FwdCfg {
  static constexpr int kWaves = W;
  static constexpr int kWavesPerSimd = 2;          // resident waves per SIMD (register budget)
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BR = 32 * kWaves;           // query rows per workgroup, 32 per wave
  static constexpr int BC = 64;                    // keys per tile
  static constexpr int NT = BC / 32;               // 32-key subtiles per tile
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BC * D;              // 16-bit elements per K or V tile
  static constexpr int NCH = D / 16;               // 16-wide k chunks of q . k
  static constexpr int NDT = D / 32;               // 32-wide output column tiles
  static constexpr int LPW = BC * CPR / kThreads;  // direct loads per wave per tile and tensor
  static constexpr int SH = (CPR == 16) ? 0 : 1;
  static_assert(LPW >= 1, "every wave loads part of each tile");
};

// LDS tiles are unpadded and row-major at 16-byte-chunk granularity, with the
// chunk index of row r XOR-ed by a row function (64 banks of 4 bytes):
//  * K, read row-wise (16 consecutive rows, one chunk each, per quarter-wave):
//    swz_k spreads 16 consecutive rows over the 16 four-bank groups;
//  * V, read with transposing loads (4 consecutive rows x 4 chunks per
//    half-wave): swz_v makes those 16 chunks land in distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  using C = FwdCfg<D>;
  return (row >> C::SH) & (C::CPR - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  using C = FwdCfg<D>;
  return (4 * (row >> C::SH)) & (C::CPR - 4);
}

// The sweep is software-pipelined: step j takes the exponentials of tile j
// on the vector ALUs while the matrix cores run the P V products of tile
// j - 1 and the scores of tile j + 1, so that each wave keeps both busy. K
// tiles are loaded two tiles ahead, V tiles one step before their use.
//
// Reference max. Any reference m gives the same O~ / l (the merges above
// hold for any m that is shared by O~ and l), so m only has to keep P finite
// and inside the 16-bit range. Step j therefore first takes P = 2^(s c2 - m)
// against the current m and keeps it when each lane's sum of its P values is
// at most kSumMax (every P is then at most kSumMax). Only otherwise -- and
// for a row's first tile -- does m move to the row max: the scores are
// formed again from K in global memory (the LDS tile is being refilled), O~
// and l are rescaled and P recomputed. With scores that are not adversarial
// this is a handful of tiles per row, and the common step forms no max.
//
// One block of BR query rows (block qb of slice bh) against the keys in
// [kfirst, klim) (kfirst a multiple of BC; the whole row is [0, Nk)). The
// slice has Nq queries and Nk keys; query i sits at position qoff + i, which
// the causal mask compares with the key index (qoff = 0 when Nq = Nk, and
// Nk - Nq for new queries appended to a cached prefix). K0, K1, V0, V1 are
// the workgroup's LDS tiles. PART = false writes O (in T,
// normalised) and LSE; PART = true writes the partial result of this key
// range in fp32 to Op / Lp: O~ / l and m + log l, or 0 and -inf for a row
// that sees none of these keys.
template <typename T, int D, int W, bool CAUSAL, bool PART>
__device__ __forceinline__ void fwd_block(const uint16_t *__restrict__ Q,
                                          const uint16_t *__restrict__ K,
                                          const uint16_t *__restrict__ V, uint16_t *__restrict__ O,
                                          float *__restrict__ LSE, float *__restrict__ Op,
                                          float *__restrict__ Lp, int Nq, int Nk, int qoff,
                                          int bh, int qb,
                                          int kfirst, int klim, float c2, uint16_t *K0,
                                          uint16_t *K1, uint16_t *V0, uint16_t *V1) {
  using C = FwdCfg<D, W>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = qb * C::BR;
  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + l32;
  const size_t base = (size_t)bh * Nq * D;   // Q, O rows of this slice
  const size_t kvbase = (size_t)bh * Nk * D;  // K, V rows
  const uint16_t *Qh = Q + base, *Kh = K + kvbase, *Vh = V + kvbase;

  // Rows past Nq are read from row Nq - 1 (clamped, always valid memory) and
  // never stored; keys past the range are masked.
  u32x4 qreg[C::NCH];
  const int qld = min(qrow, Nq - 1);
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) qreg[c] = ld128(Qh + (size_t)qld * D + 16 * c + 8 * g);

  const int kend = CAUSAL ? min(klim, qoff + q0 + C::BR) : klim;
  const int ntiles = max(kend - kfirst + C::BC - 1, 0) / C::BC;

  // Direct buffer -> LDS loads: instruction i of wave w fills LDS chunks
  // (w*LPW + i)*64 + lane; this lane fetches the global chunk that belongs
  // there under the swizzle (byte offset within the tile).
  int gk[C::LPW], gv[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int p = (w * C::LPW + i) * 64 + lane;
    const int r = p / C::CPR, sw = p % C::CPR;
    gk[i] = 2 * (r * D + 8 * (sw ^ swz_k<D>(r)));
    gv[i] = 2 * (r * D + 8 * (sw ^ swz_v<D>(r)));
  }
  // Buffer resource over the rows of tile kt that exist (below kend): the
  // range check makes the loads of rows past them -- or of a whole tile past
  // the last one -- write zeros, whose keys are masked.
  auto tile_rsrc = [&](const uint16_t *src, int kt) __attribute__((always_inline)) {
    const int kb = kfirst + kt * C::BC;
    const int rows = max(min(kend - kb, C::BC), 0);
    return make_rsrc(src + (size_t)min(kb, Nk) * D, (uint32_t)rows * D * 2);
  };
  // Load i of this wave for tile kt of one tensor into the LDS tile dst.
  auto dma = [&](const i32x4 &rs, const int (&go)[C::LPW], uint16_t *dst, int i)
      __attribute__((always_inline)) {
    buffer_load_lds16(rs, go[i], 0, dst + (w * C::LPW + i) * 512);
  };
  auto kbuf = [&](int b) { return b ? K1 : K0; };
  auto vbuf = [&](int b) { return b ? V1 : V0; };

  // Per-lane operand offsets (elements). K, row-wise: row 32t + l%32,
  // chunk 2c + g. V, transposing: rows 4g + (l%16)/4 (+8 for the upper half
  // of the operand) of each 16-key chunk, columns 32dt + 16((l/16)%2) +
  // 4(l%4); the swizzle term depends on the lane only.
  int koff[C::NCH], voff[C::NDT];
  {
    const int kx = swz_k<D>(l32);
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) koff[c] = l32 * D + 8 * ((2 * c + g) ^ kx);
    const int vr = 4 * g + (lane & 15) / 4;
    const int vx = swz_v<D>(vr);
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
      voff[dt] = vr * D + 8 * ((4 * dt + 2 * ((lane >> 4) & 1) + (lane & 3) / 2) ^ vx) +
                 4 * (lane & 1);
  }

  f32x16 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // reference: the row max when it last moved (base-2 units)
  float l_run = 0.f;        // this lane's share of the running normaliser

  constexpr int NT = C::NT;
  // S^T = K Q^T for one K tile, NT 32-key subtiles; lane: query qrow, keys
  // 8(r/4)+4g+r%4. MFMA c of subtile t is number NT c + t.
  auto s_mfma = [&](f32x16 (&sx)[NT], const uint16_t *Ks, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sx[t] = mfma32<T>(ld128(Ks + koff[c] + 32 * t * D), qreg[c], c == 0 ? kZero16 : sx[t]);
  };
  // P = 2^(s*c2 - m) for the 16 keys of chunk cc of subtile t (registers
  // 8cc .. 8cc+7: keys 16cc + 4g + (0..3) and 16cc + 8 + 4g + (0..3)),
  // rounded to T in pairs -- the B operand of O~^T += V^T P^T. The row sum
  // adds the fp32 values (the normaliser and LSE keep fp32 accuracy).
  auto p_chunk = [&](const f32x16 &sx, int cc, float mb, float &psum)
      __attribute__((always_inline)) {
    u32x4 pp;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float p0 = fast_exp2(__builtin_fmaf(sx[8 * cc + 2 * h], c2, -mb));
      const float p1 = fast_exp2(__builtin_fmaf(sx[8 * cc + 2 * h + 1], c2, -mb));
      pp[h] = pack2<T>(p0, p1);
      psum += p0 + p1;
    }
    return pp;
  };
  // O~^T += V^T P^T for chunk cc of subtile t; V^T takes the same keys for
  // column 32dt + l%32 with two transposing reads.
  auto pv_mfma = [&](const uint16_t *Vs, int t, int cc, const u32x4 &pp)
      __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
      const uint16_t *src = Vs + voff[dt] + (32 * t + 16 * cc) * D;
      o[dt] = mfma32<T>(cat(ld_tr16(src), ld_tr16(src + 8 * D)), pp, o[dt]);
    }
  };

  // A step has two parts: the previous tile's P V MFMAs (kMfmaP), then the
  // next tile's S MFMAs (kMfmaS), each with half of this tile's
  // exponentials: kValu1 / kValu2 vector instructions after each MFMA, and a
  // direct load every kDmaGap MFMAs (V loads in the first part, K in the
  // second).
  constexpr int kMfmaS = NT * C::NCH, kMfmaP = 2 * NT * C::NDT;
  constexpr int kValu1 = (D == 128) ? 3 : 6, kValu2 = (D == 128) ? 3 : 6;
  constexpr int kDmaGap1 = kMfmaP / C::LPW, kDmaGap2 = kMfmaS / C::LPW;
  // Bound on each lane's sum of P against the current reference (below the
  // fp16 maximum, 65504).
  constexpr float kSumMax = 32768.f;

  // Reference update for the scores s of one tile (a uniform branch, taken
  // for a row's first tile and when P would outgrow kSumMax): m moves to the
  // row max, O~ and l are rescaled, P and its sum are recomputed.
  auto rebase = [&](f32x16 (&s)[NT], u32x4 (&pc)[2 * NT], float &psum)
      __attribute__((always_inline)) {
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[t][r]);
    mloc = pair_max(mloc);
    const float m_cand = fmaxf(m_run, mloc * c2);
    if (m_cand > m_run) {
      const float alpha = fast_exp2(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float mb = (m_run == -INFINITY) ? 0.f : m_run;
    psum = 0.f;
#pragma unroll
    for (int k = 0; k < 2 * NT; ++k) pc[k] = p_chunk(s[k / 2], k % 2, mb, psum);
  };

  // Scores of keys past the range or (causal) after the row's position
  // become -inf. Key kb + 4g + off is visible iff off <= lim (one compare
  // per score).
  auto apply_mask = [&](f32x16 (&s)[NT], int kb) __attribute__((always_inline)) {
    if ((kb + C::BC > klim) || (CAUSAL && kb + C::BC - 1 > qoff + wq0)) {
      const int lim = (CAUSAL ? min(qoff + qrow, klim - 1) : klim - 1) - kb - 4 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 8 * (r >> 2) + (r & 3) > lim) s[t][r] = -INFINITY;
    }
  };

  // Scores of tile kt again, from K in global memory (the tile's LDS buffer
  // is being refilled): rows past Nk read row Nk - 1 and are masked.
  auto rescore = [&](f32x16 (&sr)[NT], int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = min(kb + 32 * t + l32, Nk - 1);
        sr[t] = mfma32<T>(ld128(Kh + (size_t)row * D + 16 * c + 8 * g), qreg[c],
                          c == 0 ? kZero16 : sr[t]);
      }
    apply_mask(sr, kb);
  };

  auto pv_all = [&](const u32x4 (&pp)[2 * NT], const uint16_t *Vs) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2 * NT; ++k) pv_mfma(Vs, k / 2, k % 2, pp[k]);
  };

  // One tile kt: s holds its scores (already issued), sn receives those of
  // tile kt + 1 (from K buffer b ^ 1; past the last tile the result is
  // unused), pc receives its P. The P V MFMAs of tile kt - 1 (P in pp, V in
  // V buffer b ^ 1) run in the same step, so that the exponentials of tile
  // kt overlap both kinds of MFMA.
  auto step = [&](auto first, int kt, f32x16 (&s)[NT], f32x16 (&sn)[NT], const u32x4 (&pp)[2 * NT],
                  u32x4 (&pc)[2 * NT], int b) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first)::value;
    const int kb = kfirst + kt * C::BC;
    // Every wave's loads of K (kt + 1) and V (kt - 1) have landed, and every
    // wave is done with K buffer b (read for tile kt) and V buffer b (read
    // for tile kt - 2), which receive K (kt + 2) and V (kt).
    wait_vmem_all();
    __syncthreads();
    const uint16_t *Kn = kbuf(b ^ 1), *Vp = vbuf(b ^ 1);
    const i32x4 krs = tile_rsrc(Kh, kt + 2), vrs = tile_rsrc(Vh, kt);

    __builtin_amdgcn_sched_barrier(0);
    apply_mask(s, kb);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FIRST) {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        dma(krs, gk, kbuf(b), i);
        dma(vrs, gv, vbuf(b), i);
      }
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) s_mfma(sn, Kn, c);
      float psum;
      rebase(s, pc, psum);
      l_run += psum;
    } else {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) dma(vrs, gv, vbuf(b), i);
      float psum = 0.f;
      // Part 1: the P V MFMAs of the previous tile with the first half of
      // this tile's exponentials.
      pv_all(pp, Vp);
#pragma unroll
      for (int k = 0; k < NT; ++k) pc[k] = p_chunk(s[k / 2], k % 2, m_run, psum);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < kMfmaP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < kMfmaP - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, kValu1, 0);
        if (i % kDmaGap1 == 0 && i / kDmaGap1 < C::LPW)
          __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Part 2: the next tile's S MFMAs with the second half.
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) dma(krs, gk, kbuf(b), i);
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) s_mfma(sn, Kn, c);
#pragma unroll
      for (int k = NT; k < 2 * NT; ++k) pc[k] = p_chunk(s[k / 2], k % 2, m_run, psum);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < kMfmaS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < kMfmaS - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, kValu2, 0);
        if (i % kDmaGap2 == 0 && i / kDmaGap2 < C::LPW)
          __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // P > kSumMax somewhere, or a row without a reference yet (m = -inf
      // makes its P inf or NaN).
      if (__ballot(!(psum <= kSumMax))) {
        f32x16 sr[NT];
        rescore(sr, kb);
        rebase(sr, pc, psum);
      }
      l_run += psum;
    }
  };

  f32x16 sa[NT], sb[NT];
  u32x4 pa[2 * NT], pb[2 * NT];
  {
    const i32x4 k0rs = tile_rsrc(Kh, 0), k1rs = tile_rsrc(Kh, 1);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      dma(k0rs, gk, K0, i);
      dma(k1rs, gk, K1, i);
    }
  }
  // The Q rows are used here, so that their loads are in flight with the
  // tile loads: the compiler may otherwise issue them (loads of a read-only
  // argument) after the wait below, at their first use, a second memory
  // round trip before the first tile.
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) asm volatile("" ::"v"(qreg[c]));
  wait_vmem_all();
  __syncthreads();
  // Tiles this wave computes: under the causal mask the last tiles of a
  // block can lie wholly after the wave's rows (P = 0 there), and a wave
  // none of whose rows exists (few queries, as in decoding) computes none.
  int nmine = ntiles;
  if (CAUSAL) nmine = min(ntiles, max(qoff + wq0 + 32 - kfirst + C::BC - 1, 0) / C::BC);
  if (PART && wq0 >= Nq) nmine = 0;
  if (nmine > 0) {
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) s_mfma(sa, kbuf(0), c);
    step(std::true_type{}, 0, sa, sb, pb, pa, 0);
    // Step nmine only has to finish the P V MFMAs of the wave's last tile:
    // the tile it would take next is past the wave's keys (P = 0). It runs
    // as a step of its own without the scores and exponentials, except in
    // the causal d = 64 eight-wave kernel (long rows, where the saving is
    // under 1% and that kernel measured about 1% slower with it), which runs
    // a full step there.
    constexpr bool kLastPvOnly = !(D == 64 && W == 8 && CAUSAL);
    int kt = 1;
    for (;; kt += 2) {
      if (kLastPvOnly && kt >= nmine) break;
      step(std::false_type{}, kt, sb, sa, pa, pb, 1);
      if (kt >= nmine) break;
      if (kLastPvOnly && kt + 1 >= nmine) {
        // P of the last tile to pa, where the final step reads it.
#pragma unroll
        for (int k = 0; k < 2 * NT; ++k) pa[k] = pb[k];
        ++kt;
        break;
      }
      step(std::false_type{}, kt + 1, sa, sb, pb, pa, 0);
      if (kt + 1 >= nmine) break;
    }
    if constexpr (kLastPvOnly) {
      // Step nmine: its share of the step's tile loads, then the P V MFMAs.
      const int b = kt & 1;
      wait_vmem_all();
      __syncthreads();
      const i32x4 krs = tile_rsrc(Kh, kt + 2), vrs = tile_rsrc(Vh, kt);
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        dma(krs, gk, kbuf(b), i);
        dma(vrs, gv, vbuf(b), i);
      }
      pv_all(pa, vbuf(b ^ 1));
    }
  }
  // The block's remaining steps (up to step ntiles): the wave only issues
  // its share of their tile loads and meets their barriers.
  if (ntiles > 0)
    for (int kt = nmine > 0 ? nmine + 1 : 0; kt <= ntiles; ++kt) {
      const int b = kt & 1;
      wait_vmem_all();
      __syncthreads();
      const i32x4 krs = tile_rsrc(Kh, kt + 2), vrs = tile_rsrc(Vh, kt);
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        dma(krs, gk, kbuf(b), i);
        dma(vrs, gv, vbuf(b), i);
      }
    }
  // Epilogue: O = O~ / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = pair_sum(l_run);
  const float inv = fast_rcp(l_tot);
  if (PART) {
    if (qrow < Nq) {
      const bool any = l_tot > 0.f;
      const float f = any ? inv : 0.f;
      float *Orow = Op + base + (size_t)qrow * D;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = {o[dt][4 * i] * f, o[dt][4 * i + 1] * f, o[dt][4 * i + 2] * f,
                           o[dt][4 * i + 3] * f};
          *(f32x4 *)(Orow + 32 * dt + 8 * i + 4 * g) = v;
        }
      if (g == 0)
        Lp[(size_t)bh * Nq + qrow] = any ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  // O goes out through LDS in whole rows (store_tile_rows), each wave
  // through its own 32-row half of a K or V tile buffer: wait until no wave
  // reads the tiles and no direct load still writes them.
  wait_vmem_all();
  __syncthreads();
  uint16_t *stg = (w >> 1 == 0 ? K0 : w >> 1 == 1 ? K1 : w >> 1 == 2 ? V0 : V1) + (w & 1) * 32 * D;
  store_tile_rows<T, D>(o, inv, stg, O + base + (size_t)wq0 * D, Nq - wq0, lane);
  if (qrow < Nq && g == 0) LSE[(size_t)bh * Nq + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
}

// Work units: without the causal mask, one query block. With it, block qb
// sweeps 2(qb + 1) key tiles, so blocks are paired as (nqb - 1 - p, p): every
// unit then sweeps the same number of tiles (nqb + 1 pairs), which keeps the
// two workgroup slots of each CU refilled at an even pace (with units of
// unequal length, freed slots were observed to stay empty for several
// microseconds), and halves the number of workgroup start-ups.
template <typename T, int D, int W, bool CAUSAL>
__global__ __launch_bounds__(64 * W, 2) void fwd_b16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int N,
    int nqb, int nunits, int total, float c2) {
  using C = FwdCfg<D, W>;
  // Two buffers per tensor, named separately so that the compiler can tell
  // the direct loads into one from the reads of the other.
  __shared__ __attribute__((aligned(1024))) uint16_t K0[C::TILE], K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[C::TILE], V1[C::TILE];
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nunits;
  const int u = tile - bh * nunits;
  if (!CAUSAL) {
    fwd_block<T, D, W, CAUSAL, false>(Q, K, V, O, LSE, nullptr, nullptr, N, N, 0, bh, u, 0, N, c2,
                                   K0, K1, V0, V1);
    return;
  }
  fwd_block<T, D, W, CAUSAL, false>(Q, K, V, O, LSE, nullptr, nullptr, N, N, 0, bh, nqb - 1 - u, 0,
                                 N, c2, K0, K1, V0, V1);
  if (u != nqb - 1 - u) {
    __syncthreads();  // every wave is done with the LDS tiles
    fwd_block<T, D, W, CAUSAL, false>(Q, K, V, O, LSE, nullptr, nullptr, N, N, 0, bh, u, 0, N, c2,
                                   K0, K1, V0, V1);
  }
}

// Single blocks in longest-first order over groups of S slices (causal
// only; lpt_block), one 128-row block per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(256, 3) void fwd_b16_lpt_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int N,
    int nqb, int BH, int S, int total, float c2) {
  using C = FwdCfg<D, 4>;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[C::TILE], K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[C::TILE], V1[C::TILE];
  int bh, qb;
  lpt_block(xcd_tile(blockIdx.x, total), nqb, BH, S, bh, qb);
  fwd_block<T, D, 4, true, false>(Q, K, V, O, LSE, nullptr, nullptr, N, N, 0, bh, qb, 0, N, c2,
                                  K0, K1, V0, V1);
}

// Split-key forward: the keys of every row are cut into nsplit ranges of
// split_keys keys (a multiple of the tile width), and each (slice, range,
// query block) is one workgroup, which writes its partial result in fp32:
// part s of slice bh at Op + (s * BH + bh) * Nq * D and Lp + (s * BH + bh) * Nq.
// Workgroups of one slice and range are consecutive, so they share their K
// and V tiles in one L2. The partials are combined by lse_merge_kernel.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(FwdCfg<D>::kThreads, FwdCfg<D>::kWavesPerSimd) void fwd_split_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ Op, float *__restrict__ Lp, int Nq,
    int Nk, int qoff, int BH, int nqb, int nsplit, int split_keys, int total, float c2) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[C::TILE], K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[C::TILE], V1[C::TILE];
  const int tile = xcd_tile(blockIdx.x, total);
  const int per_bh = nsplit * nqb;
  const int bh = tile / per_bh;
  const int r = tile - bh * per_bh;
  const int sp = r / nqb, qb = r - sp * nqb;
  const int kfirst = sp * split_keys;
  const int klim = min(Nk, kfirst + split_keys);
  const size_t part = (size_t)sp * BH;
  fwd_block<T, D, 4, CAUSAL, true>(Q, K, V, nullptr, nullptr, Op + part * Nq * D, Lp + part * Nq,
                                Nq, Nk, qoff, bh, qb, kfirst, klim, c2, K0, K1, V0, V1);
}

// The same queries over a single key range (all Nk keys): the block writes O
// and LSE itself, as the plain forward does, so no merge is needed.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(FwdCfg<D>::kThreads, FwdCfg<D>::kWavesPerSimd) void fwd_kv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int Nq,
    int Nk, int qoff, int nqb, int total, float c2) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[C::TILE], K1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[C::TILE], V1[C::TILE];
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nqb, qb = tile - bh * nqb;
  fwd_block<T, D, 4, CAUSAL, false>(Q, K, V, O, LSE, nullptr, nullptr, Nq, Nk, qoff, bh, qb, 0,
                                    Nk, c2, K0, K1, V0, V1);
}

// Merge of partial results over disjoint key sets, per row r and part s:
//   LSE_r = log sum_s exp(LSE_sr),  O_r = sum_s exp(LSE_sr - LSE_r) O_sr,
// the closed form of folding the two-block merge of (m, l, O~) ("Flash
// Attention" notes, section 2, parts 3.1 and 4.1) over the parts, with each
// part entering as (LSE_s, 1, O_s). Parts with LSE = -inf are empty; a row
// with only empty parts gets O = 0 and LSE = -inf. Each thread combines four
// columns of one row (HBM-bound: parts * (4 d + 4) bytes read per row).
template <typename TO>
__global__ __launch_bounds__(256) void lse_merge_kernel(const float *__restrict__ Op,
                                                         const float *__restrict__ Lp, int parts,
                                                         long rows, int d,
                                                         TO *__restrict__ O,
                                                         float *__restrict__ LSE) {
  const int tpr = d / 4;  // threads per row
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = t / tpr;
  if (row >= rows) return;
  const int c = 4 * (int)(t - row * tpr);
  float m = -INFINITY;
  for (int s = 0; s < parts; ++s) m = fmaxf(m, Lp[(size_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < parts; ++s) {
      const float ls = Lp[(size_t)s * rows + row];
      if (ls == -INFINITY) continue;
      const float wgt = fast_exp2((ls - m) * kLog2e);
      const f32x4 v = *(const f32x4 *)(Op + ((size_t)s * rows + row) * d + c);
      l += wgt;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += wgt * v[e];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if constexpr (std::is_same<TO, float>::value) {
    const f32x4 v = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *(f32x4 *)(O + (size_t)row * d + c) = v;
  } else {
    u32x2 v;
    v[0] = pack2<typename TO::Tag>(acc[0] * inv, acc[1] * inv);
    v[1] = pack2<typename TO::Tag>(acc[2] * inv, acc[3] * inv);
    *(u32x2 *)((uint16_t *)O + (size_t)row * d + c) = v;
  }
  if (c == 0) LSE[row] = l > 0.f ? m + logf(l) : -INFINITY;
}

// 16-bit output element of the merge (storage uint16_t, rounding by Tag).
template <typename T>
struct Out16 {
  typedef T Tag;
  uint16_t bits;
};

// fp32 inputs: the same sweep on v_mfma_f32_32x32x2_f32 (A: one value per
// lane, row l % 32, k = l / 32), 32-key tiles, single-buffered LDS.
template <int D>
struct FwdF32Cfg {
  static constexpr int kThreads = 256;
  static constexpr int BR = 128;
  static constexpr int BC = 32;
  static constexpr int KS = D + 2;  // bank-conflict-free A reads of K
  static constexpr int VS = D + 8;  // lane groups 0/1 read rows 4 apart: 4*VS = 32 mod 64 banks
  static constexpr int NDT = D / 32;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int N, int nqb, int total, float c2) {
  using C = FwdF32Cfg<D>;
  __shared__ float Ks[C::BC * C::KS];
  __shared__ float Vs[C::BC * C::VS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nqb;
  int qb = tile - bh * nqb;
  if (CAUSAL) qb = nqb - 1 - qb;
  const int q0 = qb * C::BR;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + l32;
  const size_t base = (size_t)bh * N * D;
  const float *Qh = Q + base, *Kh = K + base, *Vh = V + base;

  float qreg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qreg[c] = (qrow < N) ? Qh[(size_t)qrow * D + 2 * c + g] : 0.f;

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + C::BC - 1) / C::BC;
  f32x16 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // The K and V tile of step kt + 1 is loaded into registers while step kt
  // computes (thread t holds 16-byte pieces e = t, t + 256, ... of it), and
  // moved into the single LDS buffer once every wave is done with tile kt.
  constexpr int NL = C::BC * D / 4 / C::kThreads;
  f32x4 kpre[NL], vpre[NL];
  auto load_tile = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * C::kThreads;
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
      const int key = kb + row;
      kpre[i] = vpre[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        kpre[i] = *(const f32x4 *)(Kh + (size_t)key * D + col);
        vpre[i] = *(const f32x4 *)(Vh + (size_t)key * D + col);
      }
    }
  };
  if (ntiles > 0) load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int kb = kt * C::BC;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * C::kThreads;
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Ks[row * C::KS + col + u] = kpre[i][u];
        Vs[row * C::VS + col + u] = vpre[i][u];
      }
    }
    if (kt + 1 < ntiles) load_tile(kb + C::BC);
    __syncthreads();
    if (CAUSAL && kb > wq0 + 31) continue;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 2; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * C::KS + 2 * c + g], qreg[c], s, 0, 0, 0);
    const bool need_mask = (kb + C::BC > N) || (CAUSAL && kb + C::BC - 1 > wq0);
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * c2;
      if (need_mask) {
        const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= N || (CAUSAL && key > qrow)) x = -INFINITY;
      }
      s[r] = x;
      mloc = fmaxf(mloc, x);
    }
    mloc = pair_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float mb = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mb);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(s[r] - mb);
      psum += s[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    // O~^T += V^T P^T in 2-key chunks: chunk r pairs keys 8(r/4) + r%4 (lane
    // group 0) and that + 4 (group 1), i.e. this lane's own register r.
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * C::VS + 32 * dt + l32], s[r], o[dt],
                                                     0, 0, 0);
      }
  }

  const float l_tot = pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    float *Orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv, o[dt][4 * i + 2] * inv,
                   o[dt][4 * i + 3] * inv};
        *(f32x4 *)(Orow + 32 * dt + 8 * i + 4 * g) = v;
      }
    if (g == 0) LSE[(size_t)bh * N + qrow] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// fp32 forward with the keys of a row group split over the waves of one
// workgroup, for launches too small to fill the GPU with fwd_f32_kernel's
// 128-row blocks (its waves each sweep every key tile of their rows one
// after another, a latency of ntiles x 64 fp32 MFMAs). Here a workgroup
// owns 32 query rows; wave w sweeps key tiles w, w + W, w + 2W, ... of their
// range with the same per-tile arithmetic as fwd_f32_kernel, in an LDS tile
// buffer of its own (no barrier inside the sweep), and ends with its own
// running (m, l, O~). The W partial results of each row are then combined
// with the two-block merge of the online softmax ("Flash Attention" notes,
// section 2, parts 3.1 and 4.1) in closed form over the parts:
//   M = max_w m_w,  L = sum_w l_w 2^(m_w - M),  O = sum_w O~_w 2^(m_w - M) / L,
// (base-2 units, as m is kept), through LDS. A wave without tiles
// contributes m = -inf, l = 0, O~ = 0, i.e. weight 0.
template <int D>
struct FwdF32KsCfg {
  static constexpr int W = (D == 64) ? 8 : 4;  // waves (key shares) per workgroup
  static constexpr int kThreads = 64 * W;
  static constexpr int BC = 32;                // keys per tile
  static constexpr int KS = D + 2;             // row strides as in FwdF32Cfg
  static constexpr int VS = D + 8;
  static constexpr int NDT = D / 32;
  static constexpr int TILE = BC * (KS + VS);  // floats of one wave's K and V tile
  static constexpr int NL = BC * D / 4 / 64;   // 16-byte pieces per lane and tensor
  static constexpr int TPR = kThreads / 32;    // merge: threads per row
  static constexpr int CPT = D / TPR;          // merge: columns per thread
  static_assert(W * 32 * D + 2 * W * 32 <= W * TILE, "the merge reuses the tile buffers");
  static_assert(CPT % 4 == 0, "whole 16-byte column groups per merge thread");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(FwdF32KsCfg<D>::kThreads, 1) void fwd_f32_ks_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int N, int nrg, int total, float c2) {
  using C = FwdF32KsCfg<D>;
  __shared__ __attribute__((aligned(16))) float lds[C::W * C::TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nrg;
  const int q0 = (tile - bh * nrg) * 32;
  const int qrow = q0 + l32;
  const size_t base = (size_t)bh * N * D;
  const float *Qh = Q + base, *Kh = K + base, *Vh = V + base;

  // Rows past N read row N - 1 (finite values, never stored); keys past N
  // read key N - 1 and are masked (their P is 0): no branch around a load.
  float qreg[D / 2];
  const float *qsrc = Qh + (size_t)min(qrow, N - 1) * D + g;
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qreg[c] = qsrc[2 * c];

  const int kend = CAUSAL ? min(N, q0 + 32) : N;
  const int ntiles = (kend + C::BC - 1) / C::BC;
  float *Ks = lds + w * C::TILE, *Vs = Ks + C::BC * C::KS;
  f32x16 o[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = w; kt < ntiles; kt += C::W) {
    const int kb = kt * C::BC;
    // This wave's tile: lane l holds 16-byte pieces e = l, l + 64, ... (the
    // wave's own reads of the previous tile precede these writes).
#pragma unroll
    for (int i = 0; i < C::NL; ++i) {
      const int e = lane + 64 * i;
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
      const int key = min(kb + row, N - 1);
      const f32x4 kx = *(const f32x4 *)(Kh + (size_t)key * D + col);
      const f32x4 vx = *(const f32x4 *)(Vh + (size_t)key * D + col);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Ks[row * C::KS + col + u] = kx[u];
        Vs[row * C::VS + col + u] = vx[u];
      }
    }
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 2; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * C::KS + 2 * c + g], qreg[c], s, 0, 0, 0);
    const bool need_mask = (kb + C::BC > N) || (CAUSAL && kb + C::BC - 1 > q0);
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * c2;
      if (need_mask) {
        const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= N || (CAUSAL && key > qrow)) x = -INFINITY;
      }
      s[r] = x;
      mloc = fmaxf(mloc, x);
    }
    mloc = pair_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float mb = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mb);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(s[r] - mb);
      psum += s[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * C::VS + 32 * dt + l32], s[r], o[dt],
                                                     0, 0, 0);
      }
  }

  // The parts, into the tile area once every wave is done with its tiles:
  // O~_w at Op + (w*32 + row)*D (row-major), m_w and l_w of row r at
  // Mp[w*32 + r], Lp[w*32 + r].
  const float l_tot = pair_sum(l_run);
  __syncthreads();
  float *Op = lds, *Mp = lds + C::W * 32 * D, *Lp = Mp + C::W * 32;
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(f32x4 *)(Op + (w * 32 + l32) * D + 32 * dt + 8 * i + 4 * g) =
          f32x4{o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]};
  if (g == 0) {
    Mp[w * 32 + l32] = m_run;
    Lp[w * 32 + l32] = l_tot;
  }
  __syncthreads();
  // Merge: thread t takes row t / TPR, columns CPT * (t % TPR) .. + CPT - 1.
  const int row = tid / C::TPR, c0 = C::CPT * (tid % C::TPR);
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < C::W; ++v) M = fmaxf(M, Mp[v * 32 + row]);
  const float Mb = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  f32x4 acc[C::CPT / 4];
#pragma unroll
  for (int j = 0; j < C::CPT / 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < C::W; ++v) {
    const float f = fast_exp2(Mp[v * 32 + row] - Mb);
    L = __builtin_fmaf(Lp[v * 32 + row], f, L);
#pragma unroll
    for (int j = 0; j < C::CPT / 4; ++j) {
      const f32x4 x = *(const f32x4 *)(Op + (v * 32 + row) * D + c0 + 4 * j);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[j][u] = __builtin_fmaf(x[u], f, acc[j][u]);
    }
  }
  if (q0 + row < N) {
    const float inv = 1.0f / L;
    float *Orow = O + base + (size_t)(q0 + row) * D + c0;
#pragma unroll
    for (int j = 0; j < C::CPT / 4; ++j)
      *(f32x4 *)(Orow + 4 * j) =
          f32x4{acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv};
    if (c0 == 0) LSE[(size_t)bh * N + q0 + row] = (M + log2f(L)) * kLn2;
  }
}

template <typename T, int D, int W, bool CAUSAL>
static hipError_t fwd_b16_w(int BH, int N, const void *Q, const void *K, const void *V, float c2,
                            void *O, float *LSE, hipStream_t st) {
  using C = FwdCfg<D, W>;
  const int nqb = (N + C::BR - 1) / C::BR;
  const int nunits = CAUSAL ? (nqb + 1) / 2 : nqb;
  const int total = nunits * BH;
  hipLaunchKernelGGL((fwd_b16_kernel<T, D, W, CAUSAL>), dim3(total), dim3(C::kThreads), 0, st,
                     (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                     (uint16_t *)O, LSE, N, nqb, nunits, total, c2);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
static hipError_t fwd_b16(int BH, int N, const void *Q, const void *K, const void *V, float c2,
                          void *O, float *LSE, hipStream_t st) {
  if constexpr (D == 64 && CAUSAL) {
    if (use_single_block_order(D, N, CAUSAL)) {
      using C = FwdCfg<D, 4>;
      const int nqb = (N + C::BR - 1) / C::BR;
      hipLaunchKernelGGL((fwd_b16_lpt_kernel<T, D>), dim3(nqb * BH), dim3(C::kThreads), 0, st,
                         (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                         (uint16_t *)O, LSE, N, nqb, BH, single_block_group(BH, N, D), nqb * BH,
                         c2);
      return hipGetLastError();
    }
  }
  return use_256_row_blocks(BH, N, CAUSAL)
             ? fwd_b16_w<T, D, 8, CAUSAL>(BH, N, Q, K, V, c2, O, LSE, st)
             : fwd_b16_w<T, D, 4, CAUSAL>(BH, N, Q, K, V, c2, O, LSE, st);
}

template <int D, bool CAUSAL>
static hipError_t fwd_f32(int BH, int N, const void *Q, const void *K, const void *V, float c2,
                          void *O, float *LSE, hipStream_t st) {
  using C = FwdF32Cfg<D>;
  const int nqb = (N + C::BR - 1) / C::BR;
  if ((long)nqb * BH < kF32SplitBelow) {
    using S = FwdF32KsCfg<D>;
    const int nrg = (N + 31) / 32;
    const int total = nrg * BH;
    hipLaunchKernelGGL((fwd_f32_ks_kernel<D, CAUSAL>), dim3(total), dim3(S::kThreads), 0, st,
                       (const float *)Q, (const float *)K, (const float *)V, (float *)O, LSE, N,
                       nrg, total, c2);
    return hipGetLastError();
  }
  const int total = nqb * BH;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(total), dim3(C::kThreads), 0, st,
                     (const float *)Q, (const float *)K, (const float *)V, (float *)O, LSE, N,
                     nqb, total, c2);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t fwd_b16_c(int causal, int BH, int N, const void *Q, const void *K,
                            const void *V, float c2, void *O, float *LSE, hipStream_t st) {
  return causal ? fwd_b16<T, D, true>(BH, N, Q, K, V, c2, O, LSE, st)
                : fwd_b16<T, D, false>(BH, N, Q, K, V, c2, O, LSE, st);
}

// ---------------------------------------------------------------------------
// Decoding: one new query per slice (Nq = 1) over one range of cached keys.
// ---------------------------------------------------------------------------
// Per key the work is a d-element dot product and a d-element update of O,
// so reading K and V from HBM bounds the kernel, and a matrix product would
// fill one of its 32 rows. It runs on the vector units instead. A key row is
// D/8 lanes x 16 bytes; per batch each wave issues 8 loads of K and 8 of V
// per lane (KPB keys, all in flight before the first is used), forms the
// scores with a butterfly sum inside each lane group, and applies the online
// softmax ("Flash Attention" notes, section 2, part 4.2) once per batch:
// running max m (base 2), normaliser l and unnormalised O, each lane group
// holding its own keys' share of O for the 8 dims of its lanes. At the end
// the lane groups, then the four waves, are combined with the same rescaling,
// and the range's O / l and LSE go to the split workspace for
// lse_merge_kernel -- or, with a single range (Od set), straight to O
// (rounded to T) and LSE. P stays in fp32: no matrix product consumes it.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, float *__restrict__ Op, float *__restrict__ Lp,
    uint16_t *__restrict__ Od, float *__restrict__ Ld, int Nk, int BH, int nparts,
    int split_keys, float c2) {
  constexpr int LPR = D / 8;     // lanes per key row, 8 elements each
  constexpr int KPI = 64 / LPR;  // keys per load instruction: one per lane group
  constexpr int NL = 8;          // loads per tensor per batch
  constexpr int KPB = KPI * NL;  // keys per wave per batch
  __shared__ float red[4][D + 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x / nparts, sp = blockIdx.x - bh * nparts;
  const int kf = sp * split_keys, kl = min(Nk, kf + split_keys);
  const int sub = lane % LPR, grp = lane / LPR;
  const uint16_t *Kh = K + (size_t)bh * Nk * D + 8 * sub;
  const uint16_t *Vh = V + (size_t)bh * Nk * D + 8 * sub;
  // This lane's 8 query elements, times scale * log2(e): scores in base 2.
  float qf[8];
  {
    const u32x4 qv = ld128(Q + (size_t)bh * D + 8 * sub);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      qf[2 * h] = to_f32<T>((uint16_t)(qv[h] & 0xffffu)) * c2;
      qf[2 * h + 1] = to_f32<T>((uint16_t)(qv[h] >> 16)) * c2;
    }
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  // Batches are double-buffered: the loads of a wave's next batch are issued
  // before the current one is used, so they stay in flight meanwhile.
  auto load_batch = [&](int k0, u32x4 (&kr)[NL], u32x4 (&vr)[NL]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // Keys past the range read its last row again (masked below).
      const size_t key = (size_t)min(k0 + i * KPI + grp, kl - 1);
      kr[i] = ld128(Kh + key * D);
      vr[i] = ld128(Vh + key * D);
    }
  };
  auto batch = [&](int k0, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL])
      __attribute__((always_inline)) {
    float s[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float a = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        a = __builtin_fmaf(to_f32<T>((uint16_t)(kr[i][h] & 0xffffu)), qf[2 * h], a);
        a = __builtin_fmaf(to_f32<T>((uint16_t)(kr[i][h] >> 16)), qf[2 * h + 1], a);
      }
      s[i] = a;
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1)
#pragma unroll
      for (int i = 0; i < NL; ++i) s[i] += __shfl_xor(s[i], off, LPR);
    // Key k0 (lane group 0, load 0) is in the range, so the batch max is finite.
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (k0 + i * KPI + grp >= kl) s[i] = -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);  // 0 on the first batch (m = -inf)
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      s[i] = fast_exp2(s[i] - mn);
      ps += s[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        o[2 * h] = __builtin_fmaf(s[i], to_f32<T>((uint16_t)(vr[i][h] & 0xffffu)), o[2 * h]);
        o[2 * h + 1] = __builtin_fmaf(s[i], to_f32<T>((uint16_t)(vr[i][h] >> 16)), o[2 * h + 1]);
      }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) ps += __shfl_xor(ps, off);
    l = l * alpha + ps;
    m = mn;
  };
  constexpr int kStride = 4 * KPB;  // the four waves take consecutive batches
  int k0 = kf + w * KPB;
  if (k0 < kl) {
    u32x4 ka[NL], va[NL], kb[NL], vb[NL];
    load_batch(k0, ka, va);
    for (;;) {
      if (k0 + kStride < kl) load_batch(k0 + kStride, kb, vb);
      batch(k0, ka, va);
      k0 += kStride;
      if (k0 >= kl) break;
      if (k0 + kStride < kl) load_batch(k0 + kStride, ka, va);
      batch(k0, kb, vb);
      k0 += kStride;
      if (k0 >= kl) break;
    }
  }
  // The lane groups share m and l; sum their O, then combine the waves.
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off);
  if (grp == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w][8 * sub + e] = o[e];
  if (lane == 0) {
    red[w][D] = m;
    red[w][D + 1] = l;
  }
  __syncthreads();
  if (tid < D) {
    // A wave without keys has m = -inf, l = 0, O = 0 and weighs nothing;
    // wave 0 always has keys (the range is not empty).
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, red[v][D]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float f = fast_exp2(red[v][D] - M);
      L += red[v][D + 1] * f;
      acc += red[v][tid] * f;
    }
    const float lse = (M + fast_log2(L)) * kLn2;
    if (Od != nullptr) {
      Od[(size_t)bh * D + tid] = (uint16_t)(pack2<T>(acc / L, 0.f) & 0xffffu);
      if (tid == 0) Ld[bh] = lse;
    } else {
      const size_t row = (size_t)sp * BH + bh;
      Op[row * D + tid] = acc / L;
      if (tid == 0) Lp[row] = lse;
    }
  }
}

struct SplitArgs {
  int BH, Nq, Nk, qoff;
  const void *Q, *K, *V;
  float c2;
  float *Op, *Lp;
  int nsplit, split_keys;
  void *O;     // single range: final O and LSE instead of the parts
  float *LSE;
};

template <typename T, int D, bool CAUSAL>
static hipError_t fwd_split(const SplitArgs &a, hipStream_t st) {
  using C = FwdCfg<D>;
  const int nqb = (a.Nq + C::BR - 1) / C::BR;
  if (a.O != nullptr) {  // a single range, final output
    const int total = a.BH * nqb;
    hipLaunchKernelGGL((fwd_kv_kernel<T, D, CAUSAL>), dim3(total), dim3(C::kThreads), 0, st,
                       (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V,
                       (uint16_t *)a.O, a.LSE, a.Nq, a.Nk, a.qoff, nqb, total, a.c2);
    return hipGetLastError();
  }
  const int total = a.BH * a.nsplit * nqb;
  hipLaunchKernelGGL((fwd_split_kernel<T, D, CAUSAL>), dim3(total), dim3(C::kThreads), 0, st,
                     (const uint16_t *)a.Q, (const uint16_t *)a.K, (const uint16_t *)a.V, a.Op,
                     a.Lp, a.Nq, a.Nk, a.qoff, a.BH, nqb, a.nsplit, a.split_keys, total, a.c2);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t fwd_split_c(int causal, const SplitArgs &a, hipStream_t st) {
  return causal ? fwd_split<T, D, true>(a, st) : fwd_split<T, D, false>(a, st);
}

hipError_t launch_fwd_split(int dtype, int B, int H, int Nq, int Nk, int d, const void *Q,
                            const void *K, const void *V, float scale, int causal, int nsplit,
                            float *Op, float *Lp, void *O, float *LSE, hipStream_t st) {
  const SplitArgs a{B * H, Nq, Nk, causal ? Nk - Nq : 0, Q, K, V, scale * kLog2e, Op, Lp,
                    split_parts(Nk, nsplit), split_key_count(Nk, nsplit), O, LSE};
  if (Nq == 1) {
    // One query per slice (it sees every key, masked or not): the vector
    // kernel, one workgroup per slice and key range.
    const dim3 grid((unsigned)(a.BH * a.nsplit));
    const auto q = (const uint16_t *)Q, k = (const uint16_t *)K, v = (const uint16_t *)V;
    const auto od = (uint16_t *)O;
    if (dtype == kBF16 && d == 128)
      hipLaunchKernelGGL((decode_kernel<BF16, 128>), grid, dim3(256), 0, st, q, k, v, Op, Lp, od,
                         LSE, Nk, a.BH, a.nsplit, a.split_keys, a.c2);
    else if (dtype == kBF16)
      hipLaunchKernelGGL((decode_kernel<BF16, 64>), grid, dim3(256), 0, st, q, k, v, Op, Lp, od,
                         LSE, Nk, a.BH, a.nsplit, a.split_keys, a.c2);
    else if (d == 128)
      hipLaunchKernelGGL((decode_kernel<F16, 128>), grid, dim3(256), 0, st, q, k, v, Op, Lp, od,
                         LSE, Nk, a.BH, a.nsplit, a.split_keys, a.c2);
    else
      hipLaunchKernelGGL((decode_kernel<F16, 64>), grid, dim3(256), 0, st, q, k, v, Op, Lp, od,
                         LSE, Nk, a.BH, a.nsplit, a.split_keys, a.c2);
    return hipGetLastError();
  }
  if (dtype == kBF16)
    return d == 64 ? fwd_split_c<BF16, 64>(causal, a, st) : fwd_split_c<BF16, 128>(causal, a, st);
  return d == 64 ? fwd_split_c<F16, 64>(causal, a, st) : fwd_split_c<F16, 128>(causal, a, st);
}

hipError_t launch_lse_merge(int dtype, int parts, long rows, int d, const float *Op,
                            const float *Lp, void *O, float *LSE, hipStream_t st) {
  const long threads = rows * (d / 4);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (dtype == kF32)
    hipLaunchKernelGGL((lse_merge_kernel<float>), dim3(blocks), dim3(256), 0, st, Op, Lp, parts,
                       rows, d, (float *)O, LSE);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((lse_merge_kernel<Out16<BF16>>), dim3(blocks), dim3(256), 0, st, Op, Lp,
                       parts, rows, d, (Out16<BF16> *)O, LSE);
  else
    hipLaunchKernelGGL((lse_merge_kernel<Out16<F16>>), dim3(blocks), dim3(256), 0, st, Op, Lp,
                       parts, rows, d, (Out16<F16> *)O, LSE);
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                      const void *V, float scale, int causal, void *O, float *LSE,
                      hipStream_t st) {
  const int BH = B * H;
  const float c2 = scale * kLog2e;
  if (dtype == kF32) {
    if (d == 64)
      return causal ? fwd_f32<64, true>(BH, N, Q, K, V, c2, O, LSE, st)
                    : fwd_f32<64, false>(BH, N, Q, K, V, c2, O, LSE, st);
    return causal ? fwd_f32<128, true>(BH, N, Q, K, V, c2, O, LSE, st)
                  : fwd_f32<128, false>(BH, N, Q, K, V, c2, O, LSE, st);
  }
  if (dtype == kBF16)
    return d == 64 ? fwd_b16_c<BF16, 64>(causal, BH, N, Q, K, V, c2, O, LSE, st)
                   : fwd_b16_c<BF16, 128>(causal, BH, N, Q, K, V, c2, O, LSE, st);
  return d == 64 ? fwd_b16_c<F16, 64>(causal, BH, N, Q, K, V, c2, O, LSE, st)
                 : fwd_b16_c<F16, 128>(causal, BH, N, Q, K, V, c2, O, LSE, st);
}

}  // namespace fa
