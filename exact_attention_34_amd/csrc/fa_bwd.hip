// fa_bwd.hip -- backward pass of exact attention on gfx950.
//
// Follows the blocked backward of the "Flash Attention" notes (section 3,
// part 4.2, and the backward-derivation page, part 6). Per pair of tiles it
// recomputes
//   S = Q K^T,  P = exp(scale*S - LSE)            (section 3, part 4.1)
// and forms
//   dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   dK += dS^T Q,  dQ += dS K                      (derivation, parts 3-4)
// with D = rowsum(dO o O) precomputed by a separate pass (derivation, part 5).
// The scale enters dQ and dK once, at the end (the Ascend recompute article
// writes 1/sqrt(d_k) into both).
//
// The pages' loop nest (keys outer, queries inner, dQ read-modified-written
// per pair of tiles) makes every key block add into every dQ row. Here the
// work is split into two sweeps that each own their outputs, so no partial
// sum leaves a workgroup and no atomics are needed:
//   * bwd_dkdv_kernel: a workgroup owns a block of KB keys and walks the
//     query tiles, keeping dK and dV in registers (the pages' outer loop);
//   * bwd_dq_kernel: a workgroup owns a block of query rows and walks the
//     key tiles, keeping dQ in registers (recomputing S, P, dP, dS).
// The second sweep repeats the S and dP products (7 instead of 5 matrix
// products per tile pair); on this chip that is cheaper than summing dQ
// through fp32 atomics in L2, and every gradient is deterministic.

#include <limits.h>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik (fp32).
// ---------------------------------------------------------------------------
// The 8 products of one 16-byte chunk of O and dO, summed in element order
// with explicit fmas. The preprocess kernel and the dQ sweep (which forms D
// itself inside fa_bwd) both use it and reduce the chunks of a row in the
// same tree, so both give the same D bit for bit.
template <typename T>
__device__ __forceinline__ float dot8(const u32x4 &a, const u32x4 &b) {
  float acc = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc = __builtin_fmaf(to_f32<T>((uint16_t)(a[h] & 0xffffu)),
                         to_f32<T>((uint16_t)(b[h] & 0xffffu)), acc);
    acc = __builtin_fmaf(to_f32<T>((uint16_t)(a[h] >> 16)), to_f32<T>((uint16_t)(b[h] >> 16)),
                         acc);
  }
  return acc;
}

// Row sums over chunks: thread sub of a row holds chunk sub; the xor tree
// adds chunk t and t ^ off for off = TPR/2, ..., 1.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ O,
                                                      const uint16_t *__restrict__ dO,
                                                      float *__restrict__ Dvec, long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / TPR;
  const int sub = tid % TPR;
  float acc = 0.f;
  if (row < rows) acc = dot8<T>(ld128(O + row * D + 8 * sub), ld128(dO + row * D + 8 * sub));
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) Dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// Shared tile layout.
// ---------------------------------------------------------------------------
// Q, dO, K and V tiles in LDS are unpadded, row-major at 16-byte-chunk
// granularity, with the chunk index XOR-ed by swz(row). They are read two
// ways: row-wise (16 consecutive rows, one chunk each, per quarter-wave) and
// with transposing loads (4 consecutive rows x 4 chunks per half-wave). swz
// maps both access groups onto 16 distinct four-bank groups of the 64-bank
// LDS. It depends on row % 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-lane LDS byte offsets into such a tile. The swizzle only touches
// address bits that the row and column terms of one access leave zero, so
// every access is a per-lane base XOR-ed with a compile-time constant:
//  * row-wise read of row 32a + l%32, 16-byte chunk 2c + l/32:
//      (row_base() ^ 32 c) + 64 D a;
//  * transposing read (ds_read_b64_tr_b16) of rows rb + (l%16)/4, columns
//    32 dt + 16 ((l/16)%2) + 4 (l%4) .. +3, for rb = 16 b + r0 with
//    r0 < 16:  (tr_base(r0) ^ 64 dt) + 32 D b.
// The XOR terms stay below the row terms, so the row terms add: they go into
// the tile pointer and from there into the instructions' immediate offsets,
// and only one register per XOR constant is needed.
template <int D>
__device__ __forceinline__ int row_base(int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  const int f = swz<D>(l32);
  return l32 * 2 * D + 16 * (g ^ (f & 1)) + 32 * (f >> 1);
}
template <int D>
__device__ __forceinline__ int tr_base(int r0, int lane) {
  const int row = r0 + (lane & 15) / 4;
  const int cq = 2 * ((lane >> 4) & 1) + (lane & 3) / 2;  // chunk within a 64-byte column group
  const int f = swz<D>(row);
  return row * 2 * D + 16 * (cq ^ (f & 3)) + 8 * (lane & 1) + 64 * (f >> 2);
}

__device__ __forceinline__ const uint16_t *at(const uint16_t *tile, int byte_off) {
  return (const uint16_t *)((const char *)tile + byte_off);
}

// LDS chunk p (0 .. rows * CPR - 1) of a swizzled tile holds global chunk
// (p % CPR) ^ swz(row) of row p / CPR: byte offset of that chunk in a dense
// row-major source with D elements per row.
template <int D>
__device__ __forceinline__ int src_of_chunk(int p) {
  constexpr int CPR = D / 8;
  const int r = p / CPR, sw = p % CPR;
  return 2 * (r * D + 8 * (sw ^ swz<D>(r)));
}

// ---------------------------------------------------------------------------
// dK, dV: key blocks outer, query tiles inner (d = 128; d = 64 runs
// bwd_dkdv64_kernel below, on the same stream of steps).
// ---------------------------------------------------------------------------
template <int D>
struct DkdvCfg {
  static constexpr int kThreads = 512;               // 8 waves, two per SIMD
  static constexpr int KB = 128;                     // keys per workgroup, 32 per wave pair
  static constexpr int BR = 64;                      // query rows per step
  static constexpr int NT = BR / 32;                 // 32-row query subtiles per step
  static constexpr int NCH = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int QTILE = BR * D;               // 16-bit elements per Q or dO tile
  static constexpr int LPW = BR * CPR / (kThreads / 2);  // loads per role-0 wave per tile and tensor
  static constexpr int PX = NT * 16 * 64;            // floats of P handed over per key slice
  static constexpr int NBUF = 3;                     // query-tile buffers
  static_assert(LPW >= 1, "every wave loads part of each tile");
};

// The eight waves form four pairs, one per SIMD; a pair owns a slice of 32
// keys (column l % 32 of every S/P/dP/dS product) and splits the work by
// role:
//   * role 0 keeps the slice's K rows in VGPRs (B operand of S = Q K^T),
//     forms P = exp(scale S - LSE), hands P to its partner through LDS and
//     accumulates dV^T += dO^T P;
//   * role 1 keeps the V rows in VGPRs (B operand of dP = dO V^T), forms
//     dS = P o (dP - D) and accumulates dK^T += Q^T dS.
// Each product reads one operand from LDS; P and dS come out of the MFMA in
// the B-operand layout of the dV / dK products (one key per lane, 16 query
// rows per lane), and dO^T / Q^T come from transposing reads of the
// row-major tiles. Role 1 forms dK one tile late, so that in the first half
// of a step (before P is handed over) it runs the MFMAs of the previous
// tile's dK and of this tile's dP while role 0 computes exponentials, and in
// the second half its dS arithmetic runs beside role 0's dV MFMAs. Query
// tiles (Q, dO, LSE, D) are triple-buffered (the tile being read, the
// previous one for role 1's dK, and the next one being loaded).
//
// The stream of one workgroup. The kernel is persistent: workgroup w takes
// the work units w, w + G, w + 2G, ... (G workgroups, one per compute unit
// at most), each mapped XCD-aware as in the other sweeps. A unit is one key
// block, or under the causal mask the pair of blocks p and nkb - 1 - p,
// whose sweeps add up to the same length for every p. The workgroup walks
// all (block, query tile) steps of its units as one stream, so the loads of
// a block's first tiles and of its K and V rows are issued during the last
// steps of the block before, and the dK and dV of a finished block are
// stored while the next block computes. Position in the stream (wave-
// uniform): virtual workgroup id v (the stream ends at v >= total), slice
// bh, unit u, which block of the unit (half), key block kb, query tile it.
struct DkdvPos {
  int v, bh, u, half, kb, it;
};

// The stream itself: blocks of KB keys, query tiles of BR rows, nq tiles per
// slice, nkb blocks per slice, nunits units per slice, `total` units in all,
// G workgroups. Under the causal mask a block starts at its first query tile
// that holds a row at or after its first key.
template <bool CAUSAL, int KB, int BR>
struct DkdvStream {
  int nq, nkb, nunits, total, G;
  __device__ __forceinline__ int block_start(int kb) const { return CAUSAL ? kb * KB / BR : 0; }
  // The first step of virtual workgroup v's unit.
  __device__ __forceinline__ DkdvPos unit_pos(int v) const {
    DkdvPos p;
    p.v = v;
    const int t = v < total ? xcd_tile(v, total) : 0;
    p.bh = t / nunits;
    p.u = t - p.bh * nunits;
    p.half = 0;
    p.kb = p.u;
    p.it = block_start(p.u);
    return p;
  }
  // The step after p: the next query tile, the unit's second block, or the
  // workgroup's next unit (v + G; the stream ends at v >= total).
  __device__ __forceinline__ DkdvPos advance(DkdvPos p) const {
    if (p.it + 1 < nq) {
      ++p.it;
      return p;
    }
    if (CAUSAL && p.half == 0 && p.u != nkb - 1 - p.u) {
      p.half = 1;
      p.kb = nkb - 1 - p.u;
      p.it = block_start(p.kb);
      return p;
    }
    return unit_pos(p.v + G);
  }
  __device__ __forceinline__ bool last_of_block(const DkdvPos &p) const { return p.it == nq - 1; }
};

// Steps of the workgroup's stream. Query-tile buffers rotate over the steps:
// buffer b (step % 3) holds Q at qo + 2*b*QTILE, dO right after it, and LSE,
// D rows at lv + 2*b*BR; px is the P hand-over area, PX floats per key slice.
//
// The direct loads of a step's tile are issued during the step before, by
// role 0 normally, but by role 1 for the first two steps after a block ends;
// each wave waits only for loads it issued itself (then the barrier). At the
// end of a block role 0 stores dV and role 1 stores dK one step later, and
// neither waits for those stores before its next wait on loads of its own:
// a wave never issues tile loads in the two steps after it stored, so its
// waits never include store latency. (Vector-memory loads and stores of a
// wave share one counter and may complete out of order with each other, so
// a wait for loads alone is only possible when no store is outstanding.)
//
// L2: LSE holds LSE * log2(e) per row (as the dQ sweep stores it inside
// fa_bwd), so that P = 2^(S*scale*log2e - L) takes one fma per score;
// otherwise LSE is the natural-log LSE and is scaled per score.
template <typename T, int D, bool CAUSAL, bool L2>
__global__ __launch_bounds__(512, 2) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int N, int nkb, int nunits, int total, float c2, float scale) {
  using C = DkdvCfg<D>;
  constexpr int NT = C::NT;
  __shared__ __attribute__((aligned(1024))) uint16_t qo[2 * C::NBUF * C::QTILE];
  __shared__ __attribute__((aligned(256))) float lv[2 * C::NBUF * C::BR];
  __shared__ __attribute__((aligned(1024))) float px[4 * C::PX];
  // Output staging: 32 keys x 64 columns (16-bit) per key slice, used by the
  // slice's two waves at different times (separated by barriers).
  __shared__ __attribute__((aligned(1024))) uint16_t stage[4 * 32 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int l32 = lane & 31, g = lane >> 5;
  const int ks = w & 3;     // key slice: keys 32 ks .. +31 of a block
  const int role = w >> 2;  // 0: S, P, dV; 1: dP, dS, dK
  const DkdvStream<CAUSAL, C::KB, C::BR> stream{(N + C::BR - 1) / C::BR, nkb, nunits, total,
                                                 (int)gridDim.x};

  // This slice's K (role 0) or V (role 1) rows as the B operand: lane l
  // holds key kb*KB + 32 ks + l%32, 8 consecutive columns 16c + 8g .. per
  // chunk c. Keys past N read row N - 1 (masked).
  u32x4 kv[C::NCH];
  auto load_rows = [&](const DkdvPos &p) __attribute__((always_inline)) {
    const int key = min(p.kb * C::KB + 32 * ks + l32, N - 1);
    const uint16_t *src = (role == 0 ? K : V) + (size_t)p.bh * N * D + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) kv[c] = ld128(src + 16 * c + 8 * g);
  };

  // Direct buffer -> LDS loads of the query tile of step p into buffer b,
  // by the four waves of one role (r = w & 3): instruction i of wave r fills
  // LDS chunks (r*LPW + i)*64 + lane with the global chunk the swizzle puts
  // there; waves r < 2*BR/64 also load 64 LSE or D values each. The buffer
  // resources cover the rows that exist; rows past N read as zero (and are
  // masked).
  const int r4 = w & 3;
  int gq[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) gq[i] = src_of_chunk<D>((r4 * C::LPW + i) * 64 + lane);
  constexpr int kVecParts = C::BR / 64;
  auto issue = [&](int b, const DkdvPos &p) __attribute__((always_inline)) {
    uint16_t *Qb = qo + 2 * b * C::QTILE, *Ob = Qb + C::QTILE;
    const int q0 = p.it * C::BR;
    const int rows = min(N - q0, C::BR);
    const size_t base = (size_t)p.bh * N * D + (size_t)q0 * D;
    const i32x4 qrs = make_rsrc(Q + base, (uint32_t)rows * D * 2);
    const i32x4 ors = make_rsrc(dO + base, (uint32_t)rows * D * 2);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      dma_lds16(qrs, gq[i], 0, Qb + (r4 * C::LPW + i) * 512);
      dma_lds16(ors, gq[i], 0, Ob + (r4 * C::LPW + i) * 512);
    }
    if (r4 < 2 * kVecParts) {
      const int vec = r4 / kVecParts, part = r4 % kVecParts;
      const i32x4 vrs =
          make_rsrc((vec == 0 ? LSE : Dvec) + (size_t)p.bh * N + q0, (uint32_t)rows * 4);
      dma_lds4(vrs, 4 * (64 * part + lane), 0, lv + 2 * b * C::BR + vec * C::BR + 64 * part);
    }
  };

  // Row-wise reads (row 32t + l%32 of a tile, chunk 2c + g) and transposing
  // reads (rows 16cc + 4g + (0..3) and 16cc + 8 + 4g + (0..3) of subtile t:
  // the P / dS register layout), as per-lane bases XOR-ed with constants.
  const int rb = row_base<D>(lane);
  const int tb1 = tr_base<D>(4 * g, lane), tb2 = tr_base<D>(8 + 4 * g, lane);
  float *pxs = px + ks * C::PX;  // this slice's P hand-over area

  // Issue pattern of a phase of kM MFMAs, each fed by kR LDS reads issued
  // kA MFMAs ahead (LDS latency under load exceeds a few MFMAs).
  auto pipeline = [&](auto km_tag, auto kr_tag, auto ka_tag) __attribute__((always_inline)) {
    constexpr int kM = decltype(km_tag)::value, kR = decltype(kr_tag)::value;
    constexpr int kA = decltype(ka_tag)::value;
    __builtin_amdgcn_sched_group_barrier(0x100, kA * kR, 0);
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kM - kA) __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using KR = std::integral_constant<int, NT * C::NCH>;      // MFMAs of a row-wise product
  using KT = std::integral_constant<int, 2 * NT * C::NDT>;  // MFMAs of a transposed product
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I6 = std::integral_constant<int, 6>;

  // One product with an operand read row-wise from a tile: acc[t] = init[t]
  // + Σ_c tile rows (32t + l%32, chunk c) x kv[c].
  auto rows_x_kv = [&](f32x16 (&acc)[NT], const f32x16 (&init)[NT], const uint16_t *tile)
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
        acc[t] = mfma32<T>(ld128(at(tile + 32 * D * t, rb ^ (32 * c))), kv[c],
                           c == 0 ? init[t] : acc[t]);
  };
  // acc^T += tile^T x B for B in the P / dS layout (pb[t][cc]).
  auto tr_x_b = [&](f32x16 (&acc)[C::NDT], const uint16_t *tile, const u32x4 (&pb)[NT][2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
          const uint16_t *src = tile + (32 * t + 16 * cc) * D;
          acc[dt] = mfma32<T>(
              cat(ld_tr16(at(src, tb1 ^ (64 * dt))), ld_tr16(at(src, tb2 ^ (64 * dt)))),
              pb[t][cc], acc[dt]);
        }
  };
  auto pack_b = [&](const f32x16 (&x)[NT], u32x4 (&pb)[NT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 4; ++h)
          pb[t][cc][h] = pack2<T>(x[t][8 * cc + 2 * h], x[t][8 * cc + 2 * h + 1]);
  };
  // rows of subtile t, register r: 8(r/4) + 4g + r%4; LSE and D of rows
  // 8i + 4g + (0..3) are consecutive in LDS, read as one 16-byte word.
  auto vec4 = [&](const float *Lb, int off, int t, int i) __attribute__((always_inline)) {
    return *(const f32x4 *)(Lb + off + 32 * t + 8 * i + 4 * g);
  };
  // dK = scale * dK (role 1) or dV (role 0) of block (bh, kb), in halves of
  // 64 columns transposed through this slice's staging area, so that every
  // store instruction writes whole 128-byte lines (8 lanes of 16 bytes per
  // row; storing straight from the accumulator layout -- 8 bytes of each of
  // 32 rows per instruction -- cost 8 partial-line writes per line). In the
  // staging area row r (key) holds 8 chunks of 16 bytes, chunk c at
  // position c ^ (r % 8), which spreads both access patterns over the banks.
  f32x16 acc[C::NDT];  // dV^T (role 0) or dK^T (role 1): column = key, rows = d
  char *stg = (char *)(stage + ks * 32 * 64);
  auto store_acc = [&](int bh, int kb) __attribute__((always_inline)) {
    const float f = role == 0 ? 1.f : scale;
    uint16_t *out = (role == 0 ? dV : dK) + (size_t)bh * N * D;
    const int key0 = kb * C::KB + 32 * ks;
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
      // This lane's key (row l%32), columns 32 dtl + 8 i + 4 g .. +3 of the half.
#pragma unroll
      for (int dtl = 0; dtl < 2; ++dtl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dt = 2 * h + dtl, c = 4 * dtl + i;
          u32x2 a;
          a[0] = pack2<T>(acc[dt][4 * i] * f, acc[dt][4 * i + 1] * f);
          a[1] = pack2<T>(acc[dt][4 * i + 2] * f, acc[dt][4 * i + 3] * f);
          *(u32x2 *)(stg + l32 * 128 + 16 * (c ^ (l32 & 7)) + 8 * g) = a;
        }
      // Rows 8k + lane/8, chunk lane % 8: 16 bytes per lane, 8 rows per
      // instruction.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        const u32x4 v = *(const u32x4 *)(stg + r * 128 + 16 * (c ^ (r & 7)));
        if (key0 + r < N) st128_nt(out + (size_t)(key0 + r) * D + 64 * h + 8 * c, v);
      }
    }
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = kZero16;
  };
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = kZero16;

  // Who loads the tile of step n: role 1 if the step before n or the one
  // before that ended a block (lastA: step n-1, lastB: step n-2), else role 0.
  auto loader = [](bool lastA, bool lastB) { return (lastA || lastB) ? 1 : 0; };

  DkdvPos cur = stream.unit_pos(blockIdx.x);
  load_rows(cur);
  if (role == 0) issue(0, cur);
  bool mine = role == 0;     // this wave issued the loads of the current step
  bool prev_last = false;    // the step before the current one ended a block
  int b = 0;

  if (role == 0) {
    for (;;) {
      if (mine) wait_vmem_all();
      barrier_lds();  // every wave's loads landed; every wave is done with step - 2's buffer
      const uint16_t *Qs = qo + 2 * b * C::QTILE, *Os = Qs + C::QTILE;
      const float *Lb = lv + 2 * b * C::BR;
      const int q0 = cur.it * C::BR;
      const int wk0 = cur.kb * C::KB + 32 * ks;  // first key of this wave
      const int mykey = wk0 + l32;               // key of this lane's S/P column
      const bool need_mask = (q0 + C::BR > N) || (wk0 + 32 > N) || (CAUSAL && wk0 + 31 > q0);
      const bool last = stream.last_of_block(cur);
      const DkdvPos nxt = stream.advance(cur);
      const bool more = nxt.v < total;
      const int bn = b == 2 ? 0 : b + 1;
      f32x4 lse[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) lse[t][i] = vec4(Lb, 0, t, i);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s[NT];
      const f32x16 zero[NT] = {};
      rows_x_kv(s, zero, Qs);  // S = Q K^T
      pipeline(KR{}, I1{}, I6{});
      // The next block's K rows, into the registers the products above read.
      if (last && more) load_rows(nxt);
      if (need_mask) {
        // Query q0 + 4g + off sees this lane's key iff lo <= off <= hi.
        const int hi = (mykey < N ? N - 1 : -1) - q0 - 4 * g;
        const int lo = CAUSAL ? mykey - q0 - 4 * g : INT_MIN;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * t + 8 * (r >> 2) + (r & 3);
            if (off > hi || (CAUSAL && off < lo)) s[t][r] = -INFINITY;
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      // P = 2^(S*scale*log2e - LSE*log2e), handed over in fp32 (lane-major
      // 16-byte groups), and rounded to T for dV.
      u32x4 pp[NT][2];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 p;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            p[j] = fast_exp2(
                __builtin_fmaf(s[t][4 * i + j], c2, L2 ? -lse[t][i][j] : -lse[t][i][j] * kLog2e));
          *(f32x4 *)(pxs + ((t * 4 + i) * 64 + lane) * 4) = p;
#pragma unroll
          for (int j = 0; j < 4; ++j) s[t][4 * i + j] = p[j];
        }
      pack_b(s, pp);
      const bool next_mine = more && loader(last, prev_last) == 0;
      if (next_mine) issue(bn, nxt);
      barrier_lds();  // P visible to the partner
      tr_x_b(acc, Os, pp);  // dV^T += dO^T P
      pipeline(KT{}, I2{}, I4{});
      if (last) {
        // The K rows of the next block (loaded above) are waited for here,
        // before the stores, so that no later wait includes the stores.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        store_acc(cur.bh, cur.kb);
      }
      if (!more) break;
      mine = next_mine;
      prev_last = last;
      cur = nxt;
      b = bn;
    }
    barrier_lds();  // role 1 stages its last dK after this wave's last dV
  } else {
    u32x4 pd[NT][2];  // dS of the previous step, rounded to T
    const uint16_t *Qprev = qo;
    int acc_bh = -1, acc_kb = -1;  // block whose dK the accumulator holds
    int prev_bh = 0, prev_kb = 0;  // block of the previous step
    bool have_prev = false;
    for (;;) {
      if (mine) wait_vmem_all();
      barrier_lds();
      const uint16_t *Qs = qo + 2 * b * C::QTILE, *Os = Qs + C::QTILE;
      const float *Lb = lv + 2 * b * C::BR;
      const bool last = stream.last_of_block(cur);
      const DkdvPos nxt = stream.advance(cur);
      const bool more = nxt.v < total;
      const int bn = b == 2 ? 0 : b + 1;
      const bool next_mine = more && loader(last, prev_last) == 1;
      // The buffer of step - 2 is free (every wave passed the barrier
      // above after its last use): load the next step's tile into it.
      if (next_mine) issue(bn, nxt);
      if (have_prev) {
        if (acc_bh != prev_bh || acc_kb != prev_kb) {
          if (acc_bh >= 0) store_acc(acc_bh, acc_kb);
          acc_bh = prev_bh;
          acc_kb = prev_kb;
        }
        tr_x_b(acc, Qprev, pd);  // dK^T += Q^T dS of the previous step
        pipeline(KT{}, I2{}, I4{});
      }
      f32x16 dp[NT];
      const f32x16 zero[NT] = {};
      rows_x_kv(dp, zero, Os);  // dP = dO V^T
      pipeline(KR{}, I1{}, I6{});
      // The next block's V rows, into the registers the products above read.
      if (last && more) load_rows(nxt);
      barrier_lds();  // the partner's P is in LDS
      // dS = P o (dP - D), rounded to T.
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 p = *(const f32x4 *)(pxs + ((t * 4 + i) * 64 + lane) * 4);
          const f32x4 dd = vec4(Lb, C::BR, t, i);
#pragma unroll
          for (int j = 0; j < 4; ++j) dp[t][4 * i + j] = p[j] * (dp[t][4 * i + j] - dd[j]);
        }
      pack_b(dp, pd);
      __builtin_amdgcn_sched_barrier(0);
      Qprev = Qs;
      prev_bh = cur.bh;
      prev_kb = cur.kb;
      have_prev = true;
      if (!more) break;
      mine = next_mine;
      prev_last = last;
      cur = nxt;
      b = bn;
    }
    barrier_lds();  // the partner's last dV left the staging area
    if (acc_bh != prev_bh || acc_kb != prev_kb) {
      if (acc_bh >= 0) store_acc(acc_bh, acc_kb);
    }
    tr_x_b(acc, Qprev, pd);  // dK^T += Q^T dS of the last step
    pipeline(KT{}, I2{}, I4{});
    store_acc(prev_bh, prev_kb);
  }
}

// ---------------------------------------------------------------------------
// dK, dV at d = 64: symmetric waves.
// ---------------------------------------------------------------------------
// At d = 64 one wave has room for the K and the V rows of its 32 keys and
// for both accumulators, so the eight waves split a step by keys and query
// rows instead of by role: wave w owns key slice w % 4 (32 keys of the
// block) and query half w / 4 (rows 32h .. 32h + 31 of each 64-row tile),
// and forms S, P, dP, dS and the dV and dK products of that 32 x 32 piece
// itself. There is no P hand-over and one barrier per step (the tile
// rotation); the step's vector work (exponentials, dS) is half a role-0
// step's. The two waves of a key slice (one SIMD) sum their dV and dK
// partials once per block through LDS: half 1 writes, half 0 adds them to
// its own in that fixed order and stores. Loads and stores stay apart: only
// half-1 waves issue the tile loads and only half-0 waves store, so no wait
// for tile loads includes a store.
//
// The stream of steps, the work units, the tile format in LDS and the
// operand reads are those of bwd_dkdv_kernel. D - dP is formed on the MFMAs:
// the V rows are kept negated and D is the initial accumulator, so the
// products return E = D - dP, and -dS = P o E costs one multiply per score;
// dK is accumulated negated (rounding commutes with the sign) and scaled by
// -scale at the end. LSE as in bwd_dkdv_kernel (L2: already times log2(e)).
template <typename T, bool CAUSAL, bool L2>
__global__ __launch_bounds__(512, 1) void bwd_dkdv64_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const float *__restrict__ LSE, const float *__restrict__ Dvec, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, int N, int nkb, int nunits, int total, float c2, float scale) {
  constexpr int D = 64, KB = 128, BR = 64;
  constexpr int NCH = D / 16, NDT = D / 32, CPR = D / 8;
  constexpr int QTILE = BR * D;            // 16-bit elements per Q or dO tile
  constexpr int LPW = BR * CPR / 256;      // loads per loading wave per tile and tensor
  constexpr int RED = 2 * NDT * 16 * 64;   // floats of one slice's dV and dK partials
  // Two buffers (the step's tile, the next one being loaded): Q at
  // qo + 2*b*QTILE, dO right after it; LSE and D rows at lv + 2*b*BR.
  __shared__ __attribute__((aligned(1024))) uint16_t qo[2 * 2 * QTILE];
  __shared__ __attribute__((aligned(256))) float lv[2 * 2 * BR];
  __shared__ __attribute__((aligned(1024))) float red[4 * RED];
  __shared__ __attribute__((aligned(1024))) uint16_t stage[4 * 32 * D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int ks = w & 3;  // key slice: keys 32 ks .. +31 of a block
  const int hq = w >> 2;  // query half: rows 32 hq .. +31 of a tile
  const DkdvStream<CAUSAL, KB, BR> stream{(N + BR - 1) / BR, nkb, nunits, total, (int)gridDim.x};

  // This slice's K and V rows as B operands: lane l holds key
  // kb*KB + 32 ks + l%32, 8 consecutive columns 16c + 8g .. per chunk c.
  // Keys past N read row N - 1 (masked). V is negated at the block's first
  // step, where the rows are first read.
  u32x4 kr[NCH], vr[NCH];
  auto load_rows = [&](const DkdvPos &p) __attribute__((always_inline)) {
    const int key = min(p.kb * KB + 32 * ks + l32, N - 1);
    const size_t off = (size_t)p.bh * N * D + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      kr[c] = ld128(K + off + 16 * c + 8 * g);
      vr[c] = ld128(V + off + 16 * c + 8 * g);
    }
  };

  // Direct loads of step p's query tile into buffer b by the four half-1
  // waves (r = w & 3), as in bwd_dkdv_kernel; waves r < 2 also load the 64
  // LSE (r = 0) or D (r = 1) values.
  const int r4 = w & 3;
  int gq[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) gq[i] = src_of_chunk<D>((r4 * LPW + i) * 64 + lane);
  auto issue = [&](int b, const DkdvPos &p) __attribute__((always_inline)) {
    uint16_t *Qb = qo + 2 * b * QTILE, *Ob = Qb + QTILE;
    const int q0 = p.it * BR;
    const int rows = min(N - q0, BR);
    const size_t base = (size_t)p.bh * N * D + (size_t)q0 * D;
    const i32x4 qrs = make_rsrc(Q + base, (uint32_t)rows * D * 2);
    const i32x4 ors = make_rsrc(dO + base, (uint32_t)rows * D * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      dma_lds16(qrs, gq[i], 0, Qb + (r4 * LPW + i) * 512);
      dma_lds16(ors, gq[i], 0, Ob + (r4 * LPW + i) * 512);
    }
    if (r4 < 2) {
      const i32x4 vrs = make_rsrc((r4 == 0 ? LSE : Dvec) + (size_t)p.bh * N + q0, (uint32_t)rows * 4);
      dma_lds4(vrs, 4 * lane, 0, lv + 2 * b * BR + r4 * BR);
    }
  };

  const int rb = row_base<D>(lane);
  const int tb1 = tr_base<D>(4 * g, lane), tb2 = tr_base<D>(8 + 4 * g, lane);
  float *myred = red + ks * RED;
  uint16_t *stg = stage + ks * 32 * D;

  f32x16 accV[NDT], accK[NDT];  // dV^T and -dK^T / scale: column = key, rows = d
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) accV[dt] = accK[dt] = kZero16;

  DkdvPos cur = stream.unit_pos(blockIdx.x);
  load_rows(cur);
  if (hq == 1) issue(0, cur);
  int b = 0;
  for (;;) {
    if (hq == 1) wait_vmem_all();
    barrier_lds();  // the tile landed; every wave is done with the other buffer
    const uint16_t *Qs = qo + 2 * b * QTILE + 32 * D * hq;  // this wave's 32 rows
    const uint16_t *Os = Qs + QTILE;
    const float *Lb = lv + 2 * b * BR + 32 * hq;
    const int r0 = cur.it * BR + 32 * hq;  // first query row of this wave
    const int wk0 = cur.kb * KB + 32 * ks;
    const int mykey = wk0 + l32;
    const bool need_mask = (r0 + 32 > N) || (wk0 + 32 > N) || (CAUSAL && wk0 + 31 > r0);
    const bool last = stream.last_of_block(cur);
    const DkdvPos nxt = stream.advance(cur);
    const bool more = nxt.v < total;
    if (hq == 1 && more) issue(b ^ 1, nxt);
    if (cur.it == stream.block_start(cur.kb)) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int h = 0; h < 4; ++h) vr[c][h] ^= 0x80008000u;
    }
    // LSE and D of rows r0 + 8i + 4g + j (register 4i + j), 16-byte reads.
    f32x4 lse[4];
    f32x16 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lse[i] = *(const f32x4 *)(Lb + 8 * i + 4 * g);
      const f32x4 dd = *(const f32x4 *)(Lb + BR + 8 * i + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) e[4 * i + j] = dd[j];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      s = mfma32<T>(ld128(at(Qs, rb ^ (32 * c))), kr[c], c == 0 ? kZero16 : s);
    __builtin_amdgcn_sched_barrier(0);
    if (need_mask) {
      // Query r0 + 4g + off sees this lane's key iff lo <= off <= hi.
      const int hi = (mykey < N ? N - 1 : -1) - r0 - 4 * g;
      const int lo = CAUSAL ? mykey - r0 - 4 * g : INT_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + (r & 3);
        if (off > hi || (CAUSAL && off < lo)) s[r] = -INFINITY;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // E MFMAs beside the exponentials.
#pragma unroll
    for (int c = 0; c < NCH; ++c) e = mfma32<T>(ld128(at(Os, rb ^ (32 * c))), vr[c], e);
    float p[16];
    u32x4 pp[2], pd[2];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      p[r] = fast_exp2(
          __builtin_fmaf(s[r], c2, L2 ? -lse[r / 4][r % 4] : -lse[r / 4][r % 4] * kLog2e));
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h = 0; h < 4; ++h) pp[cc][h] = pack2<T>(p[8 * cc + 2 * h], p[8 * cc + 2 * h + 1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NCH - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 12, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The next block's rows, into the registers the products above read.
    if (last && more) load_rows(nxt);
    // dV^T += dO^T P beside -dS = P o E; then -dK^T += Q^T (-dS).
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t *so = Os + 16 * cc * D;
        accV[dt] = mfma32<T>(
            cat(ld_tr16(at(so, tb1 ^ (64 * dt))), ld_tr16(at(so, tb2 ^ (64 * dt)))), pp[cc],
            accV[dt]);
      }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int r = 8 * cc + 2 * h;
        pd[cc][h] = pack2<T>(p[r] * e[r], p[r + 1] * e[r + 1]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * NDT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 2 * NDT - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t *sq = Qs + 16 * cc * D;
        accK[dt] = mfma32<T>(
            cat(ld_tr16(at(sq, tb1 ^ (64 * dt))), ld_tr16(at(sq, tb2 ^ (64 * dt)))), pd[cc],
            accK[dt]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * NDT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 2 * NDT - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (last) {
      // The block's dV and dK: half 1 hands its partials to half 0.
      if (hq == 1) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 v, k;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[j] = accV[dt][4 * i + j];
              k[j] = accK[dt][4 * i + j];
            }
            *(f32x4 *)(myred + ((0 * NDT + dt) * 4 + i) * 256 + 4 * lane) = v;
            *(f32x4 *)(myred + ((1 * NDT + dt) * 4 + i) * 256 + 4 * lane) = k;
          }
      }
      barrier_lds();
      if (hq == 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 v = *(const f32x4 *)(myred + ((0 * NDT + dt) * 4 + i) * 256 + 4 * lane);
            const f32x4 k = *(const f32x4 *)(myred + ((1 * NDT + dt) * 4 + i) * 256 + 4 * lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              accV[dt][4 * i + j] += v[j];
              accK[dt][4 * i + j] += k[j];
            }
          }
        // The next block's rows are waited for here, before the stores, so
        // that no later wait includes the stores.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        const size_t o = (size_t)cur.bh * N * D + (size_t)wk0 * D;
        store_tile_rows<T, D>(accV, 1.f, stg, dV + o, N - wk0, lane);
        store_tile_rows<T, D>(accK, -scale, stg, dK + o, N - wk0, lane);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) accV[dt] = accK[dt] = kZero16;
    }
    if (!more) break;
    cur = nxt;
    b ^= 1;
  }
}

// ---------------------------------------------------------------------------
// dQ: query blocks outer, key tiles inner.
// ---------------------------------------------------------------------------
template <int D, int W = 4>
struct DqCfg {
  static constexpr int kThreads = 64 * W;          // W waves
  static constexpr int BR = 32 * W;                // query rows per workgroup, 32 per wave
  static constexpr int BC = 64;                    // keys per tile, two 32-key halves
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BC * D;              // 16-bit elements per K or V tile
  static constexpr int NCH = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int LPW = BC * CPR / kThreads;  // direct loads per wave per tile and tensor
};

// Per wave: 32 query rows, whose Q and dO rows stay in VGPRs as the B
// operands of S^T = K Q^T and dP^T = V dO^T; lane l owns query row l % 32, so
// its LSE and D are two per-lane scalars. dS^T then has one query per lane
// and 16 keys per lane in the B-operand layout of dQ^T += K^T dS^T, whose K^T
// operand comes from the same K tile with transposing reads. K and V tiles
// are double-buffered in LDS and filled by direct buffer -> LDS loads.
//
// One block of query rows (block qb of slice bh). LDS buffer b: K tile at
// kv + 2*b*TILE, V tile right after it.
template <typename T, int D, int W, bool CAUSAL, bool DFUSE>
__device__ __forceinline__ void dq_block(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ O, const float *__restrict__ LSE, float *__restrict__ Dvec,
    float *__restrict__ L2out, uint16_t *__restrict__ dQ, int N, int bh, int qb, float c2,
    float scale, uint16_t *kv) {
  using C = DqCfg<D, W>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = qb * C::BR;
  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + l32;
  const size_t base = (size_t)bh * N * D;
  const uint16_t *Qh = Q + base, *Kh = K + base, *Vh = V + base, *dOh = dO + base;

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + C::BC - 1) / C::BC;

  const i32x4 krs = make_rsrc(Kh, (uint32_t)N * D * 2);
  const i32x4 vrs = make_rsrc(Vh, (uint32_t)N * D * 2);
  int gk[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) gk[i] = src_of_chunk<D>((w * C::LPW + i) * 64 + lane);
  auto issue = [&](int b, int kt) __attribute__((always_inline)) {
    uint16_t *Kb = kv + 2 * b * C::TILE, *Vb = Kb + C::TILE;
    const int kb = kt * C::BC;
    // Byte offset of the tile in the slice: below N*D*2 < 2^32 (the slice
    // limit of the interface), so it fits the unsigned 32-bit soffset.
    const uint32_t soff = (uint32_t)kb * D * 2;
    if (kb + C::BC <= N) {
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        dma_lds16(krs, gk[i], soff, Kb + (w * C::LPW + i) * 512);
        dma_lds16(vrs, gk[i], soff, Vb + (w * C::LPW + i) * 512);
      }
    } else {
      // Tail tile: rows past N re-read row N - 1 (their keys are masked).
#pragma unroll
      for (int i = 0; i < C::LPW; ++i) {
        const int r = ((w * C::LPW + i) * 64 + lane) / C::CPR;
        const int shift = 2 * D * (min(kb + r, N - 1) - kb - r);  // <= 0
        dma_lds16(krs, gk[i] + shift, soff, Kb + (w * C::LPW + i) * 512);
        dma_lds16(vrs, gk[i] + shift, soff, Vb + (w * C::LPW + i) * 512);
      }
    }
  };
  // Rows past N are read from row N - 1 (always valid memory) and never
  // stored.
  const int qld = min(qrow, N - 1);
  u32x4 qreg[C::NCH], oreg[C::NCH], orow[DFUSE ? C::NCH : 1];
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    qreg[c] = ld128(Qh + (size_t)qld * D + 16 * c + 8 * g);
    oreg[c] = ld128(dOh + (size_t)qld * D + 16 * c + 8 * g);
  }
  const float lse2 = LSE[(size_t)bh * N + qld] * kLog2e;
  float dd;
  if constexpr (DFUSE) {
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) orow[c] = ld128(O + base + (size_t)qld * D + 16 * c + 8 * g);
  } else {
    dd = Dvec[(size_t)bh * N + qld];
  }
  // The first K/V tile goes out with the row loads (one memory round trip
  // before the first tile), and everything is waited for here with a wait
  // the compiler sees: its own waits for the rows would otherwise sit inside
  // the loop, where they would also wait for each next tile.
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // D of this row (DFUSE), formed from O and the dO chunks in registers --
  // lane g holds chunks 2c + g, so the chunk tree of the preprocess kernel
  // runs within the lane down to the last level, which joins the lane pair
  // -- and stored for the dK/dV sweep at the end of the block.
  if constexpr (DFUSE) {
    float part[C::NCH];
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) part[c] = dot8<T>(orow[c], oreg[c]);
#pragma unroll
    for (int h = C::NCH / 2; h > 0; h >>= 1)
#pragma unroll
      for (int c = 0; c < h; ++c) part[c] = part[c] + part[c + h];
    dd = pair_sum(part[0]);
  }

  const int rb = row_base<D>(lane);
  // K^T operand of dQ^T: keys 16cc + 4g + (0..3) and 16cc + 8 + 4g + (0..3)
  // of a 32-key half (the dS^T register layout), column 32dt + l%32.
  const int tb1 = tr_base<D>(4 * g, lane), tb2 = tr_base<D>(8 + 4 * g, lane);

  f32x16 dq[C::NDT];
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  // d = 64 (half the MFMAs of d = 128 per score, the same vector work): dP^T
  // starts from -D in every register, so that the MFMAs return dP - D and
  // dS costs one multiply per score.
  constexpr bool kDinit = D == 64;
  f32x16 dneg;
#pragma unroll
  for (int r = 0; r < 16; ++r) dneg[r] = -dd;

  // One 32-key half t of a tile. need_mask: the half holds keys past N or
  // (causal) past this wave's first query row. The mask is a VALU-only
  // branch, so every MFMA accumulation runs on one code path.
  auto half = [&](const uint16_t *Ks, const uint16_t *Vs, int kb, int t, bool need_mask)
      __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K Q^T and dP^T = V dO^T (minus D when kDinit); lane: query
    // qrow, keys 8(r/4)+4g+r%4.
    f32x16 s = kZero16, dp = kZero16;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      s = mfma32<T>(ld128(at(Ks + 32 * D * t, rb ^ (32 * c))), qreg[c], c == 0 ? kZero16 : s);
      dp = mfma32<T>(ld128(at(Vs + 32 * D * t, rb ^ (32 * c))), oreg[c],
                     c == 0 ? (kDinit ? dneg : kZero16) : dp);
    }
    // One operand read per MFMA, issued four MFMAs ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::NCH - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (need_mask) {
      // Key kb + 32t + 4g + off is visible iff off <= lim.
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kb - 32 * t - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
    }
    __builtin_amdgcn_sched_barrier(0);
    // P = 2^(S*scale*log2e - LSE*log2e), dS = P o (dP - D), rounded to T in
    // pairs: 16-key chunk cc = registers 8cc .. 8cc+7.
    u32x4 pk[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int r = 8 * cc + 2 * h;
        const float p0 = fast_exp2(__builtin_fmaf(s[r], c2, -lse2));
        const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], c2, -lse2));
        if constexpr (kDinit)
          pk[cc][h] = pack2<T>(p0 * dp[r], p1 * dp[r + 1]);
        else
          pk[cc][h] = pack2<T>(p0 * (dp[r] - dd), p1 * (dp[r + 1] - dd));
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        const uint16_t *src = Ks + (32 * t + 16 * cc) * D;
        dq[dt] = mfma32<T>(
            cat(ld_tr16(at(src, tb1 ^ (64 * dt))), ld_tr16(at(src, tb2 ^ (64 * dt)))), pk[cc],
            dq[dt]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::NDT - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // One tile. DIAG: the tile may hold keys after some of this wave's rows
  // (causal); a wave whose rows all precede a half skips it.
  auto tile_step = [&](const uint16_t *Ks, const uint16_t *Vs, int kt, auto diag_tag)
      __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const int kb = kt * C::BC;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int hb = kb + 32 * t;
      if (DIAG && hb > wq0 + 31) continue;
      half(Ks, Vs, kb, t, (hb + 32 > N) || (DIAG && hb + 31 > wq0));
    }
  };

  // Double-buffered sweep over the key tiles: wait for this wave's loads,
  // barrier (every wave's loads landed; every wave is done with the other
  // buffer), issue the next tile's loads into the other buffer, compute.
  // Under the causal mask the tiles from q0 on (the diagonal) run in a loop
  // of their own, so that the skipping branches (whose joins would copy the
  // dQ accumulators) stay out of the main loop.
  const int nmain = CAUSAL ? min(ntiles, q0 / C::BC) : ntiles;
  auto sweep_tile = [&](int kt, auto diag_tag) __attribute__((always_inline)) {
    const int b = kt & 1;
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < ntiles) issue(b ^ 1, kt + 1);
    const uint16_t *Ks = kv + 2 * b * C::TILE;
    tile_step(Ks, Ks + C::TILE, kt, diag_tag);
  };
  for (int kt = 0; kt < nmain; ++kt) sweep_tile(kt, std::false_type{});
  if constexpr (CAUSAL)
    for (int kt = nmain; kt < ntiles; ++kt) sweep_tile(kt, std::true_type{});

  // dQ = scale * dQ^T, transposed back and stored in whole rows through
  // this wave's 32-row share of the K/V buffers (store_tile_rows), once no
  // wave reads the tiles and no direct load still writes them.
  wait_vmem_all();
  __syncthreads();
  store_tile_rows<T, D>(dq, scale, kv + w * 32 * D, dQ + base + (size_t)wq0 * D, N - wq0, lane);
  if (DFUSE && qrow < N && g == 0) {
    Dvec[(size_t)bh * N + qrow] = dd;
    if (L2out != nullptr) L2out[(size_t)bh * N + qrow] = lse2;
  }
}

// Work units as in the forward: one query block, or under the causal mask
// the pair (nqb - 1 - p, p) of blocks with equal total length.
template <typename T, int D, int W, bool CAUSAL, bool DFUSE>
__global__ __launch_bounds__(64 * W, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ O, const float *__restrict__ LSE, float *__restrict__ Dvec,
    float *__restrict__ L2out, uint16_t *__restrict__ dQ, int N, int nqb, int nunits, int total,
    float c2, float scale) {
  using C = DqCfg<D, W>;
  __shared__ __attribute__((aligned(1024))) uint16_t kv[4 * C::TILE];
  const int tile = xcd_tile(blockIdx.x, total);
  const int bh = tile / nunits;
  const int u = tile - bh * nunits;
  if (!CAUSAL) {
    dq_block<T, D, W, CAUSAL, DFUSE>(Q, K, V, dO, O, LSE, Dvec, L2out, dQ, N, bh, u, c2, scale,
                                     kv);
    return;
  }
  dq_block<T, D, W, CAUSAL, DFUSE>(Q, K, V, dO, O, LSE, Dvec, L2out, dQ, N, bh, nqb - 1 - u, c2,
                                   scale, kv);
  if (u != nqb - 1 - u) {
    __syncthreads();  // every wave is done with the LDS tiles
    dq_block<T, D, W, CAUSAL, DFUSE>(Q, K, V, dO, O, LSE, Dvec, L2out, dQ, N, bh, u, c2, scale,
                                     kv);
  }
}

// Single blocks in longest-first order, as the forward's fwd_b16_lpt_kernel
// (causal only).
template <typename T, int D, bool DFUSE>
__global__ __launch_bounds__(256, 3) void bwd_dq_lpt_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
    const uint16_t *__restrict__ O, const float *__restrict__ LSE, float *__restrict__ Dvec,
    float *__restrict__ L2out, uint16_t *__restrict__ dQ, int N, int nqb, int BH, int S,
    int total, float c2, float scale) {
  using C = DqCfg<D, 4>;
  __shared__ __attribute__((aligned(1024))) uint16_t kv[4 * C::TILE];
  int bh, qb;
  lpt_block(xcd_tile(blockIdx.x, total), nqb, BH, S, bh, qb);
  dq_block<T, D, 4, true, DFUSE>(Q, K, V, dO, O, LSE, Dvec, L2out, dQ, N, bh, qb, c2, scale, kv);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t pre(long rows, const void *O, const void *dO, float *Dv, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t *)O, (const uint16_t *)dO, Dv, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(int dtype, int B, int H, int N, int d, const void *O,
                                 const void *dO, float *Dvec, hipStream_t st) {
  const long rows = (long)B * H * N;
  if (dtype == kBF16)
    return d == 64 ? pre<BF16, 64>(rows, O, dO, Dvec, st) : pre<BF16, 128>(rows, O, dO, Dvec, st);
  return d == 64 ? pre<F16, 64>(rows, O, dO, Dvec, st) : pre<F16, 128>(rows, O, dO, Dvec, st);
}

// Arguments shared by the two gradient sweeps.
struct BwdArgs {
  int BH, N;
  const uint16_t *Q, *K, *V, *dO;
  const float *LSE, *Dvec;
  float c2, scale;
  const uint16_t *O;  // dQ sweep only: form D from O and dO (else null)
  float *Dout;        // where that sweep writes D (else Dvec, read-only)
  float *L2out;       // dQ sweep with O: also writes LSE * log2(e) there (or null)
  const float *L2;    // dK/dV sweep: LSE * log2(e) to read instead of LSE (or null)
};

template <typename T, int D, bool CAUSAL>
static hipError_t dkdv(const BwdArgs &a, void *dK, void *dV, hipStream_t st) {
  using C = DkdvCfg<D>;
  const int nkb = (a.N + C::KB - 1) / C::KB;
  const int nunits = CAUSAL ? (nkb + 1) / 2 : nkb;
  const int total = nunits * a.BH;
  // Persistent: one workgroup per compute unit (its LDS allows no second),
  // or one per unit if there are fewer units.
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int grid = min(total, cus);
  const float *L = a.L2 != nullptr ? a.L2 : a.LSE;
  if constexpr (D == 64) {
    if (a.L2 != nullptr)
      hipLaunchKernelGGL((bwd_dkdv64_kernel<T, CAUSAL, true>), dim3(grid), dim3(512), 0, st, a.Q,
                         a.K, a.V, a.dO, L, a.Dvec, (uint16_t *)dK, (uint16_t *)dV, a.N, nkb,
                         nunits, total, a.c2, a.scale);
    else
      hipLaunchKernelGGL((bwd_dkdv64_kernel<T, CAUSAL, false>), dim3(grid), dim3(512), 0, st, a.Q,
                         a.K, a.V, a.dO, L, a.Dvec, (uint16_t *)dK, (uint16_t *)dV, a.N, nkb,
                         nunits, total, a.c2, a.scale);
  } else {
    if (a.L2 != nullptr)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, true>), dim3(grid), dim3(C::kThreads), 0,
                         st, a.Q, a.K, a.V, a.dO, L, a.Dvec, (uint16_t *)dK, (uint16_t *)dV, a.N,
                         nkb, nunits, total, a.c2, a.scale);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, false>), dim3(grid), dim3(C::kThreads), 0,
                         st, a.Q, a.K, a.V, a.dO, L, a.Dvec, (uint16_t *)dK, (uint16_t *)dV, a.N,
                         nkb, nunits, total, a.c2, a.scale);
  }
  return hipGetLastError();
}

template <typename T, int D, int W, bool CAUSAL, bool DFUSE>
static hipError_t dq_w(const BwdArgs &a, void *dQ, hipStream_t st) {
  using C = DqCfg<D, W>;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const int nunits = CAUSAL ? (nqb + 1) / 2 : nqb;
  const int total = nunits * a.BH;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, W, CAUSAL, DFUSE>), dim3(total), dim3(C::kThreads), 0,
                     st, a.Q, a.K, a.V, a.dO, a.O, a.LSE, a.Dout, a.L2out, (uint16_t *)dQ, a.N, nqb,
                     nunits, total, a.c2, a.scale);
  return hipGetLastError();
}

// Dvec read (a.Dvec) or, with a.O set, formed from O and dO and written to
// a.Dout.
template <typename T, int D, bool DFUSE>
static hipError_t dq_lpt(const BwdArgs &a, void *dQ, hipStream_t st) {
  using C = DqCfg<D, 4>;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  hipLaunchKernelGGL((bwd_dq_lpt_kernel<T, D, DFUSE>), dim3(nqb * a.BH), dim3(C::kThreads), 0,
                     st, a.Q, a.K, a.V, a.dO, a.O, a.LSE, a.Dout, a.L2out, (uint16_t *)dQ, a.N,
                     nqb, a.BH, single_block_group(a.BH, a.N, D), nqb * a.BH, a.c2, a.scale);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
static hipError_t dq(const BwdArgs &a, void *dQ, hipStream_t st) {
  if constexpr (D == 64 && CAUSAL) {
    if (use_single_block_order(D, a.N, CAUSAL))
      return a.O != nullptr ? dq_lpt<T, D, true>(a, dQ, st) : dq_lpt<T, D, false>(a, dQ, st);
  }
  const bool w8 = use_256_row_blocks(a.BH, a.N, CAUSAL);
  if (a.O != nullptr)
    return w8 ? dq_w<T, D, 8, CAUSAL, true>(a, dQ, st) : dq_w<T, D, 4, CAUSAL, true>(a, dQ, st);
  return w8 ? dq_w<T, D, 8, CAUSAL, false>(a, dQ, st) : dq_w<T, D, 4, CAUSAL, false>(a, dQ, st);
}

static BwdArgs bwd_args(int B, int H, int N, const void *Q, const void *K, const void *V,
                        const void *dO, const float *LSE, const float *Dvec, float scale) {
  return BwdArgs{B * H, N, (const uint16_t *)Q, (const uint16_t *)K, (const uint16_t *)V,
                 (const uint16_t *)dO, LSE, Dvec, scale * kLog2e, scale, nullptr,
                 const_cast<float *>(Dvec), nullptr, nullptr};
}

// Instantiates F<T, D, CAUSAL>(args...) for the run-time dtype, d, causal.
#define FA_DISPATCH(F, dtype, d, causal, ...)                                            \
  ((dtype) == kBF16                                                                     \
       ? ((d) == 64 ? ((causal) ? F<BF16, 64, true>(__VA_ARGS__)                        \
                                : F<BF16, 64, false>(__VA_ARGS__))                      \
                    : ((causal) ? F<BF16, 128, true>(__VA_ARGS__)                       \
                                : F<BF16, 128, false>(__VA_ARGS__)))                    \
       : ((d) == 64 ? ((causal) ? F<F16, 64, true>(__VA_ARGS__)                         \
                                : F<F16, 64, false>(__VA_ARGS__))                       \
                    : ((causal) ? F<F16, 128, true>(__VA_ARGS__)                        \
                                : F<F16, 128, false>(__VA_ARGS__))))

hipError_t launch_bwd_dkdv(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                           const void *V, const void *dO, const float *LSE, const float *LSE2,
                           const float *Dvec, float scale, int causal, void *dK, void *dV,
                           hipStream_t st) {
  BwdArgs a = bwd_args(B, H, N, Q, K, V, dO, LSE, Dvec, scale);
  a.L2 = LSE2;
  return FA_DISPATCH(dkdv, dtype, d, causal, a, dK, dV, st);
}

hipError_t launch_bwd_dq(int dtype, int B, int H, int N, int d, const void *Q, const void *K,
                         const void *V, const void *dO, const float *LSE, const float *Dvec,
                         float scale, int causal, void *dQ, hipStream_t st) {
  const BwdArgs a = bwd_args(B, H, N, Q, K, V, dO, LSE, Dvec, scale);
  return FA_DISPATCH(dq, dtype, d, causal, a, dQ, st);
}

hipError_t launch_bwd_dq_fused(int dtype, int B, int H, int N, int d, const void *Q,
                               const void *K, const void *V, const void *O, const void *dO,
                               const float *LSE, float *Dvec, float *LSE2, float scale,
                               int causal, void *dQ, hipStream_t st) {
  BwdArgs a = bwd_args(B, H, N, Q, K, V, dO, LSE, Dvec, scale);
  a.O = (const uint16_t *)O;
  a.Dout = Dvec;
  a.L2out = LSE2;
  return FA_DISPATCH(dq, dtype, d, causal, a, dQ, st);
}

#undef FA_DISPATCH

}  // namespace fa
