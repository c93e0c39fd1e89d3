// fa_device.h -- gfx950 device helpers for the attention kernels: vector
// types, the MFMA instructions used, 16-bit packing with round-to-nearest-even,
// the lane exchange across wave halves, and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Zero accumulator: starting an MFMA chain from it lets the compiler use the
// instruction's inline-zero accumulator operand.
constexpr f32x16 kZero16 = {};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element tags.
struct BF16 {};
struct F16 {};

// D(32x32 fp32) += A(32x16) * B(16x32), both 16-bit. Operand layout per lane l
// (wave64): A row l%32, k = 8*(l/32)..+7; B column l%32, same k.
// C/D: column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
template <typename T>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c);

template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 -> one dword of two 16-bit values (lo = a), round to nearest even.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo(x) + hi(x) for a dword of two 16-bit values (v_dot2c_f32_{bf16,f16}
// against (1, 1)): sums the rounded values in fp32.
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t x, float acc);
template <>
__device__ __forceinline__ float add_pair<BF16>(uint32_t x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}
template <>
__device__ __forceinline__ float add_pair<F16>(uint32_t x, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
}

// 16-bit -> fp32.
template <typename T>
__device__ __forceinline__ float to_f32(uint16_t h);
template <>
__device__ __forceinline__ float to_f32<BF16>(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
template <>
__device__ __forceinline__ float to_f32<F16>(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Low / high 16-bit halves of two dwords, paired into one dword.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Reductions over the lane pair (l, l ^ 32). v_permlane32_swap exchanges
// lanes 32-63 of its first operand with lanes 0-31 of its second; with both
// operands equal to x, one result holds x[l] and the other x[l ^ 32] in every
// lane, so combining the two results reduces the pair.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Swap bits 2 and 3 of a key index inside its 16-block. Row r of a 32x32
// MFMA result lives in lane group (r >> 2) & 1 at register slot
// 4 * (r >> 3) + (r & 3); storing the contraction operand of the next product
// in this order lets each lane read its 8 k-slots as one 16-byte word.
__device__ __forceinline__ int swap23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Map the linear workgroup id so that consecutive tile ids -- the tiles
// of one (batch, head) slice, which share K and V -- run on the same XCD.
__device__ __forceinline__ int xcd_tile(int wg, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = wg % kXcd, k = wg / kXcd;
  return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Single query blocks in longest-first order over groups of S slices: tile
// id t (consecutive ids on one XCD, as from xcd_tile) belongs to group
// t / (S * nqb), whose blocks go longest first across its slices: block
// nqb - 1 - r of every slice of the group before block nqb - 2 - r. Small
// groups keep few slices' K and V in an XCD's L2 at a time; the short blocks
// at the end of each group fill the slots that the long ones leave.
__device__ __forceinline__ void lpt_block(int t, int nqb, int BH, int S, int &bh, int &qb) {
  const int s0 = t / (S * nqb) * S;
  const int ns = min(S, BH - s0);
  const int k = t - s0 * nqb;
  const int r = k / ns;
  bh = s0 + (k - r * ns);
  qb = nqb - 1 - r;
}

__device__ __forceinline__ u32x4 ld128(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void st128(void *p, const u32x4 &v) { *(u32x4 *)p = v; }
// Non-temporal 16-byte store (global_store ... nt), for outputs that no
// kernel of the pass reads again: they then take less room in L2 from the
// tiles that other workgroups are still reading.
__device__ __forceinline__ void st128_nt(void *p, const u32x4 &v) {
  __builtin_nontemporal_store(v, (u32x4 *)p);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte words that source lanes i/4, 4 + i/4, 8 + i/4 and
// 12 + i/4 address. If source lane r points at row k0 + r/4, columns
// c0 + 4*(r%4) .. +3 of a row-major 16-bit tile, lane i receives rows
// k0..k0+3 of column c0 + i: four consecutive k values of one column, i.e.
// half of an MFMA operand whose contraction index runs along the tile's rows.
__device__ __forceinline__ u32x2 ld_tr16(const uint16_t *p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte-chunk swizzle for a row-major tile with a row stride of an odd
// multiple of 64 bytes. LDS has 64 banks of 4 bytes. Transposing reads
// (4 consecutive rows x 64 bytes per half-wave) are conflict-free with that
// stride; XOR-ing the chunk index with (row / 4) % 4 also spreads the rows of
// a 16-lane group of row-wise 16-byte reads over all 64 banks.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// Direct 16-byte global -> LDS load (global_load_lds_dwordx4): every lane
// reads 16 bytes at its own global address; the wave writes them to 1 KiB of
// LDS starting at lds_base (wave-uniform), lane l at lds_base + 16 l. The
// write is tracked by the vector-memory counter.
__device__ __forceinline__ void load_lds16(const void *gptr, void *lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base, 16,
                                   0, 0);
}
// Buffer resource for raw (unformatted) buffer access on gfx9: 48-bit base,
// stride 0, size in bytes (accesses at or past it read as zero), word 3 as
// the gfx9 raw-buffer format.
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Its words are wave-uniform by definition; readfirstlane keeps them in SGPRs
// even where the compiler computes a uniform value with a vector instruction.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void *lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// Direct 16-byte buffer -> LDS load (buffer_load_dwordx4 ... lds): lane l
// reads 16 bytes at byte offset voffset + soffset of the buffer and the wave
// writes them to LDS at lds_base + 16 l (lds_base wave-uniform).
__device__ __forceinline__ void buffer_load_lds16(const i32x4 &rsrc, int voffset, int soffset,
                                                  void *lds_base) {
  raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_base, 16, voffset,
                      soffset, 0, 0);
}
// The same direct loads (16 or 4 bytes per lane) written as inline assembly,
// so the compiler does not track them: it would otherwise make every later
// LDS read that it cannot prove disjoint from the destination (e.g. a buffer
// chosen at run time) wait for all outstanding vector-memory operations.
// The caller must wait for them itself (wait_vmem_all, then a barrier)
// before reading the destination. The compiler's own waits stay correct:
// vector-memory loads complete in issue order, so extra loads it does not
// know about only make its waits longer. M0 is saved and restored; its write
// needs one wait state before the load.
// A generic pointer into LDS is the shared aperture's base in the upper 32
// bits and the LDS byte offset in the lower 32, so truncating it gives the
// offset (a cast to the LDS address space would add a null-pointer check).
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ void dma_lds16(const i32x4 &rsrc, int voffset, uint32_t soffset,
                                          const void *lds_base) {
  uint32_t saved;
  // Wave-uniform by contract; kept in SGPRs (the soffset field takes no
  // literal). An unsigned byte offset: the full 32-bit range is valid.
  soffset = (uint32_t)__builtin_amdgcn_readfirstlane((int)soffset);
  uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm("" : "+s"(soffset), "+s"(m0v));
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}
__device__ __forceinline__ void dma_lds4(const i32x4 &rsrc, int voffset, uint32_t soffset,
                                          const void *lds_base) {
  uint32_t saved;
  // Wave-uniform by contract; kept in SGPRs (the soffset field takes no
  // literal). An unsigned byte offset: the full 32-bit range is valid.
  soffset = (uint32_t)__builtin_amdgcn_readfirstlane((int)soffset);
  uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
  asm("" : "+s"(soffset), "+s"(m0v));
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}
// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding vector-memory operations (direct-to-LDS loads of another
// buffer, atomics), which may keep flying across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until every vector-memory operation this wave issued has completed.
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stores a wave's 32 x D output tile, held in the layout of D/32 MFMA
// results (lane l: row l % 32; acc[dt] register r: column
// 32 dt + 8 (r / 4) + 4 (l / 32) + r % 4), times f and rounded to T, into
// rows 0 .. nrows-1 of a dense row-major [*, D] array at out. It goes
// through `lds`, a wave-private area of 32 * D 16-bit elements (16-byte
// aligned): straight from the accumulator layout a store instruction would
// write 8 bytes into each of 32 rows (a 128-byte line then takes 8 partial
// writes); read back row-major, each instruction writes 64 / (D/8) whole rows,
// 16 bytes per lane. In the LDS area row r holds its 16-byte chunks c at
// position c ^ (r % CPR), which spreads both access patterns over the banks.
// The caller makes sure no other wave uses the area meanwhile.
template <typename T, int D>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[D / 32], float f,
                                                uint16_t *lds, uint16_t *out, int nrows,
                                                int lane) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  char *st = (char *)lds;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * dt + i;  // chunk of columns 32 dt + 8 i .. +7
      u32x2 a;
      a[0] = pack2<T>(acc[dt][4 * i] * f, acc[dt][4 * i + 1] * f);
      a[1] = pack2<T>(acc[dt][4 * i + 2] * f, acc[dt][4 * i + 3] * f);
      *(u32x2 *)(st + l32 * 2 * D + 16 * (c ^ (l32 % CPR)) + 8 * g) = a;
    }
  // 64 lanes x 16 bytes = 64 / CPR rows per instruction.
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = RPI * k + lane / CPR, c = lane % CPR;
    const u32x4 v = *(const u32x4 *)(st + r * 2 * D + 16 * (c ^ (r % CPR)));
    if (r < nrows) st128_nt(out + (size_t)r * D + 8 * c, v);
  }
}

__device__ __forceinline__ u32x4 cat(const u32x2 &a, const u32x2 &b) {
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

}  // namespace fa
