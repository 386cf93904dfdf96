// Device helpers shared by the bf16 MFMA kernels (forward and backward).
//
// Conventions of the 32x32x16 bf16 MFMA on gfx950 (checked on hardware):
//   A (M x K): lane l holds A[l % 32][8*(l / 32) + e], e = 0..7
//   B (K x N): lane l holds B[8*(l / 32) + e][l % 32]
//   C (M x N): lane l, value v holds C[8*(v / 4) + 4*(l / 32) + v % 4][l % 32]
//
// Tiles staged in LDS are row-major (one row = one token, D bf16) with the
// 16-byte units of row r XOR-swizzled by swz(r), chosen so that both access
// patterns of the kernels are free of bank conflicts:
//   operand reads: 16 lanes read one unit column of 16 different rows
//     (any 16 consecutive rows) -> swz(r) takes 16 distinct values;
//   transpose reads: half a wave reads 4 consecutive rows (starting at a
//     multiple of 4) x 4 aligned units -> the 4 rows land in 4 distinct
//     aligned unit quads (for D = 64 two rows share a 256-byte bank window).
#pragma once

#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define RA_LDS __attribute__((address_space(3)))

constexpr int RSRC_WORD3 = 0x00020000;   // raw (untyped) buffer access on the gfx9 family
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2F = 0.69314718055994530942f;

// MFMA row i <- token swap23(i) (bits 2 and 3 swapped): then lane l's values
// v = 0..7 and 8..15 of a 32x32 result are 8 consecutive tokens each, exactly
// the reduction-index layout of an A or B operand.
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Transposed value tiles (rows of 64 keys = 8 units of 16 bytes): unit u of row r
// is stored at u ^ vswz(r).  An operand read has 16 lanes read one unit of 16
// consecutive rows; (row parity, u ^ vswz(r)) then takes 16 distinct values, so the
// 16 reads hit 16 distinct 16-byte bank groups of a 256-byte window.
__device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }

// Element offset of (row, col) in a swizzled tile; col is a multiple of 4.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gfx950-only builtins live in device functions: used directly in a kernel
// template body they make clang drop the kernel's host-side launch stub.

// Buffer -> LDS loads.  Lane l copies 16 (dma16) or 4 (dma4) bytes from
// base + voff into LDS at dst + 16*l (4*l); bytes at or past base + nbytes read
// as zero (buffer range check).  base, nbytes and dst must be wave-uniform.
//
// They are issued from inline assembly on purpose: the compiler cannot tell
// which LDS buffer such a load writes, so for the builtin it makes the next
// LDS read of any buffer wait for all of them (s_waitcnt vmcnt) -- which
// serialises the prefetch of the next tile with the reads of the current one.
// Here the compiler knows nothing of the LDS write, so every reader of a
// loaded tile must be ordered after the loads explicitly: wait_vmem() by the
// issuing wave, then a workgroup barrier.  ("memory" keeps the compiler from
// moving other memory accesses across them; loads it does not count only make
// its own vmcnt waits stricter, never weaker.)
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int nbytes) {
  const unsigned long long p = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffff));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = RSRC_WORD3;
  return r;
}

__device__ __forceinline__ int lds_addr(RA_LDS void* p) {
  return __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long)p);
}

// The LDS destination goes in M0 (an input operand, so the compiler sets it).
__device__ __forceinline__ void dma16(const void* base, int nbytes, RA_LDS void* dst, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(buffer_rsrc(base, nbytes)), "{m0}"(lds_addr(dst)) : "memory");
}

__device__ __forceinline__ void dma4(const void* base, int nbytes, RA_LDS void* dst, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(buffer_rsrc(base, nbytes)), "{m0}"(lds_addr(dst)) : "memory");
}

// The same with a resource built once (buffer_rsrc over a whole block) and each lane's
// byte offset within it: the range check then zero-fills everything at or past the
// block's end, and issuing a tile costs no descriptor arithmetic.
__device__ __forceinline__ void dma16r(i32x4 rsrc, RA_LDS void* dst, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr(dst)) : "memory");
}

__device__ __forceinline__ void dma4r(i32x4 rsrc, RA_LDS void* dst, int voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "{m0}"(lds_addr(dst)) : "memory");
}

__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS s16x4*)p);
}

// Both lanes of a (j, j+32) pair get the pair's maximum / sum.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// vmcnt(N), N < 16: at most N of this wave's vector memory operations still outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Operand of 8 consecutive reduction indices k0..k0+7 (k = tile rows) for
// the 32 dims c0..c0+31 (MFMA index = lane % 32), read from a swizzled
// row-major tile with two transpose reads.  In 16-lane group G of lane l,
// source lane s = l % 16 points at row k0 + 4*half + s/4 and dims
// c0 + 16*(G % 2) + 4*(s % 4); k0 must be a multiple of 8 (lanes of the
// upper half-wave use k0 + 8).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int k0, int c0, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const int col = c0 + (G & 1) * 16 + 4 * (s & 3);
  const int row = k0 + (G >> 1) * 8 + (s >> 2);
  const s16x4 lo = lds_read_tr16(tile + tile_off<D>(row, col));
  const s16x4 hi = lds_read_tr16(tile + tile_off<D>(row + 4, col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-lane byte offset, within a tile of 64 rows, of this lane's 16-byte unit
// of buffer->LDS chunk q (chunk q covers LDS units [64q, 64q + 64)).
template <int D>
__device__ __forceinline__ int chunk_voff(int q, int lane, int row_bytes) {
  const int p = q * 64 + lane;
  const int r = p / (D / 8), pu = p % (D / 8);
  return r * row_bytes + (pu ^ swz<D>(r)) * 16;
}

// Combine (lse_a) (+) (lse_b): returns lse and the weights of a and b.
__device__ __forceinline__ void lse_combine(float la, float lb, float& lse, float& wa, float& wb) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) { lse = -INFINITY; wa = 0.f; wb = 0.f; return; }
  const float ea = expf(la - mx), eb = expf(lb - mx);
  const float s = ea + eb;
  lse = mx + logf(s);
  wa = ea / s;
  wb = eb / s;
}

// Block id -> logical id so that each XCD (ids are dealt round-robin over
// the 8 XCDs) works on one contiguous range of logical ids.
__device__ __forceinline__ int xcd_logical(int i, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = i % 8, local = i / 8;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

}  // namespace ra
