// Matrix-core (MFMA) building blocks for gfx950.
//
// v_mfma_f32_32x32x16_bf16 computes D[32x32] += A[32x16] * B[16x32] per wavefront:
//   A operand: lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7   (8 bf16 = 16 bytes)
//   B operand: lane l holds B[8 * (l / 32) + j][l % 32]
//   D:         lane l, register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// Any consistent assignment of the 16 contraction indices to (l / 32, j) gives the same
// result, so A and B only have to agree with each other.
//
// ds_read_b64_tr_b16 (gfx950 transposing LDS read): within each group of 16 lanes, source lane s
// reads 4 consecutive 16-bit elements at its own address, and destination lane i receives in slot
// j the element i % 4 of source lane 4 * j + i / 4.  If source lane s points at row
// (r0 + s / 4), column (c0 + 4 * (s % 4)) of a row-major tile, destination lane i receives column
// c0 + i of rows r0 .. r0 + 3: a 4x16 block read out transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

#define MLA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// The same MFMA with its accumulator in VGPRs, for a short chain whose result the vector ALU
// reads next (attention scores).  In a kernel that keeps other accumulators in AGPRs the compiler
// selects the AGPR form for every MFMA, and each read of such a result then costs a
// v_accvgpr_read; written as inline asm with "v" operands the chain stays in VGPRs.  The compiler
// does not know these are MFMAs and inserts no wait states for them, so a chain starts with
// mfma32_v_first (zero accumulator; two wait states ahead of it for a VALU write of the
// destination) and ends with mfma32_v_last, whose s_nops (21 wait states) cover the longest
// read-after-write and write-after-read distance of this 8-pass MFMA before any other instruction
// touches the accumulator.  Between them, dependent MFMAs of the same opcode issue back to back.
__device__ __forceinline__ void mfma32_v_first(f32x16 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v(f32x16 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_v_last(f32x16 &acc, const u32x4 &a, const u32x4 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
               : "+v"(acc)
               : "v"(a), "v"(b));
}

// v_mfma_f32_16x16x32_bf16 computes D[16x16] += A[16x32] * B[32x16] per wavefront:
//   A operand: lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B operand: lane l holds B[8 * (l / 16) + j][l % 16]
//   D:         lane l, register r holds D[4 * (l / 16) + r][l % 16]
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const unsigned char *base, uint32_t byte_off) {
  return *(const MLA_LDS u32x4 *)(base + byte_off);
}

__device__ __forceinline__ void lds_write16(unsigned char *base, uint32_t byte_off, const u32x4 &v) {
  *(MLA_LDS u32x4 *)(base + byte_off) = v;
}

__device__ __forceinline__ void lds_write8(unsigned char *base, uint32_t byte_off, const u32x2 &v) {
  *(MLA_LDS u32x2 *)(base + byte_off) = v;
}

// Two transposing reads (rows r0..r0+3 then r0+4..r0+7) packed into one 8-element operand.
__device__ __forceinline__ u32x4 lds_read_tr_pair(const unsigned char *base, uint32_t off0, uint32_t off1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4 *)(base + off0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4 *)(base + off1));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// ---- buffer resources: 128-bit descriptor in SGPRs + 32-bit per-lane byte offset ---------------
// Reads past `bytes` return zero and writes past it are dropped (raw buffer, stride 0).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ int buf_load_i32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return int(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, const u32x4 &v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, const u32x2 &v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, 0);
}
// A streaming store (non-temporal hint): for outputs that no later step of the same call reads.
__device__ __forceinline__ void buf_store16_nt(rsrc_t r, const u32x4 &v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 2);
}
// A store with the system-scope cache policy (sc0 and sc1 set): the line is written through to
// memory rather than left dirty in this XCD's L2.  For rows that a later kernel reads from
// other XCDs, which cannot see this L2 anyway.
__device__ __forceinline__ void buf_store16_sys(rsrc_t r, const u32x4 &v, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 17);
}
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds_base + 16 * l
// (lds_base is wavefront-uniform and goes through M0).
//
// Issued as inline asm rather than through __builtin_amdgcn_raw_ptr_buffer_load_lds: the compiler
// treats the builtin as a pending write to all of LDS and puts s_waitcnt vmcnt(0) in front of every
// later ds_read_b64_tr_b16, which drains every prefetched tile.  The load has no register result;
// callers order it with explicit wait_vmcnt<N>() and barriers before reading the destination, and
// the "memory" clobber keeps the compiler from moving LDS accesses across it.  Because the
// compiler does not count these loads, a kernel must not leave compiler-visible vector loads
// pending across them into code that relies on the compiler's own vmcnt waits (complete such
// loads with wait_vmcnt<0>() first).
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, unsigned char *lds_base, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((MLA_LDS void *)lds_base)));
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}
// The same with the destination given as an LDS byte address (see lds_addr), which keeps the
// address arithmetic on the scalar unit without generic-to-LDS pointer conversions.
__device__ __forceinline__ void buf_load16_lds_at(rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}
// The same with the non-temporal hint, for rows that no other workgroup reads: they stream
// through instead of displacing what other workgroups and later kernels reuse from L2 and MALL.
__device__ __forceinline__ void buf_load16_lds_at_nt(rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const MLA_LDS void *)p));
}

// Workgroup order for an 8-XCD part.  Workgroups are handed to the XCDs round-robin by id, so
// ids x, x+8, x+16, ... run on XCD x and share its L2.  This maps the hardware id to a logical
// id such that XCD x receives one contiguous range of logical ids: workgroups that are adjacent
// in logical order (and read the same data) then share an L2.  It is a bijection on [0, n) for
// any n; only performance depends on the dispatch order being as assumed.
__device__ __forceinline__ int xcd_logical_id(int hw_id, int n) {
  const int x = hw_id & 7, k = hw_id >> 3;
  const int base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + k;
}

// Compiler-level memory barrier (no instruction): keeps LDS reads of a staged tile after the
// s_barrier that publishes it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Accumulator access.  MFMA results live in AGPRs; reading them through an explicit
// v_accvgpr_read pins each move to its use, so the compiler does not copy a whole accumulator
// array into VGPRs at once (which forces spills of everything else that is live).  Both helpers
// are plain register moves.
__device__ __forceinline__ float agpr_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}
__device__ __forceinline__ float agpr_write(float x) {
  float r;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of x over lanes l and l ^ 32 (one v_permlane32_swap: whichever way the halves are
// exchanged, each lane ends up holding both values, so the result is the same in both halves)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mla
