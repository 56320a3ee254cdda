// device.h -- gfx950 building blocks shared by the attention kernels.
//
// bf16 MFMA (v_mfma_f32_32x32x16_bf16), buffer-resource loads with hardware
// zero-fill past the end of a tensor, direct global->LDS loads, and the
// conversions the softmax needs.  Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 short4_lds;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr float kLog2e = 1.4426950408889634f;

// Buffer resource over [base, base + bytes).  Loads past `bytes` return zero,
// which is how every kernel here pads the ragged tail of a tile.
// Every caller passes wave-uniform values; they are read from lane 0 so that
// the compiler keeps the descriptor in scalar registers even when it cannot
// prove them uniform (e.g. after an integer division it expanded on the VALU),
// instead of wrapping each load in a loop over distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// 16 bytes from byte offset `voff` into registers (zero when out of range).
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// 16 bytes from byte offset `voff` + `soff` straight into LDS.  `dst` and
// `soff` are wave-uniform (soff, a scalar operand, saves a vector add per
// load; callers keep it below the row length, so that whether a row lies
// past the end of the resource is decided by `voff` alone); lane i's 16 bytes
// land at dst + 16 * i.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff,
                                              uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)dst, 16, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// s_waitcnt vmcnt(0) as an immediate for __builtin_amdgcn_s_waitcnt (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the other
// two at their maxima): a wait the compiler's own wait tracking sees.
constexpr int kWaitVmem0 = 0x0f70;

// The four words of the buffer resource make_rsrc builds (read from lane 0),
// for load16_to_lds_untracked.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu,
               (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// load16_to_lds issued from inline asm, so that the compiler does not track
// it: it adds no wait for it before later LDS reads (it cannot tell which LDS
// bytes a load writes when the destination stage is chosen at run time, and
// would otherwise wait for every load in flight).  The caller must wait
// (s_waitcnt vmcnt) for the load before any LDS read of the bytes it writes;
// the load writes no register.  M0 holds the wave's LDS destination.
__device__ __forceinline__ void load16_to_lds_untracked(const u32x4& r, void* dst, uint32_t voff) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst);
  // Re-read from lane 0 here so that the operand is formed in scalar registers
  // (the values may have been kept in vector registers in between).
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane(r[0]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(r[1]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(r[2]),
                    (uint32_t)__builtin_amdgcn_readfirstlane(r[3])};
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds),
      "v"(voff), "s"(rs)
      : "memory", "m0");
}

// D = A * B + C with A 32x16, B 16x32, C/D 32x32 fp32.  Lane l supplies
// A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32], e = 0..7, and
// holds D[8 * (j / 4) + 4 * (l / 32) + j % 4][l % 32] in element j.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even), packed lo | hi << 16.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// s + lo + hi of a packed bf16 pair, in fp32 (one v_dot2 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(unsigned w, float s) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), s, false);
}

// Multiply both bf16 halves of a word by 2^-s (s <= 255): a saturating
// subtract on the exponent field, exact while the result stays normal.  A
// value whose exponent field would go below 0 becomes zero; one whose field
// lands exactly on 0 keeps its 7 mantissa bits as a subnormal, i.e. m * 2^-133
// instead of (1 + m / 128) * 2^-127 -- wrong, but below 2^-126 in magnitude
// (the callers' values are at most 1 with row maxima above 2^-1, so such a
// term is negligible).  `s2` is s << 7 | s << 23.  Inputs must be >= 0.
__device__ __forceinline__ unsigned scale_pow2_down(unsigned w, unsigned s2) {
  u16x2 a = __builtin_bit_cast(u16x2, w);
  u16x2 b = __builtin_bit_cast(u16x2, s2);
  return __builtin_bit_cast(unsigned, __builtin_elementwise_sub_sat(a, b));
}

__device__ __forceinline__ float wave_swap32_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float wave_swap32_sum(float x) {
  return x + __shfl_xor(x, 32, 64);
}

// Workgroups are dealt round-robin to the 8 XCDs.  Renumber them so that a run
// of consecutive logical ids sits on one XCD (sharing its L2): physical id p
// runs on XCD p % 8; logical ids [x*per, (x+1)*per) go to XCD x.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t p, uint32_t n) {
  const uint32_t per = n / 8, rem = n % 8;
  const uint32_t x = p % 8, slot = p / 8;
  // XCDs 0..rem-1 get per+1 logical ids, the rest get per.
  const uint32_t base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + slot;
}

}  // namespace attn
