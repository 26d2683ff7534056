// Device-side helpers shared by the kernels: small vector types, the 16-bit
// MFMA wrapper, dtype packing and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace fa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));

// 16-bit MFMA operand types and helpers shared by the 16-bit kernels.
template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using vec8 = bf16x8;
};
template <>
struct Elem<false> {
  using vec8 = f16x8;
};

typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(typename Elem<BF16>::vec8 a,
                                               typename Elem<BF16>::vec8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> two 16-bit values of the storage dtype (round to
// nearest even), packed low-first into one dword.
template <bool BF16>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (BF16) {
    typedef __bf16 v2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
    v2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(unsigned, r);
  } else {
    typedef _Float16 v2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
    v2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return __builtin_bit_cast(unsigned, r);
  }
}


// Debug build only (compiled with FA_DEBUG_POISON_LDS): called by the lanes
// of a wave right before they issue an LDS DMA copy to lds_addr (lane i
// then writes BYTES bytes at lds_addr + BYTES*i). It fills exactly those
// bytes with all-ones, a NaN in fp32, bf16 and fp16, and waits until the
// fill has landed, so the copy's data is written after it. Any read of the
// destination that is not ordered after the copy's completion (a missing
// vmcnt wait or barrier) then sees NaN instead of stale data from an older
// tile, and the NaN reaches the outputs. In the normal build it is empty.
template <int BYTES>
__device__ __forceinline__ void poison_lds_before_copy(unsigned lds_addr) {
#ifdef FA_DEBUG_POISON_LDS
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword copies");
  const unsigned a = lds_addr + BYTES * (threadIdx.x & 63);
  if constexpr (BYTES == 16)
    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)a = u32x4{~0u, ~0u, ~0u, ~0u};
  else
    *(__attribute__((address_space(3))) unsigned*)(uintptr_t)a = ~0u;
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)lds_addr;
#endif
}


// The chip has 8 XCDs, each with its own L2, and consecutive workgroup ids
// are dealt to the XCDs round-robin. Work units that share K/V (the
// Q-blocks of one head) get consecutive logical ids, so this mapping sends
// a contiguous run of logical ids to one XCD: workgroup w runs logical unit
// (w % 8) * (G / 8) + w / 8. Ids past the last multiple of 8 map to
// themselves, so the mapping is a bijection of [0, G).
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int per = G >> 3;
  const int full = per << 3;
  return (w < full) ? ((w & 7) * per + (w >> 3)) : w;
}

}  // namespace fa
