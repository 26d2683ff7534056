// Sums across the lanes of a wave64 with DPP and the gfx950 lane swaps,
// not through the LDS crossbar (ds_bpermute, which __shfl_xor becomes).
//
// Each step adds a lane's value and its partner's, so every lane of a
// group ends with the same sum. Partners, in order:
//   lane ^ 1, lane ^ 2      DPP quad_perm [1,0,3,2] and [2,3,0,1]
//   lane ^ 4 (in effect)    DPP row_half_mirror: lane i of each 8 reads
//                           lane 7 - i, which lies in the other quad and
//                           (after the quad steps) holds that quad's sum
//   lane ^ 8 (in effect)    DPP row_mirror: lane i of each 16 reads 15 - i
//   lane ^ 16, lane ^ 32    v_permlane16_swap / v_permlane32_swap: of the two
//                           results one is the lane's own value and the
//                           other its partner's, so both are added
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int w = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(w);
}

// Sum over each aligned group of W lanes (W a power of two, 2 .. 64).
template <int W>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group of 2 .. 64 lanes");
  v = dpp_add<0xB1>(v);                        // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v = dpp_add<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v = dpp_add<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v = dpp_add<0x140>(v);  // row_mirror
  if constexpr (W >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
  if constexpr (W >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
  return v;
}

}  // namespace fa
