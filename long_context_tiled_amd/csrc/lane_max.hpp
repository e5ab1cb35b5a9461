// Cross-lane helper shared by the decode kernels.
#pragma once

#include "common.hpp"

namespace skipattn {

// Largest value among lanes l, l ^ 16, l ^ 32 and l ^ 48 by the gfx950 lane
// swaps (vector instructions, no LDS round trip): v_permlane16_swap with two
// copies of x leaves x of rows 0/1 (2/3) in one copy and of rows 1/0 (3/2)
// in the other, so their max is max(x, x of lane l ^ 16); the same with
// v_permlane32_swap for lane l ^ 32. The s_nop covers the wait states a
// swap needs after a vector write of its operands.
__device__ __forceinline__ float max_over_row_groups(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  const float y = fmaxf(a, b);
  float c = y, d = y;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(c), "+v"(d));
  return fmaxf(c, d);
}

}  // namespace skipattn
