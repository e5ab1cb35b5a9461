// The Sparse Activated SoftMax exponential, shared by the decodes and the
// prefill's SAS key loops.
#pragma once

#include "common.hpp"

namespace skipattn {

// Sparse Activated SoftMax exponential (TurboAttention talk page,
// "Technical Deep Dive", its Sparse Activated SoftMax part): e^-x for x >= 0
// as T[n] p(f), n = floor(x), f = x - n, with T[n] = e^-n for n < 6 and 0
// from 6 on, and p the least-squares polynomial of degree DEG for e^-f on
// [0, 1] (solution of its normal equations, rounded to fp32). The
// exponential unit gives e^-n for the integer n in one instruction, which
// here stands in for the six-entry table (the same values to fp32
// rounding); x = +inf gives 0.
// Coefficients a0 .. a_DEG of p (the prefill's generated key loop takes them
// as operands).
constexpr float kSasPoly2[3] = {0.9944886f, -0.9305485f, 0.30871853f};
constexpr float kSasPoly3[4] = {0.99961364f, -0.99204874f, 0.46246922f, -0.10250045f};

template <int DEG>
__device__ __forceinline__ float sas_poly(float f) {
  if constexpr (DEG == 2)
    return __builtin_fmaf(__builtin_fmaf(kSasPoly2[2], f, kSasPoly2[1]), f, kSasPoly2[0]);
  else
    return __builtin_fmaf(
        __builtin_fmaf(__builtin_fmaf(kSasPoly3[3], f, kSasPoly3[2]), f, kSasPoly3[1]), f,
        kSasPoly3[0]);
}

template <int DEG>
__device__ __forceinline__ float sas_exp(float x) {
  const float f = __builtin_amdgcn_fractf(x);
  const float t = exp2_fast((x - f) * -1.44269504f);
  return x < 6.f ? t * sas_poly<DEG>(f) : 0.f;
}

// sas_exp(x) * 2^e (e a small integer: an exact power-of-two factor folded
// into the table row's exponent).
template <int DEG>
__device__ __forceinline__ float sas_exp_scaled(float x, float e) {
  const float f = __builtin_amdgcn_fractf(x);
  const float t = exp2_fast(__builtin_fmaf(x - f, -1.44269504f, e));
  return x < 6.f ? t * sas_poly<DEG>(f) : 0.f;
}

}  // namespace skipattn
