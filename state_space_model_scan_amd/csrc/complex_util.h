// complex_util.h -- the complex decay exp(delta' A) and an accurate softplus,
// shared by the complex-A forward and backward kernels.
//
// Per (timestep, state) the decay is
//   exp(delta' A) = 2^(delta' Re A log2 e) * (cos 2 pi r, sin 2 pi r),
//   r = delta' Im A / (2 pi)   (revolutions; the fraction is taken),
// with the hardware exp2, sine and cosine (the latter two take revolutions).
// Where |Im A| is large the phase carries most of the rounding: a relative
// error e in delta' or in Im A / (2 pi) turns into a phase error of
// e * delta' |Im A| radians, and the gradient of delta' (which holds A a_t)
// weighs it once more by |A|.  Hence:
//   * softplus(v) = max(v, 0) + log1p(e^-|v|) everywhere, log1p(w) being
//     log(1 + w) corrected by the rounding of 1 + w: with u = fl(1 + w) and
//     c = (u - 1) - w (exact), log1p(w) = log(u) - c / u to first order (the
//     plain log2(1 + 2^x) loses up to ~30 ulp of delta' to that rounding);
//   * the backward's phase to about one rounding (cexp_turns): Im A / (2 pi)
//     held as hi + lo (the fp32 quotient and its residual), and
//     r = fract(delta' hi) + (delta' lo + the exact rounding error of
//     delta' hi, from an fma);
//   * the forward's phase as fract(delta' hi) (cexp_plain): its outputs and
//     the checkpoints the backward restarts from weigh a phase error once by
//     |A|, not twice, and the three extra operations would be a sixth of the
//     forward's issue per (timestep, state).
#pragma once

#include <hip/hip_runtime.h>

#include "device_util.h"

namespace ssm {

constexpr float kInv2PiF = 0.15915494309189535f;
constexpr float kTwoPiHi = 6.28318548202514648f;     // fp32 nearest to 2 pi
constexpr float kTwoPiLo = -1.7484555314695172e-7f;  // 2 pi - kTwoPiHi

// Im A / (2 pi) as hi + lo
struct Turns {
  float hi, lo;
};

__device__ __forceinline__ Turns turns_of(float ai) {
  const float hi = ai * kInv2PiF;
  const float lo = (fmaf(-hi, kTwoPiHi, ai) - hi * kTwoPiLo) * kInv2PiF;
  return {hi, lo};
}

// exp(dt (ar + i ai)) from ar2 = ar log2 e and hi = ai / (2 pi)
__device__ __forceinline__ void cexp_plain(float dt, float ar2, float hi, float &er, float &ei) {
  const float mag = fast_exp2(dt * ar2);
  const float r = __builtin_amdgcn_fractf(dt * hi);
  er = mag * __builtin_amdgcn_cosf(r);
  ei = mag * __builtin_amdgcn_sinf(r);
}

// exp(dt (ar + i ai)) from ar2 = ar log2 e and (hi, lo) = turns_of(ai),
// the phase to about one rounding
__device__ __forceinline__ void cexp_turns(float dt, float ar2, float hi, float lo, float &er,
                                           float &ei) {
  const float mag = fast_exp2(dt * ar2);
  const float ph = dt * hi;
  const float r = __builtin_amdgcn_fractf(ph) + fmaf(dt, lo, fmaf(dt, hi, -ph));
  er = mag * __builtin_amdgcn_cosf(r);
  ei = mag * __builtin_amdgcn_sinf(r);
}

// softplus(v) = log(1 + e^v) to a few ulp at every v (no cancellation in 1 + w)
__device__ __forceinline__ float softplus_acc(float v) {
  const float w = fast_exp2(-fabsf(v) * kLog2e);
  const float u = 1.0f + w;
  const float c = (u - 1.0f) - w;
  return fmaxf(v, 0.0f) + fmaf(fast_log2(u), kLn2, -c * fast_rcp(u));
}

}  // namespace ssm
