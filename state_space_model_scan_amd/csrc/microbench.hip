// microbench.hip -- instruction-rate and bandwidth probes (libssmmicro.so).
//
// The scan's ALU ceiling rests on three rates of the chip: plain fp32 VALU
// issue, v_exp_f32 issue, and how the two mix in the scan's own step (a
// multiply, an exp, a multiply and two FMAs per (timestep, state)).  The
// GPU cost model the Triton vector-addition tutorial sets out (compute,
// memory, overhead) needs those numbers measured, not assumed; the probes
// here measure them, together with the LDS rates of the data hand-offs and
// the device copy bandwidth.  include/ssmmicro.h documents each probe.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssmmicro.h"

namespace {

__device__ __forceinline__ void stamp(uint64_t *clk, int slot) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[2 * slot] = __builtin_amdgcn_s_memtime();
    clk[2 * slot + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

// Opaque to the optimiser: the value may have changed, so nothing computed
// from it is loop-invariant.
__device__ __forceinline__ void touch(float &v) { asm volatile("" : "+v"(v)); }

__global__ void __launch_bounds__(256) k_fma(float *out, uint64_t *clk, int iters, float a, float b) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = gid * 1e-7f + k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], a, b);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[gid] = s;
  stamp(clk, 1);
}

__global__ void __launch_bounds__(256) k_exp(float *out, uint64_t *clk, int iters) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = gid * 1e-7f + 0.1f * k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[gid] = s;
  stamp(clk, 1);
}

__global__ void __launch_bounds__(256) k_sin(float *out, uint64_t *clk, int iters) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = gid * 1e-7f + 0.1f * k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_sinf(x[k]);   // argument in revolutions
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[gid] = s;
  stamp(clk, 1);
}

// The scan step on 4 states over 8 timesteps per iteration; the step
// operands are made opaque each iteration so no exp is hoisted.
__global__ void __launch_bounds__(256) k_mix(float *out, uint64_t *clk, int iters) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float A[4], Bv[4], Cv[4], x[4], dt[8], dtu[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    A[k] = -1.0f - 0.25f * k;
    Bv[k] = 0.5f + 0.1f * k;
    Cv[k] = 0.3f - 0.05f * k;
    x[k] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dt[j] = 0.01f * (j + 1) + gid * 1e-9f;
    dtu[j] = 0.02f * (j + 1);
  }
  float acc = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      touch(dt[j]);
      touch(dtu[j]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = __builtin_amdgcn_exp2f(dt[j] * A[k]);
        x[k] = fmaf(e, x[k], Bv[k] * dtu[j]);
      }
      float y = Cv[0] * x[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) y = fmaf(Cv[k], x[k], y);
      acc += y;
    }
  }
  out[gid] = acc;
  stamp(clk, 1);
}

// The scan step of k_mix with the products B * (delta' u) of a timestep
// taken by one v_mfma_f32_16x16x4_f32 as an outer product (states x
// channels, one nonzero k), so each lane's state update reads its four
// products from the accumulators: 104 plain, 32 exps and 8 MFMAs per
// iteration.
typedef float mb_f32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) k_mixmm(float *out, uint64_t *clk, int iters) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  float A[4], Cv[4], x[4], dt[8], bsel[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    A[k] = -1.0f - 0.25f * k;
    Cv[k] = 0.3f - 0.05f * k;
    x[k] = 0.0f;
  }
  float Bl = 0.5f + 0.01f * (lane & 15);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dt[j] = 0.01f * (j + 1) + gid * 1e-9f;
    bsel[j] = lane < 16 ? 0.02f * (j + 1) : 0.0f;
  }
  float acc = 0.0f;
  const mb_f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i = 0; i < iters; ++i) {
    mb_f32x4 bx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      touch(bsel[j]);
      bx[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(Bl, bsel[j], zero4, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      touch(dt[j]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = __builtin_amdgcn_exp2f(dt[j] * A[k]);
        x[k] = fmaf(e, x[k], bx[j][k]);
      }
      float y = Cv[0] * x[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) y = fmaf(Cv[k], x[k], y);
      acc += y;
    }
  }
  out[gid] = acc;
  stamp(clk, 1);
}

template <int K>
__device__ __forceinline__ float bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}

__global__ void __launch_bounds__(256) k_dpp(float *out, uint64_t *clk, int iters) {
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  float x[8];
  const float c = 1.0f + (threadIdx.x & 15) * 1e-7f;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = gid * 1e-7f + k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = bcast<3>(x[k]) * c;
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  out[gid] = s;
  stamp(clk, 1);
}

template <int MODE>   // 0: broadcast read, 1: linear read, 2: linear 32-bit write
__global__ void __launch_bounds__(256) k_lds(float *out, uint64_t *clk, int iters) {
  __shared__ float4 s[1024];
  stamp(clk, 0);
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 1024; i += 256) s[i] = make_float4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  float acc = 0.0f;
  if constexpr (MODE == 2) {
    float *sf = reinterpret_cast<float *>(s);
    float v = gid * 1e-3f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // wave w writes its own 256-float slice; j picks one of 4 slices per wave
        sf[(w * 4 + (j & 3)) * 256 + lane * 4 + (j >> 2)] = v;
        touch(v);
      }
    }
    __syncthreads();
    acc = sf[threadIdx.x];
  } else {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int idx = MODE == 0 ? ((i * 16 + j + w) & 1023) : ((w * 256 + j * 16 + lane) & 1023);
        float4 v = s[idx];
        asm volatile("" :: "v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
      }
    }
    acc = s[threadIdx.x].x;
  }
  out[gid] = acc;
  stamp(clk, 1);
}

__global__ void __launch_bounds__(256) k_copy(uint4 *buf, uint64_t *clk, int iters, int64_t half) {
  stamp(clk, 0);
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  // four independent 16-byte loads in flight per thread (iters % 4 == 0)
  for (int i = 0; i < iters; i += 4) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = buf[gid + (i + j) * nthreads];   // < nthreads * iters == half
#pragma unroll
    for (int j = 0; j < 4; ++j) buf[half + gid + (i + j) * nthreads] = v[j];
  }
  stamp(clk, 1);
}

}  // namespace

extern "C" int ssm_microbench(int32_t kind, int32_t blocks, int32_t iters, float *out, uint64_t *clk,
                              void *stream_ptr) {
  if (blocks <= 0 || iters <= 0 || !out || !clk) return 3;
  hipStream_t st = static_cast<hipStream_t>(stream_ptr);
  const dim3 g(blocks), b(256);
  switch (kind) {
    case SSM_MB_FMA: hipLaunchKernelGGL(k_fma, g, b, 0, st, out, clk, iters, 0.999999f, 1e-7f); break;
    case SSM_MB_EXP: hipLaunchKernelGGL(k_exp, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_SIN: hipLaunchKernelGGL(k_sin, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_MIX: hipLaunchKernelGGL(k_mix, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_MIXMM: hipLaunchKernelGGL(k_mixmm, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_DPP: hipLaunchKernelGGL(k_dpp, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_LDS_BC: hipLaunchKernelGGL(k_lds<0>, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_LDS_LIN: hipLaunchKernelGGL(k_lds<1>, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_LDS_W32: hipLaunchKernelGGL(k_lds<2>, g, b, 0, st, out, clk, iters); break;
    case SSM_MB_COPY: {
      if (iters % 4 != 0) return 3;
      const int64_t half = static_cast<int64_t>(blocks) * 256 * iters;
      hipLaunchKernelGGL(k_copy, g, b, 0, st, reinterpret_cast<uint4 *>(out), clk, iters, half);
      break;
    }
    default: return 3;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
