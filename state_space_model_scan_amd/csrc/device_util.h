// device_util.h -- io element access, math and DPP helpers shared by the scan
// and conv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// io element access.  The io dtype is a template value IO: 0 = fp32, 1 =
// bf16 (the upper half of a binary32), 2 = fp16 (IEEE binary16).  A bool
// argument converts to 0 / 1.
// ---------------------------------------------------------------------------

// 16 stored bits -> float (bf16: a shift; fp16: the hardware conversion).
template <int IO>
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  if constexpr (IO == 1) return __uint_as_float(h << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
// float -> 16 stored bits, rounded to nearest, ties to even.
template <int IO>
__device__ __forceinline__ uint32_t float_to_half_bits(float v) {
  if constexpr (IO == 1) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

template <int IO, int NV>
struct RawV {  // NV consecutive io elements as loaded from memory (NV = 4 or 8)
  static_assert(NV == 4 || NV == 8, "vector width");
  static constexpr int kWords = IO ? NV / 2 : NV;
  uint32_t w[kWords];

  __device__ __forceinline__ float get(int i) const {
    if constexpr (IO == 1) {
      const uint32_t v = w[i >> 1];
      return __uint_as_float((i & 1) ? (v & 0xffff0000u) : (v << 16));
    } else if constexpr (IO == 2) {
      const uint32_t v = w[i >> 1];
      return half_bits_to_float<2>((i & 1) ? (v >> 16) : (v & 0xffffu));
    } else {
      return __uint_as_float(w[i]);
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0;
  }
  // Aligned vector load of elements [idx, idx+NV).
  __device__ __forceinline__ void load_vec(const void *base, int64_t idx) {
    const uint32_t *p = IO ? reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(base) + idx)
                             : reinterpret_cast<const uint32_t *>(static_cast<const float *>(base) + idx);
    if constexpr (kWords == 2) {
      const uint2 q = *reinterpret_cast<const uint2 *>(p);
      w[0] = q.x; w[1] = q.y;
    } else {
#pragma unroll
      for (int j = 0; j < kWords / 4; ++j) {
        const uint4 q = reinterpret_cast<const uint4 *>(p)[j];
        w[4 * j] = q.x; w[4 * j + 1] = q.y; w[4 * j + 2] = q.z; w[4 * j + 3] = q.w;
      }
    }
  }
  // Element loads of [idx, idx+cnt), zero beyond cnt (cnt may be <= 0).
  // Every element lands in a register of its own and the words are packed
  // after the last load, so no load waits on the one before it.
  __device__ __forceinline__ void load_elems(const void *base, int64_t idx, int cnt) {
    if constexpr (IO != 0) {
      uint32_t h[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) h[i] = i < cnt ? static_cast<const uint16_t *>(base)[idx + i] : 0u;
#pragma unroll
      for (int j = 0; j < kWords; ++j) w[j] = h[2 * j] | (h[2 * j + 1] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) w[i] = i < cnt ? __float_as_uint(static_cast<const float *>(base)[idx + i]) : 0u;
    }
  }
  __device__ __forceinline__ void load(const void *base, int64_t idx, int cnt, bool vec) {
    if (vec && cnt >= NV) load_vec(base, idx);
    else load_elems(base, idx, cnt);
  }
  // Element load into slot i (slot assumed zero).
  __device__ __forceinline__ void load_one(const void *base, int64_t idx, int i) {
    if constexpr (IO != 0) {
      const uint32_t h = static_cast<const uint16_t *>(base)[idx];
      w[i >> 1] |= (i & 1) ? (h << 16) : h;
    } else {
      w[i] = __float_as_uint(static_cast<const float *>(base)[idx]);
    }
  }
};

template <int IO>
using Raw8 = RawV<IO, 8>;

template <int IO>
__device__ __forceinline__ float load_io(const void *p, int64_t i) {
  if constexpr (IO != 0) return half_bits_to_float<IO>(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

// An io element's value as the bits of a binary32.
template <int IO>
__device__ __forceinline__ uint32_t load_io_bits(const void *p, int64_t i) {
  return __float_as_uint(load_io<IO>(p, i));
}

// Round to the io dtype (hardware round-to-nearest-even convert).
template <int IO>
__device__ __forceinline__ float round_io(float v) {
  if constexpr (IO != 0) return half_bits_to_float<IO>(float_to_half_bits<IO>(v));
  else return v;
}

template <int IO, int NV>
__device__ __forceinline__ void store_n(void *base, int64_t idx, const float (&v)[NV], int cnt, bool vec) {
  static_assert(NV == 4 || NV == 8, "vector width");
  if constexpr (IO != 0) {
    uint32_t pk[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i)
      pk[i] = float_to_half_bits<IO>(v[2 * i]) | (float_to_half_bits<IO>(v[2 * i + 1]) << 16);
    if (vec && cnt >= NV) {
      uint16_t *p = static_cast<uint16_t *>(base) + idx;
      if constexpr (NV == 8) *reinterpret_cast<uint4 *>(p) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      else *reinterpret_cast<uint2 *>(p) = make_uint2(pk[0], pk[1]);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i < cnt) static_cast<uint16_t *>(base)[idx + i] = static_cast<uint16_t>((i & 1) ? (pk[i >> 1] >> 16) : pk[i >> 1]);
    }
  } else {
    float *p = static_cast<float *>(base) + idx;
    if (vec && cnt >= NV) {
#pragma unroll
      for (int j = 0; j < NV / 4; ++j)
        reinterpret_cast<float4 *>(p)[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i < cnt) p[i] = v[i];
    }
  }
}

// One io element (16-bit dtypes: rounded to nearest, ties to even).
template <int IO>
__device__ __forceinline__ void store_one(void *base, int64_t idx, float v) {
  if constexpr (IO != 0) static_cast<uint16_t *>(base)[idx] = static_cast<uint16_t>(float_to_half_bits<IO>(v));
  else static_cast<float *>(base)[idx] = v;
}

template <int IO>
__device__ __forceinline__ void store8(void *base, int64_t idx, const float (&v)[8], int cnt, bool vec) {
  store_n<IO, 8>(base, idx, v, cnt, vec);
}

// ---------------------------------------------------------------------------
// math helpers (hardware exp2 / log2 / rcp)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// softplus(v) = log(1 + e^v); above 20 it equals v to fp32 precision.
__device__ __forceinline__ float softplus_f(float v) {
  const float sp = fast_log2(1.0f + fast_exp2(v * kLog2e)) * kLn2;
  return v > 20.0f ? v : sp;
}

// silu(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu_f(float v) {
  return v * fast_rcp(1.0f + fast_exp2(-v * kLog2e));
}

// ---------------------------------------------------------------------------
// DPP row broadcast: lane K of each 16-lane row to the whole row.
// ---------------------------------------------------------------------------

template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(K >= 0 && K < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}

// sum_k bcast(c, K0 + k) * x[k].  The compiler folds a DPP move into a
// multiply but not into an FMA, so the chain is written directly; the leading
// s_nop gives the two wait states a DPP source read needs after a VALU write
// of that VGPR.
template <int K0, int N>
__device__ __forceinline__ float dot_bcast(float c, const float (&x)[N]) {
  static_assert(K0 + N <= 16, "row lane");
  float y;
  if constexpr (N == 4) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %1, %2 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
        : "=&v"(y)
        : "v"(c), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]),
          "n"(K0), "n"(K0 + 1), "n"(K0 + 2), "n"(K0 + 3));
  } else if constexpr (N == 2) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %1, %2 row_newbcast:%4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
        : "=&v"(y)
        : "v"(c), "v"(x[0]), "v"(x[1]), "n"(K0), "n"(K0 + 1));
  } else if constexpr (N == 1) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "=v"(y)
        : "v"(c), "v"(x[0]), "n"(K0));
  } else {
    static_assert(N == 1 || N == 2 || N == 4, "unsupported state-group width");
  }
  return y;
}

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F &&f) {
  (f(std::integral_constant<int, I>{}), ...);
}

}  // namespace ssm
