// decode.hip -- single-step decode: selective_state_update and
// causal_conv1d_update, with their C-ABI entry points.
//
// Operations: the PaddleNLP Kernel operator-library guide names
// selective_state_update in its mamba operator list (section 4.4) and
// causal_conv1d_update with its conv_state cache and optional cache_seqlens
// ring buffer (section 4.2); include/ssmscan.h writes out what each computes.
//
// Both are HBM-bound streams over the caches: a state update reads and writes
// the fp32 state (64 bytes each way per channel at dstate 16) and touches a
// few bytes of x, dt, z and out; a conv update moves a few bytes per channel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "host_util.h"
#include "ssmscan.h"

namespace ssm {
namespace {

// ---------------------------------------------------------------------------
// selective_state_update.  Four lanes per channel, lane q holding states
// [q*NSW, q*NSW + NSW): one vector load of a wave covers 16 consecutive
// channels' state rows (1 KiB at dstate 16), fully coalesced.  The state is
// read and written with non-temporal hints: it streams through once per call,
// and keeping it out of the caches leaves them to A, B, C and the per-channel
// vectors (measured on MI355X: 180 -> 143 us for a 335 MB state, about 93% of
// a plain device copy's rate).  The C.x partial sums meet in two DPP quad
// swaps.
// ---------------------------------------------------------------------------

struct StateUpdateParams {
  float *state;
  const void *x, *dt, *B, *C, *z;
  const float *A, *D, *dt_bias;
  void *out;
  int64_t dim, ngroups;
  uint32_t per_group, dblocks;   // channels per group; blocks per batch row
  int n, softplus, vec, bcvec;
};

constexpr int kSuChannels = 64;   // channels per 256-thread block

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// NSW consecutive floats with a non-temporal (streaming) hint
template <int NSW>
struct StreamVec {
  typedef float type __attribute__((ext_vector_type(NSW)));
};
template <int NSW>
__device__ __forceinline__ void load_stream(const float *p, float (&v)[NSW]) {
  if constexpr (NSW == 1) {
    v[0] = __builtin_nontemporal_load(p);
  } else {
    const typename StreamVec<NSW>::type r =
        __builtin_nontemporal_load(reinterpret_cast<const typename StreamVec<NSW>::type *>(p));
#pragma unroll
    for (int k = 0; k < NSW; ++k) v[k] = r[k];
  }
}
template <int NSW>
__device__ __forceinline__ void store_stream(float *p, const float (&v)[NSW]) {
  if constexpr (NSW == 1) {
    __builtin_nontemporal_store(v[0], p);
  } else {
    typename StreamVec<NSW>::type r;
#pragma unroll
    for (int k = 0; k < NSW; ++k) r[k] = v[k];
    __builtin_nontemporal_store(r, reinterpret_cast<typename StreamVec<NSW>::type *>(p));
  }
}

// A block covers kSuChannels channels of one batch row (the batch index is
// uniform over the block: no per-lane 64-bit division).
template <int IO, int NSW>
__global__ void __launch_bounds__(256) state_update_kernel(const StateUpdateParams p) {
  const uint32_t b = blockIdx.x / p.dblocks;
  const uint32_t dblk = blockIdx.x - b * p.dblocks;
  const int q = threadIdx.x & 3;
  const int64_t dd = static_cast<int64_t>(dblk) * kSuChannels + (threadIdx.x >> 2);
  // lanes past the last channel repeat it without storing, so every quad
  // stays whole for the cross-lane sum
  const bool valid = dd < p.dim;
  const int64_t d = valid ? dd : p.dim - 1;
  const int64_t row = static_cast<int64_t>(b) * p.dim + d;
  const int64_t g = static_cast<uint32_t>(d) / p.per_group;
  const int n = p.n;
  const int s0 = q * NSW;

  float step = load_io<IO>(p.dt, row);
  const float xv = load_io<IO>(p.x, row);
  float h[NSW], a[NSW], Bv[NSW], Cv[NSW];
  float *srow = p.state + row * n + s0;
  const float *arow = p.A + d * n + s0;
  if (p.vec) {
    load_stream<NSW>(srow, h);
    if constexpr (NSW == 1) {
      a[0] = arow[0];
    } else {
      const typename StreamVec<NSW>::type r = *reinterpret_cast<const typename StreamVec<NSW>::type *>(arow);
#pragma unroll
      for (int k = 0; k < NSW; ++k) a[k] = r[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
      const bool sv = s0 + k < n;
      h[k] = sv ? srow[k] : 0.0f;
      a[k] = sv ? arow[k] : 0.0f;
    }
  }
  const int64_t bc = (static_cast<int64_t>(b) * p.ngroups + g) * n + s0;
  bool bc_done = false;
  if constexpr (NSW == 4) {
    if (p.bcvec) {   // a lane's four io elements of B and of C, one vector load each
      RawV<IO, 4> rb, rc;
      rb.load_vec(p.B, bc);
      rc.load_vec(p.C, bc);
#pragma unroll
      for (int k = 0; k < NSW; ++k) { Bv[k] = rb.get(k); Cv[k] = rc.get(k); }
      bc_done = true;
    }
  }
  if (!bc_done) {
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
      const bool sv = s0 + k < n;
      Bv[k] = sv ? load_io<IO>(p.B, bc + k) : 0.0f;
      Cv[k] = sv ? load_io<IO>(p.C, bc + k) : 0.0f;
    }
  }

  if (p.dt_bias) step += p.dt_bias[d];
  if (p.softplus) step = softplus_f(step);
  const float dtx = step * xv;
  float y = 0.0f;
#pragma unroll
  for (int k = 0; k < NSW; ++k) {
    const float e = fast_exp2(step * (a[k] * kLog2e));
    h[k] = fmaf(e, h[k], Bv[k] * dtx);
    y = fmaf(Cv[k], h[k], y);   // padded states: C = 0, h stays 0
  }
  if (valid) {
    if (p.vec) {
      store_stream<NSW>(srow, h);
    } else {
#pragma unroll
      for (int k = 0; k < NSW; ++k)
        if (s0 + k < n) srow[k] = h[k];
    }
  }
  // sum over the quad: swap neighbours, then swap pairs (quad_perm [1,0,3,2], [2,3,0,1])
  y += quad_dpp<0xB1>(y);
  y += quad_dpp<0x4E>(y);
  if (valid && q == 0) {
    if (p.D) y = fmaf(p.D[d], xv, y);
    if (p.z) y *= silu_f(load_io<IO>(p.z, row));
    store_one<IO>(p.out, row, y);
  }
}

// ---------------------------------------------------------------------------
// causal_conv1d_update: one thread per channel.
// ---------------------------------------------------------------------------

struct ConvUpdateParams {
  const void *x;
  void *state;
  const float *w, *bias;
  const int32_t *cache_seqlens;
  void *out;
  int64_t dim, seqlen, state_len;
  uint32_t dblocks;   // blocks of 256 channels per batch row
  int silu;
};

// raw io element copy (exact: the cache stores inputs unchanged)
template <int IO>
__device__ __forceinline__ uint32_t raw_get(const void *p, int64_t i) {
  if constexpr (IO) return static_cast<const uint16_t *>(p)[i];
  else return static_cast<const uint32_t *>(p)[i];
}
template <int IO>
__device__ __forceinline__ void raw_put(void *p, int64_t i, uint32_t v) {
  if constexpr (IO) static_cast<uint16_t *>(p)[i] = static_cast<uint16_t>(v);
  else static_cast<uint32_t *>(p)[i] = v;
}
template <int IO>
__device__ __forceinline__ float raw_float(uint32_t v) {
  if constexpr (IO != 0) return half_bits_to_float<IO>(v);
  else return __uint_as_float(v);
}

__device__ __forceinline__ int64_t ring_slot(int64_t pos, int64_t S) {
  int64_t r = pos % S;
  return r < 0 ? r + S : r;
}

// A block covers 256 channels of one batch row.
template <int IO, int W>
__global__ void __launch_bounds__(256) conv_update_kernel(const ConvUpdateParams p) {
  const uint32_t b = blockIdx.x / p.dblocks;
  const uint32_t dblk = blockIdx.x - b * p.dblocks;
  const int64_t d = static_cast<int64_t>(dblk) * 256 + threadIdx.x;
  if (d >= p.dim) return;
  const int64_t row = static_cast<int64_t>(b) * p.dim + d;
  const int64_t S = p.state_len, L = p.seqlen;
  const int64_t sbase = row * S, xbase = row * L;
  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = p.w[d * W + k];
  const float bias = p.bias ? p.bias[d] : 0.0f;

  // the W-1 inputs before the first new token, read before any cache write
  float win[W];
  uint32_t hist[W];   // their raw bits, then the first new token's
  const int64_t pos = p.cache_seqlens ? static_cast<int64_t>(p.cache_seqlens[b]) : 0;
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t slot = p.cache_seqlens ? ring_slot(pos - (W - 1) + k, S) : S - (W - 1) + k;
    hist[k] = raw_get<IO>(p.state, sbase + slot);
    win[k] = raw_float<IO>(hist[k]);
  }
  hist[W - 1] = raw_get<IO>(p.x, xbase);
  for (int64_t t = 0; t < L; ++t) {
    win[W - 1] = raw_float<IO>(t == 0 ? hist[W - 1] : raw_get<IO>(p.x, xbase + t));
    float acc = bias;
#pragma unroll
    for (int k = 0; k < W; ++k) acc = fmaf(w[k], win[k], acc);
    if (p.silu) acc = silu_f(acc);
    store_one<IO>(p.out, xbase + t, acc);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) win[k] = win[k + 1];
  }

  if (p.cache_seqlens) {
    for (int64_t t = 0; t < L; ++t)
      raw_put<IO>(p.state, sbase + ring_slot(pos + t, S), raw_get<IO>(p.x, xbase + t));
  } else if (S == W - 1 && L == 1) {
    // one new token into a cache of exactly the window: the new cache is the
    // window's last W-1 inputs, already in registers
#pragma unroll
    for (int k = 0; k < W - 1; ++k) raw_put<IO>(p.state, sbase + k, hist[k + 1]);
  } else {
    // the last S inputs of (cache, x); ascending, so every cache entry is read
    // before its slot is overwritten
    for (int64_t j = 0; j < S; ++j) {
      const int64_t src = j + L;
      const uint32_t v = src < S ? raw_get<IO>(p.state, sbase + src) : raw_get<IO>(p.x, xbase + src - S);
      raw_put<IO>(p.state, sbase + j, v);
    }
  }
}

int64_t pow2ceil64(int64_t v) {
  int64_t r = 1;
  while (r < v) r <<= 1;
  return r;
}

template <int IO>
void launch_state_update(int nsw, dim3 grid, hipStream_t s, const StateUpdateParams &p) {
  if (nsw == 4) hipLaunchKernelGGL((state_update_kernel<IO, 4>), grid, dim3(256), 0, s, p);
  else if (nsw == 2) hipLaunchKernelGGL((state_update_kernel<IO, 2>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((state_update_kernel<IO, 1>), grid, dim3(256), 0, s, p);
}

template <int IO>
void launch_conv_update(int width, dim3 grid, hipStream_t s, const ConvUpdateParams &p) {
  if (width == 4) hipLaunchKernelGGL((conv_update_kernel<IO, 4>), grid, dim3(256), 0, s, p);
  else if (width == 3) hipLaunchKernelGGL((conv_update_kernel<IO, 3>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((conv_update_kernel<IO, 2>), grid, dim3(256), 0, s, p);
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssm_state_update(const ssm_state_update_args_t *a, void *stream_ptr) {
  const int st = ssm_state_update_validate(a);
  if (st != SSM_OK) return st;
  StateUpdateParams p{};
  p.state = a->state; p.x = a->x; p.dt = a->dt; p.B = a->B; p.C = a->C; p.z = a->z;
  p.A = a->A; p.D = a->D; p.dt_bias = a->dt_bias; p.out = a->out;
  p.dim = a->dim;
  p.ngroups = a->ngroups;
  if (a->dim > 0x7fffffffLL) return SSM_ERR_SHAPE;
  p.per_group = static_cast<uint32_t>(a->dim / a->ngroups);
  const int64_t dblocks = (a->dim + kSuChannels - 1) / kSuChannels;
  p.dblocks = static_cast<uint32_t>(dblocks);
  p.n = static_cast<int>(a->dstate);
  p.softplus = a->dt_softplus;
  const int np = static_cast<int>(pow2ceil64(a->dstate < 4 ? 4 : a->dstate));
  const int nsw = np / 4;
  // vector state/A rows: every lane's NSW states are whole and aligned
  p.vec = (a->dstate == np) && aligned16(a->state) && aligned16(a->A);
  // B/C as four io elements per lane in one load (dstate 16)
  p.bcvec = (a->dstate == np) && aligned16(a->B) && aligned16(a->C);
  const int64_t blocks = a->batch * dblocks;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a->io_dtype == SSM_BF16) launch_state_update<1>(nsw, grid, stream, p);
  else if (a->io_dtype == SSM_F16) launch_state_update<2>(nsw, grid, stream, p);
  else launch_state_update<0>(nsw, grid, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

extern "C" int causal_conv1d_update(const void *x, void *conv_state, const float *weight,
                                    const float *bias, const int32_t *cache_seqlens, void *out,
                                    int64_t batch, int64_t dim, int64_t seqlen, int64_t state_len,
                                    int32_t width, int32_t io_dtype, int32_t act, void *stream_ptr) {
  const int st = causal_conv1d_update_validate(x, conv_state, weight, out, batch, dim, seqlen,
                                               state_len, width, io_dtype, act);
  if (st != SSM_OK) return st;
  ConvUpdateParams p{};
  p.x = x; p.state = conv_state; p.w = weight; p.bias = bias; p.cache_seqlens = cache_seqlens;
  p.out = out; p.dim = dim; p.seqlen = seqlen; p.state_len = state_len;
  p.silu = act == SSM_ACT_SILU;
  const int64_t dblocks = (dim + 255) / 256;
  p.dblocks = static_cast<uint32_t>(dblocks);
  const int64_t blocks = batch * dblocks;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (io_dtype == SSM_BF16) launch_conv_update<1>(width, grid, stream, p);
  else if (io_dtype == SSM_F16) launch_conv_update<2>(width, grid, stream, p);
  else launch_conv_update<0>(width, grid, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
