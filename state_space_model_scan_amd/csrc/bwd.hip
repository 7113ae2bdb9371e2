// bwd.hip -- the selective-scan backward (ssm_scan_bwd) for gfx950.
//
// Operation: the gradient of the selective-scan forward (PaddleNLP Kernel
// operator-library guide, section 4.1: the operator's backward is the
// extension's bwd entry, and last_state carries no gradient).  With
// g_t = dout_t * silu(z_t) and h_t = dL/dx_t, the adjoint of
// x_t = a_t x_{t-1} + delta'_t B_t u_t (a_t = exp(delta'_t A)) runs in
// reverse time, h_t = g_t C_t + a_{t+1} h_{t+1}; include/ssmscan.h writes out
// every gradient that follows from it.
//
// Work decomposition.  A channel (b, d) is one 16-lane row of a wave; lane s
// of the row owns state s (dstate <= 16, padded states are inert zeros), so
// a wave holds 4 channels and a 512-thread workgroup 32 channels of one
// (batch, group).  The sequence is walked in chunks of SSM_CKPT_INTERVAL = 32
// timesteps from the last to the first:
//   * per chunk every row re-runs the forward recurrence from the state the
//     forward saved at the chunk's start, keeping x_{t-1} and a_t of each
//     timestep in registers (64 VGPRs), then walks the chunk backwards;
//   * the per-(channel, timestep) scalars -- delta', delta'*u, g, u -- are
//     computed once by the lane that owns the timestep (lane j of a row owns
//     timesteps j and j+16) and handed to the row through a small per-wave
//     LDS array read 4 timesteps per vector load;
//   * sums over the states (y for dz; sum_s h B and the delta' gradient) go
//     through a per-wave LDS transpose in batches of 8 timesteps and are
//     finished by the owning lanes, which also store du, ddelta and dz;
//   * dB/dC of time-varying B/C are sums over every channel of the group:
//     the wave folds its 4 rows with the gfx950 row-swap instructions
//     (v_permlane32_swap, v_permlane16_swap) so that each lane ends with one
//     (state, timestep) value, adds it to the workgroup's LDS accumulator of
//     the chunk (an LDS atomic: the 8 waves' terms land in arrival order, so
//     dB/dC may differ between runs by rounding), and after the chunk's
//     barrier the workgroup writes its partial sums; a second kernel adds the
//     workgroups' partials in a fixed order;
//   * dA, fixed-B/C gradients, dD and d(delta_bias) are accumulated per lane
//     over the whole sequence and written as per-batch partials, summed over
//     the batch by the same second kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "host_util.h"
#include "ssmscan.h"

namespace ssm {
namespace {

constexpr int kT = SSM_CKPT_INTERVAL;   // timesteps per chunk (= checkpoint spacing)
constexpr int kWaves = 8;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kCPW = 4;                 // channels per wave (one 16-lane row each)
constexpr int kCPB = kWaves * kCPW;     // channels per workgroup
constexpr int kNP = 16;                 // lanes (states) per channel
constexpr int kRow = 36;                // padded LDS row, in floats
constexpr int kRB = 8;                  // timesteps per reduction batch
static_assert(kT == 32, "the chunk layout assumes 32 timesteps");

struct BwdParams {
  const void *u, *delta, *B, *C, *z, *dout;
  const float *A, *D, *dbias, *ckpt;
  void *du, *ddelta, *dz;
  float *pB, *pC;       // partial dB/dC: varying (b*g, nblk, n, l); fixed (b, d, n)
  float *pA;            // (b, d, n)
  float *pD, *pbias;    // (b, d)
  float *dinit;         // (b, d, n) or null
  int64_t dim, seqlen, cpg;
  int n, ngroups, nblk, nck, softplus;
};

__device__ __forceinline__ float sigmoid_f(float v) { return fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }

// v_permlane32_swap: lanes 32..63 of x trade places with lanes 0..31 of y.
__device__ __forceinline__ void swap32(float &x, float &y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
// v_permlane16_swap: rows 1 and 3 of x trade places with rows 0 and 2 of y.
__device__ __forceinline__ void swap16(float &x, float &y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

__device__ __forceinline__ void lds_add(float *p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// LDS handoff between the lanes of one wave (see scan_kernel.h).
__device__ __forceinline__ void wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <bool BF16, bool BV, bool CV>
__global__ void __launch_bounds__(kThreads) scan_bwd_kernel(const BwdParams p) {
  constexpr bool ANYV = BV || CV;
  __shared__ __align__(16) float s_bc[2][2][kNP][kRow];               // B/C tiles, double-buffered
  __shared__ __align__(16) float s_acc[ANYV ? 2 : 1][2][kNP][kT];     // dB/dC of a chunk, double-buffered
  __shared__ __align__(16) float s_cast[kWaves][4][kCPW][kT];         // delta', delta'*u, g, u
  __shared__ __align__(16) float s_red[kWaves][kCPW][kRB][kRow];      // state-sum transpose

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane >> 4, s = lane & 15;
  const int n = p.n;
  const bool sv = s < n;
  const int64_t L = p.seqlen;

  const int blk = blockIdx.x % p.nblk;
  const int bg = blockIdx.x / p.nblk;          // b * ngroups + g
  const int g = bg % p.ngroups;
  const int64_t b = bg / p.ngroups;
  const int64_t lc = static_cast<int64_t>(blk) * kCPB + w * kCPW + c;   // channel within the group
  const bool valid = lc < p.cpg;
  const int64_t dl = g * p.cpg + (valid ? lc : p.cpg - 1);
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * L;
  const int64_t bc_base = static_cast<int64_t>(bg) * n * L;

  const float Av = sv ? p.A[dl * n + s] : 0.0f;
  const float Ap = Av * kLog2e;
  const float Bf = (!BV && sv) ? load_io<BF16>(p.B, dl * n + s) : 0.0f;
  const float Cf = (!CV && sv) ? load_io<BF16>(p.C, dl * n + s) : 0.0f;
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;
  const float Dd = p.D ? p.D[dl] : 0.0f;
  const bool hz = p.z != nullptr;

  // ---- B/C tile of a chunk: thread -> (tensor, state, 2 timesteps)
  const int tq = tid >> 8;
  const int ts = (tid >> 4) & 15;
  const int tt = (tid & 15) * 2;
  const bool t_on = (tq == 0 ? BV : CV) && ts < n;
  float tile0 = 0.0f, tile1 = 0.0f;
  auto fetch_tile = [&](int ci) {
    tile0 = tile1 = 0.0f;
    if (t_on) {
      const int64_t t0 = static_cast<int64_t>(ci) * kT + tt;
      const void *src = tq == 0 ? p.B : p.C;
      const int64_t e = bc_base + ts * L + t0;
      if (t0 < L) tile0 = load_io<BF16>(src, e);
      if (t0 + 1 < L) tile1 = load_io<BF16>(src, e + 1);
    }
  };
  auto store_tile = [&](int buf) {
    *reinterpret_cast<float2 *>(&s_bc[buf][tq][ts][tt]) = make_float2(tile0, tile1);
  };

  // ---- running state of this lane
  float gcar = 0.0f;                          // h carried into the next-earlier timestep
  float dA_acc = 0.0f, dBf_acc = 0.0f, dCf_acc = 0.0f;
  float accD = 0.0f, accBias = 0.0f;          // owner sums over its timesteps

  fetch_tile(p.nck - 1);
  store_tile(0);
  if constexpr (ANYV) {
    for (int i = tid; i < 2 * 2 * kNP * kT; i += kThreads) (&s_acc[0][0][0][0])[i] = 0.0f;
  }
  __syncthreads();

  for (int k = 0; k < p.nck; ++k) {
    const int ci = p.nck - 1 - k;
    const int kb = k & 1;
    const int64_t t0 = static_cast<int64_t>(ci) * kT;
    const int len = static_cast<int>((L - t0 < kT) ? L - t0 : kT);

    // state at the chunk's start, and the next-earlier chunk's B/C tile
    const float xck = sv ? p.ckpt[(row * p.nck + ci) * n + s] : 0.0f;
    if (ci > 0) fetch_tile(ci - 1);

    // ---- owner prologue: timesteps s and s + 16 of this row
    float o_u[2], o_dout[2], o_dsp[2], o_z[2], o_dt[2], o_g[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = s + 16 * h;
      const bool on = valid && t < len;
      const int64_t e = rbase + t0 + t;
      float uu = 0.0f, dd = 0.0f, zz = 0.0f, go = 0.0f;
      if (on) {
        uu = load_io<BF16>(p.u, e);
        dd = load_io<BF16>(p.delta, e);
        go = load_io<BF16>(p.dout, e);
        if (hz) zz = load_io<BF16>(p.z, e);
      }
      const float raw = dd + bias;
      float dt = p.softplus ? softplus_f(raw) : raw;
      const float dsp = p.softplus ? sigmoid_f(raw) : 1.0f;
      const float gate = hz ? silu_f(zz) : 1.0f;
      float gg = go * gate;
      if (!on) { dt = 0.0f; gg = 0.0f; uu = 0.0f; }   // inert timestep
      o_u[h] = uu; o_dout[h] = go; o_dsp[h] = dsp; o_z[h] = zz; o_dt[h] = dt; o_g[h] = gg;
      s_cast[w][0][c][t] = dt;
      s_cast[w][1][c][t] = dt * uu;
      s_cast[w][2][c][t] = gg;
      s_cast[w][3][c][t] = uu;
    }
    wave_sync();

    const float(*bt)[kRow] = s_bc[kb][0];
    const float(*ct)[kRow] = s_bc[kb][1];

    // ---- forward re-run of the chunk
    float xs[kT], as[kT];
    float x = xck;
    float Y[2] = {0.0f, 0.0f};
#pragma unroll
    for (int t4 = 0; t4 < kT; t4 += 4) {
      const float4 dt4 = *reinterpret_cast<const float4 *>(&s_cast[w][0][c][t4]);
      const float4 du4 = *reinterpret_cast<const float4 *>(&s_cast[w][1][c][t4]);
      float4 B4 = make_float4(Bf, Bf, Bf, Bf), C4 = make_float4(Cf, Cf, Cf, Cf);
      if constexpr (BV) B4 = *reinterpret_cast<const float4 *>(&bt[s][t4]);
      if constexpr (CV) { if (hz) C4 = *reinterpret_cast<const float4 *>(&ct[s][t4]); }
      const float dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
      const float duv[4] = {du4.x, du4.y, du4.z, du4.w};
      const float Bv[4] = {B4.x, B4.y, B4.z, B4.w};
      const float Cv[4] = {C4.x, C4.y, C4.z, C4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t4 + i;
        const float a = fast_exp2(dtv[i] * Ap);
        xs[t] = x;
        as[t] = a;
        x = fmaf(a, x, duv[i] * Bv[i]);
        if (hz) s_red[w][c][t % kRB][s] = Cv[i] * x;
      }
      if (hz && (t4 % kRB) == kRB - 4) {
        // y of the batch's 8 timesteps, summed by their owners
        wave_sync();
        const int tb = t4 / kRB;
        if ((s >> 3) == (tb & 1)) {
          const float4 *r = reinterpret_cast<const float4 *>(&s_red[w][c][s & 7][0]);
          const float4 r0 = r[0], r1 = r[1], r2 = r[2], r3 = r[3];
          Y[tb >> 1] = ((r0.x + r0.y) + (r0.z + r0.w)) + ((r1.x + r1.y) + (r1.z + r1.w)) +
                       ((r2.x + r2.y) + (r2.z + r2.w)) + ((r3.x + r3.y) + (r3.z + r3.w));
        }
        wave_sync();
      }
    }
    const float x_end = x;

    // ---- dz (needs only the forward)
    if (hz) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = s + 16 * h;
        if (valid && t < len) {
          const float pre = Y[h] + Dd * o_u[h];
          const float sg = sigmoid_f(o_z[h]);
          const float dsilu = sg * (1.0f + o_z[h] * (1.0f - sg));
          store_one<BF16>(p.dz, rbase + t0 + t, o_dout[h] * pre * dsilu);
        }
      }
    }

    // ---- reverse walk of the chunk
    float pb_hi = 0.0f, pc_hi = 0.0f;   // dB/dC values of the odd timestep of a pair
    float4 dt4, du4, g4, u4, B4, C4;
#pragma unroll
    for (int t = kT - 1; t >= 0; --t) {
      const int i = t & 3;
      if (i == 3) {
        const int t4 = t - 3;
        dt4 = *reinterpret_cast<const float4 *>(&s_cast[w][0][c][t4]);
        du4 = *reinterpret_cast<const float4 *>(&s_cast[w][1][c][t4]);
        g4 = *reinterpret_cast<const float4 *>(&s_cast[w][2][c][t4]);
        u4 = *reinterpret_cast<const float4 *>(&s_cast[w][3][c][t4]);
        B4 = make_float4(Bf, Bf, Bf, Bf);
        C4 = make_float4(Cf, Cf, Cf, Cf);
        if constexpr (BV) B4 = *reinterpret_cast<const float4 *>(&bt[s][t4]);
        if constexpr (CV) C4 = *reinterpret_cast<const float4 *>(&ct[s][t4]);
      }
      const float dt = i == 0 ? dt4.x : i == 1 ? dt4.y : i == 2 ? dt4.z : dt4.w;
      const float dtu = i == 0 ? du4.x : i == 1 ? du4.y : i == 2 ? du4.z : du4.w;
      const float gg = i == 0 ? g4.x : i == 1 ? g4.y : i == 2 ? g4.z : g4.w;
      const float uu = i == 0 ? u4.x : i == 1 ? u4.y : i == 2 ? u4.z : u4.w;
      const float Bv = i == 0 ? B4.x : i == 1 ? B4.y : i == 2 ? B4.z : B4.w;
      const float Cv = i == 0 ? C4.x : i == 1 ? C4.y : i == 2 ? C4.z : C4.w;
      const float a = as[t];
      const float xp = xs[t];
      const float xt = t + 1 < kT ? xs[t + 1] : x_end;

      const float h = fmaf(gg, Cv, gcar);
      const float hax = h * (a * xp);
      dA_acc = fmaf(hax, dt, dA_acc);
      const float hB = h * Bv;
      const float q = fmaf(Av, hax, uu * hB);
      *reinterpret_cast<float2 *>(&s_red[w][c][t % kRB][2 * s]) = make_float2(hB, q);
      gcar = h * a;

      float vb = 0.0f, vc = 0.0f;
      if constexpr (BV) vb = h * dtu; else dBf_acc = fmaf(h, dtu, dBf_acc);
      if constexpr (CV) vc = gg * xt; else dCf_acc = fmaf(gg, xt, dCf_acc);
      if constexpr (ANYV) {
        if (t & 1) {
          pb_hi = vb;
          pc_hi = vc;
        } else {
          // fold the wave's 4 rows: rows of r1 / r2 after the 32-swap are
          // [dB(c0+c2), dB(c1+c3), dC(c0+c2), dC(c1+c3)] of timesteps t+1 / t
          float xa = pb_hi, ya = pc_hi;
          swap32(xa, ya);
          float r1 = xa + ya;
          float xb = vb, yb = vc;
          swap32(xb, yb);
          float r2 = xb + yb;
          swap16(r1, r2);
          const float v = r1 + r2;   // rows: dB(t+1), dB(t), dC(t+1), dC(t)
          const int rw = lane >> 4;
          lds_add(&s_acc[kb][rw >> 1][s][t + 1 - (rw & 1)], v);
        }
      }

      if ((t % kRB) == 0) {
        // sum over states of the batch [t, t+8): owners finish du, ddelta
        wave_sync();
        const int tb = t / kRB;
        if ((s >> 3) == (tb & 1)) {
          const int hh = tb >> 1;
          const int to = s + 16 * hh;
          const float4 *r = reinterpret_cast<const float4 *>(&s_red[w][c][s & 7][0]);
          float S1 = 0.0f, Q = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float4 v = r[j];
            S1 += v.x + v.z;
            Q += v.y + v.w;
          }
          if (valid && to < len) {
            const float ddl = Q * o_dsp[hh];
            store_one<BF16>(p.du, rbase + t0 + to, fmaf(o_dt[hh], S1, Dd * o_g[hh]));
            store_one<BF16>(p.ddelta, rbase + t0 + to, ddl);
            accD = fmaf(o_g[hh], o_u[hh], accD);
            accBias += ddl;
          }
        }
        wave_sync();
      }
    }

    // next tile into the other buffer; after the barrier the chunk's dB/dC
    // accumulator is complete
    if (ci > 0) store_tile(kb ^ 1);
    __syncthreads();
    if constexpr (ANYV) {
      const int fq = tid >> 8;
      const int fs = (tid >> 4) & 15;
      const int ft = (tid & 15) * 2;
      float *acc = &s_acc[kb][fq][fs][ft];
      const float v0 = acc[0], v1 = acc[1];
      acc[0] = 0.0f;
      acc[1] = 0.0f;
      if ((fq == 0 ? BV : CV) && fs < n) {
        float *dst = (fq == 0 ? p.pB : p.pC) + ((static_cast<int64_t>(bg) * p.nblk + blk) * n + fs) * L + t0 + ft;
        if (ft < len) dst[0] = v0;
        if (ft + 1 < len) dst[1] = v1;
      }
    }
  }

  // ---- per-lane results over the whole sequence
  if (valid && sv) {
    if (p.dinit) p.dinit[row * n + s] = gcar;
    p.pA[row * n + s] = dA_acc;
    if constexpr (!BV) p.pB[row * n + s] = dBf_acc;
    if constexpr (!CV) p.pC[row * n + s] = dCf_acc;
  }
  // owner sums over the row's 16 lanes
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    accD += __shfl_xor(accD, m, 16);
    accBias += __shfl_xor(accBias, m, 16);
  }
  if (valid && s == 0) {
    if (p.pD) p.pD[row] = accD;
    if (p.pbias) p.pbias[row] = accBias;
  }
}

// out[i, j] = sum_k in[i, k, j] for an (I, K, J) array, k in increasing order.
__global__ void __launch_bounds__(256) sum_mid_kernel(const float *in, float *out, int64_t I, int64_t K,
                                                      int64_t J) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= I * J) return;
  const int64_t i = e / J, j = e - i * J;
  const float *src = in + i * K * J + j;
  float acc = 0.0f;
  for (int64_t k = 0; k < K; ++k) acc += src[k * J];
  out[e] = acc;
}

using BwdFn = void (*)(const BwdParams);

template <bool BF16>
BwdFn pick_bwd(bool bv, bool cv) {
  if (bv && cv) return scan_bwd_kernel<BF16, true, true>;
  if (bv) return scan_bwd_kernel<BF16, true, false>;
  if (cv) return scan_bwd_kernel<BF16, false, true>;
  return scan_bwd_kernel<BF16, false, false>;
}

struct BwdPlan {
  int64_t cpg, nblk, nck, blocks;
  size_t nB, nC, nA, nD;   // partial element counts
  size_t bytes;
};

BwdPlan plan_bwd(const ssm_scan_bwd_args_t *a) {
  BwdPlan pl{};
  pl.cpg = a->dim / a->ngroups;
  pl.nblk = (pl.cpg + kCPB - 1) / kCPB;
  pl.nck = (a->seqlen + kT - 1) / kT;
  pl.blocks = a->batch * a->ngroups * pl.nblk;
  const size_t bgn = static_cast<size_t>(a->batch * a->ngroups) * pl.nblk * a->dstate * a->seqlen;
  const size_t bdn = static_cast<size_t>(a->batch * a->dim * a->dstate);
  pl.nB = a->B_kind == SSM_BC_VARYING ? bgn : bdn;
  pl.nC = a->C_kind == SSM_BC_VARYING ? bgn : bdn;
  pl.nA = bdn;
  pl.nD = static_cast<size_t>(a->batch * a->dim);
  // every partial array starts on a 256-byte boundary
  auto up = [](size_t e) { return (e * sizeof(float) + 255) / 256 * 256; };
  pl.bytes = up(pl.nB) + up(pl.nC) + up(pl.nA) + 2 * up(pl.nD);
  return pl;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args_t *a, size_t *bytes) {
  const int st = ssm_scan_bwd_validate(a);
  if (st != SSM_OK) return st;
  if (!bytes) return SSM_ERR_NULL;
  *bytes = plan_bwd(a).bytes;
  return SSM_OK;
}

extern "C" int ssm_scan_bwd(const ssm_scan_bwd_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_bwd_validate(a);
  if (st != SSM_OK) return st;
  const BwdPlan pl = plan_bwd(a);
  if (pl.blocks > 0x7fffffffLL || static_cast<int64_t>(pl.nB / 256) > 0x7fffffffLL) return SSM_ERR_SHAPE;
  if (a->workspace && a->workspace_bytes < pl.bytes) return SSM_ERR_WORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool bf16 = a->io_dtype == SSM_BF16;
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;

  void *ws = a->workspace;
  bool owned = false;
  if (!ws) {
    const hipError_t e = hipMallocAsync(&ws, pl.bytes, stream);
    if (e != hipSuccess) return hip_fail(e);
    owned = true;
  }
  char *base = static_cast<char *>(ws);
  auto take = [&](size_t elems) {
    float *r = reinterpret_cast<float *>(base);
    base += (elems * sizeof(float) + 255) / 256 * 256;
    return r;
  };
  BwdParams p{};
  p.u = a->u; p.delta = a->delta; p.B = a->B; p.C = a->C; p.z = a->z; p.dout = a->dout;
  p.A = a->A; p.D = a->D; p.dbias = a->delta_bias; p.ckpt = a->checkpoints;
  p.du = a->du; p.ddelta = a->ddelta; p.dz = a->dz;
  p.pB = take(pl.nB);
  p.pC = take(pl.nC);
  p.pA = take(pl.nA);
  float *pd = take(pl.nD), *pbias = take(pl.nD);
  p.pD = a->D ? pd : nullptr;
  p.pbias = a->delta_bias ? pbias : nullptr;
  p.dinit = a->dinitial_state;
  p.dim = a->dim; p.seqlen = a->seqlen; p.cpg = pl.cpg;
  p.n = static_cast<int>(a->dstate); p.ngroups = static_cast<int>(a->ngroups);
  p.nblk = static_cast<int>(pl.nblk); p.nck = static_cast<int>(pl.nck);
  p.softplus = a->delta_softplus;

  const BwdFn f = bf16 ? pick_bwd<true>(bv, cv) : pick_bwd<false>(bv, cv);
  hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(pl.blocks)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();

  auto reduce = [&](const float *in, float *out, int64_t I, int64_t K, int64_t J) {
    if (e != hipSuccess) return;
    const dim3 grid(static_cast<unsigned>((I * J + 255) / 256));
    hipLaunchKernelGGL(sum_mid_kernel, grid, dim3(256), 0, stream, in, out, I, K, J);
    e = hipGetLastError();
  };
  const int64_t bsz = a->batch, n = a->dstate, L = a->seqlen, dim = a->dim;
  if (bv) reduce(p.pB, a->dB, bsz * a->ngroups, pl.nblk, n * L);
  else reduce(p.pB, a->dB, 1, bsz, dim * n);
  if (cv) reduce(p.pC, a->dC, bsz * a->ngroups, pl.nblk, n * L);
  else reduce(p.pC, a->dC, 1, bsz, dim * n);
  reduce(p.pA, a->dA, 1, bsz, dim * n);
  if (a->D) reduce(p.pD, a->dD, 1, bsz, dim);
  if (a->delta_bias) reduce(p.pbias, a->ddelta_bias, 1, bsz, dim);

  if (owned) {
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
  }
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
