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
// a wave holds 4 channels and a 768-thread workgroup (3 waves per SIMD) 48
// channels of one (batch, group).  The sequence is walked in chunks of
// SSM_CKPT_INTERVAL = 32 timesteps from the last to the first:
//   * per chunk every row re-runs the forward recurrence from the state the
//     forward saved at the chunk's start, keeping x_{t-1} of each timestep in
//     registers (32 VGPRs), then walks the chunk backwards, recomputing the
//     decay a_t = exp(delta'_t A) (cheaper than 32 more live registers);
//   * the owned timesteps' inputs and the checkpoint of the next chunk are
//     loaded one chunk ahead;
//   * the per-(channel, timestep) scalars -- delta', delta'*u, g, u -- are
//     computed once by the lane that owns the timestep (lane j of a row owns
//     timesteps j and j+16) and stay in its registers; the row reads them by
//     DPP row broadcast (row_newbcast), mostly folded into the multiply that
//     consumes them;
//   * sums over the states (y for dz; sum_s h B and the delta' gradient) are
//     a DPP reduce-scatter over the row in batches of 16 timesteps, which
//     leaves the sum of timestep 16H + j on lane j -- its owner, which
//     stores du, ddelta and dz.  No LDS traffic and no waits inside a chunk
//     apart from the B/C tile reads and the dB/dC accumulator;
//   * dB/dC of time-varying B/C are sums over every channel of the group:
//     the wave folds its 4 rows with the gfx950 row-swap instructions
//     (v_permlane32_swap, v_permlane16_swap) so that each lane ends with one
//     (state, timestep) value, and stores it to the wave's own LDS slot of
//     the chunk; after the chunk's barrier the workgroup adds its waves'
//     slots in wave order and writes its partial sums, and a second kernel
//     adds the workgroups' partials in a fixed order (no atomics anywhere:
//     every output is bit-for-bit repeatable; LDS float atomics cost more
//     than half the kernel's time when measured);
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
constexpr int kWaves = 12;              // waves per workgroup (3 per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kCPW = 4;                 // channels per wave (one 16-lane row each)
constexpr int kCPB = kWaves * kCPW;     // channels per workgroup
constexpr int kNP = 16;                 // lanes (states) per channel
constexpr int kRow = 36;                // padded LDS row, in floats
static_assert(kT == 32, "the chunk layout assumes 32 timesteps");

struct BwdParams {
  const void *u, *delta, *B, *C, *z, *dout;
  const float *A, *D, *dbias, *ckpt;
  void *du, *ddelta, *dz;
  float *pB, *pC;       // partial dB/dC: varying (b*g, nblk, n, l); fixed (b, d, n)
  float *pA;            // (b, d, n)
  float *pD, *pbias;    // (b, d)
  float *dinit;         // (b, d, n) or null
  // sequence split: segment k >= 1's carry out of its first timestep with no
  // carry coming in (nseg, b, d, n), and its sum of delta' (nseg, b, d)
  float *loc, *ssum;
  int64_t dim, seqlen, cpg, bd;   // bd = batch * dim
  int n, ngroups, nblk, nck, softplus;
  int segc, nseg;                 // chunks per segment (after the first), segments
  int seg0;                       // chunks of segment 0
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

// One io element as stored (bf16: zero-extended 16 bits), and its value.
template <int IO>
__device__ __forceinline__ uint32_t raw_load(const void *p, int64_t i) {
  if constexpr (IO) return static_cast<const uint16_t *>(p)[i];
  else return static_cast<const uint32_t *>(p)[i];
}
template <int IO>
__device__ __forceinline__ float raw_float(uint32_t r) {
  if constexpr (IO != 0) return half_bits_to_float<IO>(r);
  else return __uint_as_float(r);
}

template <int I>
__device__ __forceinline__ float f4get(const float4 &v) {
  if constexpr (I == 0) return v.x;
  else if constexpr (I == 1) return v.y;
  else if constexpr (I == 2) return v.z;
  else return v.w;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// Lane K of the row broadcast to the row, kept in a register (for operands
// the compiler cannot fold a DPP source into).
template <int K>
__device__ __forceinline__ float bc(float v) { return dpp<0x150 + K>(v); }   // row_newbcast:K
template <int K>
__device__ __forceinline__ float row_bcast_reg(float v) {
  float r = bc<K>(v);
  asm volatile("" : "+v"(r));
  return r;
}

// v[j] is this lane's term for timestep j of a 16-timestep batch; returns the
// sum of v[s] over the row's 16 lanes for s = lane & 15.  Recursive halving:
// each step pairs lanes that differ in one lane bit (8: row_ror:8, 4:
// row_half_mirror, 2 and 1: quad permutes), every lane keeps the half of its
// values its bit selects and adds the partner's copy of that half.  In the
// first two steps the lanes of one half are whole DPP banks (bit 3: banks
// 0-1 / 2-3; bit 2: banks 0,2 / 1,3), so each kept value is two bank-masked
// DPP adds writing one register -- no selects.  The leading s_nop gives the
// two wait states a DPP source read needs after a VALU write.
__device__ __forceinline__ float row_reduce_scatter16(const float (&v)[16], int s) {
  float r8[8], r4[4], r2[2];
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(r8[0]), "=&v"(r8[1]), "=&v"(r8[2]), "=&v"(r8[3]),
        "=&v"(r8[4]), "=&v"(r8[5]), "=&v"(r8[6]), "=&v"(r8[7])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
        "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(r4[0]), "=&v"(r4[1]), "=&v"(r4[2]), "=&v"(r4[3])
      : "v"(r8[0]), "v"(r8[1]), "v"(r8[2]), "v"(r8[3]), "v"(r8[4]), "v"(r8[5]), "v"(r8[6]), "v"(r8[7]));
  const bool b1 = s & 2, b0 = s & 1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b1 ? r4[k + 2] : r4[k], send = b1 ? r4[k] : r4[k + 2];
    r2[k] = keep + dpp<0x4E>(send);           // quad_perm [2,3,0,1]
  }
  const float keep = b0 ? r2[1] : r2[0], send = b0 ? r2[0] : r2[1];
  return keep + dpp<0xB1>(send);              // quad_perm [1,0,3,2]
}

template <int IO, bool BV, bool CV, bool HZ>
__global__ void __launch_bounds__(kThreads, 3) scan_bwd_kernel(const BwdParams p) {
  constexpr bool ANYV = BV || CV;
  __shared__ __align__(16) float s_bc[2][2][kNP][kRow];               // B/C tiles, double-buffered
  // each wave's dB/dC terms of a chunk (its 4 channels summed), double-buffered
  __shared__ float s_slot[ANYV ? 2 : 1][ANYV ? kWaves : 1][2][kNP][kT + 1];

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
  const int seg = blockIdx.y;                  // this workgroup's chunks: [cbeg, cend)
  const int cbeg = seg == 0 ? 0 : p.seg0 + (seg - 1) * p.segc;
  const int clen = seg == 0 ? p.seg0 : p.segc;
  const int cend = cbeg + clen < p.nck ? cbeg + clen : p.nck;
  const int64_t lc = static_cast<int64_t>(blk) * kCPB + w * kCPW + c;   // channel within the group
  const bool valid = lc < p.cpg;
  const int64_t dl = g * p.cpg + (valid ? lc : p.cpg - 1);
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * L;
  const int64_t bc_base = static_cast<int64_t>(bg) * n * L;

  const float Av = sv ? p.A[dl * n + s] : 0.0f;
  const float Ap = Av * kLog2e;
  const float Bf = (!BV && sv) ? load_io<IO>(p.B, dl * n + s) : 0.0f;
  const float Cf = (!CV && sv) ? load_io<IO>(p.C, dl * n + s) : 0.0f;
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;
  const float Dd = p.D ? p.D[dl] : 0.0f;

  // ---- B/C tile of a chunk: thread -> (tensor, state, 2 timesteps)
  const bool t_thr = tid < 2 * kNP * kT / 2;     // 512 threads move a tile, 2 elements each
  const int tq = (tid >> 8) & 1;
  const int ts = (tid >> 4) & 15;
  const int tt = (tid & 15) * 2;
  const bool t_on = t_thr && (tq == 0 ? BV : CV) && ts < n;
  // Loads keep the raw io bits and convert at the point of use, so that no
  // wait for them lands inside the guarded load.
  uint32_t tile0 = 0, tile1 = 0;
  auto fetch_tile = [&](int ci) {
    tile0 = tile1 = 0;
    if (t_on) {
      const int64_t t0 = static_cast<int64_t>(ci) * kT + tt;
      const void *src = tq == 0 ? p.B : p.C;
      const int64_t e = bc_base + ts * L + t0;
      if (t0 < L) tile0 = raw_load<IO>(src, e);
      if (t0 + 1 < L) tile1 = raw_load<IO>(src, e + 1);
    }
  };
  auto store_tile = [&](int buf) {
    if (t_thr)
      *reinterpret_cast<float2 *>(&s_bc[buf][tq][ts][tt]) = make_float2(raw_float<IO>(tile0), raw_float<IO>(tile1));
  };

  // ---- running state of this lane
  float gcar = 0.0f;                          // h carried into the next-earlier timestep
  if (seg + 1 < p.nseg && sv) {
    // carry into this segment: the later segments' own carries, each scaled
    // by the decay of the segments between (exp2(A' * sum of delta'))
    for (int k = p.nseg - 1; k > seg; --k) {
      const int64_t r = static_cast<int64_t>(k) * p.bd + row;
      gcar = fmaf(fast_exp2(Ap * p.ssum[r]), gcar, p.loc[r * n + s]);
    }
  }
  float dA_acc = 0.0f, dBf_acc = 0.0f, dCf_acc = 0.0f;
  float accD = 0.0f, accBias = 0.0f;          // owner sums over its timesteps

  // this lane's two owned timesteps (s, s + 16) of a chunk, and the lane's
  // checkpoint: loaded one chunk ahead of their use
  uint32_t r_u[2], r_d[2], r_go[2], r_z[2];
  float r_x;
  auto fetch_own = [&](int ci) {
    const int64_t t0 = static_cast<int64_t>(ci) * kT;
    r_x = 0.0f;
    if (sv) r_x = p.ckpt[(row * p.nck + ci) * n + s];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t t = t0 + s + 16 * h;
      r_u[h] = r_d[h] = r_go[h] = r_z[h] = 0;
      if (valid && t < L) {
        r_u[h] = raw_load<IO>(p.u, rbase + t);
        r_d[h] = raw_load<IO>(p.delta, rbase + t);
        r_go[h] = raw_load<IO>(p.dout, rbase + t);
        if constexpr (HZ) r_z[h] = raw_load<IO>(p.z, rbase + t);
      }
    }
  };

  fetch_own(cend - 1);
  fetch_tile(cend - 1);
  store_tile(0);
  __syncthreads();

  for (int k = 0; k < cend - cbeg; ++k) {
    const int ci = cend - 1 - k;
    const int kb = k & 1;
    const int64_t t0 = static_cast<int64_t>(ci) * kT;
    const int len = static_cast<int>((L - t0 < kT) ? L - t0 : kT);

    // this chunk's owned inputs and checkpoint (loaded during the previous
    // chunk); then the next-earlier chunk's loads
    const float xck = r_x;
    float c_u[2], c_d[2], c_go[2], c_z[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      c_u[h] = raw_float<IO>(r_u[h]);
      c_d[h] = raw_float<IO>(r_d[h]);
      c_go[h] = raw_float<IO>(r_go[h]);
      c_z[h] = raw_float<IO>(r_z[h]);
    }
    if (ci > cbeg) {
      fetch_own(ci - 1);
      fetch_tile(ci - 1);
    }

    // ---- owner prologue: timesteps s and s + 16 of this row.  The results
    // stay in the owner's registers; the row reads them by DPP broadcast.
    float o_dt[2], o_dtu[2], o_g[2], o_u[2], o_dsp[2], o_dzf[2], o_Du[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = s + 16 * h;
      const bool on = valid && t < len;
      float uu = c_u[h];
      const float dd = c_d[h], go = c_go[h], zz = c_z[h];
      const float raw = dd + bias;
      float dt = p.softplus ? softplus_f(raw) : raw;
      const float dsp = p.softplus ? sigmoid_f(raw) : 1.0f;
      float gg = go;
      if constexpr (HZ) {
        const float sg = sigmoid_f(zz);
        gg = go * zz * sg;                                  // dout * silu(z)
        o_dzf[h] = go * sg * (1.0f + zz * (1.0f - sg));     // dout * silu'(z)
      }
      if (!on) { dt = 0.0f; gg = 0.0f; uu = 0.0f; }   // inert timestep
      o_dt[h] = dt;
      o_dtu[h] = dt * uu;
      o_g[h] = gg;
      o_u[h] = uu;
      o_dsp[h] = dsp;
      o_Du[h] = Dd * uu;
      accD = fmaf(gg, uu, accD);
    }

    const float(*bt)[kRow] = s_bc[kb][0];
    const float(*ct)[kRow] = s_bc[kb][1];

    // ---- forward re-run of the chunk
    float xs[kT];
    float x = xck;
    float Y[2] = {0.0f, 0.0f};
    float cx[16];
    float4 B4, C4;
    static_for(std::make_integer_sequence<int, kT>{}, [&](auto TT) {
      constexpr int t = decltype(TT)::value;
      constexpr int K = t & 15, H = t >> 4;
      if constexpr ((t & 3) == 0) {
        B4 = make_float4(Bf, Bf, Bf, Bf);
        C4 = make_float4(Cf, Cf, Cf, Cf);
        if constexpr (BV) B4 = *reinterpret_cast<const float4 *>(&bt[s][t]);
        if constexpr (CV && HZ) C4 = *reinterpret_cast<const float4 *>(&ct[s][t]);
      }
      const float Bv = f4get<t & 3>(B4), Cv = f4get<t & 3>(C4);
      const float a = fast_exp2(bc<K>(o_dt[H]) * Ap);
      xs[t] = x;
      x = fmaf(a, x, bc<K>(o_dtu[H]) * Bv);
      if constexpr (HZ) {
        cx[K] = Cv * x;
        if constexpr (K == 15) Y[H] = row_reduce_scatter16(cx, s);   // y of timestep 16H + s
      }
      if constexpr ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    });
    const float x_end = x;

    // ---- dz (needs only the forward)
    if constexpr (HZ) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = s + 16 * h;
        if (valid && t < len) store_one<IO>(p.dz, rbase + t0 + t, o_dzf[h] * (Y[h] + o_Du[h]));
      }
    }

    // ---- reverse walk of the chunk
    float pb_hi = 0.0f, pc_hi = 0.0f;   // dB/dC values of the odd timestep of a pair
    float hb[16], qv[16];
    static_for(std::make_integer_sequence<int, kT>{}, [&](auto RR) {
      constexpr int t = kT - 1 - decltype(RR)::value;
      constexpr int K = t & 15, H = t >> 4;
      if constexpr ((t & 3) == 3) {
        B4 = make_float4(Bf, Bf, Bf, Bf);
        C4 = make_float4(Cf, Cf, Cf, Cf);
        if constexpr (BV) B4 = *reinterpret_cast<const float4 *>(&bt[s][t - 3]);
        if constexpr (CV) C4 = *reinterpret_cast<const float4 *>(&ct[s][t - 3]);
      }
      const float Bv = f4get<t & 3>(B4), Cv = f4get<t & 3>(C4);
      const float dt = row_bcast_reg<K>(o_dt[H]);
      const float gg = row_bcast_reg<K>(o_g[H]);
      const float a = fast_exp2(dt * Ap);
      const float xp = xs[t];
      const float xt = t + 1 < kT ? xs[t + 1] : x_end;

      const float h = fmaf(gg, Cv, gcar);
      const float hax = h * (a * xp);
      dA_acc = fmaf(hax, dt, dA_acc);
      const float hB = h * Bv;
      hb[K] = hB;
      qv[K] = fmaf(Av, hax, bc<K>(o_u[H]) * hB);
      gcar = h * a;

      float vb = 0.0f, vc = 0.0f;
      // the empty asm keeps each fixed-B/C sum in step with the walk; left
      // free, the scheduler holds the chunk's products live and spills
      if constexpr (BV) {
        vb = h * bc<K>(o_dtu[H]);
      } else {
        dBf_acc = fmaf(h, bc<K>(o_dtu[H]), dBf_acc);
        asm volatile("" : "+v"(dBf_acc));
      }
      if constexpr (CV) {
        vc = gg * xt;
      } else {
        dCf_acc = fmaf(gg, xt, dCf_acc);
        asm volatile("" : "+v"(dCf_acc));
      }
      if constexpr (ANYV) {
        if constexpr (t & 1) {
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
          s_slot[kb][w][rw >> 1][s][t + 1 - (rw & 1)] = v;
        }
      }

      if constexpr (K == 0) {
        // sums over the states of timesteps [16H, 16H+16): lane s gets 16H + s
        const float S1 = row_reduce_scatter16(hb, s);
        const float Q = row_reduce_scatter16(qv, s);
        const int to = s + 16 * H;
        if (valid && to < len) {
          const float ddl = Q * o_dsp[H];
          store_one<IO>(p.du, rbase + t0 + to, fmaf(o_dt[H], S1, Dd * o_g[H]));
          store_one<IO>(p.ddelta, rbase + t0 + to, ddl);
          accBias += ddl;
        }
      }
      if constexpr ((t & 3) == 0) __builtin_amdgcn_sched_barrier(0);
    });

    // next tile into the other buffer; after the barrier the chunk's dB/dC
    // accumulator is complete
    if (ci > cbeg) store_tile(kb ^ 1);
    __syncthreads();
    if (ANYV && t_thr) {
      // the workgroup's sum: its waves' slots added in wave order
      const int fq = tq, fs = ts, ft = tt;
      float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        v0 += s_slot[kb][ww][fq][fs][ft];
        v1 += s_slot[kb][ww][fq][fs][ft + 1];
      }
      if ((fq == 0 ? BV : CV) && fs < n) {
        float *dst = (fq == 0 ? p.pB : p.pC) + ((static_cast<int64_t>(bg) * p.nblk + blk) * n + fs) * L + t0 + ft;
        if (ft < len) dst[0] = v0;
        if (ft + 1 < len) dst[1] = v1;
      }
    }
  }

  // ---- per-lane results over the segment (partials indexed (seg, b, d))
  const int64_t prow = seg * p.bd + row;
  if (valid && sv) {
    if (p.dinit && seg == 0) p.dinit[row * n + s] = gcar;
    p.pA[prow * n + s] = dA_acc;
    if constexpr (!BV) p.pB[prow * n + s] = dBf_acc;
    if constexpr (!CV) p.pC[prow * n + s] = dCf_acc;
  }
  // owner sums over the row's 16 lanes
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    accD += __shfl_xor(accD, m, 16);
    accBias += __shfl_xor(accBias, m, 16);
  }
  if (valid && s == 0) {
    if (p.pD) p.pD[prow] = accD;
    if (p.pbias) p.pbias[prow] = accBias;
  }
}

// Sequence split, first pass.  The adjoint carry is linear in what comes in
// from later timesteps: over segment k it maps an incoming carry G to
// loc_k + exp2(A' * sum_k) * G, where loc_k is the carry out of the segment's
// first timestep when G = 0 (h_t = g_t C_t + a_{t+1} h_{t+1} walked over the
// segment alone) and sum_k the segment's sum of delta'.  This kernel writes
// loc_k and sum_k for every segment k >= 1; it needs only delta, dout, z and
// C.  A 256-thread workgroup holds 16 channels of one (batch, group), one
// 16-lane row (one lane per state) each, and walks its segment in tiles of
// 64 timesteps: the tile's C (shared by the 16 channels) is loaded
// coalesced and staged through LDS, one tile ahead; lane j of a row owns
// timesteps j, j+16, j+32, j+48 of the tile, computes their delta' and
// dout * silu(z), and the row reads them by DPP broadcast.
constexpr int kCT = 64;   // timesteps per carry tile

template <int IO, bool CV, bool HZ>
__global__ void __launch_bounds__(256) seg_carry_kernel(const BwdParams p) {
  __shared__ __align__(16) float s_c[CV ? 2 : 1][kNP][kCT + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane >> 4, s = lane & 15;
  const int n = p.n;
  const bool sv = s < n;
  const int64_t L = p.seqlen;
  const int nb16 = static_cast<int>((p.cpg + 15) / 16);
  const int blk = blockIdx.x % nb16;
  const int bg = blockIdx.x / nb16;
  const int g = bg % p.ngroups;
  const int64_t b = bg / p.ngroups;
  const int64_t lc = static_cast<int64_t>(blk) * 16 + w * 4 + c;
  const bool valid = lc < p.cpg;
  const int64_t dl = g * p.cpg + (valid ? lc : p.cpg - 1);
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * L;
  const int seg = blockIdx.y + 1;
  const int64_t tbeg = (static_cast<int64_t>(p.seg0) + static_cast<int64_t>(seg - 1) * p.segc) * kT;
  const int64_t tend = tbeg + static_cast<int64_t>(p.segc) * kT < L ? tbeg + static_cast<int64_t>(p.segc) * kT : L;

  const float Ap = (sv ? p.A[dl * n + s] : 0.0f) * kLog2e;
  const float Cf = (!CV && sv) ? load_io<IO>(p.C, dl * n + s) : 0.0f;
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;

  // C tile: thread -> (state tid >> 4, timesteps 4 * (tid & 15) + 0..3);
  // rows of states >= n are staged as zeros
  const int cs = tid >> 4, ct = (tid & 15) * 4;
  const bool c_on = CV && cs < n;
  const int64_t csrc = (static_cast<int64_t>(bg) * n + (c_on ? cs : 0)) * L;
  // raw bits of the next tile: the owned timesteps' delta, dout, z and the
  // thread's four C elements
  uint32_t r_d[4], r_go[4], r_z[4], r_c[4];
  auto fetch = [&](int64_t tb) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int64_t t = tb + s + 16 * h;
      r_d[h] = r_go[h] = r_z[h] = 0;
      if (t < tend) {
        r_d[h] = raw_load<IO>(p.delta, rbase + t);
        r_go[h] = raw_load<IO>(p.dout, rbase + t);
        if constexpr (HZ) r_z[h] = raw_load<IO>(p.z, rbase + t);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r_c[j] = 0;
      if (c_on && tb + ct + j < tend) r_c[j] = raw_load<IO>(p.C, csrc + tb + ct + j);
    }
  };
  auto stage = [&](int buf) {
    if constexpr (CV)
      *reinterpret_cast<float4 *>(&s_c[buf][cs][ct]) =
          make_float4(raw_float<IO>(r_c[0]), raw_float<IO>(r_c[1]), raw_float<IO>(r_c[2]), raw_float<IO>(r_c[3]));
  };

  float gcar = 0.0f, dsum = 0.0f;
  const int ntile = static_cast<int>((tend - tbeg + kCT - 1) / kCT);
  fetch(tbeg + static_cast<int64_t>(ntile - 1) * kCT);
  stage(0);
  __syncthreads();
  for (int i = ntile - 1, k = 0; i >= 0; --i, ++k) {
    const int buf = CV ? (k & 1) : 0;
    const int64_t tb = tbeg + static_cast<int64_t>(i) * kCT;
    float o_dt[4], o_g[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float raw = raw_float<IO>(r_d[h]) + bias;
      float dt = p.softplus ? softplus_f(raw) : raw;
      const float go = raw_float<IO>(r_go[h]);
      float gg = go;
      if constexpr (HZ) {
        const float zz = raw_float<IO>(r_z[h]);
        gg = go * zz * sigmoid_f(zz);
      }
      if (tb + s + 16 * h >= tend) { dt = 0.0f; gg = 0.0f; }   // inert timestep
      o_dt[h] = dt;
      o_g[h] = gg;
      dsum += dt;
    }
    if (i > 0) fetch(tb - kCT);

    const float(*cr)[kCT + 4] = s_c[buf];
    float4 C4 = make_float4(Cf, Cf, Cf, Cf);
    static_for(std::make_integer_sequence<int, kCT>{}, [&](auto RR) {
      constexpr int t = kCT - 1 - decltype(RR)::value;
      constexpr int K = t & 15, H = t >> 4;
      if constexpr (CV && (t & 3) == 3) C4 = *reinterpret_cast<const float4 *>(&cr[s][t - 3]);
      const float h = fmaf(bc<K>(o_g[H]), f4get<t & 3>(C4), gcar);
      gcar = h * fast_exp2(bc<K>(o_dt[H]) * Ap);
    });
    if constexpr (CV) {
      if (i > 0) stage(buf ^ 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m, 16);
  const int64_t prow = static_cast<int64_t>(seg) * p.bd + row;
  if (valid && sv) p.loc[prow * n + s] = gcar;
  if (valid && s == 0) p.ssum[prow] = dsum;
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

template <int IO, bool HZ>
BwdFn pick_bc(bool bv, bool cv) {
  if (bv && cv) return scan_bwd_kernel<IO, true, true, HZ>;
  if (bv) return scan_bwd_kernel<IO, true, false, HZ>;
  if (cv) return scan_bwd_kernel<IO, false, true, HZ>;
  return scan_bwd_kernel<IO, false, false, HZ>;
}
template <int IO>
BwdFn pick_bwd(bool bv, bool cv, bool hz) {
  return hz ? pick_bc<IO, true>(bv, cv) : pick_bc<IO, false>(bv, cv);
}

template <int IO>
BwdFn pick_carry(bool cv, bool hz) {
  if (cv) return hz ? seg_carry_kernel<IO, true, true> : seg_carry_kernel<IO, true, false>;
  return hz ? seg_carry_kernel<IO, false, true> : seg_carry_kernel<IO, false, false>;
}

constexpr int kMaxSeg = 64;   // most segments the library picks by itself
constexpr int kMinSegChunks = 4;   // and the fewest chunks it gives a segment

struct BwdPlan {
  int64_t cpg, nblk, nck, blocks;
  int segc, nseg, seg0;
  size_t nB, nC, nA, nD, nLoc, nSum;   // partial element counts
  size_t bytes;
};

// Segments of the sequence split (host_util.h: split_segments,
// split_first_segment).  One 768-thread workgroup fills a compute unit; the
// carry pass over the segments after the first costs about a quarter of the
// main pass per (channel, timestep) when it fills the chip (measured).  For
// the uneven two-segment split, measured at mamba2p8b (864 workgroups, 64
// chunks; the model picks 55): first segment of 32 chunks 1.711 ms, 48:
// 1.641, 52: 1.587, 54: 1.606, 56: 1.593, 58: 1.634, 60: 1.675.
constexpr double kCarryCost = 0.25;

BwdPlan plan_bwd(const ssm_scan_bwd_args_t *a, int cus) {
  BwdPlan pl{};
  pl.cpg = a->dim / a->ngroups;
  pl.nblk = (pl.cpg + kCPB - 1) / kCPB;
  pl.nck = (a->seqlen + kT - 1) / kT;
  pl.blocks = a->batch * a->ngroups * pl.nblk;
  int64_t want = a->seq_segments > 0 ? a->seq_segments
                                     : split_segments(pl.blocks, pl.nck, cus, kCarryCost, kMaxSeg, kMinSegChunks);
  if (want > pl.nck) want = pl.nck;
  pl.segc = static_cast<int>((pl.nck + want - 1) / want);
  pl.nseg = static_cast<int>((pl.nck + pl.segc - 1) / pl.segc);   // every segment holds a chunk
  pl.seg0 = pl.segc;
  if (a->seq_segments <= 0 && pl.nseg == 2) {
    pl.seg0 = split_first_segment(pl.blocks, pl.nck, cus, kCarryCost);
    pl.segc = static_cast<int>(pl.nck - pl.seg0);
  }
  const size_t ns = static_cast<size_t>(pl.nseg);
  const size_t bgn = static_cast<size_t>(a->batch * a->ngroups) * pl.nblk * a->dstate * a->seqlen;
  const size_t bdn = static_cast<size_t>(a->batch * a->dim * a->dstate);
  pl.nB = a->B_kind == SSM_BC_VARYING ? bgn : ns * bdn;
  pl.nC = a->C_kind == SSM_BC_VARYING ? bgn : ns * bdn;
  pl.nA = ns * bdn;
  pl.nD = ns * static_cast<size_t>(a->batch * a->dim);
  pl.nLoc = pl.nseg > 1 ? ns * bdn : 0;
  pl.nSum = pl.nseg > 1 ? pl.nD : 0;
  // every partial array starts on a 256-byte boundary
  auto up = [](size_t e) { return (e * sizeof(float) + 255) / 256 * 256; };
  pl.bytes = up(pl.nB) + up(pl.nC) + up(pl.nA) + 2 * up(pl.nD) + up(pl.nLoc) + up(pl.nSum);
  return pl;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args_t *a, size_t *bytes) {
  const int st = ssm_scan_bwd_validate(a);
  if (st != SSM_OK) return st;
  if (!bytes) return SSM_ERR_NULL;
  *bytes = plan_bwd(a, cu_count_cached()).bytes;
  return SSM_OK;
}

extern "C" int ssm_scan_bwd(const ssm_scan_bwd_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_bwd_validate(a);
  if (st != SSM_OK) return st;
  const BwdPlan pl = plan_bwd(a, cu_count_cached());
  if (pl.blocks > 0x7fffffffLL || static_cast<int64_t>(pl.nB / 256) > 0x7fffffffLL ||
      static_cast<int64_t>(pl.nA / 256) > 0x7fffffffLL || pl.nseg > 65535)
    return SSM_ERR_SHAPE;
  if (!a->workspace || a->workspace_bytes < pl.bytes) return SSM_ERR_WORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;

  char *base = static_cast<char *>(a->workspace);
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
  p.loc = pl.nLoc ? take(pl.nLoc) : nullptr;
  p.ssum = pl.nSum ? take(pl.nSum) : nullptr;
  p.dinit = a->dinitial_state;
  p.dim = a->dim; p.seqlen = a->seqlen; p.cpg = pl.cpg; p.bd = a->batch * a->dim;
  p.n = static_cast<int>(a->dstate); p.ngroups = static_cast<int>(a->ngroups);
  p.nblk = static_cast<int>(pl.nblk); p.nck = static_cast<int>(pl.nck);
  p.softplus = a->delta_softplus;
  p.segc = pl.segc; p.nseg = pl.nseg; p.seg0 = pl.seg0;

  const bool hz = a->z != nullptr;
  hipError_t e = hipSuccess;
  if (pl.nseg > 1) {
    const BwdFn fc = a->io_dtype == SSM_BF16  ? pick_carry<1>(cv, hz)
                    : a->io_dtype == SSM_F16 ? pick_carry<2>(cv, hz)
                                             : pick_carry<0>(cv, hz);
    const int64_t cblocks = a->batch * a->ngroups * ((pl.cpg + 15) / 16);
    hipLaunchKernelGGL(fc, dim3(static_cast<unsigned>(cblocks), static_cast<unsigned>(pl.nseg - 1)), dim3(256), 0,
                       stream, p);
    e = hipGetLastError();
  }
  const BwdFn f = a->io_dtype == SSM_BF16  ? pick_bwd<1>(bv, cv, hz)
                 : a->io_dtype == SSM_F16 ? pick_bwd<2>(bv, cv, hz)
                                          : pick_bwd<0>(bv, cv, hz);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(pl.blocks), static_cast<unsigned>(pl.nseg)), dim3(kThreads), 0,
                       stream, p);
    e = hipGetLastError();
  }

  auto reduce = [&](const float *in, float *out, int64_t I, int64_t K, int64_t J) {
    if (e != hipSuccess) return;
    const dim3 grid(static_cast<unsigned>((I * J + 255) / 256));
    hipLaunchKernelGGL(sum_mid_kernel, grid, dim3(256), 0, stream, in, out, I, K, J);
    e = hipGetLastError();
  };
  const int64_t bsz = a->batch, n = a->dstate, L = a->seqlen, dim = a->dim;
  const int64_t kpart = pl.nseg * bsz;   // per-(segment, batch) partials
  if (bv) reduce(p.pB, a->dB, bsz * a->ngroups, pl.nblk, n * L);
  else reduce(p.pB, a->dB, 1, kpart, dim * n);
  if (cv) reduce(p.pC, a->dC, bsz * a->ngroups, pl.nblk, n * L);
  else reduce(p.pC, a->dC, 1, kpart, dim * n);
  reduce(p.pA, a->dA, 1, kpart, dim * n);
  if (a->D) reduce(p.pD, a->dD, 1, kpart, dim);
  if (a->delta_bias) reduce(p.pbias, a->ddelta_bias, 1, kpart, dim);

  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
