// bwd_complex.hip -- the gradients of the complex-A forward
// (ssm_scan_bwd_complex) for gfx950.
//
// Operation: PaddleNLP Kernel operator-library guide, section 4.1: A may be
// real or complex, and the operator's backward is the extension's bwd entry.
// With G_v = dL/dRe v + i dL/dIm v for a complex v, the adjoint of
//   x_t = a_t x_{t-1} + delta'_t B_t u_t,  a_t = exp(delta'_t A),
//   y_t = Re(sum_s C_t[s] x_t[s])
// runs in reverse time, h_t = dy_t conj(C_t) + conj(a_{t+1}) h_{t+1}, and
//   G_C_t = dy_t conj(x_t),  G_a_t = h_t conj(x_{t-1}),
//   dA += conj(delta' a) G_a,  dB_t = delta' u h_t,
//   du_t = D dy_t + delta' sum_s Re(h_t conj(B_t)),
//   d delta'_t = sum_s Re(G_a conj(A a)) + u sum_s Re(h_t conj(B_t));
// include/ssmscan.h writes out every gradient.
//
// Work decomposition: a channel is one 16-lane row of a wave, lane s owning
// complex state s (padded states are inert: A = B = C = 0 keeps them zero);
// a 512-thread workgroup holds 32 channels of one (batch, group).  The
// sequence is walked in chunks of SSM_CKPT_INTERVAL timesteps from the last
// to the first.  Per chunk every row re-runs the forward recurrence from the
// state the forward saved at the chunk's start, keeping x_{t-1} of each
// timestep in registers, then walks the chunk backwards recomputing a_t.
// The per-(channel, timestep) scalars (delta', delta' u, u, dy) are formed
// by the lane that owns the timestep (lane j owns timesteps j and j + 16)
// and read by the row through DPP row broadcasts; sums over the states
// (y for dz, the du and delta' terms) are DPP rotations within the row.
// Time-varying dB/dC sum over every channel of the group: each wave folds
// its four rows with the row-swap instructions, the workgroup adds its waves
// in order through LDS and writes its partial sums; a second kernel adds the workgroups' partials in a fixed
// order, as it adds the per-batch partials of dA, fixed dB/dC, dD and
// d(delta_bias).  No atomics: every output is bit-for-bit repeatable.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "complex_util.h"
#include "device_util.h"
#include "host_util.h"
#include "ssmscan.h"

namespace ssm {
namespace {

constexpr int kCk = SSM_CKPT_INTERVAL;   // timesteps per chunk
constexpr int kRowsPerWave = 4;          // channels per wave
constexpr int kWavesPerWG = 8;
constexpr int kChPerWG = kRowsPerWave * kWavesPerWG;
static_assert(kCk == 32, "two owned timesteps per lane of a 16-lane row");

struct CbwdParams {
  const void *u, *delta, *B, *C, *z, *dout;
  const float *A, *D, *dbias, *ckpt;
  void *du, *ddelta, *dz;
  float *dA, *dB, *dC, *dD, *ddbias, *dinit;
  float *ws_bc;               // time-varying dB/dC partials [b*g][blk][t][s][4]
  float *ws_dA, *ws_fB, *ws_fC, *ws_dD, *ws_db;   // per-(segment, batch) partials
  // sequence split: segment k >= 1's adjoint carry out of its first timestep
  // with no carry coming in, and its decay prod_t a_t, both (nseg, b, d, n, 2)
  float *loc, *pdec;
  int64_t batch, dim, seqlen, nck, cpg;
  int n, ngroups, groups_eff, nblk;
  int softplus;
  int nseg, seg0, segc;       // segments; chunks of segment 0 and of the others
};

// sum over the 16 lanes of a row, in every lane (rotations within the row)
__device__ __forceinline__ float row_sum16(float v) {
  // row rotations write every lane: no old value (see row_bc)
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, true));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, true));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, true));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, true));  // row_ror:1
  return v;
}

// lane K of each 16-lane row, in every lane of the row (DPP row_newbcast).
// It writes every lane, so no old value is needed: update_dpp with an old
// value of 0 costs a register zeroed before every broadcast.
template <int K>
__device__ __forceinline__ float row_bc(float v) {
  static_assert(K >= 0 && K < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + K, 0xf, 0xf, true));
}

// The wave's four rows (channels) summed with the gfx950 row-swap
// instructions: v_permlane32_swap trades lanes 32..63 of x with lanes 0..31
// of y, v_permlane16_swap rows 1 and 3 of x with rows 0 and 2 of y.  Of
// (v0, v1, v2, v3), row 0 of the result holds the sum of v0 over the rows,
// row 1 that of v2, row 2 that of v1, row 3 that of v3.
__device__ __forceinline__ float fold_rows4(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  const float r1 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float r2 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1), __float_as_uint(r2), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// CARRY: the carry pass of the sequence split.  Workgroup (x, y) walks
// segment y + 1 of its channels backwards from a zero carry, through the
// same adjoint steps as the backward walk (h += dy conj(C_t), then
// h <- conj(a_t) h), and stores the carry out of the segment's first
// timestep and the segment's decay prod_t a_t, multiplied up step by step as
// the walk applies it (its phase as accurate as the walk's); nothing else.
template <int IO, bool BV, bool CV, bool CARRY>
__global__ void __launch_bounds__(512) cbwd_kernel(const CbwdParams p) {
  constexpr bool ANYV = BV || CV;
  constexpr bool PART = ANYV && !CARRY;
  __shared__ float s_bc[ANYV ? 2 : 1][ANYV ? kCk : 1][16][2];       // [B, C][t][s][re, im]
  __shared__ float s_part[PART ? kWavesPerWG : 1][PART ? kCk : 1][16][4];   // per-wave (dB, dC) sums

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rw = lane >> 4, s = lane & 15;
  const int blk = blockIdx.x % p.nblk;
  const int rest = blockIdx.x / p.nblk;
  const int g = rest % p.groups_eff;
  const int64_t b = rest / p.groups_eff;
  const int64_t d_end = (g + 1) * p.cpg;
  const int64_t d = g * p.cpg + static_cast<int64_t>(blk) * kChPerWG + wave * kRowsPerWave + rw;
  const bool valid = d < d_end;
  const int64_t dl = valid ? d : d_end - 1;
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * p.seqlen;
  const int64_t L = p.seqlen;
  const int n = p.n;
  const bool sv = s < n;

  const int64_t ea = (dl * n + (sv ? s : 0)) * 2;
  const float Ar = sv ? p.A[ea] : 0.0f, Ai = sv ? p.A[ea + 1] : 0.0f;
  const float Ar2 = Ar * kLog2e;
  const Turns Atr = turns_of(Ai);
  float Bfr = 0.0f, Bfi = 0.0f, Cfr = 0.0f, Cfi = 0.0f;
  if (!BV && sv) { Bfr = load_io<IO>(p.B, ea); Bfi = load_io<IO>(p.B, ea + 1); }
  if (!CV && sv) { Cfr = load_io<IO>(p.C, ea); Cfi = load_io<IO>(p.C, ea + 1); }
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;
  const float Dd = p.D ? p.D[dl] : 0.0f;
  const int64_t bg = b * p.ngroups + g;
  const int64_t bc_base = bg * n * L * 2;   // element of (b, g, state 0, t 0, re) in a varying B/C
  const int64_t BD = p.batch * p.dim;
  const int seg = CARRY ? static_cast<int>(blockIdx.y) + 1 : static_cast<int>(blockIdx.y);
  const int64_t cbeg = seg == 0 ? 0 : p.seg0 + static_cast<int64_t>(seg - 1) * p.segc;
  const int64_t clen = seg == 0 ? p.seg0 : p.segc;
  const int64_t cend = cbeg + clen < p.nck ? cbeg + clen : p.nck;   // this workgroup's chunks [cbeg, cend)

  float hr = 0.0f, hi = 0.0f;                                 // adjoint carry
  if constexpr (!CARRY) {
    // the carry entering from the later segments: each maps an incoming
    // carry G to loc + conj(P) G, P its decay prod_t a_t
    if (seg + 1 < p.nseg && sv) {
      for (int k = p.nseg - 1; k > seg; --k) {
        const float *lc = p.loc + ((k * BD + row) * n + s) * 2;
        const float *pd = p.pdec + ((k * BD + row) * n + s) * 2;
        const float er = pd[0], ei = pd[1];
        const float nhr = fmaf(er, hr, fmaf(ei, hi, lc[0]));
        const float nhi = fmaf(er, hi, fmaf(-ei, hr, lc[1]));
        hr = nhr;
        hi = nhi;
      }
    }
  }
  float dAr = 0.0f, dAi = 0.0f, fBr = 0.0f, fBi = 0.0f, fCr = 0.0f, fCi = 0.0f;
  float accD = 0.0f, accBias = 0.0f;                           // owner lanes' sums over their timesteps
  float Pr = 1.0f, Pi = 0.0f;                                  // the segment's decay prod_t a_t (CARRY)

  for (int64_t ci = cend - 1; ci >= cbeg; --ci) {
    const int64_t c0 = ci * kCk;
    const int len = static_cast<int>((L - c0 < kCk) ? L - c0 : kCk);

    // ---- the owned timesteps' scalars (lane s owns t = s and s + 16)
    float o_dt[2], o_dtu[2], o_u[2], o_dy[2], o_dsp[2], o_dout[2], o_sg[2], o_z[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = s + 16 * k;
      o_dt[k] = o_dtu[k] = o_u[k] = o_dy[k] = o_dsp[k] = o_dout[k] = o_sg[k] = o_z[k] = 0.0f;
      if (t < len) {
        const int64_t e = rbase + c0 + t;
        const float raw = load_io<IO>(p.delta, e) + bias;
        const float uu = load_io<IO>(p.u, e);
        const float dt = p.softplus ? softplus_acc(raw) : raw;
        const float dsp = p.softplus ? fast_rcp(1.0f + fast_exp2(-raw * kLog2e)) : 1.0f;
        float dout = valid ? load_io<IO>(p.dout, e) : 0.0f;
        float dy = dout;
        if (p.z) {
          const float zz = load_io<IO>(p.z, e);
          const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
          o_sg[k] = sg;
          o_z[k] = zz;
          dy = dout * zz * sg;
        }
        o_dt[k] = dt; o_dtu[k] = dt * uu; o_u[k] = uu; o_dy[k] = dy; o_dsp[k] = dsp; o_dout[k] = dout;
      }
    }

    // ---- the chunk's B/C tile (time-varying), and the chunk start's state
    if constexpr (ANYV) {
      __syncthreads();   // the previous chunk's reads of s_bc and s_part are done
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 512 * j;           // [tensor][state][t][re, im]
        const int tensor = idx >> 10, r = idx & 1023;
        const int st = r >> 6, tc = r & 63, t = tc >> 1, comp = tc & 1;
        float v = 0.0f;
        const bool want = tensor == 0 ? (BV && !CARRY) : CV;
        if (want && st < n && t < len)
          v = load_io<IO>(tensor == 0 ? p.B : p.C, bc_base + (static_cast<int64_t>(st) * L + c0 + t) * 2 + comp);
        s_bc[tensor][t][st][comp] = v;
      }
      __syncthreads();
    }
    if constexpr (CARRY) {
      static_for(std::make_integer_sequence<int, kCk>{}, [&](auto J) {
        constexpr int t = kCk - 1 - decltype(J)::value;
        if (t < len) {
          const float dt = row_bc<t % 16>(o_dt[t / 16]);
          const float dy = row_bc<t % 16>(o_dy[t / 16]);
          float cr, cim, er, ei;
          if constexpr (CV) { cr = s_bc[1][t][s][0]; cim = s_bc[1][t][s][1]; }
          else { cr = Cfr; cim = Cfi; }
          hr = fmaf(dy, cr, hr);
          hi = fmaf(-dy, cim, hi);
          cexp_turns(dt, Ar2, Atr.hi, Atr.lo, er, ei);
          const float nhr = fmaf(er, hr, ei * hi);
          const float nhi = fmaf(er, hi, -ei * hr);
          hr = nhr;
          hi = nhi;
          const float nPr = fmaf(er, Pr, -ei * Pi);
          const float nPi = fmaf(er, Pi, ei * Pr);
          Pr = nPr;
          Pi = nPi;
        }
      });
      continue;
    }
    float xr = 0.0f, xi = 0.0f;
    if (sv) {
      const int64_t e = ((row * p.nck + ci) * n + s) * 2;
      xr = p.ckpt[e];
      xi = p.ckpt[e + 1];
    }

    auto bcoef = [&](int t, float &br, float &bi) {
      if constexpr (BV) { br = s_bc[0][t][s][0]; bi = s_bc[0][t][s][1]; }
      else { br = Bfr; bi = Bfi; }
    };
    auto ccoef = [&](int t, float &cr, float &cim) {
      if constexpr (CV) { cr = s_bc[ANYV ? 1 : 0][t][s][0]; cim = s_bc[ANYV ? 1 : 0][t][s][1]; }
      else { cr = Cfr; cim = Cfi; }
    };

    // ---- forward re-run and backward walk, in two halves of kH timesteps.
    // x_{t-1} of the half being walked is kept in registers.  The first half
    // is re-run twice, once to reach the second half's start and once to keep
    // its states: a sixth more work for half the registers the saved states
    // take, which lets two workgroups share a compute unit.
    constexpr int kH = kCk / 2;
    const float x0r = xr, x0i = xi;
    auto fstep = [&](auto TT) {   // x <- a_t x + delta'_t u_t B_t
      constexpr int t = decltype(TT)::value;
      if (t < len) {
        const float dt = row_bc<t % 16>(o_dt[t / 16]);
        const float dtu = row_bc<t % 16>(o_dtu[t / 16]);
        float er, ei, br, bi;
        cexp_turns(dt, Ar2, Atr.hi, Atr.lo, er, ei);
        bcoef(t, br, bi);
        const float nr = fmaf(er, xr, fmaf(-ei, xi, br * dtu));
        const float ni = fmaf(er, xi, fmaf(ei, xr, bi * dtu));
        xr = nr;
        xi = ni;
      }
    };
    // the owners keep y_t, the delta' term and the u term
    float r_y[2] = {0.0f, 0.0f}, r_ddt[2] = {0.0f, 0.0f}, r_du[2] = {0.0f, 0.0f};
    auto bstep = [&](auto TT, const float xpv_r, const float xpv_i) {
      constexpr int t = decltype(TT)::value;
      if (t < len) {
        const float dt = row_bc<t % 16>(o_dt[t / 16]);
        const float dtu = row_bc<t % 16>(o_dtu[t / 16]);
        const float uu = row_bc<t % 16>(o_u[t / 16]);
        const float dy = row_bc<t % 16>(o_dy[t / 16]);
        float er, ei, br, bi, cr, cim;
        cexp_turns(dt, Ar2, Atr.hi, Atr.lo, er, ei);
        bcoef(t, br, bi);
        ccoef(t, cr, cim);
        const float xpr = xpv_r, xpi = xpv_i;                  // x_{t-1}
        const float xtr = fmaf(er, xpr, fmaf(-ei, xpi, br * dtu));
        const float xti = fmaf(er, xpi, fmaf(ei, xpr, bi * dtu));
        const float yp = fmaf(cr, xtr, -cim * xti);            // Re(C x_t)
        hr = fmaf(dy, cr, hr);                                 // h_t = dy conj(C) + carry
        hi = fmaf(-dy, cim, hi);
        const float gCr = dy * xtr, gCi = -dy * xti;           // dy conj(x_t)
        const float gar = fmaf(hr, xpr, hi * xpi);             // h conj(x_{t-1})
        const float gai = fmaf(hi, xpr, -hr * xpi);
        const float war = fmaf(Ar, er, -Ai * ei), wai = fmaf(Ar, ei, Ai * er);   // A a
        const float term2 = fmaf(hr, br, hi * bi);             // Re(h conj(B))
        const float ddtp = fmaf(gar, war, fmaf(gai, wai, uu * term2));
        const float dup = dt * term2;
        dAr = fmaf(dt, fmaf(er, gar, ei * gai), dAr);          // conj(dt a) G_a
        dAi = fmaf(dt, fmaf(er, gai, -ei * gar), dAi);
        const float gBr = dtu * hr, gBi = dtu * hi;
        if constexpr (!BV) { fBr += gBr; fBi += gBi; }
        if constexpr (!CV) { fCr += gCr; fCi += gCi; }
        if constexpr (PART) {
          // row rw holds the wave's sum of component ((rw & 1) << 1) | (rw >> 1)
          // of (dB re, dB im, dC re, dC im)
          const float v = fold_rows4(BV ? gBr : 0.0f, BV ? gBi : 0.0f, CV ? gCr : 0.0f, CV ? gCi : 0.0f);
          s_part[wave][t][s][((rw & 1) << 1) | (rw >> 1)] = v;
        }
        const float nhr = fmaf(er, hr, ei * hi);               // carried: conj(a) h
        const float nhi = fmaf(er, hi, -ei * hr);
        hr = nhr;
        hi = nhi;
        const float ys = row_sum16(yp), ds = row_sum16(ddtp), us = row_sum16(dup);
        if (s == t % 16) { r_y[t / 16] = ys; r_ddt[t / 16] = ds; r_du[t / 16] = us; }
      }
    };
    float pr[kH], pim[kH];
    static_for(std::make_integer_sequence<int, kH>{}, [&](auto J) { fstep(J); });
    static_for(std::make_integer_sequence<int, kH>{}, [&](auto J) {
      constexpr int j = decltype(J)::value;
      pr[j] = xr;
      pim[j] = xi;
      fstep(std::integral_constant<int, kH + j>{});
    });
    static_for(std::make_integer_sequence<int, kH>{}, [&](auto J) {
      constexpr int j = kH - 1 - decltype(J)::value;
      bstep(std::integral_constant<int, kH + j>{}, pr[j], pim[j]);
    });
    xr = x0r;
    xi = x0i;
    static_for(std::make_integer_sequence<int, kH>{}, [&](auto J) {
      constexpr int j = decltype(J)::value;
      pr[j] = xr;
      pim[j] = xi;
      fstep(J);
    });
    static_for(std::make_integer_sequence<int, kH>{}, [&](auto J) {
      constexpr int j = kH - 1 - decltype(J)::value;
      bstep(std::integral_constant<int, j>{}, pr[j], pim[j]);
    });

    // ---- the owners' gradients of their timesteps
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = s + 16 * k;
      if (t < len && valid) {
        const int64_t e = rbase + c0 + t;
        const float ddt = r_ddt[k] * o_dsp[k];
        store_one<IO>(p.du, e, fmaf(Dd, o_dy[k], r_du[k]));
        store_one<IO>(p.ddelta, e, ddt);
        if (p.z) {
          const float pre = fmaf(Dd, o_u[k], r_y[k]);
          const float sg = o_sg[k], zz = o_z[k];
          store_one<IO>(p.dz, e, o_dout[k] * pre * sg * fmaf(zz, 1.0f - sg, 1.0f));
        }
        accD = fmaf(o_dy[k], o_u[k], accD);
        accBias += ddt;
      }
    }

    // ---- the workgroup's partial sums of time-varying dB/dC for the chunk
    if constexpr (PART) {
      __syncthreads();
      static_assert(kCk * 16 == 512, "one (timestep, state) of the chunk per thread");
      const int t = tid >> 4, st = tid & 15;
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int w = 0; w < kWavesPerWG; ++w) {
        const float4 v = *reinterpret_cast<const float4 *>(&s_part[w][t][st][0]);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      if (t < len && st < n)
        *reinterpret_cast<float4 *>(p.ws_bc + (((bg * p.nblk + blk) * L + c0 + t) * n + st) * 4) = acc;
    }
  }

  if constexpr (CARRY) {
    if (valid && sv) {
      float *lc = p.loc + ((seg * BD + row) * n + s) * 2;
      float *pd = p.pdec + ((seg * BD + row) * n + s) * 2;
      lc[0] = hr;
      lc[1] = hi;
      pd[0] = Pr;
      pd[1] = Pi;
    }
    return;
  }
  // ---- per-channel results (partials per segment and batch)
  if (valid && sv) {
    const int64_t e = ((seg * BD + row) * n + s) * 2;
    if (p.dinit && seg == 0) { p.dinit[(row * n + s) * 2] = hr; p.dinit[(row * n + s) * 2 + 1] = hi; }
    p.ws_dA[e] = dAr;
    p.ws_dA[e + 1] = dAi;
    if constexpr (!BV) { p.ws_fB[e] = fBr; p.ws_fB[e + 1] = fBi; }
    if constexpr (!CV) { p.ws_fC[e] = fCr; p.ws_fC[e + 1] = fCi; }
  }
  const float sD = row_sum16(accD), sB = row_sum16(accBias);
  if (valid && s == 0) {
    p.ws_dD[seg * BD + row] = sD;
    p.ws_db[seg * BD + row] = sB;
  }
}

// Adds the partial sums in a fixed order: per (d, s) over the batch for dA
// and fixed dB/dC; per d over the batch for dD and d(delta_bias); per
// (b*g, s, t) over the group's workgroups for time-varying dB/dC.
__global__ void __launch_bounds__(256) cbwd_sum_kernel(const CbwdParams p, int bv, int cv) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = p.n, L = p.seqlen;
  const int64_t nds = p.dim * n;
  if (i < nds) {
    float ar = 0.0f, ai = 0.0f, br = 0.0f, bi = 0.0f, cr = 0.0f, cim = 0.0f;
    for (int64_t sb = 0; sb < p.nseg * p.batch; ++sb) {   // (segment, batch) in order
      const int64_t e = (sb * nds + i) * 2;
      ar += p.ws_dA[e]; ai += p.ws_dA[e + 1];
      if (!bv) { br += p.ws_fB[e]; bi += p.ws_fB[e + 1]; }
      if (!cv) { cr += p.ws_fC[e]; cim += p.ws_fC[e + 1]; }
    }
    p.dA[2 * i] = ar; p.dA[2 * i + 1] = ai;
    if (!bv) { p.dB[2 * i] = br; p.dB[2 * i + 1] = bi; }
    if (!cv) { p.dC[2 * i] = cr; p.dC[2 * i + 1] = cim; }
  }
  if (i < p.dim) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t k = 0; k < p.nseg * p.batch; ++k) {
      sd += p.ws_dD[k * p.dim + i];
      sb += p.ws_db[k * p.dim + i];
    }
    if (p.dD) p.dD[i] = sd;
    if (p.ddbias) p.ddbias[i] = sb;
  }
  if (bv || cv) {
    const int64_t nbg = p.batch * p.ngroups;
    if (i < nbg * L * n) {
      const int64_t st = i % n, t = (i / n) % L, bgi = i / (n * L);
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      for (int blk = 0; blk < p.nblk; ++blk) {
        const float4 v = *reinterpret_cast<const float4 *>(p.ws_bc + (((bgi * p.nblk + blk) * L + t) * n + st) * 4);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      const int64_t o = ((bgi * n + st) * L + t) * 2;
      if (bv) { p.dB[o] = acc.x; p.dB[o + 1] = acc.y; }
      if (cv) { p.dC[o] = acc.z; p.dC[o + 1] = acc.w; }
    }
  }
}

using CbwdFn = void (*)(const CbwdParams);

template <int IO>
CbwdFn pick_cbwd(bool bv, bool cv) {
  if (bv && cv) return cbwd_kernel<IO, true, true, false>;
  if (bv) return cbwd_kernel<IO, true, false, false>;
  if (cv) return cbwd_kernel<IO, false, true, false>;
  return cbwd_kernel<IO, false, false, false>;
}

template <int IO>
CbwdFn pick_ccarry(bool cv) {
  return cv ? cbwd_kernel<IO, false, true, true> : cbwd_kernel<IO, false, false, true>;
}

CbwdFn cbwd_fn(int32_t io, bool bv, bool cv) {
  return io == SSM_BF16 ? pick_cbwd<1>(bv, cv) : io == SSM_F16 ? pick_cbwd<2>(bv, cv) : pick_cbwd<0>(bv, cv);
}

struct CbwdPlan {
  int groups_eff, nblk;
  int64_t cpg, nck, nwg;
  int nseg, seg0, segc;
  size_t off_bc, off_dA, off_fB, off_fC, off_dD, off_db, off_loc, off_pdec, ws_bytes;
};

// Sequence split (host_util.h: split_segments, split_first_segment).  The
// carry pass walks a chunk with the exps and the h update of the backward
// step alone, but as a chain of dependent steps behind each chunk's loads it
// takes about 0.55 of the main walk's time per chunk (measured at
// mamba2p8b_complex: 197 us for the carry of a 14-chunk segment).  There
// the library therefore keeps one pass: a split saved 113 us of the main
// kernel's 4.2 ms and its carry pass cost 197.
constexpr double kCarryCostC = 0.6;
constexpr int kMaxSegC = 64;        // most segments the library picks by itself
constexpr int kMinSegChunksC = 4;   // and the fewest chunks it gives a segment

size_t up256c(size_t v) { return (v + 255) / 256 * 256; }

CbwdPlan cbwd_plan(const ssm_scan_bwd_args_t *a, int cus) {
  CbwdPlan pl{};
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;
  pl.groups_eff = (bv || cv) ? static_cast<int>(a->ngroups) : 1;
  pl.cpg = a->dim / pl.groups_eff;
  pl.nblk = static_cast<int>((pl.cpg + kChPerWG - 1) / kChPerWG);
  pl.nck = (a->seqlen + kCk - 1) / kCk;
  pl.nwg = a->batch * pl.groups_eff * pl.nblk;
  int per_cu = blocks_per_cu(reinterpret_cast<const void *>(cbwd_fn(a->io_dtype, bv, cv)), 512);
  if (per_cu <= 0) per_cu = 2;
  const int64_t slots = static_cast<int64_t>(per_cu) * cus;
  int64_t want = a->seq_segments > 0 ? a->seq_segments
                                     : split_segments(pl.nwg, pl.nck, slots, kCarryCostC, kMaxSegC, kMinSegChunksC);
  if (want > pl.nck) want = pl.nck;
  if (want < 1) want = 1;
  pl.segc = static_cast<int>((pl.nck + want - 1) / want);
  pl.nseg = static_cast<int>((pl.nck + pl.segc - 1) / pl.segc);   // every segment holds a chunk
  pl.seg0 = pl.segc;
  if (a->seq_segments <= 0 && pl.nseg == 2) {
    pl.seg0 = split_first_segment(pl.nwg, pl.nck, slots, kCarryCostC);
    pl.segc = static_cast<int>(pl.nck - pl.seg0);
  }
  const size_t ns = static_cast<size_t>(pl.nseg);
  const size_t f = sizeof(float);
  const size_t bd = static_cast<size_t>(a->batch) * a->dim;
  const size_t per_seg = ns * bd * a->dstate * 2 * f;   // complex (segment, b, d, n)
  size_t off = 0;
  pl.off_bc = off;
  if (bv || cv) off += up256c(static_cast<size_t>(a->batch) * a->ngroups * pl.nblk * a->seqlen * a->dstate * 4 * f);
  pl.off_dA = off; off += up256c(per_seg);
  pl.off_fB = off; if (!bv) off += up256c(per_seg);
  pl.off_fC = off; if (!cv) off += up256c(per_seg);
  pl.off_dD = off; off += up256c(ns * bd * f);
  pl.off_db = off; off += up256c(ns * bd * f);
  pl.off_loc = off; if (pl.nseg > 1) off += up256c(per_seg);
  pl.off_pdec = off; if (pl.nseg > 1) off += up256c(per_seg);
  pl.ws_bytes = off;
  return pl;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssm_scan_bwd_complex_workspace_size(const ssm_scan_bwd_args_t *a, size_t *bytes) {
  const int st = ssm_scan_bwd_complex_validate(a);
  if (st != SSM_OK) return st;
  if (!bytes) return SSM_ERR_NULL;
  *bytes = cbwd_plan(a, cu_count_cached()).ws_bytes;
  return SSM_OK;
}

extern "C" int ssm_scan_bwd_complex(const ssm_scan_bwd_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_bwd_complex_validate(a);
  if (st != SSM_OK) return st;
  const CbwdPlan pl = cbwd_plan(a, cu_count_cached());
  if (!a->workspace || a->workspace_bytes < pl.ws_bytes) return SSM_ERR_WORKSPACE;
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;
  CbwdParams p{};
  p.u = a->u; p.delta = a->delta; p.B = a->B; p.C = a->C; p.z = a->z; p.dout = a->dout;
  p.A = a->A; p.D = a->D; p.dbias = a->delta_bias; p.ckpt = a->checkpoints;
  p.du = a->du; p.ddelta = a->ddelta; p.dz = a->dz;
  p.dA = a->dA; p.dB = a->dB; p.dC = a->dC; p.dD = a->dD; p.ddbias = a->ddelta_bias;
  p.dinit = a->dinitial_state;
  char *ws = static_cast<char *>(a->workspace);
  p.ws_bc = reinterpret_cast<float *>(ws + pl.off_bc);
  p.ws_dA = reinterpret_cast<float *>(ws + pl.off_dA);
  p.ws_fB = reinterpret_cast<float *>(ws + pl.off_fB);
  p.ws_fC = reinterpret_cast<float *>(ws + pl.off_fC);
  p.ws_dD = reinterpret_cast<float *>(ws + pl.off_dD);
  p.ws_db = reinterpret_cast<float *>(ws + pl.off_db);
  p.loc = pl.nseg > 1 ? reinterpret_cast<float *>(ws + pl.off_loc) : nullptr;
  p.pdec = pl.nseg > 1 ? reinterpret_cast<float *>(ws + pl.off_pdec) : nullptr;
  p.nseg = pl.nseg; p.seg0 = pl.seg0; p.segc = pl.segc;
  p.batch = a->batch; p.dim = a->dim; p.seqlen = a->seqlen;
  p.nck = pl.nck;
  p.cpg = pl.cpg;
  p.n = static_cast<int>(a->dstate); p.ngroups = static_cast<int>(a->ngroups);
  p.groups_eff = pl.groups_eff; p.nblk = pl.nblk;
  p.softplus = a->delta_softplus;
  const int64_t nwg = pl.nwg;
  int64_t nsum = a->dim * a->dstate;
  if (bv || cv) {
    const int64_t v = a->batch * a->ngroups * a->seqlen * a->dstate;
    if (v > nsum) nsum = v;
  }
  if (a->dim > nsum) nsum = a->dim;
  const int64_t sum_blocks = (nsum + 255) / 256;
  if (nwg > 0x7fffffffLL || sum_blocks > 0x7fffffffLL || pl.nseg > 65535) return SSM_ERR_SHAPE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  hipError_t e;
  if (pl.nseg > 1) {   // the carry pass over segments 1 .. nseg - 1
    CbwdFn fc = a->io_dtype == SSM_BF16 ? pick_ccarry<1>(cv) : a->io_dtype == SSM_F16 ? pick_ccarry<2>(cv)
                                                                                       : pick_ccarry<0>(cv);
    hipLaunchKernelGGL(fc, dim3(static_cast<unsigned>(nwg), static_cast<unsigned>(pl.nseg - 1)), dim3(512), 0,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  hipLaunchKernelGGL(cbwd_fn(a->io_dtype, bv, cv), dim3(static_cast<unsigned>(nwg), static_cast<unsigned>(pl.nseg)),
                     dim3(512), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  hipLaunchKernelGGL(cbwd_sum_kernel, dim3(static_cast<unsigned>(sum_blocks)), dim3(256), 0, stream, p,
                     static_cast<int>(bv), static_cast<int>(cv));
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
