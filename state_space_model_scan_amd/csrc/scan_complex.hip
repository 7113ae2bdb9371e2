// scan_complex.hip -- the selective-scan forward with complex A for gfx950,
// and its C-ABI entry point ssm_scan_fwd_complex.
//
// Operation: PaddleNLP Kernel operator-library guide, section 4.1
// (selective_scan_fn): A (dim, dstate) may be real or complex.  The page
// prints nothing more about the complex case; it is read as the same
// recurrence over the complex numbers, with B and C complex as well and the
// output the real part of the contraction (include/ssmscan.h):
//
//     x_t[s] = exp(delta'_t A[d,s]) x_{t-1}[s] + delta'_t B_t[s] u_t
//     y_t    = Re(sum_s C_t[s] x_t[s]),   out_t = (y_t + D u_t) silu(z_t)
//
// Complex values are (real, imaginary) pairs of the element type, the pair
// innermost.  The decay exp(delta' A) and delta' = softplus(delta + bias)
// are formed as complex_util.h describes: the hardware exp2, sine and cosine
// (in revolutions) on the fraction of delta' Im A / (2 pi), and the softplus
// without the cancellation of 1 + e^v.
//
// Work decomposition (the real kernel's, in scan_kernel.h): four lanes per
// channel, lane q holding complex states [q*NSW, (q+1)*NSW) in VGPRs; chunks
// of 32 timesteps, lane q owning timesteps [8q, 8q+8) of each chunk for the
// loads, delta' = softplus(delta + bias), delta'*u and the gated store;
// delta' and delta'*u reach the quad through LDS (stored by the owner once per
// chunk, read four timesteps at a time); time-varying B/C of a chunk are
// staged in the wave's LDS slice (complex pairs interleaved, as in memory)
// and read two timesteps ahead; the quad's partial Re(C.x) are summed with
// two DPP quad permutes per step and the owner of the timestep keeps the
// sum (unlike the real kernel, which sums them through LDS: here the LDS
// that would take, 8 KB a wave, is what limits the waves per compute
// unit).  The whole sequence is walked in one pass (no sequence split).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "complex_util.h"
#include "host_util.h"
#include "scan_kernel.h"
#include "ssmscan.h"

namespace ssm {
namespace {

constexpr int kBlockCh = 16;            // channels of a block: a four-lane wave's, or two eight-lane waves'
constexpr int kT = SSM_CKPT_INTERVAL;   // timesteps per chunk
static_assert(chunk_of(4) == kT && chunk_of(8) == kT, "a checkpoint at every chunk start");

// LDS floats of one wave: the B/C tile ([B, C][t][state][re, im]) and the
// delta' / delta'*u hand-off ([group of 4 timesteps][2][channel][4]).
constexpr int cplx_lds_floats(int nsw, int lpc, bool anyv) {
  return (anyv ? 2 * kT * nsw * lpc * 2 : 4) + (kT / 4) * 2 * (64 / lpc) * 4;
}

// The work of one wave: batch, B/C group and its first channel.
struct CplxWork {
  int64_t b;
  int g;
  int64_t d0;
};

struct CplxParams {
  const void *u, *delta, *B, *C, *z;
  const float *A, *D, *dbias, *init;
  void *out;
  float *last;
  float *ckpt;   // the state before every SSM_CKPT_INTERVAL-th timestep, or null
  int64_t batch, dim, seqlen, cpg, nck;
  int n, ngroups, groups_eff, nblk, nblocks;
  int softplus, vec, xcd_swizzle;
  int mix_whole, mix_small;   // mixed plan: four-lane waves, then eight-lane waves (0, 0: none)
};

// One wave's walk of its channels (LPC lanes per channel, NSW complex states
// a lane) over the whole sequence; its LDS slice is `lds`
// (cplx_lds_floats(NSW, LPC, BV || CV) floats, 16-byte aligned).
template <int IO, int NSW, int LPC, bool BV, bool CV>
__device__ __forceinline__ void cplx_body(const CplxParams &p, float *lds, const CplxWork wk) {
  constexpr bool ANYV = BV || CV;
  constexpr int KP = kp_of(LPC);        // timesteps each lane owns per chunk
  constexpr int CPW = 64 / LPC;         // channels per wave
  constexpr int NP = NSW * LPC;         // padded state count
  constexpr int PIECES = NP * (kT / 8); // B/C staging pieces: 8 timesteps of one state
  static_assert(PIECES <= 64, "one B/C piece per lane");

  // [B or C][timestep][state][re, im]
  auto sbc = [&](int tensor, int t, int st) -> float * { return lds + ((tensor * kT + t) * NP + st) * 2; };
  // delta' and delta'*u of timesteps 4g..4g+3 as [channel][4] each, for
  // every group g of the chunk (written by the owner, read by the channel's lanes)
  float *s_dd = lds + (ANYV ? 2 * kT * NP * 2 : 4);
  auto dd_at = [&](int g) -> float * { return &s_dd[g * 2 * CPW * 4]; };

  const int lane = threadIdx.x & 63;
  const int q = lane % LPC;
  const int cw_idx = lane / LPC;
  const int g = wk.g;
  const int64_t b = wk.b;
  const int64_t d_end = (g + 1) * p.cpg;
  const int64_t d = wk.d0 + cw_idx;
  const bool valid = d < d_end;
  const int64_t dl = valid ? d : d_end - 1;
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * p.seqlen;
  const int64_t seqlen = p.seqlen;
  const int s0 = q * NSW;
  const int n = p.n;
  const bool vec = p.vec != 0;

  float Ar[NSW], Ai[NSW], Bfr[NSW], Bfi[NSW], Cfr[NSW], Cfi[NSW], xr[NSW], xi[NSW];
#pragma unroll
  for (int k = 0; k < NSW; ++k) {
    const int s = s0 + k;
    const bool sv = s < n;
    const int64_t e = (dl * n + s) * 2;
    Ar[k] = sv ? p.A[e] * kLog2e : 0.0f;
    Ai[k] = sv ? p.A[e + 1] * kInv2PiF : 0.0f;
    Bfr[k] = (!BV && sv) ? load_io<IO>(p.B, e) : 0.0f;
    Bfi[k] = (!BV && sv) ? load_io<IO>(p.B, e + 1) : 0.0f;
    Cfr[k] = (!CV && sv) ? load_io<IO>(p.C, e) : 0.0f;
    Cfi[k] = (!CV && sv) ? load_io<IO>(p.C, e + 1) : 0.0f;
    xr[k] = (p.init && sv) ? p.init[(row * n + s) * 2] : 0.0f;
    xi[k] = (p.init && sv) ? p.init[(row * n + s) * 2 + 1] : 0.0f;
  }
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;
  const float Dd = p.D ? p.D[dl] : 0.0f;
  // element index of (b, g, state 0, t 0, re) in a varying B/C
  const int64_t bc_base = ((b * p.ngroups + g) * n) * seqlen * 2;

  const int own = q * KP;
  auto count = [&](int64_t c) {
    const int64_t tp0 = c + own;
    return static_cast<int>((seqlen - tp0 < KP) ? seqlen - tp0 : KP);
  };

  RawV<IO, KP> r_u, r_dl, r_z;
  r_u.zero(); r_dl.zero(); r_z.zero();
  auto fetch = [&](int64_t c) {
    const int64_t tp0 = c + own;
    const int cnt = count(c);
    r_u.load(p.u, rbase + tp0, cnt, vec);
    r_dl.load(p.delta, rbase + tp0, cnt, vec);
    if (p.z) r_z.load(p.z, rbase + tp0, cnt, vec);
  };

  // B/C tile of a chunk: lane v < PIECES loads 8 timesteps (16 io elements)
  // of one state of B and of C
  const int bc_s = lane / (kT / 8);
  const int bc_t0 = (lane % (kT / 8)) * 8;
  const bool bc_lane = ANYV && lane < PIECES;
  const bool bc_real = bc_lane && bc_s < n;
  RawV<IO, 8> rB0, rB1, rC0, rC1;
  rB0.zero(); rB1.zero(); rC0.zero(); rC1.zero();
  auto fetch_bc = [&](int64_t c) {
    if (bc_real) {
      const int64_t e = bc_base + (static_cast<int64_t>(bc_s) * seqlen + c + bc_t0) * 2;
      const int64_t left = seqlen - (c + bc_t0);
      const int ec = 2 * static_cast<int>(left < 8 ? left : 8);   // io elements in range
      if constexpr (BV) { rB0.load(p.B, e, ec, vec); rB1.load(p.B, e + 8, ec - 8, vec); }
      if constexpr (CV) { rC0.load(p.C, e, ec, vec); rC1.load(p.C, e + 8, ec - 8, vec); }
    }
  };
  auto stage_bc = [&]() {
    if (bc_lane) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const RawV<IO, 8> &sb = i < 4 ? rB0 : rB1;
        const RawV<IO, 8> &sc = i < 4 ? rC0 : rC1;
        if constexpr (BV) {
          sbc(0, bc_t0 + i, bc_s)[0] = sb.get(2 * (i & 3));
          sbc(0, bc_t0 + i, bc_s)[1] = sb.get(2 * (i & 3) + 1);
        }
        if constexpr (CV) {
          sbc(ANYV ? 1 : 0, bc_t0 + i, bc_s)[0] = sc.get(2 * (i & 3));
          sbc(ANYV ? 1 : 0, bc_t0 + i, bc_s)[1] = sc.get(2 * (i & 3) + 1);
        }
      }
    }
  };

  float dtv[KP], dtuv[KP], duv[KP], yv[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) { dtv[i] = dtuv[i] = duv[i] = yv[i] = 0.0f; }

  // FCc: a whole chunk, so no lane owns timesteps past the end
  auto prep = [&](int64_t c, auto FCc) {
    constexpr bool FC = decltype(FCc)::value;
    const int cnt = count(c);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const float uu = r_u.get(i);
      float dt = r_dl.get(i) + bias;
      if (p.softplus) dt = softplus_acc(dt);
      if (!FC && i >= cnt) dt = 0.0f;
      dtv[i] = dt;
      dtuv[i] = dt * uu;
      duv[i] = Dd * uu;
    }
  };

  struct StepIn {
    float dt, dtu, Br[NSW], Bi[NSW], Cr[NSW], Ci[NSW];
  };
  float4 dtq[2], dtuq[2];   // delta' and delta'*u of the current and next group of 4 timesteps
  auto load_in = [&](auto TT, StepIn &in) {
    constexpr int t = decltype(TT)::value;
    constexpr int gb = (t / 4) % 2;
    if constexpr (t % 4 == 0) {
      dtq[gb] = *reinterpret_cast<const float4 *>(dd_at(t / 4) + cw_idx * 4);
      dtuq[gb] = *reinterpret_cast<const float4 *>(dd_at(t / 4) + CPW * 4 + cw_idx * 4);
    }
    constexpr int e = t % 4;
    in.dt = e == 0 ? dtq[gb].x : e == 1 ? dtq[gb].y : e == 2 ? dtq[gb].z : dtq[gb].w;
    in.dtu = e == 0 ? dtuq[gb].x : e == 1 ? dtuq[gb].y : e == 2 ? dtuq[gb].z : dtuq[gb].w;
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
      if constexpr (BV) { in.Br[k] = sbc(0, t, s0 + k)[0]; in.Bi[k] = sbc(0, t, s0 + k)[1]; }
      else { in.Br[k] = Bfr[k]; in.Bi[k] = Bfi[k]; }
      if constexpr (CV) { in.Cr[k] = sbc(ANYV ? 1 : 0, t, s0 + k)[0]; in.Ci[k] = sbc(ANYV ? 1 : 0, t, s0 + k)[1]; }
      else { in.Cr[k] = Cfr[k]; in.Ci[k] = Cfi[k]; }
    }
  };

  // one timestep: complex state update, then this lane's part of Re(C.x)
  auto step = [&](auto TT, const StepIn &in) {
    constexpr int t = decltype(TT)::value;
    float y = 0.0f;
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
      float er, ei;
      cexp_plain(in.dt, Ar[k], Ai[k], er, ei);
      const float br = in.Br[k] * in.dtu, bi = in.Bi[k] * in.dtu;
      const float nr = fmaf(er, xr[k], fmaf(-ei, xi[k], br));
      const float ni = fmaf(er, xi[k], fmaf(ei, xr[k], bi));
      xr[k] = nr;
      xi[k] = ni;
      y = fmaf(in.Cr[k], nr, y);
      y = fmaf(-in.Ci[k], ni, y);
    }
    // Re(C.x) over the channel's states: lanes (0,1) and (2,3) first, then
    // the pairs (DPP quad permutes), then with eight lanes the two quads; the
    // owner of timestep t keeps it
    y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xf, 0xf, true));  // [1,0,3,2]
    y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xf, 0xf, true));  // [2,3,0,1]
    if constexpr (LPC == 8)   // and the other quad of the eight lanes (row_half_mirror)
      y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x141, 0xf, 0xf, true));
    if (q == t / KP) yv[t % KP] = y;
  };

  fetch(0);
  if constexpr (ANYV) fetch_bc(0);

  for (int64_t c = 0; c < seqlen; c += kT) {
    const int len = static_cast<int>((seqlen - c < kT) ? seqlen - c : kT);
    if (len == kT) prep(c, std::true_type{}); else prep(c, std::false_type{});
    // this lane's timesteps are groups own/4 .. own/4 + KP/4 - 1; the previous chunk's
    // reads of the rows are issued before these stores
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < KP / 4; ++j) {
      float *dp = dd_at((own >> 2) + j);
      *reinterpret_cast<float4 *>(dp + cw_idx * 4) = make_float4(dtv[4 * j], dtv[4 * j + 1], dtv[4 * j + 2], dtv[4 * j + 3]);
      *reinterpret_cast<float4 *>(dp + CPW * 4 + cw_idx * 4) =
          make_float4(dtuv[4 * j], dtuv[4 * j + 1], dtuv[4 * j + 2], dtuv[4 * j + 3]);
    }
    if constexpr (ANYV) stage_bc();
    wave_lds_sync();            // the slice is written before any lane reads it
    const RawV<IO, KP> z_cur = r_z;
    if (p.ckpt && valid) {   // the state before timestep c (the backward starts its chunks there)
      float *dst = p.ckpt + ((row * p.nck + c / kT) * n) * 2;
#pragma unroll
      for (int k = 0; k < NSW; ++k)
        if (s0 + k < n) {
          dst[(s0 + k) * 2] = xr[k];
          dst[(s0 + k) * 2 + 1] = xi[k];
        }
    }
    if (c + kT < seqlen) {
      fetch(c + kT);
      if constexpr (ANYV) fetch_bc(c + kT);
    }
    if (len == kT) {
      constexpr int AH = 2;
      StepIn in[AH + 1];
      load_in(std::integral_constant<int, 0>{}, in[0]);
      load_in(std::integral_constant<int, 1>{}, in[1]);
      static_for(std::make_integer_sequence<int, kT>{}, [&](auto TT) {
        constexpr int t = decltype(TT)::value;
        if constexpr (t + AH < kT) load_in(std::integral_constant<int, t + AH>{}, in[(t + AH) % (AH + 1)]);
        step(TT, in[t % (AH + 1)]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      static_for(std::make_integer_sequence<int, kT>{}, [&](auto TT) {
        if (decltype(TT)::value < len) {
          StepIn in1;
          load_in(TT, in1);
          step(TT, in1);
        }
      });
    }
    const int cnt = count(c);
    if (cnt > 0 && valid) {
      float o[KP];
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        float y = yv[i] + duv[i];
        if (p.z) y *= silu_f(z_cur.get(i));
        o[i] = y;
      }
      store_n<IO, KP>(p.out, rbase + c + own, o, cnt, vec);
    }
  }

  if (p.last && valid) {
#pragma unroll
    for (int k = 0; k < NSW; ++k)
      if (s0 + k < n) {
        p.last[(row * n + s0 + k) * 2] = xr[k];
        p.last[(row * n + s0 + k) * 2 + 1] = xi[k];
      }
  }
}

// 16-bit io: three waves per SIMD (at most 168 VGPRs), since the mixed plan
// needs q + 1 = 3 and the plain plan at 2.5 waves per SIMD runs its third
// waves beside the others.  fp32 io keeps its registers: under that cap its
// walk spills up to 55 dwords and the 2.8B-shaped layer ran 1235 us in the
// mixed plan against 1013 us uncapped in the plain one, so it takes the plain
// plan only.
template <int IO, int NSW, bool BV, bool CV>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(IO == SSM_F32 ? 1 : 3)))
scan_complex_kernel(const CplxParams p) {
  __shared__ __attribute__((aligned(16))) float lds[cplx_lds_floats(NSW, 4, BV || CV)];
  int bid = blockIdx.x;
  if (p.xcd_swizzle) bid = (bid & 7) * (p.nblocks >> 3) + (bid >> 3);
  const int blk = bid % p.nblk;
  const int rest = bid / p.nblk;
  CplxWork wk;
  wk.g = rest % p.groups_eff;
  wk.b = rest / p.groups_eff;
  wk.d0 = wk.g * p.cpg + static_cast<int64_t>(blk) * kBlockCh;
  cplx_body<IO, NSW, 4, BV, CV>(p, lds, wk);
}

// The mixed plan at dstate 13..16 (the real kernel's): workgroups below
// mix_whole are four-lane waves over 16-channel blocks; each block left over
// is covered by two eight-lane waves of 8 channels (two complex states per
// lane), each with about half the work, so every SIMD holds its whole waves
// and at most one half wave.
template <int IO, bool BV, bool CV>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) scan_complex_mix_kernel(const CplxParams p) {
  constexpr int L4 = cplx_lds_floats(4, 4, BV || CV), L8 = cplx_lds_floats(2, 8, BV || CV);
  __shared__ __attribute__((aligned(16))) float lds[L4 > L8 ? L4 : L8];
  const int nwhole = p.mix_whole;
  const int bid = blockIdx.x;
  const bool big = bid < nwhole;
  int unit, half = 0;
  if (big) {
    unit = p.xcd_swizzle ? (bid & 7) * (nwhole >> 3) + (bid >> 3) : bid;
  } else {
    int j = bid - nwhole;
    if (p.xcd_swizzle && p.mix_small % 8 == 0) j = (j & 7) * (p.mix_small >> 3) + (j >> 3);
    unit = nwhole + j / 2;
    half = j % 2;
  }
  const int blk = unit % p.nblk;
  const int rest = unit / p.nblk;
  CplxWork wk;
  wk.g = rest % p.groups_eff;
  wk.b = rest / p.groups_eff;
  wk.d0 = wk.g * p.cpg + static_cast<int64_t>(blk) * kBlockCh + 8 * half;
  if (big) cplx_body<IO, 4, 4, BV, CV>(p, lds, wk);
  else cplx_body<IO, 2, 8, BV, CV>(p, lds, wk);
}

using CplxFn = void (*)(const CplxParams);

template <int IO, int NSW>
CplxFn pick_cplx_bc(bool bv, bool cv) {
  if (bv && cv) return scan_complex_kernel<IO, NSW, true, true>;
  if (bv) return scan_complex_kernel<IO, NSW, true, false>;
  if (cv) return scan_complex_kernel<IO, NSW, false, true>;
  return scan_complex_kernel<IO, NSW, false, false>;
}
template <int IO>
CplxFn pick_cplx_mix(bool bv, bool cv) {
  if (bv && cv) return scan_complex_mix_kernel<IO, true, true>;
  if (bv) return scan_complex_mix_kernel<IO, true, false>;
  if (cv) return scan_complex_mix_kernel<IO, false, true>;
  return scan_complex_mix_kernel<IO, false, false>;
}
CplxFn cplx_mix_fn(int32_t io, bool bv, bool cv) {
  return io == SSM_BF16 ? pick_cplx_mix<1>(bv, cv) : io == SSM_F16 ? pick_cplx_mix<2>(bv, cv) : nullptr;
}
template <int IO>
CplxFn pick_cplx(int nsw, bool bv, bool cv) {
  if (nsw == 4) return pick_cplx_bc<IO, 4>(bv, cv);
  if (nsw == 2) return pick_cplx_bc<IO, 2>(bv, cv);
  return pick_cplx_bc<IO, 1>(bv, cv);
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssm_scan_fwd_complex(const ssm_scan_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_complex_validate(a);
  if (st != SSM_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int n = static_cast<int>(a->dstate);
  const int nsw = n > 8 ? 4 : n > 4 ? 2 : 1;   // four lanes per channel, 4*nsw >= n states
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;
  CplxParams p{};
  p.u = a->u; p.delta = a->delta; p.B = a->B; p.C = a->C; p.z = a->z;
  p.A = a->A; p.D = a->D; p.dbias = a->delta_bias; p.init = a->initial_state;
  p.out = a->out; p.last = a->last_state;
  p.ckpt = a->checkpoints;
  p.nck = (a->seqlen + SSM_CKPT_INTERVAL - 1) / SSM_CKPT_INTERVAL;
  p.batch = a->batch; p.dim = a->dim; p.seqlen = a->seqlen;
  p.n = n; p.ngroups = static_cast<int>(a->ngroups);
  p.groups_eff = (bv || cv) ? p.ngroups : 1;
  p.cpg = a->dim / p.groups_eff;
  p.nblk = static_cast<int>((p.cpg + kBlockCh - 1) / kBlockCh);
  const int64_t nblocks = a->batch * p.groups_eff * p.nblk;
  if (nblocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  p.nblocks = static_cast<int>(nblocks);
  p.softplus = a->delta_softplus;
  p.vec = (a->seqlen % 8 == 0) && aligned16(a->u) && aligned16(a->delta) && aligned16(a->out) &&
          (!a->z || aligned16(a->z)) && (!bv || aligned16(a->B)) && (!cv || aligned16(a->C));
  // mixed plan (as the real forward's), 16-bit io: q >= 2 whole waves per
  // SIMD and r blocks over become 2r half waves, provided q + 1 waves fit a SIMD
  p.mix_whole = p.mix_small = 0;
  if (nsw == 4 && a->io_dtype != SSM_F32) {
    const int simds = 4 * cu_count_cached();
    const int q = p.nblocks / simds, r = p.nblocks % simds;
    if (q >= 2 && r > 0 && 2 * r <= simds &&
        4 * (q + 1) <= blocks_per_cu(reinterpret_cast<const void *>(cplx_mix_fn(a->io_dtype, bv, cv)), 64)) {
      p.mix_whole = p.nblocks - r;
      p.mix_small = 2 * r;
    }
  }
  p.xcd_swizzle = p.mix_small ? (p.mix_whole % 8 == 0) : (p.nblocks % 8 == 0);
  CplxFn f = p.mix_small ? cplx_mix_fn(a->io_dtype, bv, cv)
           : a->io_dtype == SSM_BF16 ? pick_cplx<1>(nsw, bv, cv)
           : a->io_dtype == SSM_F16  ? pick_cplx<2>(nsw, bv, cv)
                                     : pick_cplx<0>(nsw, bv, cv);
  const int grid = p.mix_small ? p.mix_whole + p.mix_small : p.nblocks;
  hipLaunchKernelGGL(f, dim3(grid), dim3(64), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
