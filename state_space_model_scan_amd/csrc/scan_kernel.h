// scan_kernel.h -- the selective-scan forward kernel for gfx950.
//
// Operation: PaddleNLP Kernel operator-library guide, section 4.1
// (selective_scan_fn: u, delta, A, B, C, D, z, delta_bias, delta_softplus,
// last_state) with the optional section 4.2 conv prologue; the recurrence is
// the zero-order-hold discretisation written out in include/ssmscan.h.
//
// Work decomposition.  Every wave is self-contained (no barrier, no LDS
// traffic between waves):
//   * a channel (b, d) is owned by LPC adjacent lanes ("a quad" at dstate 16);
//     lane q of the quad carries states [q*NSW, (q+1)*NSW) in VGPRs and walks
//     the sequence in order -- per (timestep, state) one exp2, one multiply
//     for delta'*A, one multiply for delta'*u*B, one FMA for the state and
//     one FMA for C.x, the plain recurrence with no parallel-scan overhead;
//   * the sequence is walked in chunks of T = 8*LPC timesteps.  Lane q owns
//     timesteps [8q, 8q+8) of each chunk: it loads them as one vector per
//     input, computes delta' = softplus(delta + bias), delta'*u and D*u in
//     registers, and after the chunk gates and stores its 8 outputs;
//   * the owner writes delta' and delta'*u of its timesteps to the wave's LDS
//     slice once per chunk, and every lane of the channel reads them four
//     timesteps at a time (one 16-byte read each; cross-lane DPP moves per
//     timestep cost more); every lane writes its partial C.x to the slice,
//     and after the chunk the owner sums the LPC partials of its timesteps;
//   * time-varying B/C are the same for every channel of a wave: the wave
//     stages the chunk's B/C tile (all states) in its own LDS slice, and lane
//     q reads its NSW states of timestep t with one LDS vector load each, two
//     timesteps ahead of their use;
//   * the global loads of chunk c+1 are issued before the recurrence of chunk
//     c, so their latency hides behind it;
//   * when batch*dim is too small to fill the GPU the sequence is cut into
//     segments: a first pass (MODE_STATE) computes each segment's end state
//     from zero and its summed step; the second pass (MODE_FULL) starts every
//     segment from the exact carried state
//       x_in(k) = E_{k-1} + exp(A * S_{k-1}) * (E_{k-2} + exp(A * S_{k-2}) * ...)
//     with E_j the end state of segment j from zero and S_j its summed step:
//     the same recurrence, reassociated.
#pragma once

#include "device_util.h"
#include "ssmscan.h"

namespace ssm {

struct ScanParams {
  const void *u, *delta, *B, *C, *z, *cx;
  const float *A, *D, *dbias, *init, *cw, *cb;
  void *out;
  float *last;
  float *ws_state, *ws_sumdt;
  float *ckpt;           // saved states for the backward, or null
  int64_t batch, dim, seqlen, seg_len, cpg, nck;
  int n, n_pad, ngroups, groups_eff, nblk, nseg, nblocks;
  int softplus, conv_silu, vec, xcd_swizzle;
};

enum { MODE_STATE = 0, MODE_FULL = 1 };

constexpr int kWavesPerBlock = 1;   // every wave is independent
constexpr int kKP = 8;                                   // timesteps each lane owns per chunk
constexpr int chunk_of(int lpc) { return kKP * lpc; }    // chunk length
constexpr int channels_per_block(int lpc) { return kWavesPerBlock * 64 / lpc; }

// DPP quad_perm control word broadcasting lane SRC of each group of LPC lanes.
template <int LPC, int SRC>
constexpr int quad_bcast_ctrl() {
  if constexpr (LPC == 4) return SRC | (SRC << 2) | (SRC << 4) | (SRC << 6);
  else return SRC | (SRC << 2) | ((2 + SRC) << 4) | ((2 + SRC) << 6);   // LPC == 2
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  // every lane reads a lane of its own quad, so bound_ctrl never applies and
  // no "old" value has to be materialised
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// A broadcast value used by several multiplies: one DPP move, then plain
// operands (the empty asm keeps the compiler from folding the DPP into every
// use, which would make each of them a slower DPP instruction).
template <int CTRL>
__device__ __forceinline__ float dpp_bcast_reg(float v) {
  float r = dpp_mov<CTRL>(v);
  asm volatile("" : "+v"(r));
  return r;
}

// Keep the compiler from moving LDS accesses across this point and wait for
// this wave's LDS operations: the lanes of a wave hand data to each other
// through LDS, which per-thread alias analysis cannot see.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int IO, int NSW, int LPC, bool BV, bool CV, bool CONV, int MODE>
__global__ void __launch_bounds__(64 * kWavesPerBlock)
scan_kernel(const ScanParams p) {
  constexpr bool FULL = MODE == MODE_FULL;
  constexpr bool ANYV = BV || CV;
  constexpr int T = chunk_of(LPC);      // timesteps per chunk
  constexpr int NP = NSW * LPC;         // padded state count
  constexpr int CPW = 64 / LPC;         // channels per wave
  // B/C staging: pieces of 8 consecutive timesteps of one state
  constexpr int PIECES = NP * (T / 8);
  static_assert(PIECES <= 64, "one B/C piece per lane");
  static_assert(NSW == 1 || NSW == 2 || NSW == 4, "states per lane");

  __shared__ float s_bc[ANYV ? kWavesPerBlock : 1][ANYV ? 2 : 1][ANYV ? T : 1][ANYV ? NP : 1];
  constexpr bool XCH = LPC > 1;          // lanes of a channel exchange data
  // partial C.x of every (timestep, channel, lane) of the chunk; the row of
  // timestep t starts at t*CPW*LPC + 8*(t/8), so the owner's reads of its
  // timesteps (rows 8 apart) spread over the banks
  constexpr int YROW_SKEW = 8;
  __shared__ __attribute__((aligned(16))) float s_yp[(XCH && FULL) ? T * CPW * LPC + YROW_SKEW * (T / 8) : 4];
  auto yrow = [](int t) { return t * CPW * LPC + YROW_SKEW * (t / 8); };
  // delta' and delta'*u of timestep group g (timesteps 4g..4g+3) as
  // [channel][4] each.  In the full pass they sit in the C.x rows of the
  // group's first timesteps: every lane reads a group before the step that
  // first overwrites those rows (LDS operations of a wave complete in order).
  __shared__ __attribute__((aligned(16))) float s_dd[(XCH && !FULL) ? T * CPW * 2 : 4];
  auto dd_at = [&](int g) -> float * { return FULL ? &s_yp[yrow(4 * g)] : &s_dd[g * 2 * CPW * 4]; };

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q = lane % LPC;             // state group of this lane within its channel
  const int cw_idx = lane / LPC;        // channel within the wave

  // Block -> (batch, channel group, channel block).  Consecutive logical
  // blocks share B/C; the hardware deals blocks to the 8 XCDs round-robin, so
  // the remap keeps the blocks of one group on one XCD's L2.
  int bid = blockIdx.x;
  if (p.xcd_swizzle) bid = (bid & 7) * (p.nblocks >> 3) + (bid >> 3);
  const int blk = bid % p.nblk;
  const int rest = bid / p.nblk;
  const int g = rest % p.groups_eff;
  const int64_t b = rest / p.groups_eff;
  const int64_t d_end = (g + 1) * p.cpg;
  const int64_t d = g * p.cpg + static_cast<int64_t>(blk) * (kWavesPerBlock * CPW) + w * CPW + cw_idx;
  const bool valid = d < d_end;
  const int64_t dl = valid ? d : d_end - 1;
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * p.seqlen;
  const int64_t BD = p.batch * p.dim;
  const int seg = blockIdx.y;
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = (t_begin + p.seg_len < p.seqlen) ? t_begin + p.seg_len : p.seqlen;
  const int s0 = q * NSW;
  const int n = p.n;
  const bool vec = p.vec != 0;

  // ---- per-lane parameters
  float Ap[NSW], Bf[NSW], Cf[NSW], x[NSW];
#pragma unroll
  for (int k = 0; k < NSW; ++k) {
    const int s = s0 + k;
    const bool sv = s < n;
    Ap[k] = sv ? p.A[dl * n + s] * kLog2e : 0.0f;
    Bf[k] = (!BV && sv) ? load_io<IO>(p.B, dl * n + s) : 0.0f;
    Cf[k] = (!CV && sv) ? load_io<IO>(p.C, dl * n + s) : 0.0f;
    x[k] = 0.0f;
  }
  const float bias = p.dbias ? p.dbias[dl] : 0.0f;
  const float Dd = p.D ? p.D[dl] : 0.0f;
  float cw0 = 0, cw1 = 0, cw2 = 0, cw3 = 0, cbias = 0;
  if constexpr (CONV) {
    cw0 = p.cw[dl * 4 + 0]; cw1 = p.cw[dl * 4 + 1]; cw2 = p.cw[dl * 4 + 2]; cw3 = p.cw[dl * 4 + 3];
    cbias = p.cb ? p.cb[dl] : 0.0f;
  }
  const int64_t bc_base = ((b * p.ngroups + g) * n) * p.seqlen;

  // ---- initial state: the caller's, or the carry over earlier segments
  if (seg == 0) {
    if (p.init) {
#pragma unroll
      for (int k = 0; k < NSW; ++k)
        if (s0 + k < n) x[k] = p.init[row * n + s0 + k];
    }
  } else if constexpr (FULL) {
#pragma unroll
    for (int k = 0; k < NSW; ++k) x[k] = p.ws_state[static_cast<int64_t>(s0 + k) * BD + row];
    for (int j = 1; j < seg; ++j) {
      const float sdt = p.ws_sumdt[static_cast<int64_t>(j) * BD + row];
#pragma unroll
      for (int k = 0; k < NSW; ++k) {
        const float e = fast_exp2(sdt * Ap[k]);
        x[k] = fmaf(e, x[k], p.ws_state[(static_cast<int64_t>(j) * p.n_pad + s0 + k) * BD + row]);
      }
    }
  }

  // ---- this lane's timesteps of a chunk: [c + 8q, c + 8q + 8)
  const int own = q * kKP;
  auto count = [&](int64_t c) {
    const int64_t tp0 = c + own;
    return static_cast<int>((t_end - tp0 < kKP) ? t_end - tp0 : kKP);
  };

  // global inputs of the next chunk, loaded before the current recurrence
  RawV<IO, kKP> r_a, r_dl, r_z, r_h;   // u (or conv x), delta, z, conv halo
  r_a.zero(); r_dl.zero(); r_z.zero(); r_h.zero();
  auto fetch = [&](int64_t c) {
    const int64_t tp0 = c + own;
    const int cnt = count(c);
    r_a.load(CONV ? p.cx : p.u, rbase + tp0, cnt, vec);
    r_dl.load(p.delta, rbase + tp0, cnt, vec);
    if (FULL && p.z) r_z.load(p.z, rbase + tp0, cnt, vec);
    if constexpr (CONV) {
      // the three samples before tp0 land in slots 5..7 (zero before t = 0)
      if (vec && tp0 >= kKP) {
        r_h.load_vec(p.cx, rbase + tp0 - kKP);
      } else {
        r_h.zero();
#pragma unroll
        for (int i = kKP - 3; i < kKP; ++i) {
          const int64_t t = tp0 - kKP + i;
          if (t >= 0 && t < p.seqlen) r_h.load_one(p.cx, rbase + t, i);
        }
      }
    }
  };

  // B/C tile of a chunk: lane v < PIECES loads 8 timesteps of one state of B
  // and of C (rows of the (b, g) group), and writes them transposed to LDS.
  const int bc_s = lane / (T / 8);
  const int bc_t0 = (lane % (T / 8)) * 8;
  const bool bc_lane = ANYV && lane < PIECES;
  const bool bc_real = bc_lane && bc_s < n;
  RawV<IO, 8> r_B, r_C;
  r_B.zero(); r_C.zero();
  auto fetch_bc = [&](int64_t c) {
    if (bc_real) {
      const int64_t e = bc_base + static_cast<int64_t>(bc_s) * p.seqlen + c + bc_t0;
      const int64_t left = t_end - (c + bc_t0);
      const int cnt = static_cast<int>(left < 8 ? left : 8);
      if constexpr (BV) r_B.load(p.B, e, cnt, vec);
      if constexpr (CV && FULL) r_C.load(p.C, e, cnt, vec);
    }
  };
  auto stage_bc = [&]() {
    if (bc_lane) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (BV) s_bc[ANYV ? w : 0][0][bc_t0 + i][bc_s] = r_B.get(i);
        if constexpr (CV && FULL) s_bc[ANYV ? w : 0][ANYV ? 1 : 0][bc_t0 + i][bc_s] = r_C.get(i);
      }
    }
  };

  // per-lane chunk values for its own timesteps
  float dtv[kKP], dtuv[kKP], duv[kKP], yv[kKP];
#pragma unroll
  for (int i = 0; i < kKP; ++i) { dtv[i] = dtuv[i] = duv[i] = yv[i] = 0.0f; }

  // CSc: silu after the conv; FCc: a whole chunk, so no lane owns timesteps
  // past the end and none needs masking (compile-time constants, chosen once
  // per chunk)
  auto prep = [&](int64_t c, auto CSc, auto FCc) {
    constexpr bool CS = decltype(CSc)::value;
    constexpr bool FC = decltype(FCc)::value;
    float uu[kKP];
    if constexpr (CONV) {
      float xv[kKP + 3];
      xv[0] = r_h.get(kKP - 3); xv[1] = r_h.get(kKP - 2); xv[2] = r_h.get(kKP - 1);
#pragma unroll
      for (int i = 0; i < kKP; ++i) xv[i + 3] = r_a.get(i);
#pragma unroll
      for (int i = 0; i < kKP; ++i) {
        float acc = cbias;
        acc = fmaf(cw0, xv[i], acc);
        acc = fmaf(cw1, xv[i + 1], acc);
        acc = fmaf(cw2, xv[i + 2], acc);
        acc = fmaf(cw3, xv[i + 3], acc);
        if constexpr (CS) acc = silu_f(acc);
        uu[i] = round_io<IO>(acc);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKP; ++i) uu[i] = r_a.get(i);
    }
    const int cnt = count(c);
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      float dt = r_dl.get(i) + bias;
      if (p.softplus) dt = softplus_f(dt);
      if (!FC && i >= cnt) dt = 0.0f;
      dtv[i] = dt;
      dtuv[i] = dt * uu[i];
      duv[i] = Dd * uu[i];
    }
  };
  auto gather_y = [&]() {     // sum of the quad's partial C.x of this lane's timesteps
    if constexpr (XCH && FULL) {
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < kKP; ++i) {
        const float *yp = &s_yp[yrow(own + i) + cw_idx * LPC];
        float y = yp[0];
#pragma unroll
        for (int k = 1; k < LPC; ++k) y += yp[k];
        yv[i] = y;
      }
    }
  };

  auto epilogue = [&](int64_t c) {
    const int cnt = count(c);
    if (cnt <= 0 || !valid) return;
    float o[kKP];
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      float y = yv[i] + duv[i];
      if (p.z) y *= silu_f(r_z.get(i));
      o[i] = y;
    }
    store_n<IO, kKP>(p.out, rbase + c + own, o, cnt, vec);
  };

  float sumdt = 0.0f;   // summed delta' of the segment (MODE_STATE)

  // operands of timestep t of the chunk: (delta', delta'*u) and this lane's
  // B/C values (LDS, registers or fixed)
  struct StepIn {
    float dt, dtu, Bv[NSW], Cv[NSW];
  };
  float4 dtq[2], dtuq[2];   // delta' and delta'*u of the current and next group of 4 timesteps
  auto load_in = [&](auto TT, StepIn &in) {
    constexpr int t = decltype(TT)::value;
    if constexpr (XCH) {
      constexpr int gb = (t / 4) % 2;
      if constexpr (t % 4 == 0) {
        dtq[gb] = *reinterpret_cast<const float4 *>(dd_at(t / 4) + cw_idx * 4);
        dtuq[gb] = *reinterpret_cast<const float4 *>(dd_at(t / 4) + CPW * 4 + cw_idx * 4);
      }
      constexpr int e = t % 4;
      in.dt = e == 0 ? dtq[gb].x : e == 1 ? dtq[gb].y : e == 2 ? dtq[gb].z : dtq[gb].w;
      in.dtu = e == 0 ? dtuq[gb].x : e == 1 ? dtuq[gb].y : e == 2 ? dtuq[gb].z : dtuq[gb].w;
    } else {
      in.dt = dtv[t % kKP];
      in.dtu = dtuv[t % kKP];
    }
    if constexpr (ANYV) {
      const float *rowB = &s_bc[ANYV ? w : 0][0][t][s0];
      const float *rowC = &s_bc[ANYV ? w : 0][ANYV ? 1 : 0][t][s0];
#pragma unroll
      for (int k = 0; k < NSW; ++k) {
        in.Bv[k] = BV ? rowB[k] : Bf[k];
        in.Cv[k] = (CV && FULL) ? rowC[k] : Cf[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < NSW; ++k) { in.Bv[k] = Bf[k]; in.Cv[k] = Cf[k]; }
    }
  };

  // one timestep t (0 <= t < T) of the chunk
  auto step = [&](auto TT, const StepIn &in) {
    constexpr int t = decltype(TT)::value;
    if constexpr (!FULL) sumdt += in.dt;
#pragma unroll
    for (int k = 0; k < NSW; ++k) {
      const float e = fast_exp2(in.dt * Ap[k]);
      x[k] = fmaf(e, x[k], in.Bv[k] * in.dtu);
    }
    if constexpr (FULL) {
      float y = in.Cv[0] * x[0];
#pragma unroll
      for (int k = 1; k < NSW; ++k) y = fmaf(in.Cv[k], x[k], y);
      if constexpr (XCH) s_yp[yrow(t) + cw_idx * LPC + q] = y;
      else yv[t % kKP] = y;
    }
  };

  fetch(t_begin);
  if constexpr (ANYV) fetch_bc(t_begin);

  for (int64_t c = t_begin; c < t_end; c += T) {
    const int len = static_cast<int>((t_end - c < T) ? t_end - c : T);
    const bool csilu = CONV && p.conv_silu;
    if constexpr (FULL) {
      // the state before timestep c, every SSM_CKPT_INTERVAL timesteps
      if (p.ckpt && valid && (c % SSM_CKPT_INTERVAL) == 0) {
        float *dst = p.ckpt + (row * p.nck + c / SSM_CKPT_INTERVAL) * n;
#pragma unroll
        for (int k = 0; k < NSW; ++k)
          if (s0 + k < n) dst[s0 + k] = x[k];
      }
    }
    if (len == T) {
      if (csilu) prep(c, std::true_type{}, std::true_type{}); else prep(c, std::false_type{}, std::true_type{});
    } else {
      if (csilu) prep(c, std::true_type{}, std::false_type{}); else prep(c, std::false_type{}, std::false_type{});
    }
    if constexpr (XCH) {
      // this lane's timesteps are groups 2q and 2q+1; the previous chunk's
      // reads of the slice are issued before these stores
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float *dp = dd_at((own >> 2) + j);
        *reinterpret_cast<float4 *>(dp + cw_idx * 4) = make_float4(dtv[4 * j], dtv[4 * j + 1], dtv[4 * j + 2], dtv[4 * j + 3]);
        *reinterpret_cast<float4 *>(dp + CPW * 4 + cw_idx * 4) =
            make_float4(dtuv[4 * j], dtuv[4 * j + 1], dtuv[4 * j + 2], dtuv[4 * j + 3]);
      }
      if constexpr (!ANYV) wave_lds_sync();   // with B/C staging the sync below covers these
    }
    if constexpr (ANYV) {
      wave_lds_sync();          // the previous chunk's reads of the slice are done
      stage_bc();
      wave_lds_sync();          // the slice is written before any lane reads it
    }
    const RawV<IO, kKP> z_cur = r_z;
    if (c + T < t_end) {
      fetch(c + T);
      if constexpr (ANYV) fetch_bc(c + T);
    }
    if (len == T) {
      // whole chunk, fully unrolled; operands read from LDS two timesteps
      // ahead of their use so the LDS latency hides behind the recurrence
      constexpr int AH = 2;
      StepIn in[AH + 1];
      load_in(std::integral_constant<int, 0>{}, in[0]);
      load_in(std::integral_constant<int, 1>{}, in[1]);
      static_for(std::make_integer_sequence<int, T>{}, [&](auto TT) {
        constexpr int t = decltype(TT)::value;
        if constexpr (t + AH < T) load_in(std::integral_constant<int, t + AH>{}, in[(t + AH) % (AH + 1)]);
        step(TT, in[t % (AH + 1)]);
        // keep the lookahead loads where they are written: without the fence
        // the scheduler sinks them next to their use and every step waits on LDS
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      // ragged last chunk of a segment: timesteps past the end are skipped
      static_for(std::make_integer_sequence<int, T>{}, [&](auto TT) {
        if (decltype(TT)::value < len) {
          StepIn in1;
          load_in(TT, in1);
          step(TT, in1);
        }
      });
    }
    if constexpr (XCH && FULL) gather_y();   // sum of the quad's partial C.x
    if constexpr (FULL) {
      const RawV<IO, kKP> z_next = r_z;
      r_z = z_cur;
      epilogue(c);
      r_z = z_next;
    }
  }

  if constexpr (FULL) {
    if (p.last && seg == p.nseg - 1 && valid) {
#pragma unroll
      for (int k = 0; k < NSW; ++k)
        if (s0 + k < n) p.last[row * n + s0 + k] = x[k];
    }
  } else {
    if (valid) {
#pragma unroll
      for (int k = 0; k < NSW; ++k)
        p.ws_state[(static_cast<int64_t>(seg) * p.n_pad + s0 + k) * BD + row] = x[k];
      if (q == 0) p.ws_sumdt[static_cast<int64_t>(seg) * BD + row] = sumdt;
    }
  }
}

using ScanFn = void (*)(const ScanParams);

// Kernel instance for a plan.  (nsw, lpc) is one of (4,4), (4,2), (4,1),
// (2,1), (1,1): n_pad = nsw * lpc states.
template <int IO, int NSW, int LPC, bool BV, bool CV, bool CONV>
ScanFn pick_mode(int mode) {
  return mode == MODE_FULL ? scan_kernel<IO, NSW, LPC, BV, CV, CONV, MODE_FULL>
                           : scan_kernel<IO, NSW, LPC, BV, CV, CONV, MODE_STATE>;
}
template <int IO, int NSW, int LPC, bool BV, bool CV>
ScanFn pick_conv(bool conv, int mode) {
  return conv ? pick_mode<IO, NSW, LPC, BV, CV, true>(mode) : pick_mode<IO, NSW, LPC, BV, CV, false>(mode);
}
template <int IO, int NSW, int LPC>
ScanFn pick_bc(bool bv, bool cv, bool conv, int mode) {
  if (bv && cv) return pick_conv<IO, NSW, LPC, true, true>(conv, mode);
  if (bv) return pick_conv<IO, NSW, LPC, true, false>(conv, mode);
  if (cv) return pick_conv<IO, NSW, LPC, false, true>(conv, mode);
  return pick_conv<IO, NSW, LPC, false, false>(conv, mode);
}
template <int IO>
ScanFn pick_scan(int nsw, int lpc, bool bv, bool cv, bool conv, int mode) {
  if (nsw == 4 && lpc == 4) return pick_bc<IO, 4, 4>(bv, cv, conv, mode);
  if (nsw == 4 && lpc == 2) return pick_bc<IO, 4, 2>(bv, cv, conv, mode);
  if (nsw == 4 && lpc == 1) return pick_bc<IO, 4, 1>(bv, cv, conv, mode);
  if (nsw == 2 && lpc == 1) return pick_bc<IO, 2, 1>(bv, cv, conv, mode);
  if (nsw == 1 && lpc == 1) return pick_bc<IO, 1, 1>(bv, cv, conv, mode);
  return nullptr;
}

// Defined in scan_f32.hip / scan_bf16.hip / scan_f16.hip (one translation
// unit per io dtype).
ScanFn pick_scan_f32(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);
ScanFn pick_scan_f16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);
ScanFn pick_scan_bf16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);

}  // namespace ssm
