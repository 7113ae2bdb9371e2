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
//     the same recurrence, reassociated;
//   * when the waves do not divide evenly over the SIMDs (the Mamba-2.8B
//     layer gives 2560 waves of 16 channels for 1024 SIMDs), the channel
//     blocks left over are run by waves of eight lanes per channel (two
//     states each, 8 channels, four timesteps per lane and chunk): two such
//     waves per block, each with about half the work, so every SIMD gets its
//     whole waves plus at most one half wave (scan_mix_kernel).
#pragma once

#include "device_util.h"
#include "ssmscan.h"

namespace ssm {

struct ScanParams {
  const void *u, *delta, *B, *C, *z, *cx;
  const float *A, *D, *dbias, *init, *cw, *cb;
  void *out;
  float *last;
  float *ws_state, *ws_sumdt;   // segment plan: end states from zero, summed steps
  float *ckpt;                  // saved states for the backward, or null
  int64_t batch, dim, seqlen, seg_len, cpg, nck;
  int n, n_pad, ngroups, groups_eff, nblk, nseg, nblocks;
  int mix_whole, mix_small;     // mixed plan: four-lane waves, then eight-lane waves
  int softplus, conv_silu, xcd_swizzle;
};

enum { MODE_STATE = 0, MODE_FULL = 1 };

constexpr int kKP = 8;   // timesteps a lane owns per chunk (complex kernel; the real one uses kp_of)
// Timesteps a lane owns per chunk, and the chunk length, for LPC lanes per
// channel: 8 per lane up to four lanes per channel (chunks of 8, 16, 32), 4
// per lane with eight lanes per channel (chunks of 32), so the LDS of a wave
// stays the same.
constexpr int kp_of(int lpc) { return lpc >= 8 ? 4 : 8; }
constexpr int chunk_of(int lpc) { return kp_of(lpc) * lpc; }
constexpr int channels_per_block(int lpc) { return 64 / lpc; }

// LDS floats of one wave of the kernel: the B/C tile (both tensors), the
// partial C.x rows (full pass) or the delta' / delta'*u hand-off (state pass).
constexpr int round4(int v) { return (v + 3) / 4 * 4; }
constexpr int lds_floats(int nsw, int lpc, bool anyv, bool full) {
  return round4(anyv ? 2 * chunk_of(lpc) * nsw * lpc : 0) +
         round4((lpc > 1 && full) ? chunk_of(lpc) * 64 + 8 * (chunk_of(lpc) / 8) : 0) +
         ((lpc > 1 && !full) ? chunk_of(lpc) * (64 / lpc) * 2 : 0) + 4;
}

// The work of one wave: batch, B/C group, its first channel and its
// segment of the sequence.
struct WaveWork {
  int64_t b;
  int g;
  int64_t d0;
  int seg;
};

// Keep the compiler from moving LDS accesses across this point and wait for
// this wave's LDS operations: the lanes of a wave hand data to each other
// through LDS, which per-thread alias analysis cannot see.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// VEC: every io pointer is 16-byte aligned and seqlen % 8 == 0, so every
// owned 8-timestep range and every B/C piece is either whole or past the
// end, and is moved as one vector; otherwise element by element.
template <int IO, int NSW, int LPC, bool BV, bool CV, bool CONV, int MODE, bool VEC>
__device__ __forceinline__ void scan_body(const ScanParams &p, float *lds, const WaveWork wk) {
  constexpr bool FULL = MODE == MODE_FULL;
  constexpr bool ANYV = BV || CV;
  constexpr int kKP = kp_of(LPC);       // timesteps each lane owns per chunk
  constexpr int T = chunk_of(LPC);      // timesteps per chunk
  constexpr int NP = NSW * LPC;         // padded state count
  constexpr int CPW = 64 / LPC;         // channels per wave
  // B/C staging: pieces of 8 consecutive timesteps of one state
  constexpr int PIECES = NP * (T / 8);
  static_assert(PIECES <= 64, "one B/C piece per lane");
  static_assert(NSW == 1 || NSW == 2 || NSW == 4, "states per lane");

  // The wave's LDS (lds_floats of these parameters, 16-byte aligned):
  //   s_bc[2][T][NP]: the chunk's B and C tile, fp32;
  //   s_yp: partial C.x of every (timestep, channel, lane) of the chunk; the
  //     row of timestep t starts at t*CPW*LPC + 8*(t/8), so the owner's reads
  //     of its timesteps (rows 8 apart) spread over the banks;
  //   s_dd: the state pass's delta' / delta'*u hand-off.
  constexpr bool XCH = LPC > 1;          // lanes of a channel exchange data
  constexpr int YROW_SKEW = 8;
  float *s_bc = lds;
  float *s_yp = lds + round4(ANYV ? 2 * T * NP : 0);
  float *s_dd = s_yp + round4((XCH && FULL) ? T * CPW * LPC + YROW_SKEW * (T / 8) : 0);
  auto sbc = [&](int tensor, int t) -> float * { return s_bc + (tensor * T + t) * NP; };
  auto yrow = [](int t) { return t * CPW * LPC + YROW_SKEW * (t / 8); };
  // delta' and delta'*u of timestep group g (timesteps 4g..4g+3) as
  // [channel][4] each.  In the full pass they sit in the C.x rows of the
  // group's first timesteps: every lane reads a group before the step that
  // first overwrites those rows (LDS operations of a wave complete in order).
  auto dd_at = [&](int g) -> float * { return FULL ? &s_yp[yrow(4 * g)] : &s_dd[g * 2 * CPW * 4]; };

  const int lane = threadIdx.x & 63;
  const int q = lane % LPC;             // state group of this lane within its channel
  const int cw_idx = lane / LPC;        // channel within the wave
  const int64_t b = wk.b;
  const int g = wk.g;
  const int seg = wk.seg, nsegs = p.nseg;
  const int64_t d_end = (g + 1) * p.cpg;
  const int64_t d = wk.d0 + cw_idx;
  const bool valid = d < d_end;
  const int64_t dl = valid ? d : d_end - 1;
  const int64_t row = b * p.dim + dl;
  const int64_t rbase = row * p.seqlen;
  const int64_t BD = p.batch * p.dim;
  const int64_t t_begin = nsegs > 1 ? seg * p.seg_len : 0;
  const int64_t t_end = (nsegs > 1 && t_begin + p.seg_len < p.seqlen) ? t_begin + p.seg_len : p.seqlen;
  const int s0 = q * NSW;
  const int n = p.n;

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
  } else {
    if constexpr (FULL) {
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
  }

  // ---- this lane's timesteps of a chunk: [c + 8q, c + 8q + 8)
  const int own = q * kKP;
  auto count = [&](int64_t c) {
    const int64_t tp0 = c + own;
    return static_cast<int>((t_end - tp0 < kKP) ? t_end - tp0 : kKP);
  };

  // Raw global inputs of a chunk.  Two sets alternate (the chunk loop is
  // unrolled by two), so no loop-carried copy waits on the loads in flight.
  // D*u of the owned timesteps is kept for the epilogue only where u is not
  // in the set as loaded (conv prologue) or takes an unpacking op (16-bit
  // io); with fp32 io the epilogue forms it from the raw u, which leaves the
  // full pass enough registers for three waves per SIMD.
  constexpr bool KEEP_DU = CONV || IO != 0;
  struct RawSet {
    RawV<IO, kKP> a, dl, z, h;   // u (or conv x), delta, z, the 8 samples before (conv halo)
    RawV<IO, 8> B, C;            // this lane's piece of the chunk's B / C tile
    float du[KEEP_DU ? kKP : 1]; // D*u of the owned timesteps (prepared, for the epilogue)
  };
  // VEC: one unconditional vector load per input.  A range past the end of
  // the time range reads the row's last vector instead (those values only
  // ever meet delta' = 0, a zero input term or an output that is not
  // stored), so no load sits behind a branch and the compiler's waits count
  // exactly the loads in flight.  Otherwise element by element.
  const int64_t last_v = (t_end - 1) & ~static_cast<int64_t>(kKP - 1);   // row offset of the last vector
  const void *zsrc = p.z ? p.z : p.delta;   // without z: delta again, from cache, unused
  auto fetch = [&](RawSet &r, int64_t c) {
    const int64_t tp0 = c + own;
    if constexpr (VEC) {
      const int64_t tv = tp0 < last_v ? tp0 : last_v;
      r.a.load_vec(CONV ? p.cx : p.u, rbase + tv);
      r.dl.load_vec(p.delta, rbase + tv);
      if constexpr (FULL) r.z.load_vec(zsrc, rbase + tv);
      // the halo of the first range of a row is zeroed where it is used
      if constexpr (CONV) r.h.load_vec(p.cx, rbase + (tv >= kKP ? tv - kKP : 0));
    } else {
      const int cnt = count(c);
      r.a.load_elems(CONV ? p.cx : p.u, rbase + tp0, cnt);
      r.dl.load_elems(p.delta, rbase + tp0, cnt);
      if (FULL && p.z) r.z.load_elems(p.z, rbase + tp0, cnt);
      if constexpr (CONV) {
        // the three samples before tp0 land in slots 5..7 (zero before t = 0)
        r.h.zero();
#pragma unroll
        for (int i = kKP - 3; i < kKP; ++i) {
          const int64_t t = tp0 - kKP + i;
          if (t >= 0 && t < p.seqlen) r.h.load_one(p.cx, rbase + t, i);
        }
      }
    }
  };

  // B/C tile of a chunk: lane v < PIECES loads 8 timesteps of one state of B
  // and of C (rows of the (b, g) group), and writes them transposed to LDS.
  // With VEC every lane loads (lanes without a piece, or with a padded
  // state, read state 0's row and stage nothing or zeros).
  const int bc_s = lane / (T / 8);
  const int bc_t0 = (lane % (T / 8)) * 8;
  const bool bc_lane = ANYV && lane < PIECES;
  const bool bc_real = bc_lane && bc_s < n;
  const int64_t bc_row = bc_base + static_cast<int64_t>(bc_real ? bc_s : 0) * p.seqlen;
  auto fetch_bc = [&](RawSet &r, int64_t c) {
    if constexpr (VEC) {
      const int64_t t_last = (t_end - 1) & ~static_cast<int64_t>(7);
      const int64_t t0 = c + bc_t0 < t_last ? c + bc_t0 : t_last;
      if constexpr (BV) r.B.load_vec(p.B, bc_row + t0);
      if constexpr (CV && FULL) r.C.load_vec(p.C, bc_row + t0);
    } else {
      r.B.zero();
      r.C.zero();
      if (bc_real) {
        const int64_t left = t_end - (c + bc_t0);
        const int cnt = static_cast<int>(left < 8 ? left : 8);
        if constexpr (BV) r.B.load_elems(p.B, bc_row + c + bc_t0, cnt);
        if constexpr (CV && FULL) r.C.load_elems(p.C, bc_row + c + bc_t0, cnt);
      }
    }
  };
  auto stage_bc = [&](const RawSet &r) {
    if (bc_lane) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (BV) sbc(0, bc_t0 + i)[bc_s] = bc_real ? r.B.get(i) : 0.0f;
        if constexpr (CV && FULL) sbc(1, bc_t0 + i)[bc_s] = bc_real ? r.C.get(i) : 0.0f;
      }
    }
  };

  // per-lane chunk values for its own timesteps
  float dtv[kKP], dtuv[kKP], yv[kKP];
#pragma unroll
  for (int i = 0; i < kKP; ++i) { dtv[i] = dtuv[i] = yv[i] = 0.0f; }

  // CSc: silu after the conv; FCc: a whole chunk, so no lane owns timesteps
  // past the end and none needs masking (compile-time constants, chosen once
  // per chunk)
  auto prep = [&](RawSet &r, int64_t c, auto CSc, auto FCc) {
    constexpr bool CS = decltype(CSc)::value;
    constexpr bool FC = decltype(FCc)::value;
    float uu[kKP];
    if constexpr (CONV) {
      float xv[kKP + 3];
      const bool h_on = !VEC || c + own >= kKP;   // zero samples before t = 0
      xv[0] = h_on ? r.h.get(kKP - 3) : 0.0f;
      xv[1] = h_on ? r.h.get(kKP - 2) : 0.0f;
      xv[2] = h_on ? r.h.get(kKP - 1) : 0.0f;
#pragma unroll
      for (int i = 0; i < kKP; ++i) xv[i + 3] = r.a.get(i);
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
      for (int i = 0; i < kKP; ++i) uu[i] = r.a.get(i);
    }
    const int cnt = count(c);
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      float dt = r.dl.get(i) + bias;
      if (p.softplus) dt = softplus_f(dt);
      if (!FC && i >= cnt) dt = 0.0f;
      dtv[i] = dt;
      dtuv[i] = dt * uu[i];
      if constexpr (KEEP_DU) r.du[i] = Dd * uu[i];
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

  auto epilogue = [&](int64_t c, const RawSet &r) {
    const int cnt = count(c);
    if (cnt <= 0 || !valid) return;
    float o[kKP];
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      float y;
      if constexpr (KEEP_DU) {
        y = yv[i] + r.du[i];
      } else {
        // the product rounded on its own, as where it is kept: the same
        // output with or without the conv prologue
#pragma clang fp contract(off)
        const float du = Dd * r.a.get(i);
        y = yv[i] + du;
      }
      if (p.z) y *= silu_f(r.z.get(i));
      o[i] = y;
    }
    store_n<IO, kKP>(p.out, rbase + c + own, o, cnt, VEC);
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
      const float *rowB = sbc(0, t) + s0;
      const float *rowC = sbc(1, t) + s0;
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

  const int64_t nch = (t_end - t_begin + T - 1) / T;
  const int64_t c_last = t_begin + (nch - 1) * T;   // VEC prefetches never start past it
  // Chunk c's epilogue runs in the next chunk's body, before that body's
  // prefetch and recurrence: the output store then completes during the
  // recurrence, and no later wait for a load waits on it.  The other set
  // (nxt) still holds chunk c - T's z and D*u when the epilogue reads them,
  // and is refilled right after.
  auto body = [&](int64_t c, RawSet &cur, RawSet &nxt) {
    const int len = static_cast<int>((t_end - c < T) ? t_end - c : T);
    const bool csilu = CONV && p.conv_silu;
    if (len == T) {
      if (csilu) prep(cur, c, std::true_type{}, std::true_type{}); else prep(cur, c, std::false_type{}, std::true_type{});
    } else {
      if (csilu) prep(cur, c, std::true_type{}, std::false_type{}); else prep(cur, c, std::false_type{}, std::false_type{});
    }
    if constexpr (XCH) {
      // this lane's timesteps are groups own/4 .. own/4 + kKP/4 - 1; the
      // previous chunk's reads of the slice are issued before these stores
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < kKP / 4; ++j) {
        float *dp = dd_at((own >> 2) + j);
        *reinterpret_cast<float4 *>(dp + cw_idx * 4) = make_float4(dtv[4 * j], dtv[4 * j + 1], dtv[4 * j + 2], dtv[4 * j + 3]);
        *reinterpret_cast<float4 *>(dp + CPW * 4 + cw_idx * 4) =
            make_float4(dtuv[4 * j], dtuv[4 * j + 1], dtuv[4 * j + 2], dtuv[4 * j + 3]);
      }
      if constexpr (!ANYV) wave_lds_sync();   // with B/C staging the sync below covers these
    }
    if constexpr (ANYV) {
      wave_lds_sync();          // the previous chunk's reads of the slice are done
      stage_bc(cur);
      wave_lds_sync();          // the slice is written before any lane reads it
    }
    if constexpr (FULL) {
      if (c > t_begin) epilogue(c - T, nxt);
    }
    if constexpr (VEC) {
      const int64_t cn = c + T < c_last ? c + T : c_last;
      fetch(nxt, cn);
      if constexpr (ANYV) fetch_bc(nxt, cn);
    } else if (c + T < t_end) {
      fetch(nxt, c + T);
      if constexpr (ANYV) fetch_bc(nxt, c + T);
    }
    if constexpr (FULL) {
      // the state before timestep c, every SSM_CKPT_INTERVAL timesteps (a
      // conditional store: issued after this body's waits for loaded data)
      if (p.ckpt && valid && (c % SSM_CKPT_INTERVAL) == 0) {
        float *dst = p.ckpt + (row * p.nck + c / SSM_CKPT_INTERVAL) * n;
#pragma unroll
        for (int k = 0; k < NSW; ++k)
          if (s0 + k < n) dst[s0 + k] = x[k];
      }
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
  };

  RawSet S0, S1;
  fetch(S0, t_begin);
  if constexpr (ANYV) fetch_bc(S0, t_begin);
  for (int64_t i = 0; i < nch; i += 2) {
    body(t_begin + i * T, S0, S1);
    if (i + 1 < nch) body(t_begin + (i + 1) * T, S1, S0);
  }
  if constexpr (FULL) {
    if ((nch - 1) & 1) epilogue(c_last, S1);
    else epilogue(c_last, S0);
  }

  if constexpr (FULL) {
    if (seg == nsegs - 1) {
      if (p.last && valid) {
#pragma unroll
        for (int k = 0; k < NSW; ++k)
          if (s0 + k < n) p.last[row * n + s0 + k] = x[k];
      }
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

// The fp32-io full pass with vector io and no conv prologue needs a few
// registers more than three waves per SIMD allow; capped to three, it spills
// two values outside its loop (setup and exit).  Other instances keep the
// compiler's choice.
template <int IO, bool CONV, int MODE, bool VEC>
constexpr bool kFullF32Vec = IO == 0 && !CONV && MODE == MODE_FULL && VEC;

// One wave per workgroup.  Block -> (channel block, segment): consecutive
// logical blocks share B/C; the hardware deals blocks to the 8 XCDs
// round-robin, so the remap keeps the blocks of one group on one XCD's L2.
template <int IO, int NSW, int LPC, bool BV, bool CV, bool CONV, int MODE, bool VEC>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kFullF32Vec<IO, CONV, MODE, VEC> ? 3 : 1)))
scan_kernel(const ScanParams p) {
  __shared__ __attribute__((aligned(16))) float lds[lds_floats(NSW, LPC, BV || CV, MODE == MODE_FULL)];
  int bid = blockIdx.x;
  if (p.xcd_swizzle) bid = (bid & 7) * (p.nblocks >> 3) + (bid >> 3);
  const int blk = bid % p.nblk;
  const int rest = bid / p.nblk;
  WaveWork wk;
  wk.g = rest % p.groups_eff;
  wk.b = rest / p.groups_eff;
  wk.d0 = wk.g * p.cpg + static_cast<int64_t>(blk) * channels_per_block(LPC);
  wk.seg = static_cast<int>(blockIdx.y);
  scan_body<IO, NSW, LPC, BV, CV, CONV, MODE, VEC>(p, lds, wk);
}

// The mixed plan at dstate 16: workgroups below mix_whole are four-lane
// waves over 16-channel blocks; each 16-channel block left over is covered
// by two eight-lane waves of 8 channels (two states per lane), each with
// about half the work of a four-lane wave.  With at most one such wave per
// SIMD the load per SIMD evens out and no SIMD runs with fewer waves than
// the others until its last wave ends.
template <int IO, bool BV, bool CV, bool CONV, bool VEC>
__global__ void __launch_bounds__(64) scan_mix_kernel(const ScanParams p) {
  constexpr int L4 = lds_floats(4, 4, BV || CV, true), L8 = lds_floats(2, 8, BV || CV, true);
  __shared__ __attribute__((aligned(16))) float lds[L4 > L8 ? L4 : L8];
  const int nwhole = p.mix_whole;
  int bid = blockIdx.x;
  int unit, half = 0;
  const bool big = bid < nwhole;
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
  WaveWork wk;
  wk.g = rest % p.groups_eff;
  wk.b = rest / p.groups_eff;
  wk.d0 = wk.g * p.cpg + static_cast<int64_t>(blk) * 16 + 8 * half;
  wk.seg = 0;
  if (big) scan_body<IO, 4, 4, BV, CV, CONV, MODE_FULL, VEC>(p, lds, wk);
  else scan_body<IO, 2, 8, BV, CV, CONV, MODE_FULL, VEC>(p, lds, wk);
}

using ScanFn = void (*)(const ScanParams);

// Kernel instance for a plan.  (nsw, lpc) is one of (4,4), (4,2), (4,1),
// (2,1), (1,1): n_pad = nsw * lpc states.
template <int IO, int NSW, int LPC, bool BV, bool CV, bool CONV, bool VEC>
ScanFn pick_mode(int mode) {
  return mode == MODE_FULL ? scan_kernel<IO, NSW, LPC, BV, CV, CONV, MODE_FULL, VEC>
                           : scan_kernel<IO, NSW, LPC, BV, CV, CONV, MODE_STATE, VEC>;
}
template <int IO, int NSW, int LPC, bool BV, bool CV, bool VEC>
ScanFn pick_conv(bool conv, int mode) {
  return conv ? pick_mode<IO, NSW, LPC, BV, CV, true, VEC>(mode) : pick_mode<IO, NSW, LPC, BV, CV, false, VEC>(mode);
}
template <int IO, int NSW, int LPC, bool VEC>
ScanFn pick_bc(bool bv, bool cv, bool conv, int mode) {
  if (bv && cv) return pick_conv<IO, NSW, LPC, true, true, VEC>(conv, mode);
  if (bv) return pick_conv<IO, NSW, LPC, true, false, VEC>(conv, mode);
  if (cv) return pick_conv<IO, NSW, LPC, false, true, VEC>(conv, mode);
  return pick_conv<IO, NSW, LPC, false, false, VEC>(conv, mode);
}
template <int IO, bool VEC>
ScanFn pick_scan(int nsw, int lpc, bool bv, bool cv, bool conv, int mode) {
  if (nsw == 4 && lpc == 4) return pick_bc<IO, 4, 4, VEC>(bv, cv, conv, mode);
  if (nsw == 4 && lpc == 2) return pick_bc<IO, 4, 2, VEC>(bv, cv, conv, mode);
  if (nsw == 4 && lpc == 1) return pick_bc<IO, 4, 1, VEC>(bv, cv, conv, mode);
  if (nsw == 2 && lpc == 1) return pick_bc<IO, 2, 1, VEC>(bv, cv, conv, mode);
  if (nsw == 1 && lpc == 1) return pick_bc<IO, 1, 1, VEC>(bv, cv, conv, mode);
  return nullptr;
}

template <int IO, bool VEC>
ScanFn pick_mix(bool bv, bool cv, bool conv) {
  if (bv && cv) return conv ? scan_mix_kernel<IO, true, true, true, VEC> : scan_mix_kernel<IO, true, true, false, VEC>;
  if (bv) return conv ? scan_mix_kernel<IO, true, false, true, VEC> : scan_mix_kernel<IO, true, false, false, VEC>;
  if (cv) return conv ? scan_mix_kernel<IO, false, true, true, VEC> : scan_mix_kernel<IO, false, true, false, VEC>;
  return conv ? scan_mix_kernel<IO, false, false, true, VEC> : scan_mix_kernel<IO, false, false, false, VEC>;
}

// Defined in scan_<dtype>.hip (vector io) and scan_<dtype>_ew.hip (element
// by element): one translation unit per io dtype and load width.
ScanFn pick_scan_f32(int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec);
ScanFn pick_scan_f16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec);
ScanFn pick_scan_bf16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec);
ScanFn pick_scan_f32_ew(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);
ScanFn pick_scan_f16_ew(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);
ScanFn pick_scan_bf16_ew(int nsw, int lpc, bool bv, bool cv, bool conv, int mode);
ScanFn pick_mix_f32(bool bv, bool cv, bool conv, bool vec);
ScanFn pick_mix_f16(bool bv, bool cv, bool conv, bool vec);
ScanFn pick_mix_bf16(bool bv, bool cv, bool conv, bool vec);
ScanFn pick_mix_f32_ew(bool bv, bool cv, bool conv);
ScanFn pick_mix_f16_ew(bool bv, bool cv, bool conv);
ScanFn pick_mix_bf16_ew(bool bv, bool cv, bool conv);

}  // namespace ssm
