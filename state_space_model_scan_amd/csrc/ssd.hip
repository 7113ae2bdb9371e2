// ssd.hip -- the Mamba-2 chunked scan (ssd_scan_fwd) on the gfx950 matrix
// cores.
//
// Operation: the mamba2 chunk-scan operators the PaddleNLP Kernel
// operator-library guide lists in section 4.4 (mamba_chunk_scan_combined,
// chunk_state, state_passing), read as the selective-scan recurrence with a
// scalar decay per head; include/ssmscan.h writes it out.
//
// Evaluation (state-space duality).  Per (batch, head) and chunk of Q = 64
// tokens, with dt' the step, cs_t = A * sum_{k<=t} dt'_k inside the chunk
// and S the (headdim x dstate) state at the chunk's start:
//   M[t][tau]  = (C_t . B_tau) * exp(cs_t - cs_tau) * dt'_tau      (tau <= t)
//   Y          = M X + diag(exp(cs)) C S^T
//   S         <- exp(cs_last) S + X^T diag(exp(cs_last - cs) * dt') B
// which is the recurrence summed in another order.  The products run as
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation).  x, B and C
// are bf16 data and enter exactly; the three derived operands -- M, the
// state S in C S^T, and X scaled by the decay weights -- are split into a
// bf16 head and a bf16 tail (v = hi + lo, about 16 significant bits) and
// enter as two products each.  Rounding them to one bf16 instead costs 3-10%
// of the output (C S^T sums 128 terms with heavy cancellation); the split
// brings the error to about 1e-4.  The state stays in fp32 accumulators
// across chunks; C S^T takes its hi/lo split straight from them.
//
// Work decomposition: one 256-thread workgroup (four waves) per (batch,
// head), walking the chunks in order.  Wave w owns the chunk's tokens
// [16w, 16w+16) for M, and the head's channels [16w, 16w+16) for Y (all 64
// tokens) and for the state.  Operand layout of the 16x16x32 instruction
// (checked on the device): lane l holds A[l%16][8(l/16)+i] and
// B[8(l/16)+i][l%16] for i < 8, and accumulator i is D[4(l/16)+i][l%16].
// The products are taken transposed (G^T = B C^T, Y^T, S^T) so that each
// lane's four accumulators are consecutive elements of one LDS row and go
// out in one store; in C S^T the state operand is this lane's own
// accumulators, with the k index running over the states in their order
// and C read in the same order.  LDS matrices are row-major with each row's
// 16-byte groups (8-byte pieces for the C tile) permuted by the row index,
// so the operand reads and the transposed staging stores of X and B spread
// over the banks without padding (measured: bank conflicts were the largest
// stall before this layout).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"
#include "host_util.h"
#include "ssmscan.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = SSD_CHUNK;     // tokens per chunk
constexpr int kP = SSD_HEADDIM;   // channels per head

struct SsdParams {
  const uint16_t *x, *dt, *B, *C, *z;
  const float *A, *D, *dt_bias, *init;
  const int32_t *seq_idx;
  uint16_t *out;
  float *fin;
  float *ws_state, *ws_decay;   // sequence split: end states from zero, total decays
  const float *carried;         // chunk scan: the state entering every segment (no fold)
  int64_t seqlen, nheads, ngroups, seg_chunks;
  int D_per_channel, softplus, dt_limit, nseg;
  float dt_min, dt_max;
};

// The two launches of a sequence split: SSD_STATE finds each segment's end
// state from zero and its total decay; SSD_FULL starts every segment from the
// carried state and computes the outputs (one launch of it without a split).
enum { SSD_STATE = 0, SSD_FULL = 1 };

// element offset of (row, col) in a row-major LDS matrix whose rows hold
// ROW_LEN bf16 elements: the row's 16-byte groups are permuted by
// (row ^ row / 8) mod 8, so that both the operand reads (16 rows, one group
// each) and the transposed stores (8 rows 8 apart, 8 consecutive columns)
// spread over the banks
template <int ROW_LEN>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int GROUPS = ROW_LEN / 8;
  const int gsw = ((row ^ (row >> 3)) & 7) & (GROUPS - 1);
  return row * ROW_LEN + (col ^ (gsw << 3));
}

// element offset of (row, col) in a row-major LDS matrix of ROW_LEN bf16
// whose rows are read in 8-byte pieces: the row's 8-byte pieces are permuted
// by the row (mod 16), so 16 consecutive rows read at one column land on
// different banks (measured: permuting 16-byte groups instead left these
// reads with as many bank conflicts as no permutation)
template <int ROW_LEN>
__device__ __forceinline__ int swz8(int row, int col) {
  constexpr int PIECES = ROW_LEN / 4;
  constexpr int MASK = PIECES > 16 ? 15 : PIECES - 1;
  return row * ROW_LEN + (col ^ ((row & MASK) << 2));
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
// 8 consecutive bf16 as raw words (element i in the low / high half of word i/2)
__device__ __forceinline__ uint4 ld8_raw(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint32_t raw_word(const uint4 &q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}
__device__ __forceinline__ uint16_t raw_bits(const uint4 &q, int i) {
  const uint32_t wd = raw_word(q, i >> 1);
  return static_cast<uint16_t>((i & 1) ? (wd >> 16) : (wd & 0xffffu));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats rounded to bf16 (to nearest, ties to even) by one paired
// conversion; a in the low half
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// a ~ hi + lo and b ~ hi + lo with all four halves bf16 (hi rounded to
// nearest, lo the rounded rest), as two packed pairs: the same values as
// rounding each element on its own, in three operations per element
__device__ __forceinline__ void split_bf2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf2(a, b);
  lo = pack_bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// the 16-bit halves of two words side by side (one byte permute): the low
// halves (HIGH = false) or the high halves of a and b, a's in the low half
template <bool HIGH>
__device__ __forceinline__ uint32_t pair_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, HIGH ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// SEQ: packed sequences (seq_idx given); a template value so that the
// kernel without them keeps its registers.
template <int N, int MODE, bool SEQ>
__global__ void __launch_bounds__(256, 2) ssd_kernel(const SsdParams p) {
  constexpr bool FULL = MODE == SSD_FULL;
  constexpr int KN = N / 32;   // K steps over dstate
  constexpr int NT = N / 16;   // state tiles along dstate
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP * kQ];   // X^T   [p][t]
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * kQ];    // B^T   [n][t]
  // M [t][tau] as hi / lo bf16, and the chunk's C [t][n] (full pass only)
  __shared__ __attribute__((aligned(16))) uint16_t sM[FULL ? 2 : 1][FULL ? kQ * kQ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sC[FULL ? kQ * N : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sBrow[FULL ? kQ * N : 8];   // B [t][n] (full pass)
  __shared__ __attribute__((aligned(16))) float sCs[kQ], sDt[kQ], sW[kQ];
  __shared__ __attribute__((aligned(16))) int32_t sSid[SEQ ? kQ : 4];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, r = l & 15, kq = l >> 4;
  const int64_t bh = blockIdx.x;
  const int64_t BH = gridDim.x;
  // the full pass runs its last (in the library's own plan the longest)
  // segment's workgroups first: they are dispatched in blockIdx order
  const int seg = FULL ? static_cast<int>(gridDim.y) - 1 - static_cast<int>(blockIdx.y)
                       : static_cast<int>(blockIdx.y);
  const int64_t b = bh / p.nheads;
  const int64_t h = bh - b * p.nheads;
  const int64_t g = h / (p.nheads / p.ngroups);
  const int64_t L = p.seqlen;
  const float Ah = p.A[h];
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const int64_t xrow = p.nheads * kP;     // elements between tokens of x, z, out
  const int64_t bcrow = p.ngroups * N;    // elements between tokens of B, C
  const uint16_t *xb = p.x + (b * L * p.nheads + h) * kP;
  const uint16_t *zb = p.z ? p.z + (b * L * p.nheads + h) * kP : nullptr;
  uint16_t *ob = p.out + (b * L * p.nheads + h) * kP;
  const uint16_t *Bb = p.B + (b * L * p.ngroups + g) * N;
  const uint16_t *Cb = p.C + (b * L * p.ngroups + g) * N;
  const uint16_t *dtb = p.dt + b * L * p.nheads + h;
  const int32_t *sidb = SEQ ? p.seq_idx + b * L : nullptr;
  const bf16x8 zero8 = {};

  const int64_t nchunks = (L + kQ - 1) / kQ;
  const int64_t c_begin = seg * p.seg_chunks;
  const int64_t c_end = seg + 1 < p.nseg ? c_begin + p.seg_chunks : nchunks;

  // Token pairs and channel groups this thread stages and stores:
  // tokens 2 (tid / 8) + {0, 1}, channels 8 (tid % 8) + 0..7.
  const int xt0 = 2 * (tid >> 3), xp0 = (tid & 7) * 8;
  // D of those channels
  float Dv8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pp = xp0 + i;
    Dv8[i] = (FULL && p.D) ? (p.D_per_channel ? p.D[h * kP + pp] : p.D[h]) : 0.0f;
  }
  // Y [t][p] (fp32, 16-byte groups permuted by t): in the row-major B copy's
  // space where it fits (dstate 128), which its last reader left before M was
  // stored, so the Y stores need no barrier after the products that read M;
  // otherwise over M
  constexpr bool Y_IN_BR = FULL && kQ * N * 2 >= kQ * kP * 4;
  float *sY = Y_IN_BR ? reinterpret_cast<float *>(sBrow) : reinterpret_cast<float *>(&sM[0][0]);
  uint16_t *sBr = sBrow;   // B row-major [t][n] for the A operand of C B^T

  // state, transposed: wave w holds S[p = 16w + r][n = 16 nt + 4kq + i].
  // The state pass starts every segment from zero; the full pass starts
  // segment k from the initial state carried over segments 0..k-1:
  //   S_in(k) = E_{k-1} + P_{k-1} (E_{k-2} + P_{k-2} (... + P_0 S_init))
  // with E_j segment j's end state from zero and P_j its total decay (zero
  // where a sequence starts inside it).
  // With carried states given (the chunk scan on its own) segment k starts
  // from carried[k] as it is.
  f32x4 accs[NT];
  const int srow = (16 * w + r) * N + 4 * kq;   // this lane's first state element in a (p, n) block
  const float *start = p.carried ? p.carried + seg * BH * kP * N : p.init;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      accs[nt][i] = (FULL && start) ? start[bh * kP * N + srow + 16 * nt + i] : 0.0f;
  }
  if constexpr (FULL) {
    const int nfold = p.carried ? 0 : seg;
    for (int j = 0; j < nfold; ++j) {
      const float P = p.ws_decay[j * BH + bh];
      const float *E = p.ws_state + (j * BH + bh) * kP * N + srow;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 e4 = *reinterpret_cast<const float4 *>(E + 16 * nt);
        accs[nt][0] = fmaf(P, accs[nt][0], e4.x);
        accs[nt][1] = fmaf(P, accs[nt][1], e4.y);
        accs[nt][2] = fmaf(P, accs[nt][2], e4.z);
        accs[nt][3] = fmaf(P, accs[nt][3], e4.w);
      }
    }
  }
  __syncthreads();

  // sequence id the incoming state belongs to: the token before the segment
  // (the first token for the initial state)
  int32_t sid_prev = 0;
  if constexpr (SEQ) sid_prev = sidb[c_begin > 0 ? c_begin * kQ - 1 : 0];
  float seg_decay = 1.0f;   // product of the chunks' decays (state pass)

  constexpr int G8 = N / 8;                      // 16-byte groups per B row
  constexpr int BPIECES = (kQ / 2) * G8;        // (token pair, 16-byte group) pieces of a B tile
  constexpr int BPAIRS = (BPIECES + 255) / 256;  // pieces per thread
  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>((L - t0 < kQ) ? L - t0 : kQ);

    // ---- every global load of the chunk first, so their latencies overlap
    uint4 xr[2], zr[2], br[BPAIRS][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = xt0 + k;
      const int64_t e = (t0 + t) * xrow + xp0;
      xr[k] = t < len ? ld8_raw(xb + e) : make_uint4(0, 0, 0, 0);
      zr[k] = (FULL && zb && t < len) ? ld8_raw(zb + e) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BPAIRS; ++j) {
      const int piece = tid + 256 * j;
      const int t = 2 * (piece / G8), n0 = (piece % G8) * 8;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        br[j][k] = (piece < BPIECES && t + k < len) ? ld8_raw(Bb + (t0 + t + k) * bcrow + n0)
                                                     : make_uint4(0, 0, 0, 0);
    }
    bf16x8 cop[FULL ? KN : 1];   // this wave's C rows (tokens 16w + r)
    if constexpr (FULL) {
      const int t = 16 * w + r;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) cop[kk] = t < len ? ld8(Cb + (t0 + t) * bcrow + 32 * kk + 8 * kq) : zero8;
    }
    float dtraw = 0.0f;
    int32_t sid = 0;
    if (w == 0) {
      if (l < len) dtraw = bf2f(dtb[(t0 + l) * p.nheads]);
      if constexpr (SEQ) sid = sidb[t0 + (l < len ? l : len - 1)];
    }

    // the previous chunk's reads of the staged tiles (and, in the full pass,
    // its epilogue's reads of Y, which shares its space with the row-major B
    // copy at dstate 128 and with M otherwise) are done; the wait overlaps
    // the loads above
    __syncthreads();

    // ---- X^T and B^T into LDS, two tokens per 32-bit store
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = (i & 1) ? pair_halves<true>(raw_word(xr[0], i >> 1), raw_word(xr[1], i >> 1))
                                 : pair_halves<false>(raw_word(xr[0], i >> 1), raw_word(xr[1], i >> 1));
      *reinterpret_cast<uint32_t *>(&sXT[swz<kQ>(xp0 + i, xt0)]) = v;
    }
#pragma unroll
    for (int j = 0; j < BPAIRS; ++j) {
      const int piece = tid + 256 * j;
      if (piece >= BPIECES) break;
      const int t = 2 * (piece / G8), n0 = (piece % G8) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t v = (i & 1) ? pair_halves<true>(raw_word(br[j][0], i >> 1), raw_word(br[j][1], i >> 1))
                                   : pair_halves<false>(raw_word(br[j][0], i >> 1), raw_word(br[j][1], i >> 1));
        *reinterpret_cast<uint32_t *>(&sBT[swz<kQ>(n0 + i, t)]) = v;
      }
      if constexpr (FULL) {
#pragma unroll
        for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4 *>(&sBr[swz<N>(t + k, n0)]) = br[j][k];
      }
    }
    if constexpr (FULL) {
      // this wave's C rows (tokens 16w + r) for every wave's C S^T products
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const uint4 cw = __builtin_bit_cast(uint4, cop[kk]);
        const int rr = 16 * w + r;
        *reinterpret_cast<uint2 *>(&sC[swz8<N>(rr, 32 * kk + 8 * kq)]) = make_uint2(cw.x, cw.y);
        *reinterpret_cast<uint2 *>(&sC[swz8<N>(rr, 32 * kk + 8 * kq + 4)]) = make_uint2(cw.z, cw.w);
      }
    }
    // ---- the steps and their running sum inside the chunk (padding: dt' = 0)
    if (w == 0) {
      float dtp = 0.0f;
      if (l < len) {
        const float v = dtraw + bias;
        dtp = p.softplus ? softplus_f(v) : v;
        if (p.dt_limit) dtp = fminf(fmaxf(dtp, p.dt_min), p.dt_max);
      }
      float cs = dtp * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(cs, off);
        if (l >= off) cs += o;
      }
      sCs[l] = cs;
      sDt[l] = dtp;
      if constexpr (SEQ) sSid[l] = sid;
    }
    __syncthreads();

    const float csl = sCs[kQ - 1];
    // sequences: the chunk's last token's id, and whether the incoming state
    // reaches the end of the chunk (no sequence starts inside it)
    const int32_t sid_last = SEQ ? sSid[len - 1] : 0;
    const bool carry = !SEQ || sid_last == sid_prev;
    // the state-update weights w_t = exp(cs_last - cs_t) * dt'_t, for the
    // tokens of the chunk's last sequence
    if (tid < kQ) {
      const bool mine = !SEQ || sSid[tid] == sid_last;
      sW[tid] = mine ? fast_exp2((csl - sCs[tid]) * kLog2e) * sDt[tid] : 0.0f;
    }
    if constexpr (!FULL) __syncthreads();

    if constexpr (FULL) {
      // ---- M, from G^T = B C^T: lane holds G[t = 16w + r][tau = 16 tb + 4kq + i],
      // masked to tau <= t (and the same sequence), decayed, split, stored as
      // 4 consecutive tau.  The products read B from its row-major LDS copy,
      // an array of its own, so a wave stores its M as soon as its products
      // are done.
      const int t = 16 * w + r;
      const float cst = sCs[t];
      const int32_t sidt = SEQ ? sSid[t] : 0;
      f32x4 accg[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        accg[tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        if (tb <= w) {
          const int tau_row = 16 * tb + r;   // the B row this lane feeds as A operand
#pragma unroll
          for (int kk = 0; kk < KN; ++kk)
            accg[tb] = mfma(ld8(&sBr[swz<N>(tau_row, 32 * kk + 8 * kq)]), cop[kk], accg[tb]);
        }
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const f32x4 acc = accg[tb];
        // the four taus' cumulative steps, steps and ids, one vector read each
        const float4 cs4 = *reinterpret_cast<const float4 *>(&sCs[16 * tb + 4 * kq]);
        const float4 dt4 = *reinterpret_cast<const float4 *>(&sDt[16 * tb + 4 * kq]);
        const float csv[4] = {cs4.x, cs4.y, cs4.z, cs4.w}, dtv[4] = {dt4.x, dt4.y, dt4.z, dt4.w};
        int32_t sdv[4] = {0, 0, 0, 0};
        if constexpr (SEQ) {
          const int4 sd4 = *reinterpret_cast<const int4 *>(&sSid[16 * tb + 4 * kq]);
          sdv[0] = sd4.x; sdv[1] = sd4.y; sdv[2] = sd4.z; sdv[3] = sd4.w;
        }
        // computed for every lane of a block at or before the wave's
        // tokens and selected by the mask (no per-lane branch); the blocks
        // after them are zero
        float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (tb <= w) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tau = 16 * tb + 4 * kq + i;
            const float v = acc[i] * fast_exp2((cst - csv[i]) * kLog2e) * dtv[i];
            m[i] = (tau <= t && (!SEQ || sdv[i] == sidt)) ? v : 0.0f;
          }
        }
        uint2 hi, lo;
        split_bf2(m[0], m[1], hi.x, lo.x);
        split_bf2(m[2], m[3], hi.y, lo.y);
        const int o = swz<kQ>(t, 16 * tb + 4 * kq);
        *reinterpret_cast<uint2 *>(&sM[0][o]) = hi;
        *reinterpret_cast<uint2 *>(&sM[1][o]) = lo;
      }
      __syncthreads();

      // ---- Y^T = S C^T diag(exp(cs)) + X^T M^T for this wave's channels and
      // every token: lane holds Y[t = 16 tb + r][p = 16w + 4kq + i].
      // The state operand comes from this lane's own accumulators,
      // S[p = 16w + r][n = 16 nt + 4kq + i]: the k index of each product runs
      // over the 32 states 32kk + 16a + 4kq + j (a < 2, j < 4) in that order
      // for both operands, a permutation of the states that leaves the sum
      // unchanged; C's are the matching 8-byte pieces of its LDS rows.
      f32x4 accy[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) accy[tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        uint32_t sh[4], sl[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2)
          split_bf2(accs[2 * kk + i / 4][i % 4], accs[2 * kk + i / 4][i % 4 + 1], sh[i / 2], sl[i / 2]);
        const bf16x8 shi = __builtin_bit_cast(bf16x8, make_uint4(sh[0], sh[1], sh[2], sh[3]));
        const bf16x8 slo = __builtin_bit_cast(bf16x8, make_uint4(sl[0], sl[1], sl[2], sl[3]));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int row = 16 * tb + r;
          const uint2 c0 = *reinterpret_cast<const uint2 *>(&sC[swz8<N>(row, 32 * kk + 4 * kq)]);
          const uint2 c1 = *reinterpret_cast<const uint2 *>(&sC[swz8<N>(row, 32 * kk + 16 + 4 * kq)]);
          const bf16x8 cop8 = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
          accy[tb] = mfma(shi, cop8, accy[tb]);
          accy[tb] = mfma(slo, cop8, accy[tb]);
        }
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        // the incoming state reaches token t only inside its own sequence
        const int tt = 16 * tb + r;
        const float e = (!SEQ || sSid[SEQ ? tt : 0] == sid_prev) ? fast_exp2(sCs[tt] * kLog2e) : 0.0f;
        accy[tb] *= e;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 xop = ld8(&sXT[swz<kQ>(16 * w + r, 32 * kk + 8 * kq)]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          if (32 * kk < 16 * (tb + 1)) {   // tau blocks at or before the token block
            const int o = swz<kQ>(16 * tb + r, 32 * kk + 8 * kq);
            accy[tb] = mfma(xop, ld8(&sM[0][o]), accy[tb]);
            accy[tb] = mfma(xop, ld8(&sM[1][o]), accy[tb]);
          }
        }
      }
      if constexpr (!Y_IN_BR) __syncthreads();   // every read of M is done

      // ---- Y into LDS (the B copy's space or over M), four consecutive channels per store
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int ty = 16 * tb + r;
        const int grp = (4 * w + kq) ^ (ty & 15);   // 16-byte group of channels 16w + 4kq, permuted by t
        *reinterpret_cast<float4 *>(&sY[ty * kP + 4 * grp]) =
            make_float4(accy[tb][0], accy[tb][1], accy[tb][2], accy[tb][3]);
      }
    }
    // ---- S^T <- exp(cs_last) S^T + B^T (X w); the old state only if no
    // sequence starts inside the chunk
    const float dec = carry ? fast_exp2(csl * kLog2e) : 0.0f;
    if constexpr (!FULL) seg_decay *= dec;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) accs[nt] *= dec;
#pragma unroll
    for (int kk = 0; kk < kQ / 32; ++kk) {
      // B operand: (X w) at tokens 32kk + 8kq + i, channel 16w + r, split hi / lo
      const uint4 xt = ld8_raw(&sXT[swz<kQ>(16 * w + r, 32 * kk + 8 * kq)]);
      uint32_t xh[4], xl[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2)
        split_bf2(bf2f(raw_bits(xt, i)) * sW[32 * kk + 8 * kq + i],
                  bf2f(raw_bits(xt, i + 1)) * sW[32 * kk + 8 * kq + i + 1], xh[i / 2], xl[i / 2]);
      const bf16x8 xhi = __builtin_bit_cast(bf16x8, make_uint4(xh[0], xh[1], xh[2], xh[3]));
      const bf16x8 xlo = __builtin_bit_cast(bf16x8, make_uint4(xl[0], xl[1], xl[2], xl[3]));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 bop = ld8(&sBT[swz<kQ>(16 * nt + r, 32 * kk + 8 * kq)]);
        accs[nt] = mfma(bop, xhi, accs[nt]);
        accs[nt] = mfma(bop, xlo, accs[nt]);
      }
    }
    sid_prev = sid_last;
    if constexpr (FULL) {
      __syncthreads();   // Y is in LDS

      // ---- out = (Y + D x) * silu(z): this thread's x / z pieces, 16-byte stores
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = xt0 + k;
        if (t < len) {
          const int g0 = (xp0 >> 2) ^ (t & 15), g1 = ((xp0 >> 2) + 1) ^ (t & 15);
          const float4 y0 = *reinterpret_cast<const float4 *>(&sY[t * kP + 4 * g0]);
          const float4 y1 = *reinterpret_cast<const float4 *>(&sY[t * kP + 4 * g1]);
          float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
          // the uniform conditions outside the element loops, so the eight
          // gates' exp / rcp chains interleave
          if (p.D) {
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = fmaf(Dv8[i], bf2f(raw_bits(xr[k], i)), yv[i]);
          }
          if (zb) {
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] *= silu_f(bf2f(raw_bits(zr[k], i)));
          }
          uint32_t pk[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) pk[i / 2] = pack_bf2(yv[i], yv[i + 1]);
          *reinterpret_cast<uint4 *>(ob + (t0 + t) * xrow + xp0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
      }
    }
  }

  if constexpr (FULL) {
    if (p.fin && seg + 1 == p.nseg) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p.fin[(bh * kP + 16 * w + r) * N + 16 * nt + 4 * kq + i] = accs[nt][i];
      }
    }
  } else {
    float *E = p.ws_state + (seg * BH + bh) * kP * N + srow;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<float4 *>(E + 16 * nt) = make_float4(accs[nt][0], accs[nt][1], accs[nt][2], accs[nt][3]);
    if (tid == 0) p.ws_decay[seg * BH + bh] = seg_decay;
  }
}

// state_passing: one thread per state element of a (batch, head), the chunks
// in order; S <- P S + E is one fp32 fma, as the fold in the full pass.
__global__ void __launch_bounds__(256) ssd_state_passing_kernel(const float *states, const float *decays,
                                                                const float *init, float *carried,
                                                                float *fin, int64_t nchunks, int64_t nbh,
                                                                int64_t ps) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nbh * ps) return;
  const int64_t bh = i / ps;
  float S = init ? init[i] : 0.0f;
  for (int64_t c = 0; c < nchunks; ++c) {
    carried[c * nbh * ps + i] = S;
    S = fmaf(decays[c * nbh + bh], S, states[c * nbh * ps + i]);
  }
  if (fin) fin[i] = S;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct SsdPlan {
  int nseg;
  int64_t seg_chunks;
  size_t off_decay, ws_bytes;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

using SsdFn = void (*)(const SsdParams);

template <int N>
SsdFn ssd_fn_n(int mode, bool seq) {
  if (mode == SSD_FULL) return seq ? ssd_kernel<N, SSD_FULL, true> : ssd_kernel<N, SSD_FULL, false>;
  return seq ? ssd_kernel<N, SSD_STATE, true> : ssd_kernel<N, SSD_STATE, false>;
}

SsdFn ssd_fn(int64_t dstate, int mode, bool seq) {
  switch (dstate) {
    case 32: return ssd_fn_n<32>(mode, seq);
    case 64: return ssd_fn_n<64>(mode, seq);
    default: return ssd_fn_n<128>(mode, seq);
  }
}

// Segments: a workgroup walks its (batch, head)'s chunks in order, so with
// few (batch, head) pairs the chunks are cut into G segments of whole
// chunks: enough workgroups for 1.5 times what the GPU holds at once, each
// segment at least two chunks.  More segments only add state-pass work:
// at b=8 l=2048 h=80 n=128 (640 pairs, 512 resident) one pass took 419 us,
// 2 segments 381, 3 392, 4 399, 8 464.
SsdPlan ssd_plan(const ssd_scan_args_t *a, int cus) {
  SsdPlan pl{};
  const int64_t nchunks = (a->seqlen + kQ - 1) / kQ;
  const int64_t BH = a->batch * a->nheads;
  int G = 1;
  if (a->seq_segments >= 1) {
    G = a->seq_segments;
  } else {
    int bf = blocks_per_cu(reinterpret_cast<const void *>(ssd_fn(a->dstate, SSD_FULL, a->seq_idx != nullptr)), 256);
    if (bf <= 0) bf = 2;
    const int64_t want = static_cast<int64_t>(bf) * cus * 3 / 2;
    if (BH < want) {
      int64_t g = (want + BH - 1) / BH;
      if (g > nchunks / 2) g = nchunks / 2;
      G = g > 1 ? static_cast<int>(g) : 1;
    }
  }
  if (G > nchunks) G = static_cast<int>(nchunks);
  pl.seg_chunks = (nchunks + G - 1) / G;
  pl.nseg = static_cast<int>((nchunks + pl.seg_chunks - 1) / pl.seg_chunks);
  // The library's own two-segment plan cuts the first segment short, about
  // 9/32 of the chunks, and the last segment takes the rest: the state pass
  // shrinks with the first segment, and the full pass, which starts the long
  // segment's workgroups first, fills the compute units with the short ones
  // (ssd2p7b, measured interleaved: first segment of 16 chunks 346 us, 8:
  // 326, 9: 319, 10: 324, 11: 331, 12: 341).
  if (a->seq_segments < 1 && pl.nseg == 2) {
    int64_t first = (9 * nchunks + 16) / 32;
    if (first < 2) first = 2;
    if (first < nchunks) pl.seg_chunks = first;
  }
  if (pl.nseg > 1) {
    const size_t ns = static_cast<size_t>(pl.nseg - 1) * BH;
    pl.off_decay = up256(ns * kP * a->dstate * sizeof(float));
    pl.ws_bytes = pl.off_decay + up256(ns * sizeof(float));
  }
  return pl;
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssd_scan_workspace_size(const ssd_scan_args_t *a, size_t *bytes) {
  const int st = ssd_scan_validate(a);
  if (st != SSM_OK) return st;
  if (!bytes) return SSM_ERR_NULL;
  *bytes = ssd_plan(a, cu_count_cached()).ws_bytes;
  return SSM_OK;
}

namespace {

// the kernel parameters every launch shares
SsdParams ssd_params(const ssd_scan_args_t *a) {
  SsdParams p{};
  p.x = static_cast<const uint16_t *>(a->x);
  p.dt = static_cast<const uint16_t *>(a->dt);
  p.B = static_cast<const uint16_t *>(a->B);
  p.C = static_cast<const uint16_t *>(a->C);
  p.z = static_cast<const uint16_t *>(a->z);
  p.A = a->A; p.D = a->D; p.dt_bias = a->dt_bias; p.init = a->initial_states;
  p.seq_idx = a->seq_idx;
  p.out = static_cast<uint16_t *>(a->out);
  p.fin = a->final_states;
  p.seqlen = a->seqlen; p.nheads = a->nheads; p.ngroups = a->ngroups;
  p.D_per_channel = a->D_per_channel;
  p.softplus = a->dt_softplus;
  p.dt_limit = a->dt_limit; p.dt_min = a->dt_min; p.dt_max = a->dt_max;
  return p;
}

}  // namespace

extern "C" int ssd_chunk_state(const ssd_scan_args_t *a, int64_t chunk_size, float *states, float *decays,
                               void *stream_ptr) {
  const int st = ssd_chunk_state_validate(a, chunk_size, states, decays);
  if (st != SSM_OK) return st;
  const int64_t nchunks = (a->seqlen + chunk_size - 1) / chunk_size;
  const int64_t blocks = a->batch * a->nheads;
  if (blocks > 0x7fffffffLL || nchunks > 65535) return SSM_ERR_SHAPE;
  SsdParams p = ssd_params(a);
  p.C = nullptr; p.z = nullptr; p.D = nullptr; p.init = nullptr; p.out = nullptr; p.fin = nullptr;
  p.nseg = static_cast<int>(nchunks);
  p.seg_chunks = chunk_size / kQ;
  p.ws_state = states;
  p.ws_decay = decays;
  hipLaunchKernelGGL(ssd_fn(a->dstate, SSD_STATE, a->seq_idx != nullptr),
                     dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(nchunks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream_ptr), p);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : hip_fail(e);
}

extern "C" int ssd_state_passing(int64_t nchunks, int64_t batch, int64_t nheads, int64_t headdim,
                                 int64_t dstate, const float *states, const float *decays,
                                 const float *initial_states, float *carried, float *final_states,
                                 void *stream_ptr) {
  const int st = ssd_state_passing_validate(nchunks, batch, nheads, headdim, dstate, states, decays, carried);
  if (st != SSM_OK) return st;
  const int64_t nbh = batch * nheads, ps = headdim * dstate;
  const int64_t blocks = (nbh * ps + 255) / 256;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  hipLaunchKernelGGL(ssd_state_passing_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream_ptr), states, decays, initial_states, carried,
                     final_states, nchunks, nbh, ps);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : hip_fail(e);
}

extern "C" int ssd_chunk_scan(const ssd_scan_args_t *a, int64_t chunk_size, const float *carried,
                              void *stream_ptr) {
  const int st = ssd_chunk_scan_validate(a, chunk_size, carried);
  if (st != SSM_OK) return st;
  const int64_t nchunks = (a->seqlen + chunk_size - 1) / chunk_size;
  const int64_t blocks = a->batch * a->nheads;
  if (blocks > 0x7fffffffLL || nchunks > 65535) return SSM_ERR_SHAPE;
  SsdParams p = ssd_params(a);
  p.init = nullptr;
  p.carried = carried;
  p.nseg = static_cast<int>(nchunks);
  p.seg_chunks = chunk_size / kQ;
  hipLaunchKernelGGL(ssd_fn(a->dstate, SSD_FULL, a->seq_idx != nullptr),
                     dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(nchunks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream_ptr), p);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : hip_fail(e);
}

extern "C" int ssd_scan_fwd(const ssd_scan_args_t *a, void *stream_ptr) {
  const int st = ssd_scan_validate(a);
  if (st != SSM_OK) return st;
  const SsdPlan pl = ssd_plan(a, cu_count_cached());
  if (pl.ws_bytes > 0 && (!a->workspace || a->workspace_bytes < pl.ws_bytes)) return SSM_ERR_WORKSPACE;
  SsdParams p = ssd_params(a);
  p.nseg = pl.nseg; p.seg_chunks = pl.seg_chunks;
  if (pl.nseg > 1) {
    char *ws = static_cast<char *>(a->workspace);
    p.ws_state = reinterpret_cast<float *>(ws);
    p.ws_decay = reinterpret_cast<float *>(ws + pl.off_decay);
  }
  const int64_t blocks = a->batch * a->nheads;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const unsigned gx = static_cast<unsigned>(blocks);
  const bool seq = a->seq_idx != nullptr;
  if (pl.nseg > 1) {
    hipLaunchKernelGGL(ssd_fn(a->dstate, SSD_STATE, seq), dim3(gx, pl.nseg - 1), dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  hipLaunchKernelGGL(ssd_fn(a->dstate, SSD_FULL, seq), dim3(gx, pl.nseg), dim3(256), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
