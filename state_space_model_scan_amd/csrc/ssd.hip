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
// across chunks, with its hi/lo copy in LDS as the operand of C S^T.
//
// Work decomposition: one 256-thread workgroup (four waves) per (batch,
// head), walking the chunks in order.  Wave w owns rows [16w, 16w+16) of the
// chunk's tokens for M and Y, and rows [16w, 16w+16) of the head's channels
// for the state.  Operand layout of the 16x16x32 instruction (checked on the
// device): lane l holds A[l%16][8(l/16)+i] and B[8(l/16)+i][l%16] for
// i < 8, and accumulator i is D[4(l/16)+i][l%16].  LDS matrices are stored
// row-major with each row's 16-byte groups XOR-swizzled by the row index, so
// the operand reads (8 consecutive elements of 16 different rows) spread
// over the banks without padding.
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
  uint16_t *out;
  float *fin;
  int64_t seqlen, nheads, ngroups;
  int D_per_channel, softplus;
};

// element offset of (row, col) in a row-major LDS matrix whose rows hold
// row_len elements, 16-byte groups swizzled by the row
template <int ROW_LEN>
__device__ __forceinline__ int swz(int row, int col) {
  return row * ROW_LEN + (col ^ (((row & 7) << 3) & (ROW_LEN - 1)));
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) {
  const __bf16 h = static_cast<__bf16>(v);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
// 8 consecutive bf16 as raw words (element i in the low / high half of word i/2)
__device__ __forceinline__ uint4 ld8_raw(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint16_t raw_bits(const uint4 &q, int i) {
  const uint32_t wd = (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w;
  return static_cast<uint16_t>((i & 1) ? (wd >> 16) : (wd & 0xffffu));
}

// v ~ hi + lo with both halves bf16 (hi rounded to nearest, lo the rounded rest)
__device__ __forceinline__ void split_bf(float v, uint16_t &hi, uint16_t &lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N>
__global__ void __launch_bounds__(256, 2) ssd_kernel(const SsdParams p) {
  constexpr int KN = N / 32;   // K steps over dstate
  constexpr int NT = N / 16;   // state tiles along dstate
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP * kQ];   // X^T   [p][t]
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N * kQ];    // B^T   [n][t]
  __shared__ __attribute__((aligned(16))) uint16_t sM[2][kQ * kQ];    // M     [t][tau], hi / lo
  __shared__ __attribute__((aligned(16))) uint16_t sS[2][kP * N];     // state [p][n], hi / lo
  __shared__ float sCs[kQ], sDt[kQ], sW[kQ];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, r = l & 15, kq = l >> 4;
  const int64_t bh = blockIdx.x;
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
  const bf16x8 zero8 = {};

  // D of the channels this thread stores (8 * (tid % 8) + 0..7)
  float Dv8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pp = (tid & 7) * 8 + i;
    Dv8[i] = p.D ? (p.D_per_channel ? p.D[h * kP + pp] : p.D[h]) : 0.0f;
  }

  // state: wave w holds S[16w + 4kq + i][16 nt + r]
  f32x4 accs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = 16 * w + 4 * kq + i, n = 16 * nt + r;
      const float v = p.init ? p.init[(bh * kP + pp) * N + n] : 0.0f;
      accs[nt][i] = v;
      split_bf(v, sS[0][swz<N>(pp, n)], sS[1][swz<N>(pp, n)]);
    }
  }
  __syncthreads();

  const int64_t nchunks = (L + kQ - 1) / kQ;
  constexpr int BSEG = kQ * (N / 8) / 256;   // 16-byte pieces of the B tile per thread
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>((L - t0 < kQ) ? L - t0 : kQ);

    // ---- every global load of the chunk first, so their latencies overlap:
    // x and z (thread: tokens tid/8 and tid/8 + 32, channels 8*(tid%8)..+7),
    // the B tile, this wave's C rows (tokens 16w + r), and the steps
    uint4 xr[2], zr[2], br[BSEG];
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int t = (tid >> 3) + 32 * rep, p0 = (tid & 7) * 8;
      const int64_t e = (t0 + t) * xrow + p0;
      xr[rep] = t < len ? ld8_raw(xb + e) : make_uint4(0, 0, 0, 0);
      zr[rep] = (zb && t < len) ? ld8_raw(zb + e) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BSEG; ++j) {
      const int seg = tid + 256 * j;
      const int t = seg / (N / 8), n0 = (seg % (N / 8)) * 8;
      br[j] = t < len ? ld8_raw(Bb + (t0 + t) * bcrow + n0) : make_uint4(0, 0, 0, 0);
    }
    bf16x8 cop[KN];
    {
      const int t = 16 * w + r;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) cop[kk] = t < len ? ld8(Cb + (t0 + t) * bcrow + 32 * kk + 8 * kq) : zero8;
    }
    float dtraw = 0.0f;
    if (w == 0 && l < len) dtraw = bf2f(dtb[(t0 + l) * p.nheads]);

    // ---- X^T and B^T into LDS; the steps and their running sum inside the
    // chunk (padding: dt' = 0)
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int t = (tid >> 3) + 32 * rep, p0 = (tid & 7) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sXT[swz<kQ>(p0 + i, t)] = raw_bits(xr[rep], i);
    }
#pragma unroll
    for (int j = 0; j < BSEG; ++j) {
      const int seg = tid + 256 * j;
      const int t = seg / (N / 8), n0 = (seg % (N / 8)) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sBT[swz<kQ>(n0 + i, t)] = raw_bits(br[j], i);
    }
    if (w == 0) {
      float dtp = 0.0f;
      if (l < len) {
        const float v = dtraw + bias;
        dtp = p.softplus ? softplus_f(v) : v;
      }
      float cs = dtp * Ah;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(cs, off);
        if (l >= off) cs += o;
      }
      sCs[l] = cs;
      sDt[l] = dtp;
    }
    __syncthreads();

    const float csl = sCs[kQ - 1];
    // the state-update weights w_t = exp(cs_last - cs_t) * dt'_t
    if (tid < kQ) sW[tid] = fast_exp2((csl - sCs[tid]) * kLog2e) * sDt[tid];
    // ---- M: this wave's rows of C B^T, masked to tau <= t and decayed (the
    // B operand rows were just read into L2 by the tile load)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tau = 16 * tb + r;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (tb <= w) {
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
          const bf16x8 bop = tau < len ? ld8(Bb + (t0 + tau) * bcrow + 32 * kk + 8 * kq) : zero8;
          acc = mfma(cop[kk], bop, acc);
        }
      }
      const float cst = sCs[tau], dtt = sDt[tau];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * kq + i;
        float m = 0.0f;
        if (tb <= w && tau <= t) m = acc[i] * fast_exp2((sCs[t] - cst) * kLog2e) * dtt;
        split_bf(m, sM[0][swz<kQ>(t, tau)], sM[1][swz<kQ>(t, tau)]);
      }
    }
    __syncthreads();

    // ---- Y = diag(exp(cs)) C S^T + M X for this wave's tokens
    f32x4 accy[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      accy[pb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const int o = swz<N>(16 * pb + r, 32 * kk + 8 * kq);
        accy[pb] = mfma(cop[kk], ld8(&sS[0][o]), accy[pb]);
        accy[pb] = mfma(cop[kk], ld8(&sS[1][o]), accy[pb]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(sCs[16 * w + 4 * kq + i] * kLog2e);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) accy[pb][i] *= e;
    }
    const int kkmax = (16 * (w + 1) + 31) / 32;   // tau blocks at or before this wave's tokens
    for (int kk = 0; kk < kkmax; ++kk) {
      const int o = swz<kQ>(16 * w + r, 32 * kk + 8 * kq);
      const bf16x8 mhi = ld8(&sM[0][o]), mlo = ld8(&sM[1][o]);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        const bf16x8 xop = ld8(&sXT[swz<kQ>(16 * pb + r, 32 * kk + 8 * kq)]);
        accy[pb] = mfma(mhi, xop, accy[pb]);
        accy[pb] = mfma(mlo, xop, accy[pb]);
      }
    }
    __syncthreads();   // every read of M and of the old state is done

    // ---- Y into LDS (over M) for a coalesced epilogue
    float *sY = reinterpret_cast<float *>(&sM[0][0]);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sY[(16 * w + 4 * kq + i) * kP + 16 * pb + r] = accy[pb][i];
    }
    // ---- S <- exp(cs_last) S + (X w)^T B
    const float dec = fast_exp2(csl * kLog2e);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) accs[nt] *= dec;
#pragma unroll
    for (int kk = 0; kk < kQ / 32; ++kk) {
      // A operand: this wave's rows of (X w)^T, split into hi / lo
      const uint4 xt = ld8_raw(&sXT[swz<kQ>(16 * w + r, 32 * kk + 8 * kq)]);
      bf16x8 xhi, xlo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = bf2f(raw_bits(xt, i)) * sW[32 * kk + 8 * kq + i];
        const __bf16 hb = static_cast<__bf16>(v);
        xhi[i] = hb;
        xlo[i] = static_cast<__bf16>(v - static_cast<float>(hb));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 bop = ld8(&sBT[swz<kQ>(16 * nt + r, 32 * kk + 8 * kq)]);
        accs[nt] = mfma(xhi, bop, accs[nt]);
        accs[nt] = mfma(xlo, bop, accs[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = swz<N>(16 * w + 4 * kq + i, 16 * nt + r);
        split_bf(accs[nt][i], sS[0][o], sS[1][o]);
      }
    }
    __syncthreads();

    // ---- out = (Y + D x) * silu(z): this thread's x / z pieces, 16-byte stores
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int t = (tid >> 3) + 32 * rep, p0 = (tid & 7) * 8;
      if (t < len) {
        const float4 y0 = *reinterpret_cast<const float4 *>(&sY[t * kP + p0]);
        const float4 y1 = *reinterpret_cast<const float4 *>(&sY[t * kP + p0 + 4]);
        const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float o2[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            float y = yv[i + k];
            if (p.D) y = fmaf(Dv8[i + k], bf2f(raw_bits(xr[rep], i + k)), y);
            if (zb) y *= silu_f(bf2f(raw_bits(zr[rep], i + k)));
            o2[k] = y;
          }
          pk[i / 2] = static_cast<uint32_t>(f2bf(o2[0])) | (static_cast<uint32_t>(f2bf(o2[1])) << 16);
        }
        *reinterpret_cast<uint4 *>(ob + (t0 + t) * xrow + p0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
  }

  if (p.fin) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p.fin[(bh * kP + 16 * w + 4 * kq + i) * N + 16 * nt + r] = accs[nt][i];
    }
  }
}

}  // namespace
}  // namespace ssm

using namespace ssm;

extern "C" int ssd_scan_fwd(const ssd_scan_args_t *a, void *stream_ptr) {
  const int st = ssd_scan_validate(a);
  if (st != SSM_OK) return st;
  SsdParams p{};
  p.x = static_cast<const uint16_t *>(a->x);
  p.dt = static_cast<const uint16_t *>(a->dt);
  p.B = static_cast<const uint16_t *>(a->B);
  p.C = static_cast<const uint16_t *>(a->C);
  p.z = static_cast<const uint16_t *>(a->z);
  p.A = a->A; p.D = a->D; p.dt_bias = a->dt_bias; p.init = a->initial_states;
  p.out = static_cast<uint16_t *>(a->out);
  p.fin = a->final_states;
  p.seqlen = a->seqlen; p.nheads = a->nheads; p.ngroups = a->ngroups;
  p.D_per_channel = a->D_per_channel;
  p.softplus = a->dt_softplus;
  const int64_t blocks = a->batch * a->nheads;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (a->dstate) {
    case 32: hipLaunchKernelGGL(ssd_kernel<32>, grid, dim3(256), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(ssd_kernel<64>, grid, dim3(256), 0, stream, p); break;
    default: hipLaunchKernelGGL(ssd_kernel<128>, grid, dim3(256), 0, stream, p); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}
