// ssm_scan.hip -- host side of libssmscan.so: planning, dispatch and the
// C-ABI entry points, plus the standalone causal depthwise conv kernel.
//
// Operation: PaddleNLP Kernel operator-library guide, section 4.1
// (selective_scan_fn) and section 4.2 (causal_conv1d_fn); see
// include/ssmscan.h.  The scan kernel itself is in scan_kernel.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <unordered_map>

#include "host_util.h"
#include "scan_kernel.h"
#include "ssmscan.h"

using namespace ssm;

namespace ssm {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return SSM_ERR_HIP;
}

int cu_count_cached() {
  static std::mutex mu;
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (counts[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    counts[dev] = v;
  }
  return counts[dev];
}

int blocks_per_cu(const void *f, int block) {
  static std::mutex mu;
  static std::unordered_map<const void *, int> cache;
  if (!f) return 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(f);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, block, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  cache.emplace(f, nb);
  return nb;
}

}  // namespace ssm

namespace {

// ---------------------------------------------------------------------------
// standalone causal depthwise conv: one thread per 8 consecutive outputs.
// Optional (causal_conv1d_fn's seq_idx / initial_states / final states):
// init (b, d, 3) io prepends the three inputs before t = 0; with SEQ a tap
// contributes only when its position carries the output's sequence id; the
// thread holding the row's last output writes the last three inputs to fin.
// ---------------------------------------------------------------------------

template <int IO, bool SEQ>
__global__ void __launch_bounds__(256)
conv_kernel(const void *x, const float *wgt, const float *bias, void *out,
            int64_t rows, int64_t dim, int64_t seqlen, int silu, int vec,
            const int32_t *seq_idx, const void *init, void *fin) {
  const int64_t nt8 = (seqlen + 7) / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * nt8) return;
  const int64_t row = idx / nt8;
  const int64_t t0 = (idx - row * nt8) * 8;
  const int64_t d = row % dim;
  const int64_t rb = row * seqlen;
  const int cnt = static_cast<int>((seqlen - t0 < 8) ? seqlen - t0 : 8);
  Raw8<IO> cur, prev;
  cur.load(x, rb + t0, cnt, vec != 0);
  if (t0 >= 8 && vec) prev.load_vec(x, rb + t0 - 8);
  else prev.load_elems(x, rb + t0 - 8, t0 >= 8 ? 8 : 0);
  const float w0 = wgt[d * 4 + 0], w1 = wgt[d * 4 + 1], w2 = wgt[d * 4 + 2], w3 = wgt[d * 4 + 3];
  const float bb = bias ? bias[d] : 0.0f;
  float xv[11];
  xv[0] = prev.get(5); xv[1] = prev.get(6); xv[2] = prev.get(7);
  if (t0 == 0 && init) {
#pragma unroll
    for (int j = 0; j < 3; ++j) xv[j] = load_io<IO>(init, row * 3 + j);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i + 3] = cur.get(i);
  // sequence ids of positions t0-3 .. t0+7 (positions outside [0, seqlen)
  // hold zero inputs, so their ids do not matter)
  int32_t sid[11];
  if constexpr (SEQ) {
    const int64_t sb = (row / dim) * seqlen;
#pragma unroll
    for (int j = 0; j < 11; ++j) {
      const int64_t pos = t0 - 3 + j;
      sid[j] = (pos >= 0 && pos < seqlen) ? seq_idx[sb + pos] : 0;
    }
  }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v0 = xv[i], v1 = xv[i + 1], v2 = xv[i + 2];
    if constexpr (SEQ) {
      const int32_t me = sid[i + 3];
      if (sid[i] != me) v0 = 0.0f;
      if (sid[i + 1] != me) v1 = 0.0f;
      if (sid[i + 2] != me) v2 = 0.0f;
    }
    float acc = bb;
    acc = fmaf(w0, v0, acc);
    acc = fmaf(w1, v1, acc);
    acc = fmaf(w2, v2, acc);
    acc = fmaf(w3, xv[i + 3], acc);
    if (silu) acc = silu_f(acc);
    o[i] = acc;
  }
  store8<IO>(out, rb + t0, o, cnt, vec != 0);
  if (fin && t0 + 8 >= seqlen) {
    // the extended input at seqlen-3+j sits at xv[seqlen - t0 + j]
    const int e = static_cast<int>(seqlen - t0);
#pragma unroll
    for (int j = 0; j < 3; ++j) store_one<IO>(fin, row * 3 + j, xv[e + j]);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------


struct Plan {
  int n_pad, nsw, lpc, T;
  int groups_eff, nblk, nblocks, nseg;
  int mix_whole, mix_small;      // mixed plan: four-lane waves, eight-lane waves (0, 0: none)
  bool vec;                      // 16-byte vector io (see vector_io)
  int64_t cpg, seg_len;
  size_t ws_bytes;
};

size_t up256(size_t bytes) { return (bytes + 255) / 256 * 256; }

int pow2ceil(int v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

ScanFn pick(int io, int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec) {
  if (io == SSM_BF16) return pick_scan_bf16(nsw, lpc, bv, cv, conv, mode, vec);
  if (io == SSM_F16) return pick_scan_f16(nsw, lpc, bv, cv, conv, mode, vec);
  return pick_scan_f32(nsw, lpc, bv, cv, conv, mode, vec);
}

ScanFn pick_mixed(int io, bool bv, bool cv, bool conv, bool vec) {
  if (io == SSM_BF16) return pick_mix_bf16(bv, cv, conv, vec);
  if (io == SSM_F16) return pick_mix_f16(bv, cv, conv, vec);
  return pick_mix_f32(bv, cv, conv, vec);
}

// Every io pointer 16-byte aligned and seqlen % 8 == 0: the kernels move
// whole 8-timestep ranges as vectors.
bool vector_io(const ssm_scan_args_t *a) {
  const bool conv = a->conv_weight != nullptr;
  return (a->seqlen % 8 == 0) && aligned16(a->delta) && aligned16(a->out) &&
         (conv ? aligned16(a->conv_x) : aligned16(a->u)) && (!a->z || aligned16(a->z)) &&
         (a->B_kind != SSM_BC_VARYING || aligned16(a->B)) && (a->C_kind != SSM_BC_VARYING || aligned16(a->C));
}

// A channel's states are spread over lpc lanes of nsw states each (four
// lanes of four at dstate 16): enough waves to fill the GPU at the Mamba
// shapes, and each lane still runs several independent state chains.
Plan make_plan(const ssm_scan_args_t *a, int cus) {
  Plan pl{};
  pl.n_pad = pow2ceil(static_cast<int>(a->dstate));
  pl.vec = vector_io(a);
  switch (pl.n_pad) {
    case 16: pl.nsw = 4; pl.lpc = 4; break;
    case 8: pl.nsw = 4; pl.lpc = 2; break;
    case 4: pl.nsw = 4; pl.lpc = 1; break;
    case 2: pl.nsw = 2; pl.lpc = 1; break;
    default: pl.nsw = 1; pl.lpc = 1; break;
  }
  pl.T = chunk_of(pl.lpc);
  const bool any_varying = a->B_kind == SSM_BC_VARYING || a->C_kind == SSM_BC_VARYING;
  pl.groups_eff = any_varying ? static_cast<int>(a->ngroups) : 1;
  pl.cpg = a->dim / pl.groups_eff;
  const int cpb = channels_per_block(pl.lpc);
  pl.nblk = static_cast<int>((pl.cpg + cpb - 1) / cpb);
  pl.nblocks = static_cast<int>(a->batch * pl.groups_eff * pl.nblk);
  const int64_t waves = pl.nblocks;   // one wave per block
  // Split when the waves would leave the SIMDs short of work: the state pass
  // of a split costs more than it gains once a pass has >= ~2 waves per SIMD,
  // and narrow workloads keep gaining up to ~4-6 waves per SIMD.  The count
  // is rounded down, so the full pass never exceeds 6 waves per SIMD: just
  // above a multiple of what the SIMDs hold at once, the few waves over run
  // as a round of their own (b=1 d=2560 l=65536 fp32: 39 segments 1194 us,
  // 38 segments 1121 us).  Segments keep at least 8 chunks: shorter ones
  // spend too much on their start (the carry fold, the first chunk's loads)
  // -- at b=4 d=1536 l=2048, 8 segments ran 9% faster than 16.
  const int64_t target = 16LL * cus;
  int nseg = 1;
  if (waves < 8LL * cus) {
    const int64_t want = 3 * target / (2 * waves);
    const int64_t cap = a->seqlen / (8 * pl.T);
    nseg = static_cast<int>(want < cap ? want : cap);
    if (nseg < 1) nseg = 1;
  }
  if (a->seq_segments >= 1) nseg = a->seq_segments;
  if (nseg > a->seqlen / pl.T) nseg = static_cast<int>(a->seqlen / pl.T > 0 ? a->seqlen / pl.T : 1);
  int64_t seg_len = (a->seqlen + nseg - 1) / nseg;
  // checkpoints sit at multiples of SSM_CKPT_INTERVAL, which every chunk
  // length divides: segments then start on a checkpoint too
  const int64_t align = a->checkpoints ? SSM_CKPT_INTERVAL : pl.T;
  seg_len = (seg_len + align - 1) / align * align;
  pl.seg_len = seg_len;
  pl.nseg = static_cast<int>((a->seqlen + seg_len - 1) / seg_len);
  size_t off = pl.nseg > 1
                   ? up256(static_cast<size_t>(pl.nseg - 1) * (pl.n_pad + 1) * a->batch * a->dim * sizeof(float))
                   : 0;
  // Mixed plan (dstate 13..16, no split): with q >= 2 whole waves per SIMD
  // and r channel blocks over, r SIMDs would run a whole wave more than the
  // rest.  The r blocks become 2r eight-lane waves of 8 channels instead,
  // each about half the work of a whole wave: with 2r <= SIMDs every SIMD
  // holds q whole waves and at most one half wave -- provided q + 1 waves of
  // the kernel fit a SIMD at once (its registers and LDS decide).  At q = 1
  // the SIMDs are bound by the recurrence's latency rather than by issue, a
  // half wave takes as long as a whole one, and the plain plan is faster.
  pl.mix_whole = pl.mix_small = 0;
  if (pl.nseg == 1 && a->seq_segments == 0 && pl.nsw == 4 && pl.lpc == 4) {
    const int simds = 4 * cus;
    const int q = pl.nblocks / simds, r = pl.nblocks % simds;
    if (q >= 2 && r > 0 && 2 * r <= simds &&
        4 * (q + 1) <= blocks_per_cu(reinterpret_cast<const void *>(
                                         pick_mixed(a->io_dtype, a->B_kind == SSM_BC_VARYING,
                                                    a->C_kind == SSM_BC_VARYING, a->conv_weight != nullptr,
                                                    pl.vec)), 64)) {
      pl.mix_whole = pl.nblocks - r;
      pl.mix_small = 2 * r;
    }
  }
  pl.ws_bytes = off;
  return pl;
}

}  // namespace

extern "C" int ssm_scan_workspace_size(const ssm_scan_args_t *a, size_t *bytes) {
  const int st = ssm_scan_validate(a);
  if (st != SSM_OK) return st;
  if (!bytes) return SSM_ERR_NULL;
  *bytes = make_plan(a, cu_count_cached()).ws_bytes;
  return SSM_OK;
}

extern "C" int ssm_scan_plan(const ssm_scan_args_t *a, ssm_scan_plan_t *out) {
  const int st = ssm_scan_validate(a);
  if (st != SSM_OK) return st;
  if (!out) return SSM_ERR_NULL;
  const Plan pl = make_plan(a, cu_count_cached());
  out->segments = pl.nseg;
  out->waves = pl.mix_small ? pl.mix_whole : pl.nblocks;
  out->lanes_per_channel = pl.lpc;
  out->eight_lane_waves = pl.mix_small;
  out->workspace_bytes = pl.ws_bytes;
  return SSM_OK;
}

namespace {

// The forward for a validated call and its plan, with `ws` as the scratch
// (pl.ws_bytes of it, or none).
int scan_fwd_run(const ssm_scan_args_t *a, const Plan &pl, void *ws, void *stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

  const int io = a->io_dtype;
  const bool conv = a->conv_weight != nullptr;
  ScanParams p{};
  p.u = a->u; p.delta = a->delta; p.B = a->B; p.C = a->C; p.z = a->z;
  p.cx = a->conv_x; p.A = a->A; p.D = a->D; p.dbias = a->delta_bias;
  p.init = a->initial_state; p.cw = a->conv_weight; p.cb = a->conv_bias;
  p.out = a->out; p.last = a->last_state;
  p.batch = a->batch; p.dim = a->dim; p.seqlen = a->seqlen;
  p.seg_len = pl.seg_len; p.cpg = pl.cpg;
  p.ckpt = a->checkpoints;
  p.nck = (a->seqlen + SSM_CKPT_INTERVAL - 1) / SSM_CKPT_INTERVAL;
  p.n = static_cast<int>(a->dstate); p.n_pad = pl.n_pad; p.ngroups = static_cast<int>(a->ngroups);
  p.groups_eff = pl.groups_eff; p.nblk = pl.nblk; p.nseg = pl.nseg; p.nblocks = pl.nblocks;
  p.mix_whole = pl.mix_whole; p.mix_small = pl.mix_small;
  p.softplus = a->delta_softplus; p.conv_silu = a->conv_act == SSM_ACT_SILU;
  const bool vec = pl.vec;
  p.xcd_swizzle = pl.mix_small ? (pl.mix_whole % 8 == 0) : (pl.nblocks % 8 == 0);

  if (pl.nseg > 1) {
    float *wsf = static_cast<float *>(ws);
    p.ws_state = wsf;
    p.ws_sumdt = wsf + static_cast<size_t>(pl.nseg - 1) * pl.n_pad * a->batch * a->dim;
  }
  const int64_t grid_x = pl.mix_small ? static_cast<int64_t>(pl.mix_whole) + pl.mix_small : pl.nblocks;
  if (grid_x > 0x7fffffffLL) return SSM_ERR_SHAPE;
  const bool bv = a->B_kind == SSM_BC_VARYING, cv = a->C_kind == SSM_BC_VARYING;
  int rc = SSM_OK;
  const ScanFn f_state = pl.nseg > 1 ? pick(io, pl.nsw, pl.lpc, bv, cv, conv, MODE_STATE, vec) : nullptr;
  const ScanFn f_full = pl.mix_small ? pick_mixed(io, bv, cv, conv, vec)
                                     : pick(io, pl.nsw, pl.lpc, bv, cv, conv, MODE_FULL, vec);
  if (!f_full || (pl.nseg > 1 && !f_state)) rc = SSM_ERR_UNSUPPORTED;
  if (rc == SSM_OK && pl.nseg > 1) {
    hipLaunchKernelGGL(f_state, dim3(pl.nblocks, pl.nseg - 1), dim3(64), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e);
  }
  if (rc == SSM_OK) {
    hipLaunchKernelGGL(f_full, dim3(static_cast<unsigned>(grid_x), pl.nseg), dim3(64), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) rc = hip_fail(e);
  }
  return rc;
}

}  // namespace

// Scratch of ssm_scan_fwd_noalloc: one per device the library runs on, held
// until the process ends.  Host code must never pass `scratch` itself to a
// kernel (on the host it only names the symbol): its device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

int scratch_ptr(void **out) {
  static std::mutex mu;
  static void *ptrs[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return SSM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return SSM_OK;
}

}  // namespace

extern "C" int ssm_scan_fwd(const ssm_scan_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_validate(a);
  if (st != SSM_OK) return st;
  const Plan pl = make_plan(a, cu_count_cached());
  if (pl.ws_bytes > 0 && (!a->workspace || a->workspace_bytes < pl.ws_bytes)) return SSM_ERR_WORKSPACE;
  return scan_fwd_run(a, pl, a->workspace, stream_ptr);
}

extern "C" int ssm_scan_fwd_noalloc(const ssm_scan_args_t *a, void *stream_ptr) {
  const int st = ssm_scan_validate(a);
  if (st != SSM_OK) return st;
  const Plan pl = make_plan(a, cu_count_cached());
  if (pl.ws_bytes > kNoAllocScratchBytes) return SSM_ERR_SCRATCH;
  void *ws = nullptr;
  if (pl.ws_bytes > 0) {
    const int rc = scratch_ptr(&ws);
    if (rc != SSM_OK) return rc;
  }
  return scan_fwd_run(a, pl, ws, stream_ptr);
}

extern "C" int causal_conv1d_fwd(const void *x, const float *weight, const float *bias, void *out,
                                 int64_t batch, int64_t dim, int64_t seqlen, int32_t width,
                                 int32_t io_dtype, int32_t act, void *stream_ptr) {
  const int st = causal_conv1d_validate(x, weight, out, batch, dim, seqlen, width, io_dtype, act);
  if (st != SSM_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int64_t rows = batch * dim;
  const int64_t threads = rows * ((seqlen + 7) / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  const int vec = (seqlen % 8 == 0) && aligned16(x) && aligned16(out);
  const int silu = act == SSM_ACT_SILU;
  auto f = io_dtype == SSM_BF16 ? conv_kernel<1, false> : io_dtype == SSM_F16 ? conv_kernel<2, false>
                                                                                : conv_kernel<0, false>;
  hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     x, weight, bias, out, rows, dim, seqlen, silu, vec, nullptr, nullptr, nullptr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

extern "C" int causal_conv1d_fwd_ex(const causal_conv1d_args_t *a, void *stream_ptr) {
  const int st = causal_conv1d_ex_validate(a);
  if (st != SSM_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int64_t rows = a->batch * a->dim;
  const int64_t threads = rows * ((a->seqlen + 7) / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return SSM_ERR_SHAPE;
  const int vec = (a->seqlen % 8 == 0) && aligned16(a->x) && aligned16(a->out);
  const int silu = a->act == SSM_ACT_SILU;
  const bool seq = a->seq_idx != nullptr;
  auto f = a->io_dtype == SSM_BF16 ? (seq ? conv_kernel<1, true> : conv_kernel<1, false>)
         : a->io_dtype == SSM_F16  ? (seq ? conv_kernel<2, true> : conv_kernel<2, false>)
                                   : (seq ? conv_kernel<0, true> : conv_kernel<0, false>);
  hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a->x, a->weight, a->bias,
                     a->out, rows, a->dim, a->seqlen, silu, vec, a->seq_idx, a->initial_states, a->final_states);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

extern "C" int ssm_last_hip_error(void) { return g_last_hip_error; }
