// Host-side argument checks of the C ABI.  Plain C++: no HIP header, no device
// access, so every error path can be exercised on a machine without a GPU.
//
// What is checked follows the argument list of selective_scan_fn and
// causal_conv1d_fn (PaddleNLP Kernel operator-library guide, sections 4.1 and
// 4.2): required tensors present, positive sizes, dim divisible by the number
// of B/C groups, one of the supported io dtypes, dstate within the compiled
// range, and the conv width and activation the kernels are built for.
#include "ssmscan.h"

#include <cstdint>
#include <limits>

namespace {

bool positive(int64_t v) { return v > 0; }

// b*d*l (and friends) must fit comfortably in int64 element counts.
bool product_fits(int64_t a, int64_t b, int64_t c) {
  const int64_t lim = std::numeric_limits<int64_t>::max() / 8;
  if (a > lim / b) return false;
  const int64_t ab = a * b;
  return ab <= lim / c;
}

}  // namespace

extern "C" int ssm_scan_validate(const ssm_scan_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  if (!positive(a->batch) || !positive(a->dim) || !positive(a->seqlen) ||
      !positive(a->dstate) || !positive(a->ngroups))
    return SSM_ERR_SHAPE;
  if (a->dim % a->ngroups != 0) return SSM_ERR_SHAPE;
  if (a->seq_segments < 0) return SSM_ERR_SHAPE;
  if (!product_fits(a->batch, a->dim, a->seqlen) ||
      !product_fits(a->batch, a->ngroups * a->dstate, a->seqlen))
    return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16 && a->io_dtype != SSM_F16) return SSM_ERR_UNSUPPORTED;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if ((a->B_kind != SSM_BC_FIXED && a->B_kind != SSM_BC_VARYING) ||
      (a->C_kind != SSM_BC_FIXED && a->C_kind != SSM_BC_VARYING))
    return SSM_ERR_UNSUPPORTED;
  if (a->delta_softplus != 0 && a->delta_softplus != 1) return SSM_ERR_UNSUPPORTED;
  if (!a->delta || !a->A || !a->B || !a->C || !a->out) return SSM_ERR_NULL;
  if (a->conv_weight) {
    if (!a->conv_x) return SSM_ERR_NULL;
    if (a->conv_width != SSM_CONV_WIDTH) return SSM_ERR_UNSUPPORTED;
    if (a->conv_act != SSM_ACT_NONE && a->conv_act != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  } else if (!a->u) {
    return SSM_ERR_NULL;
  }
  return SSM_OK;
}

// selective_scan_fn with complex A (guide section 4.1): the checks of the
// real scan, with B/C holding (real, imaginary) pairs; no conv prologue and
// no checkpoints.
extern "C" int ssm_scan_complex_validate(const ssm_scan_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  const int st = ssm_scan_validate(a);
  if (st != SSM_OK) return st;
  if (!product_fits(a->batch, 2 * a->ngroups * a->dstate, a->seqlen)) return SSM_ERR_SHAPE;
  if (a->conv_weight) return SSM_ERR_UNSUPPORTED;
  if (!a->u) return SSM_ERR_NULL;
  return SSM_OK;
}

extern "C" int causal_conv1d_ex_validate(const causal_conv1d_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  const int st = causal_conv1d_validate(a->x, a->weight, a->out, a->batch, a->dim, a->seqlen, a->width,
                                        a->io_dtype, a->act);
  if (st != SSM_OK) return st;
  // the page: seq_idx excludes initial_states and the final states
  if (a->seq_idx && (a->initial_states || a->final_states)) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

extern "C" int ssm_scan_bwd_validate(const ssm_scan_bwd_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  if (!positive(a->batch) || !positive(a->dim) || !positive(a->seqlen) ||
      !positive(a->dstate) || !positive(a->ngroups))
    return SSM_ERR_SHAPE;
  if (a->dim % a->ngroups != 0) return SSM_ERR_SHAPE;
  // the per-workgroup partial sums hold up to (batch*ngroups, dim, dstate, seqlen) floats
  if (!product_fits(a->batch, a->dim, a->seqlen) ||
      !product_fits(a->batch * a->dim, a->dstate, a->seqlen))
    return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16 && a->io_dtype != SSM_F16) return SSM_ERR_UNSUPPORTED;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if ((a->B_kind != SSM_BC_FIXED && a->B_kind != SSM_BC_VARYING) ||
      (a->C_kind != SSM_BC_FIXED && a->C_kind != SSM_BC_VARYING))
    return SSM_ERR_UNSUPPORTED;
  if (a->delta_softplus != 0 && a->delta_softplus != 1) return SSM_ERR_UNSUPPORTED;
  if (a->seq_segments < 0) return SSM_ERR_SHAPE;
  if (!a->u || !a->delta || !a->A || !a->B || !a->C || !a->checkpoints || !a->dout ||
      !a->du || !a->ddelta || !a->dA || !a->dB || !a->dC)
    return SSM_ERR_NULL;
  if ((a->z && !a->dz) || (a->D && !a->dD) || (a->delta_bias && !a->ddelta_bias)) return SSM_ERR_NULL;
  return SSM_OK;
}

extern "C" int ssm_scan_bwd_complex_validate(const ssm_scan_bwd_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  const int st = ssm_scan_bwd_validate(a);
  if (st != SSM_OK) return st;
  // complex B/C are pairs: twice the elements of the real layout
  if (!product_fits(a->batch, 2 * a->ngroups * a->dstate, a->seqlen) ||
      !product_fits(a->batch * a->dim, 2 * a->dstate, a->seqlen))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

extern "C" int causal_conv1d_validate(const void *x, const float *weight, const void *out,
                                      int64_t batch, int64_t dim, int64_t seqlen,
                                      int32_t width, int32_t io_dtype, int32_t act) {
  if (!positive(batch) || !positive(dim) || !positive(seqlen)) return SSM_ERR_SHAPE;
  if (!product_fits(batch, dim, seqlen)) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16 && io_dtype != SSM_F16) return SSM_ERR_UNSUPPORTED;
  if (width != SSM_CONV_WIDTH) return SSM_ERR_UNSUPPORTED;
  if (act != SSM_ACT_NONE && act != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!x || !weight || !out) return SSM_ERR_NULL;
  return SSM_OK;
}

// selective_state_update (guide section 4.4 operator list) and
// causal_conv1d_update (section 4.2): the decode forms of the two operators.
extern "C" int ssm_state_update_validate(const ssm_state_update_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  if (!positive(a->batch) || !positive(a->dim) || !positive(a->dstate) || !positive(a->ngroups))
    return SSM_ERR_SHAPE;
  if (a->dim % a->ngroups != 0) return SSM_ERR_SHAPE;
  if (!product_fits(a->batch, a->dim, a->dstate) || !product_fits(a->batch, a->ngroups, a->dstate))
    return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16 && a->io_dtype != SSM_F16) return SSM_ERR_UNSUPPORTED;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if (a->dt_softplus != 0 && a->dt_softplus != 1) return SSM_ERR_UNSUPPORTED;
  if (!a->state || !a->x || !a->dt || !a->A || !a->B || !a->C || !a->out) return SSM_ERR_NULL;
  return SSM_OK;
}

extern "C" int causal_conv1d_update_validate(const void *x, const void *conv_state,
                                             const float *weight, const void *out,
                                             int64_t batch, int64_t dim, int64_t seqlen,
                                             int64_t state_len, int32_t width,
                                             int32_t io_dtype, int32_t act) {
  if (!positive(batch) || !positive(dim) || !positive(seqlen) || !positive(state_len))
    return SSM_ERR_SHAPE;
  if (!product_fits(batch, dim, seqlen) || !product_fits(batch, dim, state_len)) return SSM_ERR_SHAPE;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16 && io_dtype != SSM_F16) return SSM_ERR_UNSUPPORTED;
  if (width < 2 || width > SSM_CONV_WIDTH) return SSM_ERR_UNSUPPORTED;
  if (state_len < width - 1) return SSM_ERR_SHAPE;
  if (state_len > SSM_MAX_CONV_STATE) return SSM_ERR_UNSUPPORTED;
  if (act != SSM_ACT_NONE && act != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!x || !conv_state || !weight || !out) return SSM_ERR_NULL;
  return SSM_OK;
}

// Mamba-2 chunked scan (guide section 4.4 operator list).
extern "C" int ssd_scan_validate(const ssd_scan_args_t *a) {
  if (!a) return SSM_ERR_NULL;
  if (!positive(a->batch) || !positive(a->seqlen) || !positive(a->nheads) ||
      !positive(a->headdim) || !positive(a->dstate) || !positive(a->ngroups))
    return SSM_ERR_SHAPE;
  if (a->nheads % a->ngroups != 0) return SSM_ERR_SHAPE;
  if (!product_fits(a->batch * a->seqlen, a->nheads, a->headdim) ||
      !product_fits(a->batch * a->seqlen, a->ngroups, a->dstate) ||
      !product_fits(a->batch, a->nheads, a->headdim * a->dstate))
    return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (a->headdim != SSD_HEADDIM) return SSM_ERR_UNSUPPORTED;
  if (a->dstate != 32 && a->dstate != 64 && a->dstate != 128) return SSM_ERR_UNSUPPORTED;
  if (a->dt_softplus != 0 && a->dt_softplus != 1) return SSM_ERR_UNSUPPORTED;
  if (a->D_per_channel != 0 && a->D_per_channel != 1) return SSM_ERR_UNSUPPORTED;
  if (a->dt_limit != 0 && a->dt_limit != 1) return SSM_ERR_UNSUPPORTED;
  if (a->dt_limit && !(a->dt_min <= a->dt_max)) return SSM_ERR_SHAPE;
  if (a->seq_segments < 0) return SSM_ERR_SHAPE;
  if (!a->x || !a->dt || !a->A || !a->B || !a->C || !a->out) return SSM_ERR_NULL;
  const uintptr_t mis = (reinterpret_cast<uintptr_t>(a->x) | reinterpret_cast<uintptr_t>(a->B) |
                         reinterpret_cast<uintptr_t>(a->C) | reinterpret_cast<uintptr_t>(a->out) |
                         reinterpret_cast<uintptr_t>(a->z)) & 15u;
  if (mis) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

// the checks of ssd_scan_validate that the split operators share: sizes,
// dtypes, enum values, and x / dt / A / B present and aligned
static int ssd_common_validate(const ssd_scan_args_t *a, int64_t chunk_size) {
  if (!a) return SSM_ERR_NULL;
  if (!positive(a->batch) || !positive(a->seqlen) || !positive(a->nheads) ||
      !positive(a->headdim) || !positive(a->dstate) || !positive(a->ngroups))
    return SSM_ERR_SHAPE;
  if (a->nheads % a->ngroups != 0) return SSM_ERR_SHAPE;
  if (!product_fits(a->batch * a->seqlen, a->nheads, a->headdim) ||
      !product_fits(a->batch * a->seqlen, a->ngroups, a->dstate) ||
      !product_fits(a->batch, a->nheads, a->headdim * a->dstate))
    return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (a->headdim != SSD_HEADDIM) return SSM_ERR_UNSUPPORTED;
  if (a->dstate != 32 && a->dstate != 64 && a->dstate != 128) return SSM_ERR_UNSUPPORTED;
  if (a->dt_softplus != 0 && a->dt_softplus != 1) return SSM_ERR_UNSUPPORTED;
  if (a->dt_limit != 0 && a->dt_limit != 1) return SSM_ERR_UNSUPPORTED;
  if (a->dt_limit && !(a->dt_min <= a->dt_max)) return SSM_ERR_SHAPE;
  if (chunk_size <= 0 || chunk_size % SSD_CHUNK != 0) return SSM_ERR_UNSUPPORTED;
  if (!a->x || !a->dt || !a->A || !a->B) return SSM_ERR_NULL;
  const int64_t nchunks = (a->seqlen + chunk_size - 1) / chunk_size;
  if (!product_fits(nchunks, a->batch * a->nheads, a->headdim * a->dstate)) return SSM_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(a->x) | reinterpret_cast<uintptr_t>(a->B)) & 15u) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

extern "C" int ssd_chunk_state_validate(const ssd_scan_args_t *a, int64_t chunk_size, const float *states,
                                        const float *decays) {
  const int st = ssd_common_validate(a, chunk_size);
  if (st != SSM_OK) return st;
  if (!states || !decays) return SSM_ERR_NULL;
  return SSM_OK;
}

extern "C" int ssd_chunk_scan_validate(const ssd_scan_args_t *a, int64_t chunk_size, const float *carried) {
  const int st = ssd_common_validate(a, chunk_size);
  if (st != SSM_OK) return st;
  if (a->D_per_channel != 0 && a->D_per_channel != 1) return SSM_ERR_UNSUPPORTED;
  if (!a->C || !a->out || !carried) return SSM_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(a->C) | reinterpret_cast<uintptr_t>(a->out) |
       reinterpret_cast<uintptr_t>(a->z)) & 15u)
    return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

extern "C" int ssd_state_passing_validate(int64_t nchunks, int64_t batch, int64_t nheads, int64_t headdim,
                                          int64_t dstate, const float *states, const float *decays,
                                          const float *carried) {
  if (!positive(nchunks) || !positive(batch) || !positive(nheads) || !positive(headdim) || !positive(dstate))
    return SSM_ERR_SHAPE;
  if (!product_fits(nchunks, batch * nheads, headdim * dstate) || !product_fits(batch, nheads, headdim * dstate))
    return SSM_ERR_SHAPE;
  if (!states || !decays || !carried) return SSM_ERR_NULL;
  return SSM_OK;
}

extern "C" const char *ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "bad shape (size <= 0, dim not divisible by ngroups, or too large)";
    case SSM_ERR_UNSUPPORTED: return "unsupported argument (dtype, dstate > 16, conv width or cache length out of range, or enum value)";
    case SSM_ERR_HIP: return "HIP runtime error";
    case SSM_ERR_WORKSPACE: return "workspace smaller than required";
    case SSM_ERR_SCRATCH: return "plan needs more scratch than the built-in no-allocation buffer holds";
    default: return "unknown status";
  }
}

extern "C" int ssm_abi_version(void) { return SSM_ABI_VERSION; }
