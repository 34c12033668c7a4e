// Host-only part of the C ABI: argument validation, geometry, workspace sizes and
// status strings.  Built without HIP so that it can also be linked into host tests.
#include <math.h>
#include <string.h>

#include "../../include/vmoba.h"
#include "geometry.h"
#include "internal.h"

namespace vmoba {

int validate_problem(const vmoba_problem* p) {
  if (!p) return VMOBA_ERR_NULL;
  if (p->batch <= 0 || p->heads <= 0 || p->T <= 0 || p->H <= 0 || p->W <= 0 ||
      p->bt <= 0 || p->bh <= 0 || p->bw <= 0 || p->layer_idx < 0)
    return VMOBA_ERR_SHAPE;
  if (p->T % p->bt || p->H % p->bh || p->W % p->bw) return VMOBA_ERR_SHAPE;
  if (p->dtype != VMOBA_BF16 && p->dtype != VMOBA_FP32) return VMOBA_ERR_DTYPE;
  if (p->grad_dtype != VMOBA_BF16 && p->grad_dtype != VMOBA_FP32) return VMOBA_ERR_DTYPE;
  if (p->dtype == VMOBA_FP32 && p->grad_dtype != VMOBA_FP32) return VMOBA_ERR_DTYPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VMOBA_ERR_HEAD_DIM;
  const int mode = p->layer_idx % 3;
  if (mode == 0 && (p->bh != p->H || p->bw != p->W)) return VMOBA_ERR_MODE;
  if (mode == 1 && p->bt != p->T) return VMOBA_ERR_MODE;
  // Every element count and index used on the device stays below 2^31.  The products are
  // formed with a saturating multiply (all factors are positive here), so no intermediate
  // overflows whatever the sizes.
  constexpr int64_t kLim = int64_t(1) << 31;
  auto mul = [](int64_t a, int64_t b) -> int64_t {
    return a >= kLim || b >= kLim || a * b >= kLim ? kLim : a * b;
  };
  const int64_t L = mul(mul(p->T, p->H), p->W);
  const int64_t elems = mul(mul(mul(p->batch, L), p->heads), p->head_dim);
  const int64_t nb = mul(mul(p->T / p->bt, p->H / p->bh), p->W / p->bw);
  const int64_t groups = mul(p->batch, p->heads);
  if (L >= kLim || elems >= kLim || mul(groups, L) >= kLim ||
      mul(mul(groups, nb), nb) >= kLim || mul(nb, nb) >= kLim)
    return VMOBA_ERR_OVERFLOW;
  return VMOBA_OK;
}

Geom make_geom(const vmoba_problem* p) {
  Geom g;
  g.B = p->batch;
  g.Hh = p->heads;
  g.D = p->head_dim;
  g.T = p->T;
  g.H = p->H;
  g.W = p->W;
  g.L = p->T * p->H * p->W;
  g.bt = p->bt;
  g.bh = p->bh;
  g.bw = p->bw;
  g.nt = p->T / p->bt;
  g.nh = p->H / p->bh;
  g.nw = p->W / p->bw;
  g.Nb = g.nt * g.nh * g.nw;
  g.S = p->bt * p->bh * p->bw;
  g.mode = p->layer_idx % 3;
  g.dtype = p->dtype;
  g.grad_dtype = p->grad_dtype;
  g.div_S = make_fastdiv(uint32_t(g.S));
  g.div_nhnw = make_fastdiv(uint32_t(g.nh * g.nw));
  g.div_nw = make_fastdiv(uint32_t(g.nw));
  g.div_bhbw = make_fastdiv(uint32_t(g.bh * g.bw));
  g.div_bw = make_fastdiv(uint32_t(g.bw));
  return g;
}


int workspace_bytes(const vmoba_problem* p, int op, size_t* bytes) {
  const Geom g = make_geom(p);
  const size_t groups = size_t(g.B) * g.Hh;
  switch (op) {
    case VMOBA_OP_POOL:
    case VMOBA_OP_SPARSE_FWD:
    case VMOBA_OP_DENSE_FWD:
      *bytes = 0;
      return VMOBA_OK;
    case VMOBA_OP_SELECT:
      // block scores, fp32 per head group, then the pool tables and a row bitmap (global
      // strategies) or a row bitmap and three floats per row (local ones)
      *bytes = select_ws(g);
      return VMOBA_OK;
    case VMOBA_OP_SPARSE_BWD:
    case VMOBA_OP_DENSE_BWD:
      // delta = rowsum(dO * O), fp32 [B][Hh][L]
      *bytes = align256(groups * size_t(g.L) * sizeof(float));
      return VMOBA_OK;
    case VMOBA_OP_SELECT_TOKENS:
      *bytes = token_select_ws(g);
      return VMOBA_OK;
    case VMOBA_OP_TOKEN_FWD:
    case VMOBA_OP_TOKEN_BWD: {
      // the token mask re-indexed by list position, u32 [B*Hh][L][ceil(N_b/32)]; the
      // backward adds delta
      const size_t words = (size_t(g.Nb) + 31) / 32;
      *bytes = align256(groups * size_t(g.L) * words * 4);
      if (op == VMOBA_OP_TOKEN_BWD) *bytes += align256(groups * size_t(g.L) * sizeof(float));
      return VMOBA_OK;
    }
    default:
      return VMOBA_ERR_OP;
  }
}

}  // namespace vmoba

extern "C" {

const char* vmoba_version(void) { return "vmoba-gfx950 0.1.0"; }

const char* vmoba_status_string(int status) {
  switch (status) {
    case VMOBA_OK: return "ok";
    case VMOBA_ERR_NULL: return "null pointer argument";
    case VMOBA_ERR_SHAPE: return "bad shape: sizes must be positive and the block shape must divide (T, H, W)";
    case VMOBA_ERR_MODE: return "block shape does not match the partition mode layer_idx % 3";
    case VMOBA_ERR_TAU: return "tau must be finite and in (0, 1]";
    case VMOBA_ERR_DTYPE: return "unsupported dtype";
    case VMOBA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case VMOBA_ERR_WORKSPACE: return "workspace too small";
    case VMOBA_ERR_OVERFLOW: return "problem too large for 32-bit indexing";
    case VMOBA_ERR_HIP: return "HIP runtime error";
    case VMOBA_ERR_OP: return "unknown op";
    case VMOBA_ERR_SELECT: return "unknown selection mode or top-k count < 1";
    case VMOBA_ERR_SCRATCH: return "problem needs more delta rows than the no-allocation backward's fixed scratch holds (B * Hh * L * 4 bytes > VMOBA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int vmoba_validate(const vmoba_problem* p) { return vmoba::validate_problem(p); }

int vmoba_num_blocks(const vmoba_problem* p, int32_t* nb) {
  int st = vmoba::validate_problem(p);
  if (st) return st;
  if (!nb) return VMOBA_ERR_NULL;
  *nb = vmoba::make_geom(p).Nb;
  return VMOBA_OK;
}

int vmoba_workspace_size(const vmoba_problem* p, int op, size_t* bytes) {
  int st = vmoba::validate_problem(p);
  if (st) return st;
  if (!bytes) return VMOBA_ERR_NULL;
  return vmoba::workspace_bytes(p, op, bytes);
}

}  // extern "C"
