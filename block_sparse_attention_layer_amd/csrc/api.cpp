// Entry points of the C ABI declared in include/vmoba.h: host-side argument checks,
// then the kernel launchers.  Nothing is enqueued when a check fails.
#include <math.h>

#include "../../include/vmoba.h"
#include "internal.h"

using namespace vmoba;

namespace {

int check_common(const vmoba_problem* p) { return validate_problem(p); }

int check_blocks(const vmoba_problem* p) {
  const Geom g = make_geom(p);
  return g.Nb <= kMaxBlocks ? VMOBA_OK : VMOBA_ERR_SHAPE;
}

int check_ws(const vmoba_problem* p, int op, const void* ws, size_t ws_bytes) {
  size_t need = 0;
  int st = workspace_bytes(p, op, &need);
  if (st) return st;
  if (need > ws_bytes) return VMOBA_ERR_WORKSPACE;
  if (need > 0 && !ws) return VMOBA_ERR_NULL;
  return VMOBA_OK;
}

// Token-granular calls: bf16, N_b <= kMaxBlocks, and the mask and score tables within the
// 32-bit ranges the kernels use.
int check_tokens(const vmoba_problem* p) {
  if (p->dtype != VMOBA_BF16) return VMOBA_ERR_DTYPE;
  const Geom g = make_geom(p);
  if (g.Nb > kMaxBlocks) return VMOBA_ERR_SHAPE;
  const int64_t G = int64_t(g.B) * g.Hh;
  const int64_t words = (int64_t(g.Nb) + 31) / 32;
  if (G * g.L * g.Nb >= (int64_t(1) << 31) || G * g.L * words * 4 >= (int64_t(1) << 32))
    return VMOBA_ERR_OVERFLOW;
  return VMOBA_OK;
}

}  // namespace

extern "C" {

int vmoba_partition_pool(const vmoba_problem* p, const void* q, const void* k,
                         float* q_pool, float* k_pool, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if (!q || !k || !q_pool || !k_pool) return VMOBA_ERR_NULL;
  return launch_pool(make_geom(p), q, k, q_pool, k_pool, stream);
}

int vmoba_select(const vmoba_problem* p, const float* q_pool, const float* k_pool,
                 float tau, int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr,
                 int32_t* row_idx, float* head_stats, float* norm_scores, void* ws,
                 size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  if (!(tau > 0.0f) || !(tau <= 1.0f) || !isfinite(tau)) return VMOBA_ERR_TAU;
  if (!q_pool || !k_pool || !row_ptr || !col_idx || !col_ptr || !row_idx || !head_stats)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_SELECT, ws, ws_bytes))) return st;
  return launch_select(make_geom(p), q_pool, k_pool, VMOBA_SEL_THRESHOLD_GLOBAL, tau, 0,
                       row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores, ws,
                       stream);
}

int vmoba_select_mode(const vmoba_problem* p, const float* q_pool, const float* k_pool,
                      int mode, float tau, int32_t topk, int32_t* row_ptr, int32_t* col_idx,
                      int32_t* col_ptr, int32_t* row_idx, float* head_stats,
                      float* norm_scores, void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  const bool thr = mode == VMOBA_SEL_THRESHOLD_GLOBAL || mode == VMOBA_SEL_THRESHOLD_LOCAL;
  const bool tk = mode == VMOBA_SEL_TOPK_GLOBAL || mode == VMOBA_SEL_TOPK_LOCAL;
  if (!thr && !tk) return VMOBA_ERR_SELECT;
  if (thr && (!(tau > 0.0f) || !(tau <= 1.0f) || !isfinite(tau))) return VMOBA_ERR_TAU;
  if (tk && topk < 1) return VMOBA_ERR_SELECT;
  if (!q_pool || !k_pool || !row_ptr || !col_idx || !col_ptr || !row_idx || !head_stats)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_SELECT, ws, ws_bytes))) return st;
  return launch_select(make_geom(p), q_pool, k_pool, mode, thr ? tau : 0.0f,
                       tk ? topk : 0, row_ptr, col_idx, col_ptr, row_idx, head_stats,
                       norm_scores, ws, stream);
}

int vmoba_sparse_attn_fwd(const vmoba_problem* p, const void* q, const void* k,
                          const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                          void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  if (!q || !k || !v || !row_ptr || !col_idx || !o || !lse) return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_SPARSE_FWD, ws, ws_bytes))) return st;
  return launch_attn_fwd(make_geom(p), false, q, k, v, row_ptr, col_idx, o, lse, ws,
                         stream);
}

int vmoba_sparse_attn_bwd(const vmoba_problem* p, const void* q, const void* k,
                          const void* v, const void* o, const float* lse,
                          const void* dout, const int32_t* row_ptr,
                          const int32_t* col_idx, const int32_t* col_ptr,
                          const int32_t* row_idx, void* dq, void* dk, void* dv, void* ws,
                          size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  if (!q || !k || !v || !o || !lse || !dout || !row_ptr || !col_idx || !col_ptr ||
      !row_idx || !dq || !dk || !dv)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_SPARSE_BWD, ws, ws_bytes))) return st;
  const Geom g = make_geom(p);
  float* delta = static_cast<float*>(ws);
  if ((st = launch_bwd_delta(g, o, dout, delta, stream))) return st;
  return launch_bwd_dkdv_dq(g, q, k, v, lse, delta, dout, row_ptr, col_idx, col_ptr, row_idx,
                            dq, dk, dv, stream);
}

int vmoba_sparse_attn_bwd_delta(const vmoba_problem* p, const void* o, const void* dout,
                                float* delta, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if (!o || !dout || !delta) return VMOBA_ERR_NULL;
  return launch_bwd_delta(make_geom(p), o, dout, delta, stream);
}

int vmoba_sparse_attn_bwd_dkdv(const vmoba_problem* p, const void* q, const void* k,
                               const void* v, const float* lse, const float* delta,
                               const void* dout, const int32_t* col_ptr,
                               const int32_t* row_idx, void* dk, void* dv, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  if (!q || !k || !v || !lse || !delta || !dout || !col_ptr || !row_idx || !dk || !dv)
    return VMOBA_ERR_NULL;
  return launch_bwd_dkdv(make_geom(p), false, q, k, v, lse, delta, dout, col_ptr, row_idx,
                         dk, dv, stream);
}

int vmoba_sparse_attn_bwd_dq(const vmoba_problem* p, const void* q, const void* k,
                             const void* v, const float* lse, const float* delta,
                             const void* dout, const int32_t* row_ptr,
                             const int32_t* col_idx, void* dq, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_blocks(p))) return st;
  if (!q || !k || !v || !lse || !delta || !dout || !row_ptr || !col_idx || !dq)
    return VMOBA_ERR_NULL;
  return launch_bwd_dq(make_geom(p), false, q, k, v, lse, delta, dout, row_ptr, col_idx, dq,
                       stream);
}

int vmoba_dense_attn_fwd(const vmoba_problem* p, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  int st = check_common(p);
  if (st) return st;
  if (!q || !k || !v || !o || !lse) return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_DENSE_FWD, ws, ws_bytes))) return st;
  return launch_attn_fwd(make_geom(p), true, q, k, v, nullptr, nullptr, o, lse, ws,
                         stream);
}

int vmoba_dense_attn_bwd(const vmoba_problem* p, const void* q, const void* k,
                         const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_DENSE_BWD, ws, ws_bytes))) return st;
  const Geom g = make_geom(p);
  float* delta = static_cast<float*>(ws);
  if ((st = launch_bwd_delta(g, o, dout, delta, stream))) return st;
  if ((st = launch_bwd_dkdv(g, true, q, k, v, lse, delta, dout, nullptr, nullptr, dk, dv,
                            stream)))
    return st;
  return launch_bwd_dq(g, true, q, k, v, lse, delta, dout, nullptr, nullptr, dq, stream);
}

int vmoba_select_tokens(const vmoba_problem* p, const void* q, const float* k_pool, float tau,
                        uint32_t* token_mask, int32_t* row_ptr, int32_t* col_idx,
                        int32_t* col_ptr, int32_t* row_idx, float* head_stats, void* ws,
                        size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_tokens(p))) return st;
  if (!(tau > 0.0f) || !(tau <= 1.0f) || !isfinite(tau)) return VMOBA_ERR_TAU;
  if (!q || !k_pool || !token_mask || !row_ptr || !col_idx || !col_ptr || !row_idx ||
      !head_stats)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_SELECT_TOKENS, ws, ws_bytes))) return st;
  return launch_select_tokens(make_geom(p), q, k_pool, tau, token_mask, row_ptr, col_idx,
                              col_ptr, row_idx, head_stats, ws, stream);
}

int vmoba_token_attn_fwd(const vmoba_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const uint32_t* token_mask, void* o, float* lse, void* ws,
                         size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_tokens(p))) return st;
  if (make_geom(p).S < 4) return VMOBA_ERR_SHAPE;
  if (!q || !k || !v || !row_ptr || !col_idx || !token_mask || !o || !lse)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_TOKEN_FWD, ws, ws_bytes))) return st;
  const Geom g = make_geom(p);
  uint32_t* posmask = static_cast<uint32_t*>(ws);
  if ((st = launch_token_posmask(g, row_ptr, col_idx, token_mask, posmask, stream))) return st;
  return launch_token_attn_fwd(g, q, k, v, row_ptr, col_idx, posmask, o, lse, stream);
}

int vmoba_token_attn_bwd(const vmoba_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* col_ptr, const int32_t* row_idx,
                         const uint32_t* token_mask, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream) {
  int st = check_common(p);
  if (st) return st;
  if ((st = check_tokens(p))) return st;
  if (make_geom(p).S < 4) return VMOBA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !row_ptr || !col_idx || !col_ptr ||
      !row_idx || !token_mask || !dq || !dk || !dv)
    return VMOBA_ERR_NULL;
  if ((st = check_ws(p, VMOBA_OP_TOKEN_BWD, ws, ws_bytes))) return st;
  const Geom g = make_geom(p);
  const size_t words = (size_t(g.Nb) + 31) / 32;
  uint32_t* posmask = static_cast<uint32_t*>(ws);
  float* delta = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                          align256(size_t(g.B) * g.Hh * g.L * words * 4));
  if ((st = launch_token_posmask(g, row_ptr, col_idx, token_mask, posmask, stream))) return st;
  if ((st = launch_bwd_delta(g, o, dout, delta, stream))) return st;
  if ((st = launch_token_bwd_dkdv(g, q, k, v, lse, delta, dout, col_ptr, row_idx, token_mask,
                                  dk, dv, stream)))
    return st;
  return launch_token_bwd_dq(g, q, k, v, lse, delta, dout, row_ptr, col_idx, posmask, dq,
                             stream);
}

}  // extern "C"
