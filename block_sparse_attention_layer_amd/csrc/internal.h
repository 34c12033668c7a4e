// Internal interface between the C ABI (api.cpp, validate.cpp) and the kernel
// launchers (*.hip).  Host code only; no HIP types so that it builds with g++.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/vmoba.h"
#include "geometry.h"

namespace vmoba {

// Largest block count the selection and sparse attention calls accept: the selection
// kernel keeps the N_b x N_b pair bitmap of one head in LDS (128 KiB at 1024 blocks).
constexpr int kMaxBlocks = 1024;

// Workspace buffers start on 256-byte boundaries.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int validate_problem(const vmoba_problem* p);
Geom make_geom(const vmoba_problem* p);
int workspace_bytes(const vmoba_problem* p, int op, size_t* bytes);

// Launchers: enqueue on `stream` (a hipStream_t) and return VMOBA_OK or VMOBA_ERR_HIP.
int launch_pool(const Geom& g, const void* q, const void* k, float* q_pool,
                float* k_pool, void* stream);

// mode: vmoba_selection; tau for the threshold modes, topk for the top-k modes.
int launch_select(const Geom& g, const float* q_pool, const float* k_pool, int mode, float tau,
                  int topk, int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr,
                  int32_t* row_idx, float* head_stats, float* norm_scores, void* ws,
                  void* stream);

// Workspace sizes of the selection calls (select.hip).
size_t select_ws(const Geom& g);

// Token-granular selection (select.hip); token_select_ws is its workspace size.
size_t token_select_ws(const Geom& g);
int launch_select_tokens(const Geom& g, const void* q, const float* k_pool, float tau,
                         uint32_t* tokmask, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* col_ptr, int32_t* row_idx, float* head_stats, void* ws,
                         void* stream);

// Attention under a token mask (attn_fwd.hip / attn_bwd.hip, bf16): the list-position
// mask from the key-block mask, the forward, and the two gradient kernels.
int launch_token_posmask(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx,
                         const uint32_t* tokmask, uint32_t* posmask, void* stream);
int launch_token_attn_fwd(const Geom& g, const void* q, const void* k, const void* v,
                          const int32_t* row_ptr, const int32_t* col_idx,
                          const uint32_t* posmask, void* o, float* lse, void* stream);
int launch_token_bwd_dkdv(const Geom& g, const void* q, const void* k, const void* v,
                          const float* lse, const float* delta, const void* dout,
                          const int32_t* col_ptr, const int32_t* row_idx,
                          const uint32_t* tokmask, void* dk, void* dv, void* stream);
int launch_token_bwd_dq(const Geom& g, const void* q, const void* k, const void* v,
                        const float* lse, const float* delta, const void* dout,
                        const int32_t* row_ptr, const int32_t* col_idx,
                        const uint32_t* posmask, void* dq, void* stream);

int launch_attn_fwd(const Geom& g, bool dense, const void* q, const void* k,
                    const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                    void* o, float* lse, void* ws, void* stream);

int launch_bwd_delta(const Geom& g, const void* o, const void* dout, float* delta,
                     void* stream);

int launch_bwd_dkdv(const Geom& g, bool dense, const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dout,
                    const int32_t* col_ptr, const int32_t* row_idx, void* dk, void* dv,
                    void* stream);

int launch_bwd_dq(const Geom& g, bool dense, const void* q, const void* k, const void* v,
                  const float* lse, const float* delta, const void* dout,
                  const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* stream);

// The sparse dK/dV and dQ of one backward, dQ on a second stream of the device (forked
// from and joined back into `stream`), or both on `stream` when no second stream is had.
int launch_bwd_dkdv_dq(const Geom& g, const void* q, const void* k, const void* v,
                       const float* lse, const float* delta, const void* dout,
                       const int32_t* row_ptr, const int32_t* col_idx,
                       const int32_t* col_ptr, const int32_t* row_idx, void* dq, void* dk,
                       void* dv, void* stream);

}  // namespace vmoba
