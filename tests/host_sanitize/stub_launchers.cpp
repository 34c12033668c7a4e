// Host-only stand-ins for the kernel launchers of the C ABI, for a sanitizer build of the
// host code (api.cpp, validate.cpp) with g++: each records that it was called and checks
// that the host code handed it the pointers the call needs.  Nothing here touches a GPU.
#include <stdio.h>
#include <stdlib.h>

#include "../../block_sparse_attention_layer_amd/csrc/internal.h"

int g_launches = 0;

#define NEED(x)                                                          \
  do {                                                                   \
    if (!(x)) {                                                          \
      fprintf(stderr, "%s: launcher got a null %s\n", __func__, #x);    \
      abort();                                                           \
    }                                                                    \
  } while (0)

namespace vmoba {

size_t select_ws(const Geom& g) {
  const size_t G = size_t(g.B) * g.Hh, nb = size_t(g.Nb);
  return align256(G * nb * nb * 4) + align256(G * nb * 16) + align256(G * 4096);
}

size_t token_select_ws(const Geom& g) {
  const size_t G = size_t(g.B) * g.Hh;
  return align256(G * size_t(g.L) * g.Nb * 4) + align256(G * 4096);
}

int launch_pool(const Geom& g, const void* q, const void* k, float* qp, float* kp, void*) {
  NEED(g.Nb > 0 && q && k && qp && kp);
  return ++g_launches, VMOBA_OK;
}

int launch_select(const Geom& g, const float* qp, const float* kp, int mode, float, int,
                  int32_t* rp, int32_t* ci, int32_t* cp, int32_t* ri, float* hs, float*,
                  void* ws, void*) {
  NEED(g.Nb > 0 && g.Nb <= kMaxBlocks && qp && kp && rp && ci && cp && ri && hs && ws);
  NEED(mode >= 0 && mode <= 3);
  return ++g_launches, VMOBA_OK;
}

int launch_select_tokens(const Geom& g, const void* q, const float* kp, float, uint32_t* tm,
                         int32_t* rp, int32_t* ci, int32_t* cp, int32_t* ri, float* hs,
                         void* ws, void*) {
  NEED(g.Nb > 0 && q && kp && tm && rp && ci && cp && ri && hs && ws);
  return ++g_launches, VMOBA_OK;
}

int launch_token_posmask(const Geom&, const int32_t* rp, const int32_t* ci, const uint32_t* tm,
                         uint32_t* pm, void*) {
  NEED(rp && ci && tm && pm);
  return ++g_launches, VMOBA_OK;
}

int launch_token_attn_fwd(const Geom&, const void* q, const void* k, const void* v,
                          const int32_t* rp, const int32_t* ci, const uint32_t* pm, void* o,
                          float* lse, void*) {
  NEED(q && k && v && rp && ci && pm && o && lse);
  return ++g_launches, VMOBA_OK;
}

int launch_token_bwd_dkdv(const Geom&, const void* q, const void* k, const void* v,
                          const float* lse, const float* delta, const void* dout,
                          const int32_t* cp, const int32_t* ri, const uint32_t* tm, void* dk,
                          void* dv, void*) {
  NEED(q && k && v && lse && delta && dout && cp && ri && tm && dk && dv);
  return ++g_launches, VMOBA_OK;
}

int launch_token_bwd_dq(const Geom&, const void* q, const void* k, const void* v,
                        const float* lse, const float* delta, const void* dout,
                        const int32_t* rp, const int32_t* ci, const uint32_t* pm, void* dq,
                        void*) {
  NEED(q && k && v && lse && delta && dout && rp && ci && pm && dq);
  return ++g_launches, VMOBA_OK;
}

int launch_attn_fwd(const Geom&, bool dense, const void* q, const void* k, const void* v,
                    const int32_t* rp, const int32_t* ci, void* o, float* lse, void*, void*) {
  NEED(q && k && v && o && lse && (dense || (rp && ci)));
  return ++g_launches, VMOBA_OK;
}

int launch_bwd_delta(const Geom&, const void* o, const void* dout, float* delta, void*) {
  NEED(o && dout && delta);
  return ++g_launches, VMOBA_OK;
}

int launch_bwd_dkdv(const Geom&, bool dense, const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dout, const int32_t* cp,
                    const int32_t* ri, void* dk, void* dv, void*) {
  NEED(q && k && v && lse && delta && dout && dk && dv && (dense || (cp && ri)));
  return ++g_launches, VMOBA_OK;
}

int launch_bwd_dq(const Geom&, bool dense, const void* q, const void* k, const void* v,
                  const float* lse, const float* delta, const void* dout, const int32_t* rp,
                  const int32_t* ci, void* dq, void*) {
  NEED(q && k && v && lse && delta && dout && dq && (dense || (rp && ci)));
  return ++g_launches, VMOBA_OK;
}

int launch_bwd_dkdv_dq(const Geom&, const void* q, const void* k, const void* v,
                       const float* lse, const float* delta, const void* dout,
                       const int32_t* rp, const int32_t* ci, const int32_t* cp,
                       const int32_t* ri, void* dq, void* dk, void* dv, void*) {
  NEED(q && k && v && lse && delta && dout && rp && ci && cp && ri && dq && dk && dv);
  return g_launches += 2, VMOBA_OK;
}

}  // namespace vmoba
