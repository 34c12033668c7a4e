// Host driver of the sanitizer build: every entry point of api.cpp and validate.cpp with
// valid arguments and with each argument error, the workspace sizes of every op, every
// status string, and the geometry helpers (block map a bijection onto the tokens and
// inverted by token_block; fast division exact).  Built with address and undefined-
// behaviour sanitizers that abort on the first report; prints "ok" at the end.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/vmoba.h"
#include "../../block_sparse_attention_layer_amd/csrc/geometry.h"

extern int g_launches;

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond);      \
      g_fail = 1;                                                      \
    }                                                                  \
  } while (0)

static vmoba_problem prob(int B, int Hh, int d, int T, int H, int W, int l, int bt, int bh,
                          int bw, int dt = VMOBA_BF16, int gdt = VMOBA_BF16) {
  vmoba_problem p;
  p.batch = B; p.heads = Hh; p.head_dim = d; p.T = T; p.H = H; p.W = W; p.layer_idx = l;
  p.bt = bt; p.bh = bh; p.bw = bw; p.dtype = dt; p.grad_dtype = gdt;
  return p;
}

// a pointer that is never dereferenced (the launchers are stand-ins)
static char g_dummy[64];
#define F ((void*)g_dummy)
#define FI ((int32_t*)g_dummy)
#define FF ((float*)g_dummy)
#define FU ((uint32_t*)g_dummy)

// call `fn` with argument i replaced by NULL for each pointer argument: every such call
// must return VMOBA_ERR_NULL and enqueue nothing
template <typename Fn>
static void each_null(int n, Fn fn) {
  for (int i = 0; i < n; ++i) {
    const int before = g_launches;
    EXPECT(fn(i) == VMOBA_ERR_NULL);
    EXPECT(g_launches == before);
  }
}

static void check_entry_points(const vmoba_problem& p) {
  size_t ws_sel = 0, ws_bwd = 0, ws_tok = 0, ws_tf = 0, ws_tb = 0, ws = 0;
  EXPECT(vmoba_workspace_size(&p, VMOBA_OP_SELECT, &ws_sel) == VMOBA_OK);
  EXPECT(vmoba_workspace_size(&p, VMOBA_OP_SPARSE_BWD, &ws_bwd) == VMOBA_OK);
  EXPECT(vmoba_workspace_size(&p, VMOBA_OP_SELECT_TOKENS, &ws_tok) == VMOBA_OK);
  EXPECT(vmoba_workspace_size(&p, VMOBA_OP_TOKEN_FWD, &ws_tf) == VMOBA_OK);
  EXPECT(vmoba_workspace_size(&p, VMOBA_OP_TOKEN_BWD, &ws_tb) == VMOBA_OK);
  for (int op = 0; op <= 8; ++op) EXPECT(vmoba_workspace_size(&p, op, &ws) == VMOBA_OK);
  EXPECT(vmoba_workspace_size(&p, 9, &ws) == VMOBA_ERR_OP);
  EXPECT(vmoba_workspace_size(&p, -1, &ws) == VMOBA_ERR_OP);
  EXPECT(vmoba_workspace_size(&p, 0, nullptr) == VMOBA_ERR_NULL);
  int32_t nb = 0;
  EXPECT(vmoba_num_blocks(&p, &nb) == VMOBA_OK && nb > 0);

  int before = g_launches;
  EXPECT(vmoba_partition_pool(&p, F, F, FF, FF, nullptr) == VMOBA_OK);
  EXPECT(g_launches == before + 1);
  each_null(4, [&](int i) {
    void* a[4] = {F, F, F, F};
    a[i] = nullptr;
    return vmoba_partition_pool(&p, a[0], a[1], (float*)a[2], (float*)a[3], nullptr);
  });

  auto sel = [&](int i, float tau, size_t n) {
    void* a[8] = {F, F, F, F, F, F, F, F};
    if (i >= 0) a[i] = nullptr;
    return vmoba_select(&p, (float*)a[0], (float*)a[1], tau, (int32_t*)a[2], (int32_t*)a[3],
                        (int32_t*)a[4], (int32_t*)a[5], (float*)a[6], nullptr, a[7], n,
                        nullptr);
  };
  before = g_launches;
  EXPECT(sel(-1, 0.25f, ws_sel) == VMOBA_OK);
  EXPECT(sel(-1, 1.0f, ws_sel) == VMOBA_OK);
  EXPECT(g_launches == before + 2);
  before = g_launches;
  each_null(8, [&](int i) { return sel(i, 0.25f, ws_sel); });
  EXPECT(sel(-1, 0.0f, ws_sel) == VMOBA_ERR_TAU);
  EXPECT(sel(-1, 1.0001f, ws_sel) == VMOBA_ERR_TAU);
  EXPECT(sel(-1, NAN, ws_sel) == VMOBA_ERR_TAU);
  EXPECT(sel(-1, INFINITY, ws_sel) == VMOBA_ERR_TAU);
  if (ws_sel > 0) EXPECT(sel(-1, 0.25f, ws_sel - 1) == VMOBA_ERR_WORKSPACE);
  EXPECT(g_launches == before);

  for (int mode = -1; mode <= 4; ++mode) {
    for (int k : {-1, 0, 1, 1 << 30}) {
      for (float tau : {0.0f, 0.25f, 2.0f}) {
        const bool thr = mode == 0 || mode == 2, tk = mode == 1 || mode == 3;
        int want = VMOBA_OK;
        if (!thr && !tk) want = VMOBA_ERR_SELECT;
        else if (thr && !(tau > 0.0f && tau <= 1.0f)) want = VMOBA_ERR_TAU;
        else if (tk && k < 1) want = VMOBA_ERR_SELECT;
        before = g_launches;
        EXPECT(vmoba_select_mode(&p, FF, FF, mode, tau, k, FI, FI, FI, FI, FF, nullptr, F,
                                 ws_sel, nullptr) == want);
        EXPECT(g_launches == before + (want == VMOBA_OK ? 1 : 0));
      }
    }
  }

  before = g_launches;
  EXPECT(vmoba_sparse_attn_fwd(&p, F, F, F, FI, FI, F, FF, nullptr, 0, nullptr) == VMOBA_OK);
  EXPECT(g_launches == before + 1);
  each_null(7, [&](int i) {
    void* a[7] = {F, F, F, F, F, F, F};
    a[i] = nullptr;
    return vmoba_sparse_attn_fwd(&p, a[0], a[1], a[2], (int32_t*)a[3], (int32_t*)a[4], a[5],
                                 (float*)a[6], nullptr, 0, nullptr);
  });

  auto bwd = [&](int i, size_t n) {
    void* a[14] = {F, F, F, F, F, F, F, F, F, F, F, F, F, F};
    if (i >= 0) a[i] = nullptr;
    return vmoba_sparse_attn_bwd(&p, a[0], a[1], a[2], a[3], (float*)a[4], a[5],
                                 (int32_t*)a[6], (int32_t*)a[7], (int32_t*)a[8],
                                 (int32_t*)a[9], a[10], a[11], a[12], a[13], n, nullptr);
  };
  before = g_launches;
  EXPECT(bwd(-1, ws_bwd) == VMOBA_OK);
  EXPECT(g_launches == before + 3);
  each_null(13, [&](int i) { return bwd(i, ws_bwd); });
  before = g_launches;
  EXPECT(bwd(-1, ws_bwd - 1) == VMOBA_ERR_WORKSPACE);
  EXPECT(bwd(13, ws_bwd) == VMOBA_ERR_NULL);
  EXPECT(g_launches == before);

  before = g_launches;
  EXPECT(vmoba_sparse_attn_bwd_delta(&p, F, F, FF, nullptr) == VMOBA_OK);
  EXPECT(vmoba_sparse_attn_bwd_dkdv(&p, F, F, F, FF, FF, F, FI, FI, F, F, nullptr) == VMOBA_OK);
  EXPECT(vmoba_sparse_attn_bwd_dq(&p, F, F, F, FF, FF, F, FI, FI, F, nullptr) == VMOBA_OK);
  EXPECT(g_launches == before + 3);
  each_null(3, [&](int i) {
    void* a[3] = {F, F, F};
    a[i] = nullptr;
    return vmoba_sparse_attn_bwd_delta(&p, a[0], a[1], (float*)a[2], nullptr);
  });
  each_null(10, [&](int i) {
    void* a[10] = {F, F, F, F, F, F, F, F, F, F};
    a[i] = nullptr;
    return vmoba_sparse_attn_bwd_dkdv(&p, a[0], a[1], a[2], (float*)a[3], (float*)a[4], a[5],
                                      (int32_t*)a[6], (int32_t*)a[7], a[8], a[9], nullptr);
  });
  each_null(9, [&](int i) {
    void* a[9] = {F, F, F, F, F, F, F, F, F};
    a[i] = nullptr;
    return vmoba_sparse_attn_bwd_dq(&p, a[0], a[1], a[2], (float*)a[3], (float*)a[4], a[5],
                                    (int32_t*)a[6], (int32_t*)a[7], a[8], nullptr);
  });

  before = g_launches;
  EXPECT(vmoba_dense_attn_fwd(&p, F, F, F, F, FF, nullptr, 0, nullptr) == VMOBA_OK);
  EXPECT(vmoba_dense_attn_bwd(&p, F, F, F, F, FF, F, F, F, F, F, ws_bwd, nullptr) == VMOBA_OK);
  EXPECT(g_launches == before + 4);
  EXPECT(vmoba_dense_attn_bwd(&p, F, F, F, F, FF, F, F, F, F, F, ws_bwd - 1, nullptr) ==
         VMOBA_ERR_WORKSPACE);

  // token-granular calls: bf16 only
  const bool bf = p.dtype == VMOBA_BF16;
  before = g_launches;
  const int st = vmoba_select_tokens(&p, F, FF, 0.25f, FU, FI, FI, FI, FI, FF, F, ws_tok,
                                     nullptr);
  EXPECT(st == (bf ? VMOBA_OK : VMOBA_ERR_DTYPE));
  const int sf = vmoba_token_attn_fwd(&p, F, F, F, FI, FI, FU, F, FF, F, ws_tf, nullptr);
  const int sb = vmoba_token_attn_bwd(&p, F, F, F, F, FF, F, FI, FI, FI, FI, FU, F, F, F, F,
                                      ws_tb, nullptr);
  const int S = p.bt * p.bh * p.bw;
  const int want_attn = !bf ? VMOBA_ERR_DTYPE : (S < 4 ? VMOBA_ERR_SHAPE : VMOBA_OK);
  EXPECT(sf == want_attn && sb == want_attn);
  EXPECT(g_launches == before + (bf ? 1 : 0) + (want_attn == VMOBA_OK ? 2 + 4 : 0));
  if (bf && S >= 4) {
    before = g_launches;
    EXPECT(vmoba_token_attn_fwd(&p, F, F, F, FI, FI, FU, F, FF, F, ws_tf - 1, nullptr) ==
           VMOBA_ERR_WORKSPACE);
    EXPECT(vmoba_token_attn_bwd(&p, F, F, F, F, FF, F, FI, FI, FI, FI, nullptr, F, F, F, F,
                                ws_tb, nullptr) == VMOBA_ERR_NULL);
    EXPECT(g_launches == before);
  }
}

static void check_geometry(int T, int H, int W, int bt, int bh, int bw) {
  vmoba_problem p = prob(1, 1, 64, T, H, W, 2, bt, bh, bw);
  EXPECT(vmoba_validate(&p) == VMOBA_OK);
  vmoba::Geom g{};
  g.T = T; g.H = H; g.W = W; g.L = T * H * W; g.bt = bt; g.bh = bh; g.bw = bw;
  g.nt = T / bt; g.nh = H / bh; g.nw = W / bw; g.Nb = g.nt * g.nh * g.nw; g.S = bt * bh * bw;
  g.div_S = vmoba::make_fastdiv(g.S); g.div_nhnw = vmoba::make_fastdiv(g.nh * g.nw);
  g.div_nw = vmoba::make_fastdiv(g.nw); g.div_bhbw = vmoba::make_fastdiv(bh * bw);
  g.div_bw = vmoba::make_fastdiv(bw);
  std::vector<int> seen(size_t(g.L), 0);
  for (int j = 0; j < g.Nb; ++j)
    for (int r = 0; r < g.S; ++r) {
      const int x = vmoba::block_base(g, j) + vmoba::block_offset(g, r);
      EXPECT(x >= 0 && x < g.L);
      if (x < 0 || x >= g.L) return;
      seen[size_t(x)]++;
      EXPECT(vmoba::token_block(g, x) == j);
    }
  for (int x = 0; x < g.L; ++x) EXPECT(seen[size_t(x)] == 1);
}

int main() {
  // problems: fp32 tiny, bf16 at d = 64 and 128, the three partition modes, large sizes
  const vmoba_problem probs[] = {
      prob(1, 2, 64, 4, 8, 8, 2, 2, 4, 4, VMOBA_FP32, VMOBA_FP32),
      prob(2, 3, 64, 4, 8, 8, 0, 1, 8, 8),
      prob(1, 12, 128, 21, 30, 52, 1, 21, 6, 4, VMOBA_BF16, VMOBA_FP32),
      prob(1, 12, 128, 24, 36, 64, 2, 4, 6, 8),
      prob(1, 12, 128, 21, 45, 80, 2, 3, 9, 8),
      prob(1, 1, 128, 2, 2, 2, 2, 1, 1, 1),           // blocks of one token
  };
  for (const auto& p : probs) {
    EXPECT(vmoba_validate(&p) == VMOBA_OK);
    check_entry_points(p);
  }
  // argument errors of the problem itself win over every other check
  vmoba_problem bad = probs[3];
  bad.T = 25;
  EXPECT(vmoba_validate(&bad) == VMOBA_ERR_SHAPE);
  EXPECT(vmoba_sparse_attn_fwd(&bad, F, F, F, FI, FI, F, FF, nullptr, 0, nullptr) ==
         VMOBA_ERR_SHAPE);
  bad = probs[3]; bad.head_dim = 96;
  EXPECT(vmoba_validate(&bad) == VMOBA_ERR_HEAD_DIM);
  bad = probs[3]; bad.dtype = 7;
  EXPECT(vmoba_validate(&bad) == VMOBA_ERR_DTYPE);
  bad = probs[3]; bad.layer_idx = 0;
  EXPECT(vmoba_validate(&bad) == VMOBA_ERR_MODE);
  EXPECT(vmoba_validate(nullptr) == VMOBA_ERR_NULL);
  // int32 ranges: 2^31 elements and more are rejected, without overflow in the check
  vmoba_problem big = prob(4096, 64, 128, 64, 64, 64, 2, 1, 1, 1);
  EXPECT(vmoba_validate(&big) == VMOBA_ERR_OVERFLOW);
  big = prob(0x7fffffff, 0x7fffffff, 128, 0x7fffffff, 0x7fffffff, 0x7fffffff, 2, 1, 1, 1);
  EXPECT(vmoba_validate(&big) == VMOBA_ERR_OVERFLOW);
  // more than the attention calls' block limit
  vmoba_problem many = prob(1, 1, 64, 1, 1, 1025, 2, 1, 1, 1);
  EXPECT(vmoba_validate(&many) == VMOBA_OK);
  size_t n = 0;
  EXPECT(vmoba_workspace_size(&many, VMOBA_OP_SELECT, &n) == VMOBA_OK);
  EXPECT(vmoba_select(&many, FF, FF, 0.25f, FI, FI, FI, FI, FF, nullptr, F, n, nullptr) ==
         VMOBA_ERR_SHAPE);
  // every status string, including unknown values
  for (int s = -3; s < 20; ++s) {
    const char* m = vmoba_status_string(s);
    EXPECT(m != nullptr && strlen(m) > 0);
  }
  EXPECT(strncmp(vmoba_version(), "vmoba", 5) == 0);
  // geometry
  check_geometry(4, 8, 8, 2, 4, 4);
  check_geometry(24, 36, 64, 4, 6, 8);
  check_geometry(21, 45, 80, 3, 9, 8);
  check_geometry(21, 30, 52, 21, 6, 4);
  check_geometry(6, 18, 16, 3, 9, 8);
  for (uint32_t d : {1u, 2u, 3u, 7u, 192u, 216u, 1512u, 82944u, 122500u, 0x7fffffffu}) {
    const vmoba::FastDiv f = vmoba::make_fastdiv(d);
    for (uint32_t x : {0u, 1u, d - 1, d, d + 1, 3 * d + 5, 0x7ffffffeu, 0x7fffffffu})
      if (x <= 0x7fffffffu) EXPECT(vmoba::fd_div(x, f) == x / d);
  }
  if (g_fail) return 1;
  printf("ok %d launches\n", g_launches);
  return 0;
}
