// Problem geometry shared by the host validation code and the kernels.
//
// Partition of the (T, H, W) latent into bt x bh x bw blocks (papernotes 关键设计 1):
// block j sits at grid cell (jt, jh, jw) of the (T/bt, H/bh, W/bw) grid, row-major;
// token r inside a block sits at offset (dt, dh, dw), row-major.  The token index is
//   x = base(j) + off(r),  base(j) = (jt*bt*H + jh*bh)*W + jw*bw,
//                          off(r)  = (dt*H + dh)*W + dw,
// which is ((jt*bt + dt)*H + jh*bh + dh)*W + jw*bw + dw written as two terms.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define VMOBA_HD __host__ __device__ __forceinline__
#else
#define VMOBA_HD inline
#endif

namespace vmoba {

// Division of 0 <= n < 2^31 by a fixed 1 <= d < 2^31 with one high multiply, an add and
// a shift: s = ceil(log2 d), m = floor(2^32 * (2^s - d) / d) + 1, n / d = (hi(n*m) + n) >> s
// (Granlund & Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  f.s = s;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

VMOBA_HD uint32_t fd_div(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t hi = __umulhi(n, f.m);
#else
  uint32_t hi = uint32_t((uint64_t(n) * f.m) >> 32);
#endif
  return (hi + n) >> f.s;
}

struct Geom {
  int32_t B, Hh, D, T, H, W, L;
  int32_t bt, bh, bw;       // block shape
  int32_t nt, nh, nw;       // block grid
  int32_t Nb, S;            // blocks, tokens per block
  int32_t mode, dtype, grad_dtype;
  FastDiv div_S, div_nhnw, div_nw, div_bhbw, div_bw;
};

// Token index of position r inside block j.
VMOBA_HD int32_t block_base(const Geom& g, uint32_t j) {
  uint32_t jt = fd_div(j, g.div_nhnw);
  uint32_t rem = j - jt * uint32_t(g.nh * g.nw);
  uint32_t jh = fd_div(rem, g.div_nw);
  uint32_t jw = rem - jh * uint32_t(g.nw);
  return int32_t((jt * g.bt * g.H + jh * g.bh) * g.W + jw * g.bw);
}

// Block of token x (inverse of base + offset).
VMOBA_HD int32_t token_block(const Geom& g, int32_t x) {
  const int32_t hw = g.H * g.W;
  const int32_t t = x / hw, rem = x - t * hw;
  const int32_t h = rem / g.W, w = rem - h * g.W;
  return ((t / g.bt) * g.nh + h / g.bh) * g.nw + w / g.bw;
}

VMOBA_HD int32_t block_offset(const Geom& g, uint32_t r) {
  uint32_t dt = fd_div(r, g.div_bhbw);
  uint32_t rem = r - dt * uint32_t(g.bh * g.bw);
  uint32_t dh = fd_div(rem, g.div_bw);
  uint32_t dw = rem - dh * uint32_t(g.bw);
  return int32_t((dt * g.H + dh) * g.W + dw);
}

}  // namespace vmoba
