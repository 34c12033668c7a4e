// Block-sparse (and dense) flash attention forward for gfx950.
//
// papernotes 方法详解/整体框架 and paperlayer §3.1: each query block attends only to the
// tokens of its selected key blocks; the output keeps full attention's shape.
//
// bf16 kernel, per workgroup: NW waves x 32 queries of one query block, all sharing the
// block's key stream.  Per key tile (KT = 32*KSUB keys) the workgroup stages K row-major
// and V transposed in LDS (double-buffered, padded rows, global loads of tile t+1 in
// flight while tile t is computed).  Each wave computes S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 with its Q fragments held in registers, so every lane owns
// one query column: the online-softmax max needs one exchange between the two lane
// halves, the row sum none until the end, and rescaling O is a per-lane multiply.
// P^T stays in registers as the B operand of O^T += V^T P^T; the k-order of that product
// is permuted to match the S^T accumulator layout, and the V^T reads follow the same
// permutation.  exp2 with the log2(e)/sqrt(d) scale folded into one FMA; fp32
// accumulation throughout; O rescaled by 1/l and written back in natural token order
// with LSE = m/sqrt(d) + ln l.
#include <math.h>

#include <type_traits>

#include "attn_common.h"

namespace vmoba {

template <int D, int NW, int KSUB, bool DENSE, bool TAB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(AttnParams a) {
  constexpr int NT = NW * 64;
  constexpr int QT = NW * 32;
  constexpr int KT = KSUB * 32;
  constexpr int ROWB = D * 2;                // bytes per tile row
  constexpr int RPI = 1024 / ROWB;           // tile rows per wave load instruction
  constexpr int LPW = KT / (NW * RPI);       // load instructions per wave per tensor
  static_assert(KT % (NW * RPI) == 0, "tile rows split over waves");
  constexpr int TILE = KT * ROWB;            // bytes of one K or V tile
  // lazy rescale: keep the running max until a score exceeds it by 2^8 in exp2 units
  constexpr float kRescaleLog2 = 8.0f;

  // two pipeline stages as separate objects, so the compiler can tell that reads of one
  // stage do not depend on the direct-to-LDS loads in flight into the other
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILE];
  __shared__ int32_t cols[DENSE ? 1 : kMaxBlocks];        // base token of listed blocks
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];      // block_offset(r), r < S
  __shared__ int32_t scratch[NW];

  const Geom& g = a.g;
  const int rows = DENSE ? 1 : g.Nb;
  int bid = xcd_item(blockIdx.x, g.B * g.Hh, rows * a.tiles);
  if (bid < 0) return;
  const int qt = bid % a.tiles;
  bid /= a.tiles;
  const int iblk = bid % rows;
  const int grp = bid / rows;

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.out);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  // key stream: compacted block list -> base tokens; offsets of tokens inside a block
  int nkeys;
  if constexpr (DENSE) {
    nkeys = g.L;
  } else {
    int start, len;
    list_range(g, a.row_ptr, grp, iblk, &start, &len);
    const int kept = compact_list<NT>(a.col_idx + size_t(grp) * g.Nb * g.Nb + start, len,
                                      g.Nb, cols, scratch);
    for (int i = tid; i < kept; i += NT) cols[i] = block_base(g, uint32_t(cols[i]));
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r));
    __syncthreads();
    nkeys = kept * g.S;
  }
  const int ntiles = (nkeys + KT - 1) / KT;

  // this lane's query, Q fragments in registers (B operand of S^T = K Q^T)
  const int qlim = DENSE ? g.L : g.S;
  const int rq = qt * QT + w * 32 + l32;
  const bool qvalid = rq < qlim;
  const int rqc = qvalid ? rq : 0;
  const int32_t xq = DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  const int32_t qoff = row_offset(g, grp, xq);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + qoff + s * 16 + half * 8));

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // LDS read offsets of this lane (stage, sub-tile and k-step add immediates)
  const int grp16 = lane >> 4, sl = lane & 15;
  const int krow = l32 * ROWB, kswz = swz<D>(l32) ^ half;
  const int vkey0 = 4 * half + (sl >> 2);
  const int vc0 = 2 * (grp16 & 1) + ((sl & 3) >> 1);
  const int vbase_lo = TILE + vkey0 * ROWB + (sl & 1) * 8;
  const int vsw_lo = swz<D>(vkey0), vsw_hi = swz<D>(vkey0 + 8);

  // loader: this lane fetches chunk (lane % CPR) ^ swz(row) of rows r_i = lrow0 + i*RPI;
  // the stream position of row i in tile t is t*KT + r_i, tracked as (block, offset)
  constexpr int CPR = D / 8;
  const int lrow0 = w * (KT / NW) + lane / CPR;
  const int lcp = lane % CPR;
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  // Row addresses are computed first, without divergent branches, and the loads are
  // issued back to back afterwards: a branch join between one row's load and the next
  // row's address arithmetic would make the compiler wait for the load in flight.
  auto issue_tile = [&](int t, unsigned char* smem) {
    int32_t off[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = min(t * KT + lrow0 + i * RPI, nkeys - 1);   // ragged end repeats
      int32_t x = p;
      if constexpr (!DENSE) {
        const uint32_t pb = fd_div(uint32_t(p), g.div_S);
        const uint32_t rr = uint32_t(p) - pb * uint32_t(g.S);
        x = cols[pb] + (TAB ? offtab[rr] : block_offset(g, rr));
      }
      off[i] = x;
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = lrow0 + i * RPI;
      const int32_t o = gbase + off[i] * hstride + (lcp ^ swz<D>(r)) * 8;
      const int dst = (w * (KT / NW) + i * RPI) * ROWB;   // wave-uniform
      load_to_lds16(K + o, smem + dst);
      load_to_lds16(V + o, smem + TILE + dst);
    }
  };

  const float c2 = a.scale_log2;
  const float thr = kRescaleLog2 / c2;

  // S^T of the tile in stage ST: keys along MFMA rows, this lane's query in the column
  auto scores = [&](auto STc, f32x16* sacc) {
    const unsigned char* smem = decltype(STc)::value ? stage1 : stage0;
    constexpr int SB = 0;
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kt][v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        // chunk 2s + half of row l32 sits at position (2s) ^ swz(l32) ^ half
        const int ko = krow + 16 * ((2 * s) ^ kswz);
        const bf16x8 ka = as_bf16x8(
            *reinterpret_cast<const u32x4*>(smem + SB + kt * 32 * ROWB + ko));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[kt], 0, 0, 0);
      }
    }
  };
  auto mask_tail = [&](int t, f32x16* sacc) {
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = t * KT + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (key >= nkeys) sacc[kt][v] = -INFINITY;
      }
  };
  auto tile_max = [&](const f32x16* sacc) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  auto exps = [&](f32x16* sacc) {
    const float moff = m_run * c2;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kt][v], c2, -moff));
        sacc[kt][v] = pv;
        psum += pv;
      }
    return psum;
  };
  auto rescale_to = [&](float m_new) {
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    m_run = m_new;
  };
  // O^T += V^T P^T, 16 keys per step; V^T fragments by transposing reads
  auto pv_update = [&](auto STc, const f32x16* sacc) {
    const unsigned char* smem = decltype(STc)::value ? stage1 : stage0;
    constexpr int SB = 0;
#pragma unroll
    for (int ks = 0; ks < 2 * KSUB; ++ks) {
      const int kt = ks >> 1, g0 = (ks & 1) * 8;
      u32x4 pw;
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(sacc[kt][g0 + 2 * e], sacc[kt][g0 + 2 * e + 1]);
      const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int c = dt * 4 + vc0;
        const u32x2 lo = lds_read_tr16(smem + SB + ks * 16 * ROWB + vbase_lo + 16 * (c ^ vsw_lo));
        const u32x2 hi = lds_read_tr16(smem + SB + ks * 16 * ROWB + vbase_lo + 8 * ROWB +
                                       16 * (c ^ vsw_hi));
        const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
      }
    }
  };

  // one tile: FIRST sets the running max from the tile; later tiles keep it unless their
  // max exceeds it by more than the lazy-rescale margin
  auto step = [&](auto STc, auto FIRSTc, auto LASTc, int t) {
    constexpr int ST = decltype(STc)::value;
    constexpr bool FIRST = decltype(FIRSTc)::value, LAST = decltype(LASTc)::value;
    if (t + 1 < ntiles) issue_tile(t + 1, ST ? stage0 : stage1);
    f32x16 sacc[KSUB];
    scores(STc, sacc);
    if (LAST && t * KT + KT > nkeys) mask_tail(t, sacc);
    if constexpr (FIRST) {
      m_run = tile_max(sacc);
    } else {
      const float mx = tile_max(sacc);
      const bool grow = mx > m_run + thr;
      if (__ballot(grow)) rescale_to(grow ? mx : m_run);   // wave-uniform; rare
    }
    l_run += exps(sacc);
    pv_update(STc, sacc);
    wait_lds_loads();
    __syncthreads();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (ntiles > 0) issue_tile(0, stage0);
  wait_lds_loads();
  __syncthreads();
  if (ntiles == 1) {
    step(S0{}, T_{}, T_{}, 0);
  } else if (ntiles > 1) {
    step(S0{}, T_{}, F_{}, 0);
    int t = 1;
    for (; t + 1 < ntiles - 1; t += 2) {
      step(S1{}, F_{}, F_{}, t);
      step(S0{}, F_{}, F_{}, t + 1);
    }
    if (t < ntiles - 1) {
      step(S1{}, F_{}, F_{}, t);
      ++t;
    }
    if (t & 1) step(S1{}, F_{}, T_{}, t);
    else step(S0{}, F_{}, T_{}, t);
  }

  // finalise
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = nkeys == 0;
  const float inv = empty ? 0.f : 1.0f / l_tot;
  if (qvalid) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = dt * 32 + gq * 8 + half * 4;
        u32x2 out;
        out[0] = pack_bf16x2(oacc[dt][4 * gq + 0] * inv, oacc[dt][4 * gq + 1] * inv);
        out[1] = pack_bf16x2(oacc[dt][4 * gq + 2] * inv, oacc[dt][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(O + qoff + d0) = out;
      }
    if (half == 0)
      a.lse[size_t(grp) * g.L + xq] = empty ? -INFINITY : m_run * a.scale + logf(l_tot);
  }
}

// fp32 instance (VALU, one query per lane): the plain online-softmax recurrence over the
// same key stream, for fp32 inputs.
template <int D, bool DENSE>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnParams a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  __shared__ int32_t cols[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t scratch[1];
  const Geom& g = a.g;
  const int rows = DENSE ? 1 : g.Nb;
  int bid = blockIdx.x;
  const int qt = bid % a.tiles;
  bid /= a.tiles;
  const int iblk = bid % rows;
  const int grp = bid / rows;
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  float* O = static_cast<float*>(a.out);

  int nkeys;
  if constexpr (DENSE) {
    nkeys = g.L;
  } else {
    int start, len;
    list_range(g, a.row_ptr, grp, iblk, &start, &len);
    nkeys = compact_list<64>(a.col_idx + size_t(grp) * g.Nb * g.Nb + start, len, g.Nb, cols,
                             scratch) * g.S;
  }
  const int qlim = DENSE ? g.L : g.S;
  const int rq = qt * 64 + threadIdx.x;
  const bool qvalid = rq < qlim;
  const int rqc = qvalid ? rq : 0;
  const int32_t xq = DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  const int32_t qoff = row_offset(g, grp, xq);
  float qv[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = Q[qoff + d] * a.scale;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t0 = 0; t0 < nkeys; t0 += KT) {
    for (int idx = threadIdx.x; idx < KT * D; idx += 64) {
      const int kk = idx / D, d = idx % D;
      const int p = t0 + kk;
      float kv = 0.f, vv = 0.f;
      if (p < nkeys) {
        const int32_t x = DENSE ? p : stream_token(g, cols, uint32_t(p));
        const int32_t off = row_offset(g, grp, x) + d;
        kv = K[off];
        vv = V[off];
      }
      ks[kk][d] = kv;
      vs[kk][d] = vv;
    }
    __syncthreads();
    const int n = min(KT, nkeys - t0);
    for (int kk = 0; kk < n; ++kk) {
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], ks[kk][d], s);
      const float mn = fmaxf(m, s);
      const float al = expf(m - mn);
      const float p = expf(s - mn);
      l = l * al + p;
      for (int d = 0; d < D; ++d) acc[d] = acc[d] * al + p * vs[kk][d];
      m = mn;
    }
    __syncthreads();
  }
  if (qvalid) {
    const float inv = nkeys ? 1.0f / l : 0.f;
    for (int d = 0; d < D; ++d) O[qoff + d] = acc[d] * inv;
    a.lse[size_t(grp) * g.L + xq] = nkeys ? m + logf(l) : -INFINITY;
  }
}

template <int D, int NW, int KSUB, bool DENSE>
static void launch_fwd_bf16(AttnParams& a, hipStream_t s) {
  const Geom& g = a.g;
  const int qlim = DENSE ? g.L : g.S;
  a.tiles = (qlim + NW * 32 - 1) / (NW * 32);
  const int rows = DENSE ? 1 : g.Nb;
  const int grid = xcd_grid(g.B * g.Hh, rows * a.tiles);
  if (!DENSE && g.S <= kOffsetTable)
    attn_fwd_bf16_kernel<D, NW, KSUB, DENSE, !DENSE><<<grid, NW * 64, 0, s>>>(a);
  else
    attn_fwd_bf16_kernel<D, NW, KSUB, DENSE, false><<<grid, NW * 64, 0, s>>>(a);
}

template <int D, bool DENSE>
static void launch_fwd_f32(AttnParams& a, hipStream_t s) {
  const Geom& g = a.g;
  const int qlim = DENSE ? g.L : g.S;
  a.tiles = (qlim + 63) / 64;
  const int rows = DENSE ? 1 : g.Nb;
  attn_fwd_f32_kernel<D, DENSE><<<g.B * g.Hh * rows * a.tiles, 64, 0, s>>>(a);
}

int launch_attn_fwd(const Geom& g, bool dense, const void* q, const void* k,
                    const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                    void* o, float* lse, void* ws, void* stream) {
  (void)ws;
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams a{};
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = o;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.scale = 1.0f / sqrtf(float(g.D));
  a.scale_log2 = kLog2e * a.scale;
  if (g.dtype == VMOBA_BF16) {
    if (g.D == 128) {
      if (dense) launch_fwd_bf16<128, 4, 2, true>(a, s);
      else launch_fwd_bf16<128, 4, 2, false>(a, s);
    } else {
      if (dense) launch_fwd_bf16<64, 4, 2, true>(a, s);
      else launch_fwd_bf16<64, 4, 2, false>(a, s);
    }
  } else {
    if (g.D == 128) {
      if (dense) launch_fwd_f32<128, true>(a, s);
      else launch_fwd_f32<128, false>(a, s);
    } else {
      if (dense) launch_fwd_f32<64, true>(a, s);
      else launch_fwd_f32<64, false>(a, s);
    }
  }
  return launch_status();
}

}  // namespace vmoba
