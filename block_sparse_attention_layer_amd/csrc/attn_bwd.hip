// Block-sparse (and dense) flash attention backward for gfx950, with the block selection
// held constant (it is not differentiated):
//   P = exp(q.k/sqrt(d) - lse),  dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO * O),
//   dS = P * (dP - delta),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
//
// Three kernels, no atomics, deterministic:
//  * delta_kernel: delta per query row (16 lanes per row, shuffle reduction).
//  * dkdv kernel (key-major, over the column lists): each wave owns 32 keys of one key
//    block with K and V as register-resident MFMA B operands; the workgroup streams the
//    query tokens of every query block that selected this key block (tiles of 32 cross
//    block boundaries), staging Q and dO in LDS both row-major (A operands of S = Q K^T
//    and dP = dO V^T) and transposed (A operands of dV^T += dO^T P and dK^T += Q^T dS).
//    S, P, dP and dS live with one key per lane, so P and dS feed the next MFMA straight
//    from registers; LSE and delta per query come from LDS.
//  * dq kernel (query-major, over the row lists): the forward's layout (one query per
//    lane, Q and dO fragments in registers); K and V are staged row-major for
//    S^T = K Q^T and dP^T = V dO^T, and K once more transposed for dQ^T += K^T dS^T.
#include <math.h>

#include <type_traits>

#include "attn_common.h"

namespace vmoba {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// The split kernels pass P between their two roles as fp16: P lies in [0, 1], where fp16
// keeps 11 significant bits (2^-12 relative rounding) down to 2^-14 and an absolute 2^-25
// below, against the 2^-9 of the bf16 rounding dS takes next; it halves the exchange's LDS
// traffic against fp32.
// two fp32 values rounded to nearest-even fp16, packed (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
// half e of a packed fp16 pair times x, in fp32 (one v_fma_mix_f32: the +0 addend keeps it
// a fused operation, exact up to the one fp32 rounding)
__device__ __forceinline__ float mul_f16(uint32_t packed, int e, float x) {
  const f16x2 h = __builtin_bit_cast(f16x2, packed);
  return __builtin_fmaf(float(h[e]), x, 0.0f);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(Geom g, const T* __restrict__ o,
                                                    const T* __restrict__ dout,
                                                    float* __restrict__ delta) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LPR = D / VEC;  // lanes per row
  const int row = (blockIdx.x * 256 + threadIdx.x) / LPR;  // (b*L + x)*Hh + h
  const int c = threadIdx.x % LPR;
  const int nrows = g.B * g.L * g.Hh;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 ov = *reinterpret_cast<const u32x4*>(o + size_t(row) * D + c * VEC);
    const u32x4 dv = *reinterpret_cast<const u32x4*>(dout + size_t(row) * D + c * VEC);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += bf16_to_f32(ov[e] & 0xffffu) * bf16_to_f32(dv[e] & 0xffffu);
        acc += bf16_to_f32(ov[e] >> 16) * bf16_to_f32(dv[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += __uint_as_float(ov[e]) * __uint_as_float(dv[e]);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && c == 0) {
    const int h = row % g.Hh;
    const int bx = row / g.Hh;  // b*L + x
    const int b = bx / g.L, x = bx - b * g.L;
    delta[(size_t(b) * g.Hh + h) * g.L + x] = acc;
  }
}

// Store four consecutive gradient values as bf16 (round to nearest even) or fp32.
template <typename GT>
__device__ __forceinline__ void store4(GT* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(GT) == 2) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  }
}

// ---------------------------------------------------------------------------------
// dK, dV: one wave per 32 keys, query stream from the column list of the key block.
// TOK: token-granular selection, a query token's pairs with this key block kept only where
// its key-block mask has the block's bit.
template <int D, int NW, bool DENSE, bool TAB, typename GT, bool TOK = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_bf16_kernel(AttnParams a) {
  constexpr int NT = NW * 64;
  constexpr int QT = 32;                     // queries per tile
  constexpr int ROWB = D * 2;
  constexpr int RPI = 1024 / ROWB;
  constexpr int LPW = QT / (NW * RPI);
  static_assert(QT % (NW * RPI) == 0, "tile rows split over waves");
  constexpr int TILE = QT * ROWB;
  static_assert(NW >= 3 && QT <= 64, "LSE, delta and mask words are loaded by waves 0-2");
  // per stage: Q tile, dO tile, then 64 floats of LSE and 64 of delta (one wave's load
  // each; lanes 32-63 repeat the first 32), and with TOK 64 mask words
  constexpr int STAGE = 2 * TILE + (TOK ? 3 : 2) * 64 * 4;

  // two pipeline stages as separate objects (see the forward kernel)
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[STAGE];
  // V rows of this workgroup's keys (B operands of dP = dO V^T), loaded once
  __shared__ __attribute__((aligned(1024))) unsigned char vtile[NW * 32 * ROWB];
  __shared__ int32_t rows_l[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];   // block_offset(r), r < S
  __shared__ int32_t scratch[NW];

  const Geom& g = a.g;
  int grp, jblk, kt;
  if constexpr (DENSE) {
    const int bid = xcd_item(blockIdx.x, g.B * g.Hh, a.tiles);
    if (bid < 0) return;
    kt = bid % a.tiles;
    jblk = 0;
    grp = bid / a.tiles;
  } else {
    SparseItem it;
    if (!sparse_item<NT>(g, a.col_ptr, a.tiles, a.ordered != 0, rows_l, scratch, &it)) return;
    grp = it.grp;
    jblk = it.blk;
    kt = it.tile;
  }

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ dO = static_cast<const uint16_t*>(a.dout);
  GT* __restrict__ dK = static_cast<GT*>(a.dk);
  GT* __restrict__ dV = static_cast<GT*>(a.dv);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * D) * 2u;   // < 2^32 (validated)
  const BufRes rQ = buffer_res(Q, tbytes), rO = buffer_res(dO, tbytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // the wave index, known uniform
  const int l32 = lane & 31, half = lane >> 5;

  int nq;
  if constexpr (DENSE) {
    nq = g.L;
  } else {
    int start, len;
    list_range(g, a.col_ptr, grp, jblk, &start, &len);
    const int kept = compact_list<NT>(a.row_idx + size_t(grp) * g.Nb * g.Nb + start, len,
                                      g.Nb, rows_l, scratch);
    for (int i = tid; i < kept; i += NT) rows_l[i] = block_base(g, uint32_t(rows_l[i]));
    if (kept == 0 && tid == 0) rows_l[0] = 0;   // token 0: address of an empty stream
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r));
    __syncthreads();
    nq = kept * g.S;
  }
  const int ntiles = (nq + QT - 1) / QT;

  // this lane's key: K and V fragments as B operands (lane = key, 8 d per k-step)
  const int klim = DENSE ? g.L : g.S;
  const int rk = kt * NW * 32 + w * 32 + l32;
  const bool kvalid = rk < klim;
  // A wave whose 32 keys all lie past the block's end (the ragged last key tile) only
  // takes its share of the loads and the barriers; its SIMD's matrix core goes to the
  // other workgroup's wave.
  const bool wave_busy = kt * NW * 32 + w * 32 < klim;
  const int rkc = kvalid ? rk : 0;
  const int32_t xk = DENSE ? rkc : block_base(g, jblk) + block_offset(g, rkc);
  const int32_t koff = row_offset(g, grp, xk);
  bf16x8 kf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(K + koff + s * 16 + half * 8));
  {
    // this wave's 32 V rows into vtile (row = wave*32 + key lane), swizzled like a tile
    constexpr int CPR0 = D / 8;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = w * 32 + i * RPI + lane / CPR0;
      const int rr = kt * NW * 32 + r;
      const int rrc = rr < klim ? rr : 0;
      const int32_t x = DENSE ? rrc : block_base(g, jblk) + block_offset(g, rrc);
      const int32_t off = row_offset(g, grp, x) + ((lane % CPR0) ^ swz<D>(r)) * 8;
      load_to_lds16(buffer_res(V, tbytes), 2u * uint32_t(off), vtile + (w * 32 + i * RPI) * ROWB);
    }
  }
  const unsigned char* vrow = vtile;
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dkacc[dt][v] = 0.f;
      dvacc[dt][v] = 0.f;
    }

  const float* lse_g = a.lse + size_t(grp) * g.L;
  const float* dl_g = a.delta + size_t(grp) * g.L;
  const BufRes rL = buffer_res(lse_g, uint32_t(g.L) * 4u);
  const BufRes rD = buffer_res(dl_g, uint32_t(g.L) * 4u);
  // key-block mask words: G * L * mwords * 4 < 2^32 bytes (validated)
  const BufRes rM = buffer_res(a.tokmask, uint32_t(g.B * g.Hh * g.L * a.mwords) * 4u);
  const uint32_t mword = uint32_t(grp * g.L) * uint32_t(a.mwords) + uint32_t(jblk >> 5);
  constexpr int CPR = D / 8;
  const int lrow0 = w * (QT / NW) + lane / CPR;
  const int lcp = lane % CPR;
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nq - 1, 0);   // positions past the end repeat the last query
  auto qtoken = [&](int p) -> int32_t {
    if constexpr (DENSE) {
      return p;
    } else {
      const uint32_t bi = fd_div(uint32_t(p), g.div_S);
      const uint32_t r = uint32_t(p) - bi * uint32_t(g.S);
      return rows_l[bi] + (TAB ? offtab[r] : block_offset(g, r));
    }
  };
  // element offsets of this lane's Q/dO rows of tile t, and the token of its LSE/delta
  auto tile_offsets = [&](int t, int32_t (&o)[LPW], int32_t& xl) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = lrow0 + i * RPI;
      o[i] = gbase + qtoken(min(t * QT + r, plast)) * hstride + (lcp ^ swz<D>(r)) * 8;
    }
    xl = qtoken(min(t * QT + l32, plast));
  };
  auto issue_offsets = [&](const int32_t (&o)[LPW], int32_t xl, unsigned char* sb) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int dst = (w * (QT / NW) + i * RPI) * ROWB;
      load_to_lds16(rQ, 2u * uint32_t(o[i]), sb + dst);
      load_to_lds16(rO, 2u * uint32_t(o[i]), sb + TILE + dst);
    }
    // LSE and delta of the tile's queries; a scalar branch keeps the descriptors uniform
    if (wu == 0) load_to_lds4(rL, 4u * uint32_t(xl), sb + 2 * TILE);
    if (wu == 1) load_to_lds4(rD, 4u * uint32_t(xl), sb + 2 * TILE + 64 * 4);
    if constexpr (TOK)
      if (wu == 2)
        load_to_lds4(rM, 4u * (mword + uint32_t(xl) * uint32_t(a.mwords)),
                     sb + 2 * TILE + 2 * 64 * 4);
  };
  auto issue_tile = [&](int t, unsigned char* sb) {
    int32_t o[LPW], xl;
    tile_offsets(t, o, xl);
    issue_offsets(o, xl, sb);
  };

  const float c2 = a.scale_log2;
  const int grp16 = lane >> 4, sl = lane & 15;
  auto step = [&](auto STc, int t) {
    constexpr int ST = decltype(STc)::value;
    __builtin_amdgcn_sched_barrier(0);   // keep the steps from being interleaved
    unsigned char* const cur = ST ? stage1 : stage0;
    unsigned char* const nxt = ST ? stage0 : stage1;
    if (t + 1 < ntiles) issue_tile(t + 1, nxt);
    if (wave_busy) {
    const unsigned char* qb = cur;
    const unsigned char* ob = cur + TILE;
    const float* lse_s = reinterpret_cast<const float*>(cur + 2 * TILE);
    const float* dl_s = lse_s + 64;

    f32x16 sacc, dpacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sacc[v] = 0.f;
      dpacc[v] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int o = tile_off<D>(l32, 2 * s + half);
      const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(qb + o));
      const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(ob + o));
      const bf16x8 vb16 = as_bf16x8(*reinterpret_cast<const u32x4*>(
          vrow + tile_off<D>(w * 32 + l32, 2 * s + half)));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[s], sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vb16, dpacc, 0, 0, 0);
    }
    // sacc[v]: query 8*(v/4) + 4*half + v%4 of the tile; key = this lane
    __builtin_amdgcn_sched_barrier(0);   // bound the live range of the LSE/delta reads
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float4 l4 = *reinterpret_cast<const float4*>(lse_s + gq * 8 + half * 4);
      const float4 d4 = *reinterpret_cast<const float4*>(dl_s + gq * 8 + half * 4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * gq + r;
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[v], c2, -lv[r] * kLog2e));
        sacc[v] = pv;
        dpacc[v] = pv * (dpacc[v] - dv4[r]);
      }
    }
    if (t * QT + QT > nq) {   // ragged last tile (uniform branch): no P, dS past the end
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (t * QT + 8 * (v >> 2) + 4 * half + (v & 3) >= nq) {
          sacc[v] = 0.f;
          dpacc[v] = 0.f;
        }
    }
    if constexpr (TOK) {   // queries that did not select this key block: no P, no dS
      const uint32_t* mk_s = reinterpret_cast<const uint32_t*>(cur + 2 * TILE + 2 * 64 * 4);
      const uint32_t jb = uint32_t(jblk) & 31u;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const u32x4 m4 = *reinterpret_cast<const u32x4*>(mk_s + gq * 8 + half * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (!((m4[r] >> jb) & 1u)) {
            sacc[4 * gq + r] = 0.f;
            dpacc[4 * gq + r] = 0.f;
          }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int g0 = ks * 8;
      u32x4 pw, sw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = pack_bf16x2(sacc[g0 + 2 * e], sacc[g0 + 2 * e + 1]);
        sw[e] = pack_bf16x2(dpacc[g0 + 2 * e], dpacc[g0 + 2 * e + 1]);
      }
      const bf16x8 pb = as_bf16x8(pw), sbf = as_bf16x8(sw);
      const int q0 = ks * 16 + 4 * half + (sl >> 2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int c = dt * 4 + 2 * (grp16 & 1) + ((sl & 3) >> 1);
        const int bo = (sl & 1) * 8;
        const int o0 = tile_off<D>(q0, c) + bo, o1 = tile_off<D>(q0 + 8, c) + bo;
        const u32x2 olo = lds_read_tr16(ob + o0), ohi = lds_read_tr16(ob + o1);
        const u32x2 qlo = lds_read_tr16(qb + o0), qhi = lds_read_tr16(qb + o1);
        dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(u32x4{olo[0], olo[1], ohi[0], ohi[1]}), pb, dvacc[dt], 0, 0, 0);
        dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}), sbf, dkacc[dt], 0, 0, 0);
      }
    }
    }
    wait_lds_loads();
    __syncthreads();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (ntiles > 0) issue_tile(0, stage0);
  wait_lds_loads();
  __syncthreads();
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(S0{}, t);
    step(S1{}, t + 1);
  }
  if (t < ntiles) step(S0{}, t);

  if (kvalid) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = dt * 32 + gq * 8 + half * 4;
        const float sc = a.scale;
        store4(dK + koff + d0, dkacc[dt][4 * gq] * sc, dkacc[dt][4 * gq + 1] * sc,
               dkacc[dt][4 * gq + 2] * sc, dkacc[dt][4 * gq + 3] * sc);
        store4(dV + koff + d0, dvacc[dt][4 * gq], dvacc[dt][4 * gq + 1],
               dvacc[dt][4 * gq + 2], dvacc[dt][4 * gq + 3]);
      }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV for d = 128 on v_mfma_f32_16x16x32_bf16.  A workgroup covers four key groups of
// 16*KS keys; as launched (KS = 3), 192 keys (a whole 192-token block) in groups of 48, so
// every Q / dO fragment a wave reads from LDS feeds three products.
//
// Per 32-query tile and key group:
//   S = Q K^T and dP = dO V^T as 2 query sub-tiles x 3 key sub-tiles x 4 d-steps (A = Q or
//   dO rows from LDS, B = the group's K or V columns in registers); the accumulator gives
//   lane l the key l % 16 of each key sub-tile and queries 4*(l/16) + 0..3 of each query
//   sub-tile;
//   P = exp(S / sqrt(d) - lse), dS = P (dP - delta), packed with their k order permuted to
//   the accumulator layout (k position 8g + e is query 4g + e for e < 4 and 16 + 4g + e - 4
//   otherwise): they are the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A
//   operands (dO^T, Q^T) come from two transposing reads each that follow the same
//   permutation.
//
// The work of a key group is split over two waves on one SIMD (waves kg and kg + 4 of 8):
//   role P (waves 0-3): S, P, dV^T += dO^T P; writes P (rounded to fp16, accumulator
//     layout) to an LDS exchange buffer;
//   role dS (waves 4-7): dP of tile t, and one step later, once role P's P of tile t has
//     been published by the step barrier, dS and dK^T += Q^T dS.  Its dP accumulators
//     start at -delta of their queries, so the products give dP - delta and dS is one
//     multiply a value.
// Each wave holds one accumulator (96 registers a lane) and one of K or V, so two waves
// fit a SIMD (256 registers each): the SIMD's matrix core alternates between them while
// each one's vector work (the softmax, or the dS) runs beside the other's products.  One
// wave holding both accumulators (192 registers) leaves one wave per SIMD, which measured
// 9 % slower.  The arithmetic of every element is the same either way.
//
// LDS tiles: row r holds one query (256 bytes, 16 chunks of 16 bytes), chunk c at position
// c ^ 2 (r & 7).  Both access patterns run free of bank conflicts with it (the bank-conflict
// counter reads zero for each pattern in isolation on gfx950): row reads, 16 bytes a lane
// from one chunk column of 16 consecutive rows, and transposing reads, 8 bytes a lane from
// 4 rows x 32 bytes per 16 lanes.  The position sets that look distinct on paper are not
// enough: c ^ (2 (r & 7) | (r >> 3)) halves the rate of the row reads.
__device__ __forceinline__ int swz16(int r) { return 2 * (r & 7); }

// Stages: the Q/dO/LSE/delta of tile t are read by role P at step t and by role dS at
// steps t and t+1, so step t refills the stage of tile t-2 with tile t+2 (four stages;
// the loads of a tile have two steps to land).  The exchange buffer alternates with the
// tile's parity: role P writes tile t's half at step t, role dS reads it at step t+1,
// and role P overwrites it at step t+2, after the barrier that ends step t+1.
// TOK: token-granular selection; role P keeps P only where the query token's key-block
// mask has this block's bit (dS then vanishes with it).  Wave 2 loads the tile's mask
// words into its slot instead of an LSE copy.
template <bool DENSE, bool TAB, typename GT, bool TOK = false, bool ALN = false, int KS = 3>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_split_bf16_kernel(AttnParams a) {
  constexpr int D = 128, NW = 8, NT = 512, NKG = 4;
  // KS: key sub-tiles of 16 per wave
  constexpr int KW = 16 * KS;                // keys per key group
  constexpr int KWG = NKG * KW;              // keys per workgroup
  constexpr int QT = 32;                     // queries per tile
  constexpr int ROWB = D * 2;
  constexpr int TILE = QT * ROWB;            // bytes of one Q or dO tile
  constexpr int LPW = QT / (NW * 4);         // load instructions per wave per tensor
  static_assert(LPW == 1, "one row group per wave");
  constexpr int NS = 4;                      // pipeline stages
  constexpr int PER_TILE = 2 * LPW + 1;      // loads per wave per tile
  // per stage: Q tile, dO tile, then eight 64-float slots: LSE (even waves), delta (odd);
  // every wave loads one slot so that all waves count the same loads per tile
  constexpr int STAGE = 2 * TILE + NW * 64 * 4;
  constexpr int XF = 2 * KS * 4 * 64;        // values of P one key group passes a tile

  __shared__ __attribute__((aligned(1024))) unsigned char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[STAGE];
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2][NKG][XF / 2];   // P, fp16 pairs
  __shared__ int32_t rows_l[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];
  __shared__ int32_t scratch[NW];
  auto stage = [&](auto Ic) -> unsigned char* {
    constexpr int I = decltype(Ic)::value % NS;
    if constexpr (I == 0) return stage0;
    else if constexpr (I == 1) return stage1;
    else if constexpr (I == 2) return stage2;
    else return stage3;
  };

  const Geom& g = a.g;
  int grp, jblk, kt;
  if constexpr (DENSE) {
    const int bid = xcd_item(blockIdx.x, g.B * g.Hh, a.tiles);
    if (bid < 0) return;
    kt = bid % a.tiles;
    jblk = 0;
    grp = bid / a.tiles;
  } else {
    SparseItem it;
    if (!sparse_item<NT>(g, a.col_ptr, a.tiles, a.ordered != 0, rows_l, scratch, &it)) return;
    grp = it.grp;
    jblk = it.blk;
    kt = it.tile;
  }

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ dO = static_cast<const uint16_t*>(a.dout);
  GT* __restrict__ dK = static_cast<GT*>(a.dk);
  GT* __restrict__ dV = static_cast<GT*>(a.dv);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * D) * 2u;   // < 2^32 (validated)
  const BufRes rQ = buffer_res(Q, tbytes), rO = buffer_res(dO, tbytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int kg = wu & (NKG - 1);
  const bool role_p = wu < NKG;              // wave-uniform
  const int g16 = lane >> 4, i16 = lane & 15;

  int nq;
  if constexpr (DENSE) {
    nq = g.L;
  } else {
    int start, len;
    list_range(g, a.col_ptr, grp, jblk, &start, &len);
    const int kept = compact_list<NT>(a.row_idx + size_t(grp) * g.Nb * g.Nb + start, len,
                                      g.Nb, rows_l, scratch);
    for (int i = tid; i < kept; i += NT) rows_l[i] = block_base(g, uint32_t(rows_l[i]));
    if (kept == 0 && tid == 0) rows_l[0] = 0;   // token 0: address of an empty stream
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r));
    __syncthreads();
    nq = kept * g.S;
  }
  const int ntiles = __builtin_amdgcn_readfirstlane((nq + QT - 1) / QT);

  // this wave's keys: K (role P) or V (role dS) columns, the B operands, in registers
  const int klim = DENSE ? g.L : g.S;
  const int kbase = kt * KWG + kg * KW;
  const bool wave_busy = kbase < klim;   // otherwise: loads and barriers only
  auto key_token = [&](int ks) -> int32_t {
    const int rk = kbase + ks * 16 + i16;
    const int rkc = rk < klim ? rk : 0;
    return DENSE ? rkc : block_base(g, jblk) + block_offset(g, rkc);
  };
  const uint16_t* __restrict__ KV = role_p ? K : V;
  bf16x8 kvf[KS][D / 32];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int32_t koff = row_offset(g, grp, key_token(ks));
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      kvf[ks][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(KV + koff + s * 32 + g16 * 8));
  }
  // dV^T (role P) or dK^T (role dS) of this wave's keys
  f32x4 acc[D / 16][KS];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc[ds][ks] = f32x4{0.f, 0.f, 0.f, 0.f};

  // query stream loader: one instruction moves 4 rows; lane L fills row L/16 at chunk
  // position L % 16 (logical chunk (L % 16) ^ swz16(row))
  const float* lse_g = a.lse + size_t(grp) * g.L;
  const float* dl_g = a.delta + size_t(grp) * g.L;
  const BufRes rL = buffer_res(lse_g, uint32_t(g.L) * 4u);
  const BufRes rD = buffer_res(dl_g, uint32_t(g.L) * 4u);
  // key-block mask words: G * L * mwords * 4 < 2^32 bytes (validated)
  const BufRes rM = buffer_res(a.tokmask, TOK ? uint32_t(g.B * g.Hh * g.L * a.mwords) * 4u : 0u);
  const uint32_t mword = TOK ? uint32_t(grp * g.L) * uint32_t(a.mwords) + uint32_t(jblk >> 5) : 0u;
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nq - 1, 0);   // positions past the end repeat the last query
  const int lrow = w * (QT / NW) + g16;
  const int chunk = (i16 ^ swz16(lrow)) * 8;
  auto qtoken = [&](int p) -> int32_t {
    if constexpr (DENSE) {
      return p;
    } else {
      const uint32_t bi = fd_div(uint32_t(p), g.div_S);
      const uint32_t r = uint32_t(p) - bi * uint32_t(g.S);
      return rows_l[bi] + (TAB ? offtab[r] : block_offset(g, r));
    }
  };
  // element offset of this lane's Q/dO row of tile t, and the token of its LSE/delta
  // ALN (blocks a multiple of the tile): tile t lies in one list entry, at rows aln_rr.. of
  // it; the entry and row advance by one tile a call (calls come in tile order) and stop
  // at the last tile, which the tiles past the end repeat
  int aln_pb = 0, aln_rr = 0;
  auto tile_offsets = [&](int t, int32_t& o, int32_t& xl) {
    if constexpr (ALN) {
      const int32_t rb = rows_l[aln_pb];
      o = gbase + (rb + offtab[aln_rr + lrow]) * hstride;
      xl = rb + offtab[aln_rr + (lane & 31)];
      if (t + 1 < ntiles) {
        aln_rr += QT;
        if (aln_rr == g.S) {
          aln_rr = 0;
          ++aln_pb;
        }
      }
      return;
    }
    o = gbase + qtoken(min(t * QT + lrow, plast)) * hstride;
    xl = qtoken(min(t * QT + (lane & 31), plast));
  };
  auto issue_offsets = [&](int32_t o, int32_t xl, unsigned char* sb) {
    const int dst = wu * (QT / NW) * ROWB;
    load_to_lds16(rQ, 2u * uint32_t(o + chunk), sb + dst);
    load_to_lds16(rO, 2u * uint32_t(o + chunk), sb + TILE + dst);
    // scalar branch: the descriptor stays uniform
    if (TOK && wu == 2)
      load_to_lds4(rM, 4u * (mword + uint32_t(xl) * uint32_t(a.mwords)),
                   sb + 2 * TILE + wu * 64 * 4);
    else if (wu & 1) load_to_lds4(rD, 4u * uint32_t(xl), sb + 2 * TILE + wu * 64 * 4);
    else load_to_lds4(rL, 4u * uint32_t(xl), sb + 2 * TILE + wu * 64 * 4);
  };
  auto issue_tile = [&](int t, unsigned char* sb) {
    int32_t o, xl;
    tile_offsets(t, o, xl);
    issue_offsets(o, xl, sb);
  };

  // LDS read offsets of this lane: row reads of d-step s (query sub-tile 0), transposing
  // reads of d-tile ds
  int roff[D / 32], toff[D / 16];
  {
    const int rrd = i16 * ROWB;
    const int rsw = swz16(i16);
    const int trow = 4 * g16 + (i16 >> 2);
    const int trd = trow * ROWB + 8 * (i16 & 1);
    const int tsw = swz16(trow);
    const int tc = (i16 & 3) >> 1;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) roff[s] = rrd + 16 * ((4 * s + g16) ^ rsw);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) toff[ds] = trd + 16 * ((2 * ds + tc) ^ tsw);
  }
  const float c2 = a.scale_log2;

  using Acc = f32x4[2][KS];
  // S = Q K^T (role P, rows of the Q tile) or dP = dO V^T (role dS, rows of the dO tile)
  auto products = [&](const unsigned char* rows, Acc& sacc, const f32x4 (&init)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[qs][ks] = init[qs];
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const int o = qs * 16 * ROWB + roff[s];
        const bf16x8 ra = as_bf16x8(*reinterpret_cast<const u32x4*>(rows + o));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[qs][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra, kvf[ks][s], sacc[qs][ks],
                                                                 0, 0, 0);
      }
  };
  // acc^T += X^T B over the tile whose rows are in `rows` (dO for role P, Q for role dS)
  auto accumulate = [&](const unsigned char* rows, const bf16x8 (&bop)[KS])
      __attribute__((always_inline)) {
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const int o = toff[ds];
      const u32x2 lo = lds_read_tr16(rows + o), hi = lds_read_tr16(rows + o + 16 * ROWB);
      const bf16x8 xt = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[ds][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xt, bop[ks], acc[ds][ks], 0, 0, 0);
    }
  };
  // k order of the B operands permuted to the accumulator layout: position 8g + e is
  // query 4g + e (e < 4) of query sub-tile 0 and 4g + e - 4 of sub-tile 1
  auto pack = [&](const float (&v)[2][KS][4], bf16x8 (&out)[KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      out[ks] = as_bf16x8(u32x4{pack_bf16x2(v[0][ks][0], v[0][ks][1]),
                                pack_bf16x2(v[0][ks][2], v[0][ks][3]),
                                pack_bf16x2(v[1][ks][0], v[1][ks][1]),
                                pack_bf16x2(v[1][ks][2], v[1][ks][3])});
  };
  // role P, tile t in stage sb: P to the exchange buffer, dV^T += dO^T P (sacc: the
  // registers role dS keeps its dP in)
  auto step_p = [&](const unsigned char* sb, uint32_t* xb, Acc& sacc)
      __attribute__((always_inline)) {
    const f32x4 zero[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    products(sb, sacc, zero);
    const float* lse_s = reinterpret_cast<const float*>(sb + 2 * TILE);
    float pv[2][KS][4];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float4 l4 = *reinterpret_cast<const float4*>(lse_s + qs * 16 + 4 * g16);
      const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
      bool keep[4] = {true, true, true, true};
      if constexpr (TOK) {   // select, not multiply: an empty row has lse = -inf
        const u32x4 m4 = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const uint32_t*>(sb + 2 * TILE + 2 * 64 * 4) + qs * 16 + 4 * g16);
        const uint32_t jb = uint32_t(jblk) & 31u;
#pragma unroll
        for (int i = 0; i < 4; ++i) keep[i] = (m4[i] >> jb) & 1u;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[qs][ks][i] = __builtin_amdgcn_exp2f(fmaf(sacc[qs][ks][i], c2, -lv[i]));
          if constexpr (TOK) pv[qs][ks][i] = keep[i] ? pv[qs][ks][i] : 0.f;
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      *reinterpret_cast<u32x4*>(xb + (ks * 64 + lane) * 4) =
          u32x4{pack_f16x2(pv[0][ks][0], pv[0][ks][1]), pack_f16x2(pv[0][ks][2], pv[0][ks][3]),
                pack_f16x2(pv[1][ks][0], pv[1][ks][1]), pack_f16x2(pv[1][ks][2], pv[1][ks][3])};
    bf16x8 pb[KS];
    pack(pv, pb);
    accumulate(sb + TILE, pb);
  };
  // role dS: dS of the previous tile (its stage sbp, its P in xb) from dprev, then the
  // dP of the current tile (stage sb) into dprev, then dK^T += Q^T dS
  auto finish_ds = [&](const unsigned char* sbp, const uint32_t* xb, const Acc& dprev,
                       bf16x8 (&sbf)[KS]) __attribute__((always_inline)) {
    (void)sbp;
    float sv[2][KS][4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 p4 = *reinterpret_cast<const u32x4*>(xb + (ks * 64 + lane) * 4);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int i = 0; i < 4; ++i)   // P (dP - delta)
          sv[qs][ks][i] = mul_f16(p4[2 * qs + (i >> 1)], i & 1, dprev[qs][ks][i]);
    }
    pack(sv, sbf);
  };

  // The last tile of a ragged stream: wave 0, whose load filled the LSE slot, writes
  // +inf over the positions past the end once its load has landed (before the barrier
  // that publishes the tile): P = 0 there, and so dS = 0.
  const int tail = nq % QT;
  auto mask_tail = [&](unsigned char* sb, int t) __attribute__((always_inline)) {
    if (tail != 0 && t == ntiles - 1 && wu == 0) {
      if (lane >= tail && lane < QT)
        reinterpret_cast<float*>(sb + 2 * TILE)[lane] = __builtin_inff();
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
    }
  };

  int32_t noff, nxl;
  Acc dprev;   // role dS: dP of the previous tile (role P: its S)
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dprev[qs][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // one loop per role (the branch outside the loop keeps each loop's registers its own);
  // both loops pass the same barriers
  auto run = [&](auto RPc) __attribute__((always_inline)) {
    constexpr bool RP = decltype(RPc)::value;
    auto step = [&](auto STc, int t) __attribute__((always_inline)) {
      constexpr int ST = decltype(STc)::value;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lds<PER_TILE>();   // this wave's loads of tile t have landed
      mask_tail(stage(STc), t);
      pipeline_barrier();
      issue_offsets(noff, nxl, stage(std::integral_constant<int, ST + 2>{}));
      tile_offsets(t + 3, noff, nxl);
      if (wave_busy) {
        if constexpr (RP) {
          step_p(stage(STc), &xbuf[ST & 1][kg][0], dprev);
        } else {
          bf16x8 sbf[KS];
          if (t > 0) finish_ds(stage(std::integral_constant<int, ST + NS - 1>{}),
                               &xbuf[(ST + 1) & 1][kg][0], dprev, sbf);
          // dP - delta: the accumulators start at -delta of the tile's queries
          const float* dl_s = reinterpret_cast<const float*>(stage(STc) + 2 * TILE) + 64;
          f32x4 nd[2];
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) {
            const float4 d4 = *reinterpret_cast<const float4*>(dl_s + qs * 16 + 4 * g16);
            nd[qs] = f32x4{-d4.x, -d4.y, -d4.z, -d4.w};
          }
          products(stage(STc) + TILE, dprev, nd);
          if (t > 0) accumulate(stage(std::integral_constant<int, ST + NS - 1>{}), sbf);
        }
      }
    };
    issue_tile(0, stage0);
    issue_tile(1, stage1);
    tile_offsets(2, noff, nxl);
    int t = 0;
    for (; t + NS <= ntiles; t += NS) {
      step(I0{}, t);
      step(I1{}, t + 1);
      step(I2{}, t + 2);
      step(I3{}, t + 3);
    }
    if (t < ntiles) step(I0{}, t);
    if (t + 1 < ntiles) step(I1{}, t + 1);
    if (t + 2 < ntiles) step(I2{}, t + 2);
  };
  if (role_p) run(std::true_type{});
  else run(std::false_type{});
  // role dS: the dS and dK^T of the last tile, once its P is published
  wait_vmcnt_lds<0>();   // also: the loads past the end land before the LDS is released
  __syncthreads();
  if (wave_busy && !role_p && ntiles > 0) {
    const int last = ntiles - 1;
    bf16x8 sbf[KS];
    const uint32_t* xb = &xbuf[last & 1][kg][0];
    switch (last & 3) {
      case 0: finish_ds(stage0, xb, dprev, sbf); accumulate(stage0, sbf); break;
      case 1: finish_ds(stage1, xb, dprev, sbf); accumulate(stage1, sbf); break;
      case 2: finish_ds(stage2, xb, dprev, sbf); accumulate(stage2, sbf); break;
      default: finish_ds(stage3, xb, dprev, sbf); accumulate(stage3, sbf); break;
    }
  }

  // dV^T (role P) or dK^T (role dS): lane l holds key l%16 of sub-tile ks,
  // d = 16 ds + 4 (l/16) + 0..3
  GT* __restrict__ out = role_p ? dV : dK;
  const float osc = role_p ? 1.0f : a.scale;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (kbase + ks * 16 + i16 < klim) {
      const int32_t koff = row_offset(g, grp, key_token(ks));
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const int d0 = ds * 16 + 4 * g16;
        store4(out + koff + d0, acc[ds][ks][0] * osc, acc[ds][ks][1] * osc,
               acc[ds][ks][2] * osc, acc[ds][ks][3] * osc);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// dQ for d = 128 on v_mfma_f32_16x16x32_bf16, the layout of the 48-query forward: a
// workgroup covers 192 queries (a whole 192-token block) in four query groups of 48
// (three 16-query sub-tiles), streaming the keys of the row list in tiles of 32.  Per
// tile and query group:
//   S^T = K Q^T and dP^T = V dO^T as 2 key sub-tiles x 3 query sub-tiles x 4 d-steps
//   (A = K or V rows from LDS, B = the group's Q or dO columns in registers); the
//   accumulator gives lane l the query l % 16 of each query sub-tile and keys
//   4 (l/16) + 0..3 of each key sub-tile;
//   P = exp(S / sqrt(d) - lse), dS = P (dP - delta), packed with their k order permuted
//   to the accumulator layout (as P in the forward): the B operand of dQ^T += K^T dS^T,
//   whose A operand K^T comes from two transposing reads of the K tile.
// The work of a query group is split over two waves on one SIMD (waves qg and qg + 4):
//   role P (waves 0-3): S and dP of tile t (its dP^T accumulators start at -delta of their
//     queries), P, and dS = P (dP - delta) from the fp32 P, packed in bf16 as the B
//     operands of the dQ product and written to an LDS exchange buffer;
//   role dQ (waves 4-7): one step later, once the step barrier has published that dS,
//     dQ^T += K^T dS^T.
// Role P holds the group's Q and dO columns, role dQ the dQ accumulator (96 registers a
// lane), so two waves fit a SIMD, all eight waves have queries at 192-token blocks, and
// each K/V tile is loaded once per block.  The roles run 48 and 24 products a step, and
// all the vector work is role P's: role dQ's step is its LDS reads (the exchange and the
// transposing K reads) and its products.  The K tile is read row-wise and transposed
// (swizzle swz16); the V tile only row-wise (same swizzle).  Stages as in the split dK/dV
// kernel: the K tile of tile t is read at steps t and t+1, step t refills the stage of
// tile t-2 with tile t+2.
// TOK: token-granular selection; role P keeps P only at the list positions its query
// selected (the query's row of the list-position mask, two words cached per sub-tile and
// refetched when a tile moves into another 32-position window).
template <bool DENSE, bool TAB, typename GT, bool TOK = false, bool ALN = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_split_bf16_kernel(AttnParams a) {
  constexpr int D = 128, NW = 8, NT = 512, NQG = 4;
  constexpr int M = 3;                       // query sub-tiles per group
  constexpr int QW = 16 * M;                 // queries per group
  constexpr int QT = NQG * QW;               // queries per workgroup
  constexpr int KT = 32;                     // keys per tile
  constexpr int ROWB = D * 2;
  constexpr int TILE = KT * ROWB;            // bytes of one K or V tile
  constexpr int LPW = KT / (NW * 4);         // load instructions per wave per tensor
  static_assert(LPW == 1, "one row group per wave");
  constexpr int NS = 4;                      // pipeline stages
  constexpr int PER_TILE = 2 * LPW;          // loads per wave per tile
  constexpr int XF = 2 * M * 4 * 64;         // values of dS one query group passes a tile

  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2][NQG][XF / 2];   // dS, bf16 pairs
  __shared__ int32_t cols[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];
  __shared__ int32_t scratch[NW];
  auto stage = [&](auto Ic) -> unsigned char* {
    constexpr int I = decltype(Ic)::value % NS;
    if constexpr (I == 0) return stage0;
    else if constexpr (I == 1) return stage1;
    else if constexpr (I == 2) return stage2;
    else return stage3;
  };

  const Geom& g = a.g;
  int grp, iblk, qt;
  if constexpr (DENSE) {
    const int bid = xcd_item(blockIdx.x, g.B * g.Hh, a.tiles);
    if (bid < 0) return;
    qt = bid % a.tiles;
    iblk = 0;
    grp = bid / a.tiles;
  } else {
    SparseItem it;
    if (!sparse_item<NT>(g, a.row_ptr, a.tiles, a.ordered != 0, cols, scratch, &it)) return;
    grp = it.grp;
    iblk = it.blk;
    qt = it.tile;
  }

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ dO = static_cast<const uint16_t*>(a.dout);
  GT* __restrict__ dQ = static_cast<GT*>(a.dq);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * D) * 2u;   // < 2^32 (validated)
  const BufRes rK = buffer_res(K, tbytes), rV = buffer_res(V, tbytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int qg = wu & (NQG - 1);
  const bool role_p = wu < NQG;              // wave-uniform
  const int g16 = lane >> 4, i16 = lane & 15;

  int nkeys;
  if constexpr (DENSE) {
    nkeys = g.L;
  } else {
    int start, len;
    list_range(g, a.row_ptr, grp, iblk, &start, &len);
    const int kept = compact_list<NT>(a.col_idx + size_t(grp) * g.Nb * g.Nb + start, len,
                                      g.Nb, cols, scratch);
    // ALN: the tables hold element offsets (token times the row stride, plus the head's
    // base in cols), so a tile's row offset is one addition
    const int32_t hs = ALN ? g.Hh * D : 1, gb = ALN ? row_offset(g, grp, 0) : 0;
    for (int i = tid; i < kept; i += NT) cols[i] = gb + block_base(g, uint32_t(cols[i])) * hs;
    if (kept == 0 && tid == 0) cols[0] = gb;   // token 0: loads of an empty stream
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r)) * hs;
    __syncthreads();
    nkeys = kept * g.S;
  }
  const int ntiles = __builtin_amdgcn_readfirstlane((nkeys + KT - 1) / KT);

  // this lane's query in each sub-tile (role P holds its Q and dO fragments)
  const int qlim = DENSE ? g.L : g.S;
  const int qbase = qt * QT + qg * QW;
  const bool wave_busy = qbase < qlim;   // otherwise: loads and barriers only
  auto query_token = [&](int m) -> int32_t {
    const int rq = qbase + m * 16 + i16;
    const int rqc = rq < qlim ? rq : 0;
    return DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  };

  // loader: one instruction moves 4 rows; lane L fills row L/16 at chunk position L % 16
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nkeys - 1, 0);   // positions past the end repeat the last key
  const int lrow = w * (KT / NW) + g16;
  const int chunk = (i16 ^ swz16(lrow)) * 8;
  // ALN (blocks a multiple of the tile): as in the dK/dV kernel
  int aln_pb = 0, aln_rr = 0;
  auto tile_offsets = [&](int t) -> int32_t {
    if constexpr (ALN) {
      const int32_t o = cols[aln_pb] + offtab[aln_rr + lrow];
      if (t + 1 < ntiles) {
        aln_rr += KT;
        if (aln_rr == g.S) {
          aln_rr = 0;
          ++aln_pb;
        }
      }
      return o;
    }
    const int p = min(t * KT + lrow, plast);
    int32_t x = p;
    if constexpr (!DENSE) {
      const uint32_t pb = fd_div(uint32_t(p), g.div_S);
      const uint32_t rr = uint32_t(p) - pb * uint32_t(g.S);
      x = cols[pb] + (TAB ? offtab[rr] : block_offset(g, rr));
    }
    return gbase + x * hstride;
  };
  auto issue_offsets = [&](int32_t o, unsigned char* sb) {
    const int dst = wu * (KT / NW) * ROWB;   // wave-uniform
    load_to_lds16(rK, 2u * uint32_t(o + chunk), sb + dst);
    load_to_lds16(rV, 2u * uint32_t(o + chunk), sb + TILE + dst);
  };

  // LDS read offsets of this lane: K/V rows of d-step s (key sub-tile 0), and the K^T
  // reads of d-tile ds (keys 0..15; +16 rows for keys 16..31)
  int roff[D / 32], toff[D / 16];
  {
    const int rsw = swz16(i16);
    const int trow = 4 * g16 + (i16 >> 2);
    const int tsw = swz16(trow);
    const int tc = (i16 & 3) >> 1;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) roff[s] = i16 * ROWB + 16 * ((4 * s + g16) ^ rsw);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      toff[ds] = trow * ROWB + 8 * (i16 & 1) + 16 * ((2 * ds + tc) ^ tsw);
  }
  const float c2 = a.scale_log2;

  using Acc = f32x4[2][M];
  using Frag = bf16x8[M][D / 32];
  // S^T = K Q^T (rows of the K tile, B = Q) or dP^T = V dO^T (rows of the V tile, B = dO),
  // the accumulator of key sub-tile ks and query sub-tile m starting at init[ks][m]
  auto products = [&](const unsigned char* rows, const Frag& bf, Acc& sacc, const Acc& init)
      __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < M; ++m) sacc[ks][m] = init[ks][m];
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ra = as_bf16x8(*reinterpret_cast<const u32x4*>(
            rows + ks * 16 * ROWB + roff[s]));
#pragma unroll
        for (int m = 0; m < M; ++m)
          sacc[ks][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra, bf[m][s], sacc[ks][m],
                                                                0, 0, 0);
      }
  };
  PosMask pm[TOK ? M : 1];
  if constexpr (TOK) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      pm[m].init(a.posmask + size_t(grp * g.L + query_token(m)) * a.mwords, a.mwords);
  }
  // role P, tile t in stage sb: S and dP, then dS = P (dP - delta) packed as the B operands
  // of dQ^T += K^T dS^T, to the exchange buffer (keys past the end, and with TOK unselected
  // list positions: P = 0, by a select since an empty row has lse = -inf, and so dS = 0)
  auto step_p = [&](const unsigned char* sb, uint32_t* xb, int t, const Frag& qf,
                    const Frag& df, const float (&lse2)[M], const float (&ndl)[M])
      __attribute__((always_inline)) {
    // S starts at -inf for the keys past the end of the ragged last tile (never with ALN:
    // the stream is a multiple of the tile), so that their P is 0; dP starts at -delta
    Acc s0, d0;
    float kb[2][4] = {};
    if (!ALN && t * KT + KT > nkeys) {   // uniform
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kb[ks][i] = t * KT + ks * 16 + 4 * g16 + i >= nkeys ? -INFINITY : 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        s0[ks][m] = f32x4{kb[ks][0], kb[ks][1], kb[ks][2], kb[ks][3]};
        d0[ks][m] = f32x4{ndl[m], ndl[m], ndl[m], ndl[m]};
      }
    Acc sacc, dacc;
    products(sb, qf, sacc, s0);
    products(sb + TILE, df, dacc, d0);   // dP^T - delta
    bool b0[TOK ? M : 1], b1[TOK ? M : 1];
    int bh = 0;   // the boundary, counted from this lane's first key
    if constexpr (TOK) {
      const int li0 = int(fd_div(uint32_t(t * KT), g.div_S));
#pragma unroll
      for (int m = 0; m < M; ++m) {
        pm[m].fetch(li0);
        b0[m] = pm[m].keep(li0);
        b1[m] = pm[m].keep(li0 + 1);
      }
      bh = (li0 + 1) * g.S - t * KT - 4 * g16;
    }
    float pv[2][M][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[ks][m][i] = __builtin_amdgcn_exp2f(fmaf(sacc[ks][m][i], c2, -lse2[m]));
          if constexpr (TOK) pv[ks][m][i] = ((ks * 16 + i) < bh ? b0[m] : b1[m]) ? pv[ks][m][i] : 0.f;
        }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float d[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) d[ks][i] = pv[ks][m][i] * dacc[ks][m][i];
      *reinterpret_cast<u32x4*>(xb + (m * 64 + lane) * 4) =
          u32x4{pack_bf16x2(d[0][0], d[0][1]), pack_bf16x2(d[0][2], d[0][3]),
                pack_bf16x2(d[1][0], d[1][1]), pack_bf16x2(d[1][2], d[1][3])};
    }
  };
  // role dQ: the packed dS of a tile from the exchange buffer
  auto read_ds = [&](const uint32_t* xb, bf16x8 (&sbf)[M]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      sbf[m] = as_bf16x8(*reinterpret_cast<const u32x4*>(xb + (m * 64 + lane) * 4));
  };

  int32_t noff;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // one loop per role (the branch outside the loop keeps each loop's registers its own);
  // both loops pass the same barriers
  auto run = [&](auto RPc) __attribute__((always_inline)) {
    constexpr bool RP = decltype(RPc)::value;
    // role P: Q and dO fragments, lse * log2(e) and -delta of this lane's queries
    Frag qf, df;
    float lse2[M], ndl[M];
    if constexpr (RP) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int32_t x = query_token(m);
        const int32_t qoff = row_offset(g, grp, x);
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          qf[m][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + qoff + s * 32 + g16 * 8));
          df[m][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(dO + qoff + s * 32 + g16 * 8));
        }
        lse2[m] = a.lse[size_t(grp) * g.L + x] * kLog2e;
        ndl[m] = -a.delta[size_t(grp) * g.L + x];
      }
    }
    f32x4 qacc[RP ? 1 : M][RP ? 1 : D / 16];   // role dQ: dQ^T
    if constexpr (!RP) {
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) qacc[m][ds] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // dQ^T += K^T dS^T over the K tile in stage sb
    auto accumulate = [&](const unsigned char* sb, const bf16x8 (&sbf)[M])
        __attribute__((always_inline)) {
      if constexpr (!RP) {
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          const u32x2 lo = lds_read_tr16(sb + toff[ds]);
          const u32x2 hi = lds_read_tr16(sb + toff[ds] + 16 * ROWB);
          const bf16x8 kt = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int m = 0; m < M; ++m)
            qacc[m][ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, sbf[m], qacc[m][ds],
                                                                  0, 0, 0);
        }
      }
    };
    auto step = [&](auto STc, int t) __attribute__((always_inline)) {
      constexpr int ST = decltype(STc)::value;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lds<PER_TILE>();   // this wave's loads of tile t have landed
      pipeline_barrier();
      issue_offsets(noff, stage(std::integral_constant<int, ST + 2>{}));
      noff = tile_offsets(t + 3);
      if (wave_busy) {
        if constexpr (RP) {
          step_p(stage(STc), &xbuf[ST & 1][qg][0], t, qf, df, lse2, ndl);
        } else if (t > 0) {   // the previous tile's dS, posted by role P before this barrier
          bf16x8 sbf[M];
          read_ds(&xbuf[(ST + 1) & 1][qg][0], sbf);
          accumulate(stage(std::integral_constant<int, ST + NS - 1>{}), sbf);
        }
      }
    };
    issue_offsets(tile_offsets(0), stage0);
    issue_offsets(tile_offsets(1), stage1);
    noff = tile_offsets(2);
    int t = 0;
    for (; t + NS <= ntiles; t += NS) {
      step(I0{}, t);
      step(I1{}, t + 1);
      step(I2{}, t + 2);
      step(I3{}, t + 3);
    }
    if (t < ntiles) step(I0{}, t);
    if (t + 1 < ntiles) step(I1{}, t + 1);
    if (t + 2 < ntiles) step(I2{}, t + 2);
    // role dQ: the dQ^T of the last tile, once its dS is published
    wait_vmcnt_lds<0>();   // also: the loads past the end land before the LDS is released
    __syncthreads();
    if constexpr (!RP) {
      if (wave_busy && ntiles > 0) {
        const int last = ntiles - 1;
        bf16x8 sbf[M];
        read_ds(&xbuf[last & 1][qg][0], sbf);
        switch (last & 3) {
          case 0: accumulate(stage0, sbf); break;
          case 1: accumulate(stage1, sbf); break;
          case 2: accumulate(stage2, sbf); break;
          default: accumulate(stage3, sbf); break;
        }
      }
      // dQ^T: lane l holds query l%16 of sub-tile m, d = 16 ds + 4 (l/16) + 0..3
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (qbase + m * 16 + i16 < qlim) {
          const int32_t qoff = row_offset(g, grp, query_token(m));
#pragma unroll
          for (int ds = 0; ds < D / 16; ++ds) {
            const int d0 = ds * 16 + 4 * g16;
            const float sc = a.scale;
            store4(dQ + qoff + d0, qacc[m][ds][0] * sc, qacc[m][ds][1] * sc,
                   qacc[m][ds][2] * sc, qacc[m][ds][3] * sc);
          }
        }
      }
    }
  };
  if (role_p) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------------
// dQ: one wave per 32 queries, key stream from the row list of the query block.
// TOK: token-granular selection, as in the forward (list-position mask of the query).
// NS: K/V tile stages.  With 4, step t waits only for this wave's loads of tile t, passes
// a barrier and refills the stage of tile t-1 with tile t+3 (as the forward does).  With
// 2 (the TOK instances, whose per-query mask-word loads would interleave with the tile
// loads on the same counter), the loads of tile t+1 are in flight during tile t and the
// step ends waiting for all of them.
template <int D, int NW, int KSUB, bool DENSE, bool TAB, typename GT, bool TOK = false,
          int NS = 2, bool ALN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_bf16_kernel(AttnParams a) {
  constexpr int NT = NW * 64;
  constexpr int QT = NW * 32;
  constexpr int KT = KSUB * 32;
  constexpr int ROWB = D * 2;
  constexpr int RPI = 1024 / ROWB;
  constexpr int LPW = KT / (NW * RPI);
  static_assert(KT % (NW * RPI) == 0, "tile rows split over waves");
  constexpr int TILE = KT * ROWB;

  static_assert(NS == 2 || (NS == 4 && !TOK), "stages");
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[NS > 2 ? 2 * TILE : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[NS > 2 ? 2 * TILE : 1];
  auto stage = [&](auto Ic) -> unsigned char* {
    constexpr int I = decltype(Ic)::value % NS;
    if constexpr (I == 0) return stage0;
    else if constexpr (I == 1) return stage1;
    else if constexpr (I == 2) return stage2;
    else return stage3;
  };
  __shared__ int32_t cols[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];   // block_offset(r), r < S
  __shared__ int32_t scratch[NW];

  const Geom& g = a.g;
  int grp, iblk, qt;
  if constexpr (DENSE) {
    const int bid = xcd_item(blockIdx.x, g.B * g.Hh, a.tiles);
    if (bid < 0) return;
    qt = bid % a.tiles;
    iblk = 0;
    grp = bid / a.tiles;
  } else {
    SparseItem it;
    if (!sparse_item<NT>(g, a.row_ptr, a.tiles, a.ordered != 0, cols, scratch, &it)) return;
    grp = it.grp;
    iblk = it.blk;
    qt = it.tile;
  }

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ dO = static_cast<const uint16_t*>(a.dout);
  GT* __restrict__ dQ = static_cast<GT*>(a.dq);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * D) * 2u;   // < 2^32 (validated)
  const BufRes rK = buffer_res(K, tbytes), rV = buffer_res(V, tbytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  int nkeys;
  if constexpr (DENSE) {
    nkeys = g.L;
  } else {
    int start, len;
    list_range(g, a.row_ptr, grp, iblk, &start, &len);
    const int kept = compact_list<NT>(a.col_idx + size_t(grp) * g.Nb * g.Nb + start, len,
                                      g.Nb, cols, scratch);
    // ALN: the tables hold element offsets (token times the row stride, plus the head's
    // base in cols), so a tile's row offsets are one addition
    const int32_t hs = ALN ? g.Hh * D : 1, gb = ALN ? row_offset(g, grp, 0) : 0;
    for (int i = tid; i < kept; i += NT) cols[i] = gb + block_base(g, uint32_t(cols[i])) * hs;
    if (kept == 0 && tid == 0) cols[0] = gb;   // token 0: address of an empty stream
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r)) * hs;
    __syncthreads();
    nkeys = kept * g.S;
  }
  const int ntiles = __builtin_amdgcn_readfirstlane((nkeys + KT - 1) / KT);

  const int qlim = DENSE ? g.L : g.S;
  const int rq = qt * QT + w * 32 + l32;
  const bool qvalid = rq < qlim;
  // waves with no valid query only load and synchronise (see the dK/dV kernel)
  const bool wave_busy = qt * QT + w * 32 < qlim;
  const int rqc = qvalid ? rq : 0;
  const int32_t xq = DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  const int32_t qoff = row_offset(g, grp, xq);
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + qoff + s * 16 + half * 8));
    df[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(dO + qoff + s * 16 + half * 8));
  }
  const float lse2 = a.lse[size_t(grp) * g.L + xq] * kLog2e;
  const float dl = a.delta[size_t(grp) * g.L + xq];
  // token-granular selection: this lane's row of the list-position mask
  const uint32_t pmrow = uint32_t(grp * g.L + xq) * uint32_t(a.mwords);

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqacc[dt][v] = 0.f;

  constexpr int CPR = D / 8;
  const int lrow0 = w * (KT / NW) + lane / CPR;
  const int lcp = lane % CPR;
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nkeys - 1, 0);   // positions past the end repeat the last key
  // element offsets of this lane's K/V rows of tile t (addresses first, loads back to back)
  // ALN (blocks a multiple of the tile): tile t lies in one list entry, at rows aln_rr.. of
  // it; the entry and row advance by one tile a call (calls come in tile order) and stop
  // at the last tile, which the tiles past the end repeat
  int aln_pb = 0, aln_rr = 0;
  auto tile_offsets = [&](int t, int32_t (&o)[LPW]) {
    if constexpr (ALN) {
      const int32_t cb = cols[aln_pb];
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = lrow0 + i * RPI;
        o[i] = cb + offtab[aln_rr + r] + (lcp ^ swz<D>(r)) * 8;
      }
      if (t + 1 < ntiles) {
        aln_rr += KT;
        if (aln_rr == g.S) {
          aln_rr = 0;
          ++aln_pb;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = lrow0 + i * RPI;
      const int p = min(t * KT + r, plast);
      int32_t x = p;
      if constexpr (!DENSE) {
        const uint32_t bi = fd_div(uint32_t(p), g.div_S);
        const uint32_t rr = uint32_t(p) - bi * uint32_t(g.S);
        x = cols[bi] + (TAB ? offtab[rr] : block_offset(g, rr));
      }
      o[i] = gbase + x * hstride + (lcp ^ swz<D>(r)) * 8;
    }
  };
  auto issue_offsets = [&](const int32_t (&o)[LPW], unsigned char* sb) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int dst = (w * (KT / NW) + i * RPI) * ROWB;
      load_to_lds16(rK, 2u * uint32_t(o[i]), sb + dst);
      load_to_lds16(rV, 2u * uint32_t(o[i]), sb + TILE + dst);
    }
  };
  int32_t noff[LPW];   // addresses of the next tile, computed one step ahead

  const float c2 = a.scale_log2;
  const int grp16 = lane >> 4, sl = lane & 15;
  // lane offsets of the K^T reads of key sub-tile 0 (the swizzle repeats every 16 rows,
  // so sub-tile ks adds 16 ks rows): key 4 (l/32) + (l%16)/4 (+8 for the upper half),
  // chunk 4 dt + 2 ((l/16) % 2) + (l%4)/2, 8 bytes at (l%2) * 8
  int trlo[D / 32], trhi[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int key0 = 4 * half + (sl >> 2);
    const int c = dt * 4 + 2 * (grp16 & 1) + ((sl & 3) >> 1);
    const int bo = (sl & 1) * 8;
    trlo[dt] = tile_off<D>(key0, c) + bo;
    trhi[dt] = tile_off<D>(key0 + 8, c) + bo;
  }
  auto compute = [&](const unsigned char* cur, int t, uint32_t pw0, uint32_t pw1)
      __attribute__((always_inline)) {
    // token-granular selection: which of this lane's keys its query selected, worked out
    // before the products take the registers (one bit per key)
    uint32_t keepbits = ~0u;
    if constexpr (TOK) {
      keepbits = 0u;
      const uint32_t p0 = uint32_t(t * KT);
      const int wi = int(fd_div(p0, g.div_S)) >> 5;
      const uint32_t w0 = pw0, w1 = pw1;
      if (g.S >= KT) {
        // the tile spans list positions li0 (offsets below the boundary) and li0 + 1: two
        // mask bits, and one compare a key
        const int li0 = int(fd_div(p0, g.div_S));
        const int r0 = li0 - 32 * wi, r1 = r0 + 1;
        const uint32_t b0 = (w0 >> r0) & 1u;
        const uint32_t b1 = (((r1 < 32) ? w0 : w1) >> (r1 & 31)) & 1u;
        const int bh = (li0 + 1) * g.S - int(p0) - 4 * half;   // from this lane's first key
#pragma unroll
        for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            keepbits |= ((kk * 32 + 8 * (v >> 2) + (v & 3)) < bh ? b0 : b1) << (kk * 16 + v);
      } else {
        // opaque per-tile base: otherwise the 16 per-key lane offsets are hoisted out of
        // the loop into 16 registers
        uint32_t pb = p0 + 4 * half;
        asm volatile("" : "+v"(pb));
#pragma unroll
        for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t p = pb + (kk * 32 + 8 * (v >> 2) + (v & 3));
            const int rel = int(fd_div(p, g.div_S)) - 32 * wi;
            keepbits |= ((((rel < 32) ? w0 : w1) >> (rel & 31)) & 1u) << (kk * 16 + v);
          }
      }
      // keep the computation here: sunk to its use it lands where registers are scarcest
      asm volatile("" : "+v"(keepbits));
    }
    const unsigned char* kb = cur;
    const unsigned char* vb = cur + TILE;
    // K and V fragments in four batches of d-steps, each read ahead of its products, and
    // the K^T reads of dQ right after.
    // dP accumulators start at -delta of this lane's query: the products give dP - delta
    f32x16 sacc[KSUB], dpacc[KSUB];
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[kk][v] = 0.f;
        dpacc[kk][v] = -dl;
      }
    constexpr int NB = 4;   // batches of d-steps
#pragma unroll
    for (int hb = 0; hb < NB; ++hb) {
      constexpr int HS = D / 16 / NB;   // d-steps per batch
      bf16x8 ka[KSUB][HS], va[KSUB][HS];
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
        for (int j = 0; j < HS; ++j) {
          const int o = tile_off<D>(kk * 32 + l32, 2 * (hb * HS + j) + half);
          ka[kk][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + o));
          va[kk][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(vb + o));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
        for (int j = 0; j < HS; ++j) {
          sacc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk][j], qf[hb * HS + j],
                                                             sacc[kk], 0, 0, 0);
          dpacc[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk][j], df[hb * HS + j],
                                                              dpacc[kk], 0, 0, 0);
        }
    }
    bf16x8 kt[2 * KSUB][D / 32];   // K^T fragments of dQ^T += K^T dS^T (transposing reads)
    // this tile's copies of the lane offsets: opaque, so that the stage base is added at
    // the read (immediate offset) instead of hoisting one address per stage and offset
    int tl[D / 32], th[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      tl[dt] = trlo[dt];
      th[dt] = trhi[dt];
      asm volatile("" : "+v"(tl[dt]), "+v"(th[dt]));
    }
#pragma unroll
    for (int ks = 0; ks < 2 * KSUB; ++ks) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x2 lo = lds_read_tr16(kb + tl[dt] + ks * 16 * ROWB);
        const u32x2 hi = lds_read_tr16(kb + th[dt] + ks * 16 * ROWB);
        kt[ks][dt] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kk][v], c2, -lse2));
        dpacc[kk][v] = pv * dpacc[kk][v];   // P (dP - delta)
      }
    if (t * KT + KT > nkeys) {   // ragged last tile (uniform branch): no dS past the end
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (t * KT + kk * 32 + 8 * (v >> 2) + 4 * half + (v & 3) >= nkeys) dpacc[kk][v] = 0.f;
    }
    if constexpr (TOK) {   // list positions this lane's query did not select: no dS
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((keepbits >> (kk * 16 + v)) & 1u)) dpacc[kk][v] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 2 * KSUB; ++ks) {
      const int kk = ks >> 1, g0 = (ks & 1) * 8;
      u32x4 sw;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sw[e] = pack_bf16x2(dpacc[kk][g0 + 2 * e], dpacc[kk][g0 + 2 * e + 1]);
      const bf16x8 sbf = as_bf16x8(sw);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[ks][dt], sbf, dqacc[dt], 0, 0, 0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if constexpr (NS == 2) {
    auto step = [&](auto STc, int t) {
      constexpr int ST = decltype(STc)::value;
      __builtin_amdgcn_sched_barrier(0);   // keep the steps from being interleaved
      unsigned char* const cur = ST ? stage1 : stage0;
      unsigned char* const nxt = ST ? stage0 : stage1;
      // the two mask words of this tile, loaded before the next tile's loads are issued
      // so that waiting for them does not wait for those
      uint32_t pw0 = 0u, pw1 = 0u;
      if constexpr (TOK) {
        const int wi = int(fd_div(uint32_t(t * KT), g.div_S)) >> 5;
        pw0 = wi < a.mwords ? a.posmask[pmrow + wi] : 0u;
        pw1 = wi + 1 < a.mwords ? a.posmask[pmrow + wi + 1] : 0u;
      }
      if (t + 1 < ntiles) {
        issue_offsets(noff, nxt);
        tile_offsets(t + 2, noff);
      }
      if (wave_busy) compute(cur, t, pw0, pw1);
      wait_lds_loads();
      __syncthreads();
    };
    tile_offsets(0, noff);
    if (ntiles > 0) issue_offsets(noff, stage0);
    tile_offsets(1, noff);
    wait_lds_loads();
    __syncthreads();
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      step(S0{}, t);
      step(S1{}, t + 1);
    }
    if (t < ntiles) step(S0{}, t);
  } else {
    // tiles are loaded unconditionally, one a step; positions past the end repeat the
    // last key and are never used
    constexpr int PER_TILE = 2 * LPW;   // loads per wave per tile
    auto step = [&](auto STc, int t) {
      constexpr int ST = decltype(STc)::value;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lds<(NS - 2) * PER_TILE>();   // this wave's loads of tile t have landed
      pipeline_barrier();
      issue_offsets(noff, stage(std::integral_constant<int, ST + NS - 1>{}));
      tile_offsets(t + NS, noff);
      if (wave_busy) compute(stage(STc), t, 0u, 0u);
    };
    tile_offsets(0, noff);
    issue_offsets(noff, stage0);
    tile_offsets(1, noff);
    issue_offsets(noff, stage1);
    tile_offsets(2, noff);
    issue_offsets(noff, stage2);
    tile_offsets(3, noff);
    int t = 0;
    for (; t + NS <= ntiles; t += NS) {
      step(S0{}, t);
      step(S1{}, t + 1);
      step(S2{}, t + 2);
      step(S3{}, t + 3);
    }
    if (t < ntiles) step(S0{}, t);
    if (t + 1 < ntiles) step(S1{}, t + 1);
    if (t + 2 < ntiles) step(S2{}, t + 2);
    wait_vmcnt_lds<0>();   // the loads past the end land before the LDS is released
  }
  if (qvalid) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = dt * 32 + gq * 8 + half * 4;
        const float sc = a.scale;
        store4(dQ + qoff + d0, dqacc[dt][4 * gq] * sc, dqacc[dt][4 * gq + 1] * sc,
               dqacc[dt][4 * gq + 2] * sc, dqacc[dt][4 * gq + 3] * sc);
      }
  }
}

// ---------------------------------------------------------------------------------
// fp32 instances (VALU): the same recurrences one query (dQ) or one key (dK, dV) per lane.
template <int D, bool DENSE>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(AttnParams a) {
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
  const float* dO = static_cast<const float*>(a.dout);
  float* dQ = static_cast<float*>(a.dq);
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
  float qv[D], dov[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = Q[qoff + d];
    dov[d] = dO[qoff + d];
    acc[d] = 0.f;
  }
  const float lse = a.lse[size_t(grp) * g.L + xq];
  const float dl = a.delta[size_t(grp) * g.L + xq];
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
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(qv[d], ks[kk][d], s);
        dp = fmaf(dov[d], vs[kk][d], dp);
      }
      const float p = expf(s * a.scale - lse);
      const float ds = p * (dp - dl);
      for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ks[kk][d], acc[d]);
    }
    __syncthreads();
  }
  if (qvalid)
    for (int d = 0; d < D; ++d) dQ[qoff + d] = acc[d] * a.scale;
}

template <int D, bool DENSE>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(AttnParams a) {
  constexpr int QT = 32;
  __shared__ float qs[QT][D];
  __shared__ float os[QT][D];
  __shared__ float ls[QT], dls[QT];
  __shared__ int32_t rows_l[DENSE ? 1 : kMaxBlocks];
  __shared__ int32_t scratch[1];
  const Geom& g = a.g;
  const int nrow = DENSE ? 1 : g.Nb;
  int bid = blockIdx.x;
  const int kt = bid % a.tiles;
  bid /= a.tiles;
  const int jblk = bid % nrow;
  const int grp = bid / nrow;
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  const float* dO = static_cast<const float*>(a.dout);
  float* dK = static_cast<float*>(a.dk);
  float* dV = static_cast<float*>(a.dv);
  int nq;
  if constexpr (DENSE) {
    nq = g.L;
  } else {
    int start, len;
    list_range(g, a.col_ptr, grp, jblk, &start, &len);
    nq = compact_list<64>(a.row_idx + size_t(grp) * g.Nb * g.Nb + start, len, g.Nb, rows_l,
                          scratch) * g.S;
  }
  const int klim = DENSE ? g.L : g.S;
  const int rk = kt * 64 + threadIdx.x;
  const bool kvalid = rk < klim;
  const int rkc = kvalid ? rk : 0;
  const int32_t xk = DENSE ? rkc : block_base(g, jblk) + block_offset(g, rkc);
  const int32_t koff = row_offset(g, grp, xk);
  float kv[D], vv[D], dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    kv[d] = K[koff + d];
    vv[d] = V[koff + d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const float* lse_g = a.lse + size_t(grp) * g.L;
  const float* dl_g = a.delta + size_t(grp) * g.L;
  for (int t0 = 0; t0 < nq; t0 += QT) {
    for (int idx = threadIdx.x; idx < QT * D; idx += 64) {
      const int qq = idx / D, d = idx % D;
      const int p = t0 + qq;
      float qval = 0.f, oval = 0.f;
      if (p < nq) {
        const int32_t x = DENSE ? p : stream_token(g, rows_l, uint32_t(p));
        const int32_t off = row_offset(g, grp, x) + d;
        qval = Q[off];
        oval = dO[off];
        if (d == 0) {
          ls[qq] = lse_g[x];
          dls[qq] = dl_g[x];
        }
      }
      qs[qq][d] = qval;
      os[qq][d] = oval;
    }
    __syncthreads();
    const int n = min(QT, nq - t0);
    for (int qq = 0; qq < n; ++qq) {
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(qs[qq][d], kv[d], s);
        dp = fmaf(os[qq][d], vv[d], dp);
      }
      const float p = expf(s * a.scale - ls[qq]);
      const float ds = p * (dp - dls[qq]);
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(p, os[qq][d], dv[d]);
        dk[d] = fmaf(ds, qs[qq][d], dk[d]);
      }
    }
    __syncthreads();
  }
  if (kvalid)
    for (int d = 0; d < D; ++d) {
      dK[koff + d] = dk[d] * a.scale;
      dV[koff + d] = dv[d];
    }
}

// ---------------------------------------------------------------------------------
template <typename T, int D>
static void launch_delta(const Geom& g, const void* o, const void* dout, float* delta,
                         hipStream_t s) {
  constexpr int LPR = D / (16 / sizeof(T));
  const size_t rows = size_t(g.B) * g.L * g.Hh;
  const int grid = int((rows * LPR + 255) / 256);
  delta_kernel<T, D><<<grid, 256, 0, s>>>(g, static_cast<const T*>(o),
                                         static_cast<const T*>(dout), delta);
}

template <bool DENSE, typename GT, bool TOK = false, int KS = 3>
static void launch_dkdv_split_bf16(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  const int lim = DENSE ? g.L : g.S;
  const int rows = DENSE ? 1 : g.Nb;
  constexpr int KWG = 4 * 16 * KS;   // keys a workgroup
  a.tiles = (lim + KWG - 1) / KWG;
  const int grid = launch_grid<DENSE>(a, rows);
  if (!DENSE && g.S <= kOffsetTable && g.S % 32 == 0)
    attn_bwd_dkdv_split_bf16_kernel<DENSE, !DENSE, GT, TOK, !DENSE, KS><<<grid, 512, 0, s>>>(a);
  else if (!DENSE && g.S <= kOffsetTable)
    attn_bwd_dkdv_split_bf16_kernel<DENSE, !DENSE, GT, TOK, false, KS><<<grid, 512, 0, s>>>(a);
  else
    attn_bwd_dkdv_split_bf16_kernel<DENSE, false, GT, TOK, false, KS><<<grid, 512, 0, s>>>(a);
}

template <int D, bool DENSE, typename GT, bool TOK = false>
static void launch_dkdv_bf16(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  constexpr int NWK = 4;
  const int lim = DENSE ? g.L : g.S;
  if constexpr (D == 128) {
    // 192 keys a workgroup (key groups of 48) when 192-key tiles pad a block no more
    // than 128-key ones.  (The same kernel with key groups of 32 for the other blocks
    // measured no faster than this 32-key kernel inside a whole step.)
    if ((lim + 191) / 192 * 192 <= (lim + 127) / 128 * 128) {
      launch_dkdv_split_bf16<DENSE, GT, TOK, 3>(a, s);
      return;
    }
  }
  const int rows = DENSE ? 1 : g.Nb;
  a.tiles = (lim + NWK * 32 - 1) / (NWK * 32);
  const int grid = launch_grid<DENSE>(a, rows);
  if (!DENSE && g.S <= kOffsetTable)
    attn_bwd_dkdv_bf16_kernel<D, NWK, DENSE, !DENSE, GT, TOK><<<grid, NWK * 64, 0, s>>>(a);
  else
    attn_bwd_dkdv_bf16_kernel<D, NWK, DENSE, false, GT, TOK><<<grid, NWK * 64, 0, s>>>(a);
}

template <bool DENSE, typename GT, bool TOK = false>
static void launch_dq_split_bf16(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  const int lim = DENSE ? g.L : g.S;
  const int rows = DENSE ? 1 : g.Nb;
  a.tiles = (lim + 191) / 192;
  const int grid = launch_grid<DENSE>(a, rows);
  if (!DENSE && g.S <= kOffsetTable && g.S % 32 == 0)
    attn_bwd_dq_split_bf16_kernel<DENSE, !DENSE, GT, TOK, !DENSE><<<grid, 512, 0, s>>>(a);
  else if (!DENSE && g.S <= kOffsetTable)
    attn_bwd_dq_split_bf16_kernel<DENSE, !DENSE, GT, TOK><<<grid, 512, 0, s>>>(a);
  else
    attn_bwd_dq_split_bf16_kernel<DENSE, false, GT, TOK><<<grid, 512, 0, s>>>(a);
}

template <int D, bool DENSE, typename GT, bool TOK = false>
static void launch_dq_bf16(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  constexpr int KSUB = D == 128 ? 1 : 2;   // staging needs KSUB*32*D/8 to split over 4 waves
  const int lim = DENSE ? g.L : g.S;
  if constexpr (D == 128) {
    // 192 queries a workgroup (query groups of 48) when 192-query tiles pad a block no
    // more than 128-query ones (the rule of the forward and dK/dV), and either 128-query
    // tiles would leave more than an eighth of their query slots empty or the launch has
    // at least 1,024 of these workgroups (four rounds at one a CU): with fewer, the
    // 32-query kernel's smaller workgroups (two a CU) end the launch sooner
    const int p128 = (lim + 127) / 128 * 128;
    const int t192 = (lim + 191) / 192;
    const long wgs = long(g.B) * g.Hh * (DENSE ? 1 : g.Nb) * t192;
    if (t192 * 192 <= p128 && ((p128 - lim) * 8 > p128 || wgs >= 1024)) {
      // (this implies lim > 128, as the token instance's two-position key tiles need)
      launch_dq_split_bf16<DENSE, GT, TOK>(a, s);
      return;
    }
  }
  const int rows = DENSE ? 1 : g.Nb;
  a.tiles = (lim + 127) / 128;
  const int grid = launch_grid<DENSE>(a, rows);
  constexpr int NS = TOK ? 2 : 4;
  if (!DENSE && g.S <= kOffsetTable && g.S % (KSUB * 32) == 0)
    attn_bwd_dq_bf16_kernel<D, 4, KSUB, DENSE, !DENSE, GT, TOK, NS, !DENSE>
        <<<grid, 256, 0, s>>>(a);
  else if (!DENSE && g.S <= kOffsetTable)
    attn_bwd_dq_bf16_kernel<D, 4, KSUB, DENSE, !DENSE, GT, TOK, NS><<<grid, 256, 0, s>>>(a);
  else
    attn_bwd_dq_bf16_kernel<D, 4, KSUB, DENSE, false, GT, TOK, NS><<<grid, 256, 0, s>>>(a);
}

template <int D, bool DENSE>
static void launch_dkdv_f32(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  const int lim = DENSE ? g.L : g.S;
  const int rows = DENSE ? 1 : g.Nb;
  a.tiles = (lim + 63) / 64;
  attn_bwd_dkdv_f32_kernel<D, DENSE><<<g.B * g.Hh * rows * a.tiles, 64, 0, s>>>(a);
}

template <int D, bool DENSE>
static void launch_dq_f32(AttnParams a, hipStream_t s) {
  const Geom& g = a.g;
  const int lim = DENSE ? g.L : g.S;
  const int rows = DENSE ? 1 : g.Nb;
  a.tiles = (lim + 63) / 64;
  attn_bwd_dq_f32_kernel<D, DENSE><<<g.B * g.Hh * rows * a.tiles, 64, 0, s>>>(a);
}

// Instantiate launcher L<D, DENSE, GT> for the problem's head_dim, mode and grad type.
#define VMOBA_DISPATCH_BF16(L, a, s, dense)                                      \
  do {                                                                          \
    const bool g32_ = (a).g.grad_dtype == VMOBA_FP32;                           \
    if ((a).g.D == 128) {                                                       \
      if (dense) { if (g32_) L<128, true, float>(a, s); else L<128, true, uint16_t>(a, s); } \
      else { if (g32_) L<128, false, float>(a, s); else L<128, false, uint16_t>(a, s); }    \
    } else {                                                                    \
      if (dense) { if (g32_) L<64, true, float>(a, s); else L<64, true, uint16_t>(a, s); }   \
      else { if (g32_) L<64, false, float>(a, s); else L<64, false, uint16_t>(a, s); }      \
    }                                                                           \
  } while (0)

#define VMOBA_DISPATCH_F32(L, a, s, dense)                                       \
  do {                                                                          \
    if ((a).g.D == 128) { if (dense) L<128, true>(a, s); else L<128, false>(a, s); } \
    else { if (dense) L<64, true>(a, s); else L<64, false>(a, s); }             \
  } while (0)

static AttnParams bwd_params(const Geom& g, const void* q, const void* k, const void* v,
                             const float* lse, const float* delta, const void* dout) {
  AttnParams a{};
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = const_cast<float*>(lse);
  a.delta = const_cast<float*>(delta);
  a.scale = 1.0f / sqrtf(float(g.D));
  a.scale_log2 = kLog2e * a.scale;
  return a;
}

int launch_bwd_delta(const Geom& g, const void* o, const void* dout, float* delta,
                     void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.dtype == VMOBA_BF16) {
    if (g.D == 128) launch_delta<uint16_t, 128>(g, o, dout, delta, s);
    else launch_delta<uint16_t, 64>(g, o, dout, delta, s);
  } else {
    if (g.D == 128) launch_delta<float, 128>(g, o, dout, delta, s);
    else launch_delta<float, 64>(g, o, dout, delta, s);
  }
  return launch_status();
}

int launch_bwd_dkdv(const Geom& g, bool dense, const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dout,
                    const int32_t* col_ptr, const int32_t* row_idx, void* dk, void* dv,
                    void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams a = bwd_params(g, q, k, v, lse, delta, dout);
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.dk = dk;
  a.dv = dv;
  if (g.dtype == VMOBA_BF16) VMOBA_DISPATCH_BF16(launch_dkdv_bf16, a, s, dense);
  else VMOBA_DISPATCH_F32(launch_dkdv_f32, a, s, dense);
  return launch_status();
}

int launch_bwd_dq(const Geom& g, bool dense, const void* q, const void* k, const void* v,
                  const float* lse, const float* delta, const void* dout,
                  const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams a = bwd_params(g, q, k, v, lse, delta, dout);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.dq = dq;
  if (g.dtype == VMOBA_BF16) VMOBA_DISPATCH_BF16(launch_dq_bf16, a, s, dense);
  else VMOBA_DISPATCH_F32(launch_dq_f32, a, s, dense);
  return launch_status();
}

// dK/dV and dQ side by side: dQ on a second stream of the device, forked from `stream`
// after what is already queued there (delta) and joined back into it.  The two kernels
// read the same inputs and write disjoint outputs; each fills one workgroup a CU, so
// running them together lets the second fill the CUs the first leaves idle at its tail.
// The second stream is made once per host thread and device (default priority) and kept
// until the process ends: a stream shared between threads would take one thread's work
// into another thread's graph capture while that capture runs.  It is not made while
// `stream` is being captured.  The fork and join events are made and released per call.
// Without a second stream the two run one after the other on `stream`.
namespace {
constexpr int kMaxSideDevices = 64;
thread_local hipStream_t t_side[kMaxSideDevices] = {};

// create: whether a missing stream may be made now (not while `stream` is being captured)
hipStream_t side_stream(int dev, bool create) {
  if (dev < 0 || dev >= kMaxSideDevices) return nullptr;
  if (!t_side[dev] && create) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    hipStream_t s = nullptr;
    const hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return nullptr;
    t_side[dev] = s;
  }
  return t_side[dev];
}
}  // namespace

int launch_bwd_dkdv_dq(const Geom& g, const void* q, const void* k, const void* v,
                       const float* lse, const float* delta, const void* dout,
                       const int32_t* row_ptr, const int32_t* col_idx,
                       const int32_t* col_ptr, const int32_t* row_idx, void* dq, void* dk,
                       void* dv, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  const bool have_dev =
      s ? hipStreamGetDevice(s, &dev) == hipSuccess : hipGetDevice(&dev) == hipSuccess;
  // (the null stream is never captured; asking about it could fail while another stream
  // is captured, and leave that error for the launch checks below)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const bool capturing =
      s && (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone);
  hipStream_t side = have_dev ? side_stream(dev, !capturing) : nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  if (side && (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess ||
               hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess)) {
    if (fork) (void)hipEventDestroy(fork);
    side = nullptr;
  }
  if (!side) {
    int st = launch_bwd_dkdv(g, false, q, k, v, lse, delta, dout, col_ptr, row_idx, dk, dv,
                             stream);
    if (st) return st;
    return launch_bwd_dq(g, false, q, k, v, lse, delta, dout, row_ptr, col_idx, dq, stream);
  }
  int st = VMOBA_OK;
  if (hipEventRecord(fork, s) != hipSuccess || hipStreamWaitEvent(side, fork, 0) != hipSuccess)
    st = VMOBA_ERR_HIP;
  if (!st)
    st = launch_bwd_dkdv(g, false, q, k, v, lse, delta, dout, col_ptr, row_idx, dk, dv,
                         stream);
  if (!st) st = launch_bwd_dq(g, false, q, k, v, lse, delta, dout, row_ptr, col_idx, dq, side);
  // the join is recorded even after a failed launch, so that `stream` never runs ahead of
  // work queued on the second stream
  if (hipEventRecord(join, side) != hipSuccess || hipStreamWaitEvent(s, join, 0) != hipSuccess)
    st = st ? st : VMOBA_ERR_HIP;
  (void)hipEventDestroy(fork);
  (void)hipEventDestroy(join);
  return st;
}

// Token-granular selection: dK/dV over the column lists under the key-block mask, dQ over
// the row lists under the list-position mask (bf16 only).
int launch_token_bwd_dkdv(const Geom& g, const void* q, const void* k, const void* v,
                          const float* lse, const float* delta, const void* dout,
                          const int32_t* col_ptr, const int32_t* row_idx,
                          const uint32_t* tokmask, void* dk, void* dv, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams a = bwd_params(g, q, k, v, lse, delta, dout);
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.tokmask = tokmask;
  a.mwords = (g.Nb + 31) / 32;
  a.dk = dk;
  a.dv = dv;
  const bool g32 = g.grad_dtype == VMOBA_FP32;
  if (g.D == 128) {
    if (g32) launch_dkdv_bf16<128, false, float, true>(a, s);
    else launch_dkdv_bf16<128, false, uint16_t, true>(a, s);
  } else {
    if (g32) launch_dkdv_bf16<64, false, float, true>(a, s);
    else launch_dkdv_bf16<64, false, uint16_t, true>(a, s);
  }
  return launch_status();
}

int launch_token_bwd_dq(const Geom& g, const void* q, const void* k, const void* v,
                        const float* lse, const float* delta, const void* dout,
                        const int32_t* row_ptr, const int32_t* col_idx,
                        const uint32_t* posmask, void* dq, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  AttnParams a = bwd_params(g, q, k, v, lse, delta, dout);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.posmask = posmask;
  a.mwords = (g.Nb + 31) / 32;
  a.dq = dq;
  const bool g32 = g.grad_dtype == VMOBA_FP32;
  if (g.D == 128) {
    if (g32) launch_dq_bf16<128, false, float, true>(a, s);
    else launch_dq_bf16<128, false, uint16_t, true>(a, s);
  } else {
    if (g32) launch_dq_bf16<64, false, float, true>(a, s);
    else launch_dq_bf16<64, false, uint16_t, true>(a, s);
  }
  return launch_status();
}

}  // namespace vmoba
