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

// TOK: token-granular selection, the keys of list position li kept only where bit li of
// the query token's position-mask row is set.
template <int D, int NW, int KSUB, int NS, bool DENSE, bool TAB, bool TOK = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(AttnParams a) {
  constexpr int NT = NW * 64;
  constexpr int QT = NW * 32;
  constexpr int KT = KSUB * 32;
  constexpr int ROWB = D * 2;                // bytes per tile row
  constexpr int RPI = 1024 / ROWB;           // tile rows per wave load instruction
  constexpr int LPW = KT / (NW * RPI);       // load instructions per wave per tensor
  static_assert(KT % (NW * RPI) == 0, "tile rows split over waves");
  static_assert(NS >= 2 && NS <= 4, "stages");
  constexpr int TILE = KT * ROWB;            // bytes of one K or V tile
  // lazy rescale: keep the running max until a score exceeds it by 2^8 in exp2 units
  constexpr float kRescaleLog2 = 8.0f;

  // Pipeline stages as separate objects, so that the compiler can tell that reading one
  // stage does not depend on the direct-to-LDS loads in flight into another.
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[NS > 2 ? 2 * TILE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[NS > 3 ? 2 * TILE : 16];
  __shared__ int32_t cols[DENSE ? 1 : kMaxBlocks];        // base token of listed blocks
  __shared__ int32_t offtab[TAB ? kOffsetTable : 1];      // block_offset(r), r < S
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
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.out);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * g.D) * 2u;   // < 2^32 (validated)
  const BufRes rK = buffer_res(K, tbytes), rV = buffer_res(V, tbytes);

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
    if (kept == 0 && tid == 0) cols[0] = 0;   // token 0: loads of an empty stream
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
  // A wave whose 32 queries all lie past the block's end (the ragged last query tile)
  // only takes its share of the loads and the barriers: skipping the arithmetic leaves
  // its SIMD's matrix core to the other workgroup's wave.
  const bool wave_busy = qt * QT + w * 32 < qlim;
  const int rqc = qvalid ? rq : 0;
  const int32_t xq = DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  const int32_t qoff = row_offset(g, grp, xq);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + qoff + s * 16 + half * 8));
  PosMask pm;
  if constexpr (TOK) pm.init(a.posmask + (size_t(grp) * g.L + xq) * a.mwords, a.mwords);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // LDS read offsets of this lane (sub-tile and k-step add immediates)
  const int grp16 = lane >> 4, sl = lane & 15;
  const int krow = l32 * ROWB, kswz = swz<D>(l32) ^ half;
  const int vkey0 = 4 * half + (sl >> 2);
  const int vc0 = 2 * (grp16 & 1) + ((sl & 3) >> 1);
  const int vbase_lo = TILE + vkey0 * ROWB + (sl & 1) * 8;
  const int vsw_lo = swz<D>(vkey0), vsw_hi = swz<D>(vkey0 + 8);

  // loader: this lane fetches chunk (lane % CPR) ^ swz(row) of rows lrow0 + i*RPI of the
  // tile.  Row addresses are computed first, without divergent branches, and the loads
  // issued back to back afterwards: a branch join between one row's load and the next
  // row's address arithmetic would make the compiler wait for the load in flight.
  // Positions past the stream's end repeat its last token (an empty stream reads token
  // 0), so every tile, also one past the end, is a valid load and the pipeline issues
  // one tile per step unconditionally.
  constexpr int CPR = D / 8;
  const int lrow0 = w * (KT / NW) + lane / CPR;
  const int lcp = lane % CPR;
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nkeys - 1, 0);
  // element offsets (shared by K and V) of this lane's rows of tile t
  auto tile_offsets = [&](int t, int32_t (&o)[LPW]) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int p = min(t * KT + lrow0 + i * RPI, plast);
      int32_t x = p;
      if constexpr (!DENSE) {
        const uint32_t pb = fd_div(uint32_t(p), g.div_S);
        const uint32_t rr = uint32_t(p) - pb * uint32_t(g.S);
        x = cols[pb] + (TAB ? offtab[rr] : block_offset(g, rr));
      }
      o[i] = gbase + x * hstride + (lcp ^ swz<D>(lrow0 + i * RPI)) * 8;
    }
  };
  auto issue_offsets = [&](const int32_t (&o)[LPW], unsigned char* smem) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int dst = (w * (KT / NW) + i * RPI) * ROWB;   // wave-uniform
      load_to_lds16(rK, 2u * uint32_t(o[i]), smem + dst);
      load_to_lds16(rV, 2u * uint32_t(o[i]), smem + TILE + dst);
    }
  };
  auto issue_tile = [&](int t, unsigned char* smem) {
    int32_t o[LPW];
    tile_offsets(t, o);
    issue_offsets(o, smem);
  };

  const float c2 = a.scale_log2;
  const float thr = kRescaleLog2 / c2;

  // K fragments of a tile (A operand of S^T = K Q^T): chunk 2s + half of row l32 sits at
  // chunk position (2s) ^ swz(l32) ^ half
  auto load_k = [&](const unsigned char* smem, bf16x8 (&kf)[KSUB][D / 16]) {
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        kf[kt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            smem + kt * 32 * ROWB + krow + 16 * ((2 * s) ^ kswz)));
  };
  auto scores = [&](const bf16x8 (&kf)[KSUB][D / 16], f32x16 (&acc)[KSUB]) {
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[kt][v] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt][s], qf[s], acc[kt], 0, 0, 0);
    }
  };
  // keys of the ragged last tile past the stream's end score -inf
  auto mask_tail = [&](f32x16 (&acc)[KSUB], int t) {
    if (t * KT + KT > nkeys) {
#pragma unroll
      for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t * KT + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (key >= nkeys) acc[kt][v] = -INFINITY;
        }
    }
  };
  // token-granular selection: keys of list positions this lane's query did not select
  auto mask_tokens = [&](f32x16 (&acc)[KSUB], int t) {
    if constexpr (TOK) {
      const uint32_t p0 = uint32_t(t * KT);
      const int li0 = int(fd_div(p0, g.div_S));
      pm.fetch(li0);
      if (g.S >= KT) {
        // the tile spans list positions li0 (offsets below bnd) and li0 + 1 only: two
        // mask bits a tile, and one compare a key against the boundary
        const bool b0 = pm.keep(li0), b1 = pm.keep(li0 + 1);
        const int bh = (li0 + 1) * g.S - t * KT - 4 * half;   // from this lane's first key
#pragma unroll
        for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const bool kp = (kt * 32 + 8 * (v >> 2) + (v & 3)) < bh ? b0 : b1;
            if (!kp) acc[kt][v] = -INFINITY;
          }
      } else {
        uint32_t pb = p0 + 4 * half;   // opaque, so the per-key offsets are not hoisted
        asm volatile("" : "+v"(pb));
#pragma unroll
        for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t p = pb + (kt * 32 + 8 * (v >> 2) + (v & 3));
            if (!pm.keep(int(fd_div(p, g.div_S)))) acc[kt][v] = -INFINITY;
          }
      }
    }
  };
  // max over this lane's own 16*KSUB scores of the tile (lane l ^ 32 holds the other keys
  // of the same query)
  auto tile_max = [&](const f32x16 (&acc)[KSUB]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KSUB; ++kt)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = max3f(mx, acc[kt][v], acc[kt][v + 1]);
    return mx;
  };
  // lazy rescale: keep the running max unless the tile's max exceeds it by the margin
  // (every lane on the first tile, rarely afterwards).  The query's max exceeds the margin
  // exactly when one of its two lanes' maxima does; the two are combined only here.
  auto maybe_rescale = [&](float mx) {
    if (__ballot(mx > m_run + thr)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const bool grow = mx > m_run + thr;
      const float m_new = grow ? mx : m_run;
      // (with token masks a lane that has seen only masked keys keeps m = -inf, and
      // -inf - -inf would make its alpha NaN)
      const float alpha = (TOK && !grow) ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
      m_run = m_new;
    }
  };
  // P = exp2(S c2 - m c2), summed into l and packed to bf16 pairs (B operand of O^T += V^T P^T)
  auto softmax_pack = [&](const f32x16 (&acc)[KSUB], u32x4 (&pw)[2 * KSUB]) {
    // (with token masks a query may have seen only masked keys so far: m = -inf, P = 0)
    const float moff = (TOK && m_run == -INFINITY) ? 0.f : m_run * c2;
    // the row sum takes the same bf16 P as the product with V, two at a time
    float psum = l_run;
#pragma unroll
    for (int ks = 0; ks < 2 * KSUB; ++ks) {
      const int kt = ks >> 1, g0 = (ks & 1) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(acc[kt][g0 + 2 * e], c2, -moff));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(acc[kt][g0 + 2 * e + 1], c2, -moff));
        pw[ks][e] = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(pw[ks][e], psum);
      }
    }
    l_run = psum;
  };
  // O^T += V^T P^T, 16 keys per step; V^T fragments by transposing reads
  auto pv_update = [&](const unsigned char* smem, const u32x4 (&pw)[2 * KSUB]) {
#pragma unroll
    for (int ks = 0; ks < 2 * KSUB; ++ks) {
      const bf16x8 pb = as_bf16x8(pw[ks]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int c = dt * 4 + vc0;
        const u32x2 lo = lds_read_tr16(smem + ks * 16 * ROWB + vbase_lo + 16 * (c ^ vsw_lo));
        const u32x2 hi = lds_read_tr16(smem + ks * 16 * ROWB + vbase_lo + 8 * ROWB +
                                       16 * (c ^ vsw_hi));
        const bf16x8 va = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
      }
    }
  };

  // Software pipeline over key tiles.  Tile t sits in stage t % NS; tiles up to t + NS - 2
  // are in flight.  Step t: wait for tile t+1, barrier, refill the stage of tile t-1 with
  // tile t+NS-1 (its addresses were computed one step earlier), then compute S(t+1) on the matrix cores while the vector unit turns S(t)
  // into P(t), and finish with O += P(t) V(t).  S(t) itself was computed in step t-1.
  static_assert(NS == 4, "the step loop is unrolled over four stages");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int32_t noff[LPW];   // offsets of the tile the next step loads
  auto step = [&](auto STc, int t, f32x16 (&cur)[KSUB], f32x16 (&nxt)[KSUB]) {
    constexpr int ST = decltype(STc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_lds<(NS - 3) * 2 * LPW>();   // this wave's loads of tile t+1 have landed
    pipeline_barrier();
    issue_offsets(noff, stage(std::integral_constant<int, ST + NS - 1>{}));
    tile_offsets(t + NS, noff);   // the next step's loads; the lookups finish meanwhile
    if (wave_busy) {
      bf16x8 kf[KSUB][D / 16];
      load_k(stage(std::integral_constant<int, ST + 1>{}), kf);
      mask_tail(cur, t);
      mask_tokens(cur, t);
      maybe_rescale(tile_max(cur));
      u32x4 pw[2 * KSUB];
      scores(kf, nxt);
      softmax_pack(cur, pw);
      pv_update(stage(STc), pw);
    }
  };

  // prologue: tiles 0 .. NS-2 in flight, S(0)
  issue_tile(0, stage0);
  issue_tile(1, stage1);
  issue_tile(2, stage2);
  tile_offsets(NS - 1, noff);
  f32x16 sa[KSUB], sb[KSUB];
  wait_vmcnt_lds<(NS - 2) * 2 * LPW>();
  pipeline_barrier();
  if (wave_busy) {
    bf16x8 kf[KSUB][D / 16];
    load_k(stage0, kf);
    scores(kf, sa);
  }
  int t = 0;
  for (; t + NS <= ntiles; t += NS) {
    step(I0{}, t, sa, sb);
    step(I1{}, t + 1, sb, sa);
    step(I2{}, t + 2, sa, sb);
    step(I3{}, t + 3, sb, sa);
  }
  if (t < ntiles) step(I0{}, t, sa, sb);
  if (t + 1 < ntiles) step(I1{}, t + 1, sb, sa);
  if (t + 2 < ntiles) step(I2{}, t + 2, sa, sb);

  // finalise; the loads of the tiles past the end must land before the workgroup's LDS
  // is released
  wait_vmcnt_lds<0>();
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = nkeys == 0 || (TOK && !(l_tot > 0.f));
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

// ---------------------------------------------------------------------------------
// d = 128 on v_mfma_f32_16x16x32_bf16: each wave owns M sub-tiles of 16 queries, so a
// workgroup covers 64*M queries (a whole 192-token block at M = 3).  Every K and V^T
// fragment read from LDS feeds M products, and each staged K/V tile serves 64*M queries,
// which cuts both the LDS reads per pair and the tile loads per query against 32 queries
// per wave.
//
// Per 32-key tile and wave: S^T = K Q^T as 2 key sub-tiles x M query sub-tiles x 4 d-steps
// (A = K rows from LDS, B = this wave's Q columns in registers); the accumulator gives lane
// l the query l % 16 of each sub-tile and keys 4*(l/16) + 0..3 of each key sub-tile.  The
// row max reduces over the lane's 8 values and then over the four 16-lane groups (two
// permlane swaps).  P stays in registers as the B operand of O^T += V^T P^T with its k order
// permuted to the accumulator layout (k position 8g + e is key 4g + e for e < 4 and
// 16 + 4g + e - 4 otherwise); the V^T operand comes from two transposing reads that follow
// the same permutation.
//
// LDS tiles: row r holds one token (256 bytes, 16 chunks of 16 bytes).  K chunk c of row r
// sits at position c ^ (r & 15), so the 16 rows of a K fragment read hit 16 different bank
// groups; V chunk c of row r sits at c ^ 2 (r & 7), so the 8 rows x 32 bytes of a
// half-wave's transposing read cover all 64 banks.
template <int M, int NS, bool DENSE, bool TAB, bool ALN = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd16_bf16_kernel(AttnParams a) {
  constexpr int D = 128, NW = 4, NT = 256;
  constexpr int QW = 16 * M;                 // queries per wave
  constexpr int QT = NW * QW;                // queries per workgroup
  constexpr int KT = 32;                     // keys per tile
  constexpr int ROWB = D * 2;
  constexpr int TILE = KT * ROWB;            // bytes of one K or V tile
  constexpr int LPW = KT / (NW * 4);         // load instructions per wave per tensor
  static_assert(NS == 4, "the step loop is unrolled over four stages");
  constexpr float kRescaleLog2 = 8.0f;

  // one __shared__ object per stage: the compiler tells direct-to-LDS loads apart from LDS
  // reads only by object, so with one array for all stages it would make every step wait
  // for all loads in flight (vmcnt(0)) before its first LDS read
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[2 * TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[2 * TILE];
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
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.out);
  const uint32_t tbytes = uint32_t(g.B * g.L * g.Hh * g.D) * 2u;   // < 2^32 (validated)
  const BufRes rK = buffer_res(K, tbytes), rV = buffer_res(V, tbytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // w, known to be wave-uniform
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
    // base in cols), so a tile's row offsets are one addition
    const int32_t hs = ALN ? g.Hh * D : 1, gb = ALN ? row_offset(g, grp, 0) : 0;
    for (int i = tid; i < kept; i += NT) cols[i] = gb + block_base(g, uint32_t(cols[i])) * hs;
    if (kept == 0 && tid == 0) cols[0] = gb;   // token 0: loads of an empty stream
    if constexpr (TAB)
      for (int r = tid; r < g.S; r += NT) offtab[r] = block_offset(g, uint32_t(r)) * hs;
    __syncthreads();
    nkeys = kept * g.S;
  }
  const int ntiles = __builtin_amdgcn_readfirstlane((nkeys + KT - 1) / KT);

  // this lane's query in each sub-tile; Q fragments (B operands) in registers
  const int qlim = DENSE ? g.L : g.S;
  const int qbase = qt * QT + w * QW;
  const bool wave_busy = qbase < qlim;   // otherwise: loads and barriers only
  auto query_token = [&](int m) -> int32_t {   // token of this lane's query in sub-tile m
    const int rq = qbase + m * 16 + i16;
    const int rqc = rq < qlim ? rq : 0;
    return DENSE ? rqc : block_base(g, iblk) + block_offset(g, rqc);
  };
  bf16x8 qf[M][D / 32];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int32_t qoff = row_offset(g, grp, query_token(m));
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[m][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(Q + qoff + s * 32 + g16 * 8));
  }

  f32x4 oacc[M][D / 16];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) oacc[m][ds] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max, and derived from it (updated only when it moves): the rescale
  // threshold m + thr and the exponent offset m * c2
  float m_run[M], l_run[M], m_thr[M], m_off[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    m_run[m] = -INFINITY;
    l_run[m] = 0.f;
    m_thr[m] = -INFINITY;
    m_off[m] = -INFINITY;
  }

  // loader: one instruction moves 4 rows; lane L fills row L/16 at chunk position L % 16
  const int32_t hstride = g.Hh * D;
  const int32_t gbase = row_offset(g, grp, 0);
  const int plast = max(nkeys - 1, 0);
  int kchunk[LPW], vchunk[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = w * (KT / NW) + i * 4 + g16;
    kchunk[i] = (i16 ^ (r & 15)) * 8;
    vchunk[i] = (i16 ^ (2 * (r & 7))) * 8;
  }
  // ALN (blocks a multiple of the tile): tile t lies in one list entry, at rows
  // aln_rr.. of it; the entry and row advance by one tile a call (calls come in tile
  // order) and stop at the last tile, which the tiles past the end repeat
  int aln_pb = 0, aln_rr = 0;
  const int aln_row = w * (KT / NW) + g16;   // this lane's row of the tile, first load
  auto tile_offsets = [&](int t, int32_t (&o)[LPW]) {
    if constexpr (ALN) {
      const int32_t cb = cols[aln_pb];
#pragma unroll
      for (int i = 0; i < LPW; ++i) o[i] = cb + offtab[aln_rr + aln_row + i * 4];
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
      const int p = min(t * KT + w * (KT / NW) + i * 4 + g16, plast);
      int32_t x = p;
      if constexpr (!DENSE) {
        const uint32_t pb = fd_div(uint32_t(p), g.div_S);
        const uint32_t rr = uint32_t(p) - pb * uint32_t(g.S);
        x = cols[pb] + (TAB ? offtab[rr] : block_offset(g, rr));
      }
      o[i] = gbase + x * hstride;
    }
  };
  auto issue_offsets = [&](const int32_t (&o)[LPW], unsigned char* smem) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int dst = (wu * (KT / NW) + i * 4) * ROWB;   // wave-uniform
      load_to_lds16(rK, 2u * uint32_t(o[i] + kchunk[i]), smem + dst);
      load_to_lds16(rV, 2u * uint32_t(o[i] + vchunk[i]), smem + TILE + dst);
    }
  };
  auto issue_tile = [&](int t, unsigned char* smem) {
    int32_t o[LPW];
    tile_offsets(t, o);
    issue_offsets(o, smem);
  };

  // LDS read offsets: K fragment (key sub-tile ks, d-step s) of lane l is row ks*16 + l%16,
  // chunk 4s + l/16; the V^T reads of lane l name row 4*(l/16) + (l%16)/4 (+16 for keys
  // 16..31) and the 8 bytes at d = 16 dsub + 4 (l % 4)
  const int krd = i16 * ROWB;
  const int vrow = 4 * g16 + (i16 >> 2);
  const int vrd = TILE + vrow * ROWB + 8 * (i16 & 1);
  const int vsw = 2 * (vrow & 7);
  const int vc = (i16 & 3) >> 1;

  // per-lane LDS offsets inside a stage, formed once: K fragment of d-step s (key sub-tile
  // 0; sub-tile 1 is 16 rows further), V^T read of d-tile ds (keys 0..15; +16 rows for keys
  // 16..31).  The stage and sub-tile parts are constants of each unrolled step.
  int koff[D / 32], voff[D / 16];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) koff[s] = krd + 16 * ((4 * s + g16) ^ i16);
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) voff[ds] = vrd + 16 * ((2 * ds + vc) ^ vsw);

  const float c2 = a.scale_log2;
  const float thr = kRescaleLog2 / c2;

  auto compute = [&](const unsigned char* sm, int t) {
    f32x4 sacc[2][M];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < M; ++m) sacc[ks][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the K fragments of one 16-key sub-tile at a time, read ahead of its products (the
    // second sub-tile's reads overlap the first one's products)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 ka[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        ka[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(sm + ks * 16 * ROWB + koff[s]));
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int m = 0; m < M; ++m)
          sacc[ks][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qf[m][s], sacc[ks][m],
                                                                0, 0, 0);
    }
    // V^T fragments, read here so that their latency hides behind the softmax
    bf16x8 va[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const u32x2 lo = lds_read_tr16(sm + voff[ds]);
      const u32x2 hi = lds_read_tr16(sm + 16 * ROWB + voff[ds]);
      va[ds] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    if (!ALN && t * KT + KT > nkeys) {   // ragged last tile: keys past the end score -inf
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t * KT + ks * 16 + 4 * g16 + i >= nkeys) {
#pragma unroll
            for (int m = 0; m < M; ++m) sacc[ks][m][i] = -INFINITY;
          }
    }
    // per query: max over the lane's 8 scores, then over the four 16-lane groups.  A row's
    // max exceeds m_run + thr exactly when one of its four lanes' maxima does, so the sparse
    // kernels test the lanes' own maxima and exchange them only to rescale (the dense one
    // exchanges them first: deferred, its registers spill inside the loop)
    auto row_max = [&](float v) __attribute__((always_inline)) {
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
      v = __builtin_elementwise_maximum(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
      return __builtin_elementwise_maximum(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    };
    float mx[M];
    bool any = false;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = max3f(sacc[0][m][0], sacc[0][m][1], sacc[0][m][2]);
      v = max3f(v, sacc[0][m][3], sacc[1][m][0]);
      v = max3f(v, sacc[1][m][1], sacc[1][m][2]);
      v = __builtin_elementwise_maximum(v, sacc[1][m][3]);
      mx[m] = DENSE ? row_max(v) : v;
      any |= mx[m] > m_thr[m];
    }
    // lazy rescale (wave-uniform): every sub-tile on the first tile, rarely afterwards
    if (__ballot(any)) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = DENSE ? mx[m] : row_max(mx[m]);
        const float m_new = v > m_thr[m] ? v : m_run[m];
        const float alpha = __builtin_amdgcn_exp2f((m_run[m] - m_new) * c2);
        l_run[m] *= alpha;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) oacc[m][ds] *= alpha;
        m_run[m] = m_new;
        m_thr[m] = m_new + thr;
        m_off[m] = m_new * c2;
      }
    }
    // P = exp2(S c2 - m c2), packed in the permuted k order
    u32x4 pw[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float moff = m_off[m];
      float p[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p[ks][i] = __builtin_amdgcn_exp2f(fmaf(sacc[ks][m][i], c2, -moff));
      pw[m] = u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
      // the sparse kernels' row sum takes the same bf16 P as the product with V, two at a
      // time (the dense one sums the fp32 P: with the dot products its registers spill)
      if constexpr (DENSE) {
        l_run[m] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                    ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      } else {
        float l = l_run[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) l = sum_bf16x2(pw[m][j], l);
        l_run[m] = l;
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int m = 0; m < M; ++m)
        oacc[m][ds] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ds], as_bf16x8(pw[m]),
                                                              oacc[m][ds], 0, 0, 0);
  };

  // pipeline: tile t in stage t % 4, tiles t+1, t+2 in flight while t is computed
  int32_t noff[LPW];
  auto step = [&](auto STc, int t) {
    constexpr int ST = decltype(STc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_lds<(NS - 2) * 2 * LPW>();   // this wave's loads of tile t have landed
    pipeline_barrier();
    issue_offsets(noff, stage(std::integral_constant<int, ST + NS - 1>{}));
    tile_offsets(t + NS, noff);
    if (wave_busy) compute(stage(STc), t);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  issue_tile(0, stage(std::integral_constant<int, 0>{}));
  issue_tile(1, stage(std::integral_constant<int, 1>{}));
  issue_tile(2, stage(std::integral_constant<int, 2>{}));
  tile_offsets(NS - 1, noff);
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
  // the loads of the tiles past the end must land before the LDS is released
  wait_vmcnt_lds<0>();

  // finalise: row sums over the four lane groups, O / l in natural token order, LSE
  const bool empty = nkeys == 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float l = l_run[m];
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l),
                                                      false, false);
    l = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                      false, false);
    l = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    const float inv = empty ? 0.f : 1.0f / l;
    if (qbase + m * 16 + i16 < qlim) {
      const int32_t xq = query_token(m);
      const int32_t qoff = row_offset(g, grp, xq);
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        u32x2 out;
        out[0] = pack_bf16x2(oacc[m][ds][0] * inv, oacc[m][ds][1] * inv);
        out[1] = pack_bf16x2(oacc[m][ds][2] * inv, oacc[m][ds][3] * inv);
        *reinterpret_cast<u32x2*>(O + qoff + ds * 16 + 4 * g16) = out;
      }
      if (g16 == 0)
        a.lse[size_t(grp) * g.L + xq] = empty ? -INFINITY : m_run[m] * a.scale + logf(l);
    }
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

template <int D, int NW, int KSUB, int NS, bool DENSE, bool TOK = false>
static void launch_fwd_bf16(AttnParams& a, hipStream_t s) {
  const Geom& g = a.g;
  const int qlim = DENSE ? g.L : g.S;
  a.tiles = (qlim + NW * 32 - 1) / (NW * 32);
  const int rows = DENSE ? 1 : g.Nb;
  const int grid = launch_grid<DENSE>(a, rows);
  if (!DENSE && g.S <= kOffsetTable)
    attn_fwd_bf16_kernel<D, NW, KSUB, NS, DENSE, !DENSE, TOK><<<grid, NW * 64, 0, s>>>(a);
  else
    attn_fwd_bf16_kernel<D, NW, KSUB, NS, DENSE, false, TOK><<<grid, NW * 64, 0, s>>>(a);
}

template <int M, bool DENSE>
static void launch_fwd16_bf16(AttnParams& a, hipStream_t s) {
  const Geom& g = a.g;
  const int qlim = DENSE ? g.L : g.S;
  a.tiles = (qlim + 64 * M - 1) / (64 * M);
  const int rows = DENSE ? 1 : g.Nb;
  const int grid = launch_grid<DENSE>(a, rows);
  if (!DENSE && g.S <= kOffsetTable && g.S % 32 == 0)
    attn_fwd16_bf16_kernel<M, 4, DENSE, !DENSE, !DENSE><<<grid, 256, 0, s>>>(a);
  else if (!DENSE && g.S <= kOffsetTable)
    attn_fwd16_bf16_kernel<M, 4, DENSE, !DENSE><<<grid, 256, 0, s>>>(a);
  else
    attn_fwd16_bf16_kernel<M, 4, DENSE, false><<<grid, 256, 0, s>>>(a);
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
    // 32-key tiles, 4 stages: three tiles of loads in flight behind the one in use
    if (g.D == 128) {
      // 48 queries per wave when 192-query tiles pad no more than 128-query ones
      const int qlim = dense ? g.L : g.S;
      const bool m3 = (qlim + 191) / 192 * 192 <= (qlim + 127) / 128 * 128;
      if (m3) {
        if (dense) launch_fwd16_bf16<3, true>(a, s);
        else launch_fwd16_bf16<3, false>(a, s);
      } else if (dense) {
        launch_fwd_bf16<128, 4, 1, 4, true>(a, s);
      } else if (qlim > 128 && qlim <= 256) {
        // blocks of 193-256 tokens: eight waves, one workgroup a block, so the block's
        // key list is streamed once instead of by two workgroups (216-token blocks: 3-5 %)
        launch_fwd_bf16<128, 8, 1, 4, false>(a, s);
      } else {
        launch_fwd_bf16<128, 4, 1, 4, false>(a, s);
      }
    } else {
      if (dense) launch_fwd_bf16<64, 4, 2, 4, true>(a, s);
      else launch_fwd_bf16<64, 4, 2, 4, false>(a, s);
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

// Token-granular selection: the list-position mask of every query token from its key-block
// mask and its block's list (entries outside [0, N_b) skipped, as the attention kernels
// skip them).  One wave per token; bits are gathered in LDS, then written as whole words.
__global__ __launch_bounds__(256) void token_posmask_kernel(Geom g, const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col_idx,
                                                            const uint32_t* __restrict__ tokmask,
                                                            uint32_t* __restrict__ posmask) {
  __shared__ uint32_t words[4][kMaxBlocks / 32];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = blockIdx.y;
  const int x = blockIdx.x * 4 + w;
  const int W = (g.Nb + 31) / 32;
  for (int i = lane; i < W; i += 64) words[w][i] = 0u;
  __syncthreads();
  if (x < g.L) {
    const int blk = token_block(g, x);
    int start, len;
    list_range(g, row_ptr, grp, blk, &start, &len);
    const int32_t* lst = col_idx + size_t(grp) * g.Nb * g.Nb + start;
    const uint32_t* tm = tokmask + (size_t(grp) * g.L + x) * W;
    int pos = 0;
    for (int base = 0; base < len; base += 64) {
      const int i = base + lane;
      const int32_t j = i < len ? lst[i] : -1;
      const bool ok = j >= 0 && j < g.Nb;
      const unsigned long long vm = __ballot(ok);
      const int li = pos + __popcll(vm & ((1ull << lane) - 1ull));
      if (ok && ((tm[j >> 5] >> (j & 31)) & 1u)) atomicOr(&words[w][li >> 5], 1u << (li & 31));
      pos += __popcll(vm);
    }
  }
  __syncthreads();
  if (x < g.L) {
    uint32_t* dst = posmask + (size_t(grp) * g.L + x) * W;
    for (int i = lane; i < W; i += 64) dst[i] = words[w][i];
  }
}

int launch_token_posmask(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx,
                         const uint32_t* tokmask, uint32_t* posmask, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((g.L + 3) / 4, g.B * g.Hh);
  token_posmask_kernel<<<grid, 256, 0, s>>>(g, row_ptr, col_idx, tokmask, posmask);
  return launch_status();
}

int launch_token_attn_fwd(const Geom& g, const void* q, const void* k, const void* v,
                          const int32_t* row_ptr, const int32_t* col_idx,
                          const uint32_t* posmask, void* o, float* lse, void* stream) {
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
  a.posmask = posmask;
  a.mwords = (g.Nb + 31) / 32;
  a.scale = 1.0f / sqrtf(float(g.D));
  a.scale_log2 = kLog2e * a.scale;
  if (g.D == 128) launch_fwd_bf16<128, 4, 1, 4, false, true>(a, s);
  else launch_fwd_bf16<64, 4, 2, 4, false, true>(a, s);
  return launch_status();
}

}  // namespace vmoba
