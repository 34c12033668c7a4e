// Block selection with the cumulative-mass threshold (papernotes 关键设计 2 and 3;
// paperlayer §3.3-§3.4) and the other strategies of the ablation.
//
// Scores: block_scores_kernel computes s_ij = <Qbar_i, Kbar_j> / sqrt(d) for one 32 x 32
// tile of one head group per wave, on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), so
// the products and sums keep fp32 precision; the selection compares masses near tau.
//
// Global strategies (threshold + global, the method's; top-k + global): the N_b x N_b
// pool of a head group goes through the pool selection further down, spread over many
// workgroups:
//   1. m = max s; each pair's mass e = exp(s - m) is held as a 64-bit fixed-point integer,
//      so every mass sum is exact and independent of summation order.
//   2. The cutoff pair is found without sorting: the fp32 scores are mapped to
//      order-preserving 32-bit keys, and four 8-bit radix passes build per-digit
//      (count, mass) histograms of the still-undecided keys, walking down from the
//      largest digit until the running mass reaches ceil(tau * sum e) (top-k: the
//      running count reaches k).  What remains is the key of the k*-th pair; exact ties at
//      that key are taken in ascending linear index i*N_b + j, as many as needed.
//   3. The prefix plus the diagonal go to a row bitmap (wave ballots in linear order),
//      and emit_lists_kernel turns the bitmap into CSR and CSC (row and column counts, an
//      exclusive scan, an ascending walk per row / column).
// Up to kSingleSelectBlocks blocks, single_select_kernel does all of this in one
// workgroup per head group, in LDS.  The pool passes also select over the token-granular
// pool (query tokens x key blocks).
//
// Local strategies (threshold + local, top-k + local): every query block's row of N_b
// scores is its own pool, normalised by a softmax over the row.  select_local_kernel
// gives each row one wave; a pair is kept iff the fixed-point mass (threshold) or the
// number (top-k) of the row's pairs that precede it in the order (higher score, or the
// same score at a lower key index) is below the target.  Each lane counts that for its
// pairs against the whole row staged in LDS.  The rows go to the bitmap, and
// emit_lists_kernel turns it into CSR and CSC as above.
#include <math.h>

#include <algorithm>

#include "device_common.h"

namespace vmoba {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(64) void block_scores_kernel(int Nb, const float* __restrict__ qp,
                                                          const float* __restrict__ kp,
                                                          float* __restrict__ scores,
                                                          float scale) {
  const int lane = threadIdx.x;
  const int i0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const int grp = blockIdx.z;
  const int half = lane >> 5;
  const int ri = i0 + (lane & 31), rj = j0 + (lane & 31);
  const float* qrow = qp + (size_t(grp) * Nb + min(ri, Nb - 1)) * D + half * (D / 2);
  const float* krow = kp + (size_t(grp) * Nb + min(rj, Nb - 1)) * D + half * (D / 2);
  const bool qok = ri < Nb, kok = rj < Nb;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  // Lane half `half` feeds d in [half*D/2, (half+1)*D/2): A and B use the same d for the
  // same k slot, so the contraction covers every d once.
#pragma unroll 4
  for (int c = 0; c < D / 2; c += 4) {
    float4 a = *reinterpret_cast<const float4*>(qrow + c);
    float4 bb = *reinterpret_cast<const float4*>(krow + c);
    if (!qok) a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!kok) bb = make_float4(0.f, 0.f, 0.f, 0.f);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bb.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bb.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bb.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bb.w, acc, 0, 0, 0);
  }
  // acc[v] holds row i0 + 8*(v/4) + 4*half + v%4, column j0 + lane%32.
  if (rj < Nb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (i < Nb) scores[(size_t(grp) * Nb + i) * Nb + rj] = acc[v] * scale;
    }
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr double kMassUnit = 17592186044416.0;  // 2^44 (a local pool of <= 1024 pairs)

__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t fixed_mass(float s, float m) {
  const float e = expf(s - m);
  return uint64_t(double(e) * kMassUnit + 0.5);
}

// Shared memory of single_select_kernel and emit_lists_kernel.
struct SelShared {
  uint32_t cnt[256];
  unsigned long long mass[256];
  float redf[kSelWaves];
  unsigned long long redu[kSelWaves];
  uint32_t redi[kSelWaves];
  // selection state (written by thread 0)
  float m;
  unsigned long long Z, R, above_mass, tie_mass;
  uint32_t prefix, above_cnt, tie_cnt, take_ties, select_all, tie_seen;
  int32_t row_cnt[kMaxBlocks];
  int32_t col_cnt[kMaxBlocks];
};

// Add (1, mass) to digit `dg` of the histogram for every lane with `match`.  Lanes of a
// wave that share a digit (typical for the leading digit, whose bits hold the sign and
// exponent) are summed first and added by one leader; after four rounds the remaining
// lanes, whose digits are spread out, add directly.
__device__ __forceinline__ void histogram_add(uint32_t* cnt, unsigned long long* hmass,
                                              bool match, uint32_t dg,
                                              unsigned long long mass) {
  const int lane = threadIdx.x & 63;
  unsigned long long active = __ballot(match);
  for (int round = 0; round < 4 && active; ++round) {
    const int leader = __ffsll((long long)active) - 1;
    const uint32_t ldg = __shfl(dg, leader);
    const bool same = match && dg == ldg;
    const unsigned long long smask = __ballot(same);
    const unsigned long long msum = wave_sum_u64(same ? mass : 0ull);
    if (lane == leader) {
      atomicAdd(&cnt[ldg], uint32_t(__popcll(smask)));
      atomicAdd(&hmass[ldg], msum);
    }
    match = match && !same;
    active &= ~smask;
  }
  if (match) {
    atomicAdd(&cnt[dg], 1u);
    atomicAdd(&hmass[dg], mass);
  }
}

__device__ __forceinline__ void histogram_add(SelShared& sh, bool match, uint32_t dg,
                                              unsigned long long mass) {
  histogram_add(sh.cnt, sh.mass, match, dg, mass);
}

__device__ float block_max(float v, SelShared& sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.redf[w] = v;
  __syncthreads();
  float r = sh.redf[0];
  for (int i = 1; i < kSelWaves; ++i) r = fmaxf(r, sh.redf[i]);
  __syncthreads();
  return r;
}

__device__ unsigned long long block_sum_u64(unsigned long long v, SelShared& sh) {
  v = wave_sum_u64(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh.redu[w] = v;
  __syncthreads();
  unsigned long long r = 0;
  for (int i = 0; i < kSelWaves; ++i) r += sh.redu[i];
  __syncthreads();
  return r;
}

// Exclusive scan of one int per thread (thread order); returns the block total in *total.
__device__ int block_excl_scan(int v, SelShared& sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.redi[w] = uint32_t(x);
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    if (i < w) off += int(sh.redi[i]);
    tot += int(sh.redi[i]);
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// The global strategies for small pools (N_b <= kSingleSelectBlocks): one 1024-thread
// workgroup per head group runs the whole decision in LDS: max and total mass, the four
// digit passes, ties in linear order into an LDS pair bitmap, then CSR and CSC.  Below a
// few hundred blocks this beats the pool passes, whose dozen dependent launches cost more
// than the pool itself.
template <bool TOPK>
__global__ __launch_bounds__(kSelThreads) void single_select_kernel(
    int Nb, float tau, int topk, const float* __restrict__ scores, int32_t* __restrict__ row_ptr,
    int32_t* __restrict__ col_idx, int32_t* __restrict__ col_ptr,
    int32_t* __restrict__ row_idx, float* __restrict__ head_stats,
    float* __restrict__ norm_scores) {
  __shared__ SelShared sh;
  extern __shared__ uint32_t bits[];  // N_b*N_b-bit pair bitmap, padded to 64-bit words
  const int grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = Nb * Nb;
  const float* s = scores + size_t(grp) * N;

  // 1. max and total fixed-point mass
  float mx = -INFINITY;
  for (int idx = tid; idx < N; idx += kSelThreads) mx = fmaxf(mx, s[idx]);
  mx = block_max(mx, sh);
  unsigned long long z = 0;
  for (int idx = tid; idx < N; idx += kSelThreads) z += fixed_mass(s[idx], mx);
  z = block_sum_u64(z, sh);
  if (tid == 0) {
    sh.m = mx;
    sh.Z = z;
    if constexpr (TOPK) {
      sh.R = (unsigned long long)topk;   // a count of pairs
      sh.select_all = topk >= N ? 1u : 0u;
    } else {
      const double r = ceil(double(tau) * double(z));
      sh.R = (unsigned long long)r;
      sh.select_all = (tau >= 1.0f || sh.R > z) ? 1u : 0u;
    }
    sh.prefix = 0;
    sh.above_cnt = 0;
    sh.above_mass = 0;
  }
  __syncthreads();

  // 2. four radix passes over the order keys, most significant digit first
  if (!sh.select_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
      for (int d = tid; d < 256; d += kSelThreads) {
        sh.cnt[d] = 0;
        sh.mass[d] = 0;
      }
      __syncthreads();
      const uint32_t prefix = sh.prefix;
      for (int base = 0; base < N; base += kSelThreads) {
        const int idx = base + tid;
        const float sv = idx < N ? s[idx] : -INFINITY;
        const uint32_t key = order_key(sv);
        const bool match = idx < N && (key & hi_mask) == prefix;
        const uint32_t dg = (key >> shift) & 0xffu;
        const unsigned long long ms = match ? fixed_mass(sv, mx) : 0ull;
        histogram_add(sh, match, dg, ms);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned long long acc = sh.above_mass;
        uint32_t cnt = sh.above_cnt;
        int dg = 255;
        for (; dg >= 0; --dg) {
          const bool reach = TOPK ? cnt + sh.cnt[dg] >= sh.R : acc + sh.mass[dg] >= sh.R;
          if (reach && sh.cnt[dg] > 0) break;
          acc += sh.mass[dg];
          cnt += sh.cnt[dg];
        }
        if (dg < 0) {
          sh.select_all = 1u;  // rounding kept the total below the target
        } else {
          sh.above_mass = acc;
          sh.above_cnt = cnt;
          sh.prefix = prefix | (uint32_t(dg) << shift);
          sh.tie_cnt = sh.cnt[dg];
          sh.tie_mass = sh.mass[dg];
        }
      }
      __syncthreads();
      if (sh.select_all) break;
    }
  }
  if (tid == 0 && !sh.select_all) {
    // all tied pairs share one score, hence one fixed-point mass
    const unsigned long long e1 = sh.tie_mass / sh.tie_cnt;
    const unsigned long long need = sh.R - (TOPK ? sh.above_cnt : sh.above_mass);
    unsigned long long t = TOPK ? need : (e1 ? (need + e1 - 1) / e1 : 1);
    if (t < 1) t = 1;
    if (t > sh.tie_cnt) t = sh.tie_cnt;
    sh.take_ties = uint32_t(t);
  }
  if (tid == 0) sh.tie_seen = 0;
  __syncthreads();

  // 3. compaction in linear order into the LDS bitmap
  const bool all = sh.select_all != 0;
  const uint32_t kstar = sh.prefix;
  const uint32_t take = all ? 0u : sh.take_ties;
  const int lane = tid & 63, w = tid >> 6;
  const float inv_z = float(kMassUnit / double(sh.Z));
  for (int base = 0; base < N; base += kSelThreads) {
    const int idx = base + tid;
    const bool in = idx < N;
    const float sv = in ? s[idx] : -INFINITY;
    const uint32_t key = order_key(sv);
    const bool tie = in && !all && key == kstar;
    // rank of this tie among ties in linear order
    const unsigned long long tmask = __ballot(tie);
    const int before_in_wave = __popcll(tmask & ((1ull << lane) - 1ull));
    if (lane == 0) sh.redi[w] = uint32_t(__popcll(tmask));
    __syncthreads();
    int before = int(sh.tie_seen);
    int total = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      if (i < w) before += int(sh.redi[i]);
      total += int(sh.redi[i]);
    }
    const int rank = before + before_in_wave;
    const int i_row = in ? idx / Nb : 0;
    const bool diag = in && (idx - i_row * Nb) == i_row;
    const bool sel = in && (all || key > kstar || (tie && uint32_t(rank) < take) || diag);
    const unsigned long long smask = __ballot(sel);
    if (lane == 0) {
      const int word = (base >> 5) + 2 * w;
      bits[word] = uint32_t(smask);
      bits[word + 1] = uint32_t(smask >> 32);
    }
    if (norm_scores && in) norm_scores[size_t(grp) * N + idx] = expf(sv - sh.m) * inv_z;
    __syncthreads();
    if (tid == 0) sh.tie_seen += uint32_t(total);
    __syncthreads();
  }

  // 4. CSR / CSC from the bitmap
  for (int i = tid; i < Nb; i += kSelThreads) {
    int rc = 0, cc = 0;
    for (int j = 0; j < Nb; ++j) {
      const int ir = i * Nb + j, ic = j * Nb + i;
      rc += (bits[ir >> 5] >> (ir & 31)) & 1u;
      cc += (bits[ic >> 5] >> (ic & 31)) & 1u;
    }
    sh.row_cnt[i] = rc;
    sh.col_cnt[i] = cc;
  }
  __syncthreads();
  int32_t* rp = row_ptr + size_t(grp) * (Nb + 1);
  int32_t* cp = col_ptr + size_t(grp) * (Nb + 1);
  // Nb <= kMaxBlocks = kSelThreads: one entry per thread
  {
    const int rc = tid < Nb ? sh.row_cnt[tid] : 0;
    const int cc = tid < Nb ? sh.col_cnt[tid] : 0;
    int rtot = 0, ctot = 0;
    const int roff = block_excl_scan(rc, sh, &rtot);
    const int coff = block_excl_scan(cc, sh, &ctot);
    __syncthreads();
    if (tid < Nb) {
      sh.row_cnt[tid] = roff;
      sh.col_cnt[tid] = coff;
      rp[tid] = roff;
      cp[tid] = coff;
    }
    if (tid == 0) {
      rp[Nb] = rtot;
      cp[Nb] = ctot;
      if (head_stats) {
        float* hs = head_stats + size_t(grp) * 4;
        const double zz = double(sh.Z);
        if (all) {
          hs[0] = float(N);
          hs[2] = 1.0f;
          hs[3] = 0.0f;
        } else {
          const unsigned long long e1 = sh.tie_mass / sh.tie_cnt;
          hs[0] = float(sh.above_cnt + sh.take_ties);
          hs[2] = float(double(sh.above_mass + e1 * sh.take_ties) / zz);
          hs[3] = float(double(e1) / zz);
        }
        hs[1] = float(rtot);
      }
    }
  }
  __syncthreads();
  int32_t* ci = col_idx + size_t(grp) * N;
  int32_t* ri = row_idx + size_t(grp) * N;
  for (int i = tid; i < Nb; i += kSelThreads) {
    int pr = sh.row_cnt[i], pc = sh.col_cnt[i];
    for (int j = 0; j < Nb; ++j) {
      const int ir = i * Nb + j, ic = j * Nb + i;
      if ((bits[ir >> 5] >> (ir & 31)) & 1u) ci[pr++] = j;
      if ((bits[ic >> 5] >> (ic & 31)) & 1u) ri[pc++] = j;
    }
  }
}

// One wave per query-block row; U = ceil(N_b / 64) pairs per lane.  rowstats[G][N_b][3] =
// {prefix length, prefix mass fraction, smallest normalised score in the prefix}.
template <bool TOPK, int U>
__global__ __launch_bounds__(256) void select_local_kernel(
    int Nb, float tau, int topk, const float* __restrict__ scores, uint32_t* __restrict__ bitmap,
    float* __restrict__ rowstats, float* __restrict__ norm_scores) {
  constexpr int WPB = 4;
  __shared__ float vs[WPB][64 * U];
  __shared__ unsigned long long es[WPB][64 * U];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = blockIdx.y;
  const int i = blockIdx.x * WPB + w;
  if (i >= Nb) return;   // a whole wave; nothing below synchronises across waves
  const float* srow = scores + (size_t(grp) * Nb + i) * Nb;

  float v[U];
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = lane + 64 * u;
    v[u] = j < Nb ? srow[j] : -INFINITY;
    mx = fmaxf(mx, v[u]);
  }
  mx = wave_max(mx);
  unsigned long long e[U], z = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = lane + 64 * u;
    e[u] = j < Nb ? fixed_mass(v[u], mx) : 0ull;
    z += e[u];
    vs[w][j] = v[u];
    es[w][j] = e[u];
  }
  z = wave_sum_u64(z);
  // the wave's own LDS writes become visible to its other lanes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  unsigned long long target;
  bool all;
  if constexpr (TOPK) {
    target = (unsigned long long)topk;
    all = topk >= Nb;
  } else {
    target = (unsigned long long)ceil(double(tau) * double(z));
    all = tau >= 1.0f || target > z;
  }
  // mass (threshold) or count (top-k) of the row's pairs ahead of each of this lane's
  unsigned long long before[U];
#pragma unroll
  for (int u = 0; u < U; ++u) before[u] = 0;
  for (int jj = 0; jj < Nb; ++jj) {
    const float vj = vs[w][jj];
    const unsigned long long ej = TOPK ? 1ull : es[w][jj];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = lane + 64 * u;
      if (vj > v[u] || (vj == v[u] && jj < j)) before[u] += ej;
    }
  }

  const int W = (Nb + 31) / 32;
  uint32_t* brow = bitmap + (size_t(grp) * Nb + i) * W;
  const float inv_z = float(kMassUnit / double(z));
  unsigned long long pmass = 0;
  int pcnt = 0;
  float vmin = INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = lane + 64 * u;
    const bool in = j < Nb;
    const bool pre = in && (all || before[u] < target);
    const bool sel = pre || (in && j == i);
    const unsigned long long bm = __ballot(sel);
    if (lane == 0) {
      if (2 * u < W) brow[2 * u] = uint32_t(bm);
      if (2 * u + 1 < W) brow[2 * u + 1] = uint32_t(bm >> 32);
    }
    pcnt += __popcll(__ballot(pre));
    if (pre) {
      pmass += e[u];
      vmin = fminf(vmin, float(double(e[u]) / double(z)));
    }
    if (norm_scores && in)
      norm_scores[(size_t(grp) * Nb + i) * Nb + j] = expf(v[u] - mx) * inv_z;
  }
  pmass = wave_sum_u64(pmass);
  vmin = -wave_max(-vmin);
  if (lane == 0) {
    float* rs = rowstats + (size_t(grp) * Nb + i) * 3;
    rs[0] = float(pcnt);
    rs[1] = float(double(pmass) / double(z));
    rs[2] = pcnt ? vmin : 0.0f;
  }
}

// CSR and CSC of one head group from a row-aligned pair bitmap (N_b rows of
// ceil(N_b/32) words), plus head_stats = {sum of prefix lengths, nnz, mean prefix mass,
// mean smallest prefix score} over the rows (rowstats and head_stats may be null).
__global__ __launch_bounds__(kSelThreads) void emit_lists_kernel(
    int Nb, const uint32_t* __restrict__ bitmap, const float* __restrict__ rowstats,
    int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ col_ptr, int32_t* __restrict__ row_idx,
    float* __restrict__ head_stats) {
  __shared__ SelShared sh;
  extern __shared__ uint32_t bits[];
  const int grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = (Nb + 31) / 32;
  const uint32_t* src = bitmap + size_t(grp) * Nb * W;
  for (int x = tid; x < Nb * W; x += kSelThreads) bits[x] = src[x];
  __syncthreads();
  auto bit = [&](int i, int j) { return (bits[i * W + (j >> 5)] >> (j & 31)) & 1u; };
  for (int i = tid; i < Nb; i += kSelThreads) {
    int rc = 0, cc = 0;
    for (int x = 0; x < W; ++x) rc += __popc(bits[i * W + x]);
    for (int r = 0; r < Nb; ++r) cc += bit(r, i);
    sh.row_cnt[i] = rc;
    sh.col_cnt[i] = cc;
  }
  __syncthreads();
  int32_t* rp = row_ptr + size_t(grp) * (Nb + 1);
  int32_t* cp = col_ptr + size_t(grp) * (Nb + 1);
  float ks = 0.f, ms = 0.f, vsum = 0.f;
  for (int i = tid; i < Nb && rowstats; i += kSelThreads) {
    const float* rs = rowstats + (size_t(grp) * Nb + i) * 3;
    ks += rs[0];
    ms += rs[1];
    vsum += rs[2];
  }
  {
    const int rc = tid < Nb ? sh.row_cnt[tid] : 0;
    const int cc = tid < Nb ? sh.col_cnt[tid] : 0;
    int rtot = 0, ctot = 0;
    const int roff = block_excl_scan(rc, sh, &rtot);
    const int coff = block_excl_scan(cc, sh, &ctot);
    ks = wave_sum(ks);
    ms = wave_sum(ms);
    vsum = wave_sum(vsum);
    __syncthreads();
    if (tid < Nb) {
      sh.row_cnt[tid] = roff;
      sh.col_cnt[tid] = coff;
      rp[tid] = roff;
      cp[tid] = coff;
    }
    if ((tid & 63) == 0) {   // Nb <= kMaxBlocks = kSelThreads: sums of the first waves
      sh.redf[tid >> 6] = ks;
      sh.redi[tid >> 6] = 0;
    }
    __syncthreads();
    if (tid == 0) {
      rp[Nb] = rtot;
      cp[Nb] = ctot;
    }
    __syncthreads();
    if ((tid & 63) == 0) sh.redf[tid >> 6] = ms;
    __syncthreads();
    float mtot = 0.f;
    if (tid == 0)
      for (int x = 0; x < kSelWaves; ++x) mtot += sh.redf[x];
    __syncthreads();
    if ((tid & 63) == 0) sh.redf[tid >> 6] = vsum;
    __syncthreads();
    float vtot = 0.f;
    if (tid == 0)
      for (int x = 0; x < kSelWaves; ++x) vtot += sh.redf[x];
    __syncthreads();
    if ((tid & 63) == 0) sh.redf[tid >> 6] = ks;
    __syncthreads();
    if (tid == 0 && head_stats) {
      float ktot = 0.f;
      for (int x = 0; x < kSelWaves; ++x) ktot += sh.redf[x];
      float* hs = head_stats + size_t(grp) * 4;
      hs[0] = ktot;
      hs[1] = float(rtot);
      hs[2] = mtot / float(Nb);
      hs[3] = vtot / float(Nb);
    }
  }
  __syncthreads();
  int32_t* ci = col_idx + size_t(grp) * Nb * Nb;
  int32_t* ri = row_idx + size_t(grp) * Nb * Nb;
  for (int i = tid; i < Nb; i += kSelThreads) {
    int pr = sh.row_cnt[i], pc = sh.col_cnt[i];
    for (int j = 0; j < Nb; ++j) {
      if (bit(i, j)) ci[pr++] = j;
      if (bit(j, i)) ri[pc++] = j;
    }
  }
}

// ---------------------------------------------------------------------------------
// Pool selection over many workgroups.  A head group's pool is `rows` x N_b scores in
// row-major order (linear index row * N_b + j): the N_b x N_b block pairs of the global
// strategies (rows = query blocks, forced pair (i, i)), or the L x N_b (query token, key
// block) pairs of the token-granular reading of papernotes 关键设计 2 (rows = tokens, forced
// pair (x, block(x))).  The decision is the threshold (or top-k) rule of the single-head
// description above:
//   scores             block_scores_kernel / token_scores_kernel, which also record the
//                      head's maximum as an atomic maximum of order keys;
//   pool_hist_kernel   one per 8-bit digit: (count, fixed-point mass) histograms of the keys
//                      that match the digits decided so far, merged with global atomics
//                      (integer sums, so the order of the atomics does not matter);
//   pool_step_kernel   one wave per head group finds where the walk down the merged
//                      histogram from the top digit reaches the target mass (or count);
//   pool_ties_*        only when the cut falls inside a run of equal keys: the ranks of the
//                      tied pairs in linear order (per-chunk counts, then a scan);
//   pool_emit_kernel   the row bitmap [G][rows][W] (W = ceil(N_b/32) words per row) and,
//                      for token rows, the union bitmap of every query block;
//   emit_lists_kernel  CSR / CSC of the block bitmap; pool_stats_kernel the head stats.
// A chunk is `rpc` consecutive rows (a multiple of 4: one quarter per wave).  Masses are
// integers in units of 2^-unit_log2 of the largest one, with unit_log2 chosen per pool so
// that a head's total stays below 2^63.
struct PoolState {
  unsigned long long R, above_mass, tie_mass, Z;
  uint32_t mkey, prefix, above_cnt, tie_cnt, take, select_all, need_rank, nnz;
};

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t pool_mass(float s, float m, double unit) {
  return uint64_t(double(expf(s - m)) * unit + 0.5);
}

// largest power-of-two unit with npairs * unit < 2^63 (at most 2^44)
inline double pool_unit(double npairs) {
  int b = 0;
  while (b < 62 && double(uint64_t(1) << b) < npairs) ++b;
  return ldexp(1.0, std::min(44, 62 - b));
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

__global__ void pool_max_kernel(int N, const float* __restrict__ scores,
                                PoolState* __restrict__ st) {
  const int grp = blockIdx.y;
  float mx = -INFINITY;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    mx = fmaxf(mx, scores[size_t(grp) * N + i]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) atomicMax(&st[grp].mkey, order_key(mx));
}

constexpr int kScoreTiles = 3;   // tiles of 32 key blocks per wave of token_scores_kernel

template <int D, typename T>
__global__ __launch_bounds__(64) void token_scores_kernel(Geom g, const T* __restrict__ q,
                                                          const float* __restrict__ kp,
                                                          float* __restrict__ scores,
                                                          PoolState* __restrict__ st,
                                                          float scale) {
  // one wave: 32 tokens against kScoreTiles tiles of 32 blocks; each Q fragment feeds the
  // tiles' independent product chains (each tile's chain is the same as alone)
  constexpr int JT = kScoreTiles;
  const int lane = threadIdx.x;
  const int x0 = blockIdx.x * 32, j00 = blockIdx.y * 32 * JT;
  const int grp = blockIdx.z;
  const int half = lane >> 5;
  const int rx = x0 + (lane & 31);
  const int b = grp / g.Hh, h = grp - b * g.Hh;
  const T* qrow = q + ((size_t(b) * g.L + min(rx, g.L - 1)) * g.Hh + h) * D + half * (D / 2);
  const bool qok = rx < g.L;
  const float* krow[JT];
  bool kok[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int rj = j00 + jt * 32 + (lane & 31);
    kok[jt] = rj < g.Nb;
    krow[jt] = kp + (size_t(grp) * g.Nb + min(rj, g.Nb - 1)) * D + half * (D / 2);
  }
  f32x16_t acc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[jt][v] = 0.f;
  // lane half `half` feeds d in [half*D/2, (half+1)*D/2) for both operands
#pragma unroll 2
  for (int c = 0; c < D / 2; c += 4) {
    float4 a;
    if constexpr (sizeof(T) == 2) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(qrow + c);
      a = make_float4(bf16_to_f32(w[0] & 0xffffu), bf16_to_f32(w[0] >> 16),
                      bf16_to_f32(w[1] & 0xffffu), bf16_to_f32(w[1] >> 16));
    } else {
      a = *reinterpret_cast<const float4*>(qrow + c);
    }
    if (!qok) a = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 bb[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      bb[jt] = *reinterpret_cast<const float4*>(krow[jt] + c);
      if (!kok[jt]) bb[jt] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bb[jt].x, acc[jt], 0, 0, 0);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bb[jt].y, acc[jt], 0, 0, 0);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bb[jt].z, acc[jt], 0, 0, 0);
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) acc[jt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bb[jt].w, acc[jt], 0, 0, 0);
  }
  // acc[jt][v]: token x0 + 8*(v/4) + 4*half + v%4, block j00 + 32 jt + lane%32
  float mx = -INFINITY;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    if (kok[jt]) {
      const int rj = j00 + jt * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int x = x0 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (x < g.L) {
          const float sv = acc[jt][v] * scale;
          scores[(size_t(grp) * g.L + x) * g.Nb + rj] = sv;
          mx = fmaxf(mx, sv);
        }
      }
    }
  }
  mx = wave_max(mx);
  if (lane == 0) atomicMax(&st[grp].mkey, order_key(mx));
}

// Digit pass: histogram of digit (key >> shift) & 255 over the pairs whose higher digits
// equal the prefix decided so far (pass 0: every pair).
__global__ __launch_bounds__(256) void pool_hist_kernel(int rows, int Nb, int rpc, int shift,
                                                        double unit,
                                                        const float* __restrict__ scores,
                                                        const PoolState* __restrict__ st,
                                                        uint32_t* __restrict__ hcnt,
                                                        unsigned long long* __restrict__ hmass) {
  __shared__ uint32_t cnt[256];
  __shared__ unsigned long long mass[256];
  const int grp = blockIdx.y;
  const PoolState S = st[grp];
  if (S.select_all) return;
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  mass[tid] = 0;
  __syncthreads();
  const float m = key_to_float(S.mkey);
  const uint32_t hi_mask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
  const size_t N = size_t(rows) * Nb;
  const size_t begin = size_t(blockIdx.x) * rpc * Nb;
  const size_t end = min(N, begin + size_t(rpc) * Nb);
  const float* s = scores + size_t(grp) * N;
  // four coalesced loads in flight per thread before any is used (the counts and the
  // fixed-point masses are integers, so the order of the additions does not matter)
  constexpr int U = 4;
  for (size_t base = begin; base < end; base += U * 256) {
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t idx = base + u * 256 + tid;
      sv[u] = idx < end ? s[idx] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = base + u * 256 + tid < end;
      const uint32_t key = order_key(sv[u]);
      const bool match = in && (key & hi_mask) == S.prefix;
      const uint32_t dg = (key >> shift) & 0xffu;
      histogram_add(cnt, mass, match, dg, match ? pool_mass(sv[u], m, unit) : 0ull);
    }
  }
  __syncthreads();
  if (cnt[tid]) {
    atomicAdd(&hcnt[grp * 256 + tid], cnt[tid]);
    atomicAdd(&hmass[grp * 256 + tid], mass[tid]);
  }
}

// After digit pass `pass`: pick the digit where the running mass (topk > 0: count)
// reaches the target.  One wave per head group: the lanes copy the merged histogram to
// LDS and clear it for the next pass, then lane 0 walks the copy.
// Inclusive prefix sum over the 64 lanes of a wave (lane 0 first), of a 64-bit value.
__device__ __forceinline__ unsigned long long wave_prefix_u64(unsigned long long v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t lo = __shfl_up(uint32_t(v), off, 64);
    const uint32_t hi = __shfl_up(uint32_t(v >> 32), off, 64);
    if (lane >= off) v += (static_cast<unsigned long long>(hi) << 32) | lo;
  }
  return v;
}

// The walk down the merged histogram, one wave per head group: lane L holds digits
// 255 - 4L ... 252 - 4L.  A prefix sum over the lanes gives every lane the mass and count
// of the digits above its four; each lane then tests its digits in descending order for
// the stop rule (a non-empty digit at which the running mass, or count, reaches the
// target), and the lowest lane with a hit holds the digit the sequential walk from the
// top digit stops at.
__global__ __launch_bounds__(64) void pool_step_kernel(int pass, float tau, int topk,
                                                       double npairs,
                                                       PoolState* __restrict__ st,
                                                       uint32_t* __restrict__ hcnt,
                                                       unsigned long long* __restrict__ hmass) {
  const int grp = blockIdx.x, lane = threadIdx.x;
  uint32_t* gc = hcnt + grp * 256;
  unsigned long long* gm = hmass + grp * 256;
  uint32_t c4[4];
  unsigned long long m4[4];
  uint32_t csum = 0;
  unsigned long long msum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = 255 - 4 * lane - j;
    c4[j] = gc[d];
    m4[j] = gm[d];
    gc[d] = 0u;
    gm[d] = 0ull;
    csum += c4[j];
    msum += m4[j];
  }
  PoolState S = st[grp];
  const bool count = topk > 0;
  const unsigned long long mincl = wave_prefix_u64(msum, lane);
  const unsigned long long cincl = wave_prefix_u64(csum, lane);
  if (pass == 0) {   // every pair matched: the histogram holds the whole pool
    const unsigned long long z = __shfl(uint32_t(mincl), 63, 64) |
                                 (static_cast<unsigned long long>(
                                      __shfl(uint32_t(mincl >> 32), 63, 64)) << 32);
    S.Z = z;
    if (count) {
      S.R = (unsigned long long)topk;
      S.select_all = double(topk) >= npairs ? 1u : 0u;
    } else {
      S.R = (unsigned long long)ceil(double(tau) * double(z));
      S.select_all = (tau >= 1.0f || S.R > z) ? 1u : 0u;
    }
    S.above_mass = 0;
    S.above_cnt = 0;
    S.prefix = 0;
  }
  if (S.select_all) {   // uniform
    if (lane == 0 && pass == 0) st[grp] = S;
    return;
  }
  // this lane's digits in descending order, from the totals above them
  unsigned long long acc = S.above_mass + (mincl - msum);
  uint32_t n = S.above_cnt + uint32_t(cincl - csum);
  int hit = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool reach = count ? n + c4[j] >= S.R : acc + m4[j] >= S.R;
    if (hit < 0 && c4[j] > 0 && reach) hit = j;
    if (hit < 0) {
      acc += m4[j];
      n += c4[j];
    }
  }
  const uint64_t hits = __ballot(hit >= 0);
  if (hits == 0) {   // rounding kept the total below the target
    if (lane == 0) {
      S.select_all = 1u;
      st[grp] = S;
    }
    return;
  }
  if (lane != __builtin_ctzll(hits)) return;
  const int dg = 255 - 4 * lane - hit;
  S.above_mass = acc;
  S.above_cnt = n;
  S.prefix |= uint32_t(dg) << (24 - 8 * pass);
  S.tie_cnt = c4[hit];
  S.tie_mass = m4[hit];
  if (pass == 3) {
    // all tied pairs share one score, hence one fixed-point mass
    const unsigned long long e1 = S.tie_mass / S.tie_cnt;
    const unsigned long long need = S.R - (count ? S.above_cnt : S.above_mass);
    unsigned long long t = count ? need : (e1 ? (need + e1 - 1) / e1 : 1);
    if (t < 1) t = 1;
    if (t > S.tie_cnt) t = S.tie_cnt;
    S.take = uint32_t(t);
    S.need_rank = S.take < S.tie_cnt ? 1u : 0u;
  }
  st[grp] = S;
}

// Tied pairs (key equal to the cut) per chunk, when only some of them are taken.
__global__ __launch_bounds__(256) void pool_ties_count_kernel(int rows, int Nb, int rpc,
                                                              const float* __restrict__ scores,
                                                              const PoolState* __restrict__ st,
                                                              uint32_t* __restrict__ chunkcnt) {
  __shared__ uint32_t red[4];
  const int grp = blockIdx.y;
  const PoolState S = st[grp];
  if (S.select_all || !S.need_rank) return;
  const int tid = threadIdx.x;
  const size_t N = size_t(rows) * Nb;
  const size_t begin = size_t(blockIdx.x) * rpc * Nb;
  const size_t end = min(N, begin + size_t(rpc) * Nb);
  const float* s = scores + size_t(grp) * N;
  uint32_t n = 0;
  for (size_t idx = begin + tid; idx < end; idx += 256) n += order_key(s[idx]) == S.prefix;
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  if ((tid & 63) == 0) red[tid >> 6] = n;
  __syncthreads();
  if (tid == 0) chunkcnt[size_t(grp) * gridDim.x + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// Exclusive scan of the per-chunk tie counts of one head group (one workgroup each).
__global__ __launch_bounds__(256) void pool_ties_scan_kernel(int nchunks,
                                                             const PoolState* __restrict__ st,
                                                             uint32_t* __restrict__ chunkcnt) {
  __shared__ uint32_t part[256];
  const int grp = blockIdx.x;
  if (st[grp].select_all || !st[grp].need_rank) return;
  const int tid = threadIdx.x;
  uint32_t* c = chunkcnt + size_t(grp) * nchunks;
  const int per = (nchunks + 255) / 256;
  const int lo = min(nchunks, tid * per), hi = min(nchunks, lo + per);
  uint32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += c[i];
  part[tid] = sum;
  __syncthreads();
  uint32_t off = 0;
  for (int i = 0; i < tid; ++i) off += part[i];
  for (int i = lo; i < hi; ++i) {
    const uint32_t v = c[i];
    c[i] = off;
    off += v;
  }
}

// Row bitmap, union bitmap (token rows) and pair count.  Wave w of a chunk handles its
// quarter of the chunk's rows in order; each row's N_b pairs go 64 per ballot.
template <bool TOKROWS>
__global__ __launch_bounds__(256) void pool_emit_kernel(Geom g, int rows, int rpc,
                                                        const float* __restrict__ scores,
                                                        PoolState* __restrict__ st,
                                                        const uint32_t* __restrict__ chunkoff,
                                                        uint32_t* __restrict__ rowbits,
                                                        uint32_t* __restrict__ qbits) {
  __shared__ uint32_t wties[4];
  const int grp = blockIdx.y;
  const PoolState S = st[grp];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool all = S.select_all != 0;
  const uint32_t kstar = S.prefix;
  const uint32_t take = all ? 0u : S.take;
  const bool ranked = !all && S.need_rank;
  const int Nb = g.Nb, W = (Nb + 31) / 32;
  const size_t N = size_t(rows) * Nb;
  const float* s = scores + size_t(grp) * N;
  const int rpw = rpc / 4;
  const int x0 = blockIdx.x * rpc + w * rpw;
  const int x1 = min(rows, x0 + rpw);
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t rank = 0;
  if (ranked) {   // ties before this wave's rows: earlier chunks, then earlier waves
    uint32_t n = 0;
    for (int x = x0; x < x1; ++x)
      for (int jc = 0; jc < Nb; jc += 64) {
        const int j = jc + lane;
        n += __popcll(__ballot(j < Nb && order_key(s[size_t(x) * Nb + j]) == kstar));
      }
    if (lane == 0) wties[w] = n;
    __syncthreads();
    rank = chunkoff[size_t(grp) * gridDim.x + blockIdx.x];
    for (int i = 0; i < w; ++i) rank += wties[i];
  }
  uint32_t nnz = 0;
  for (int x = x0; x < x1; ++x) {
    const int bx = TOKROWS ? token_block(g, x) : x;   // the row's forced column
    uint32_t* rb = rowbits + (size_t(grp) * rows + x) * W;
    uint32_t* qb = qbits + (size_t(grp) * Nb + bx) * W;
    for (int jc = 0; jc < Nb; jc += 64) {
      const int j = jc + lane;
      const bool in = j < Nb;
      const float sv = in ? s[size_t(x) * Nb + j] : -INFINITY;
      const uint32_t key = order_key(sv);
      const bool tie = in && !all && key == kstar;
      const unsigned long long tb = __ballot(tie);
      const uint32_t r = rank + uint32_t(__popcll(tb & lt));
      rank += uint32_t(__popcll(tb));
      const bool sel = in && (all || key > kstar || (tie && r < take) || j == bx);
      const unsigned long long sb = __ballot(sel);
      nnz += uint32_t(__popcll(sb));
      const int wd = (jc >> 5) + (lane & 1);
      const uint32_t word = (lane & 1) ? uint32_t(sb >> 32) : uint32_t(sb);
      if (lane < 2 && wd < W) {
        rb[wd] = word;
        if (TOKROWS && word) atomicOr(&qb[wd], word);
      }
    }
  }
  if (lane == 0 && nnz) atomicAdd(&st[grp].nnz, nnz);
}

// head_stats = {k*, nnz, prefix mass, cutoff score}; and, if asked, the normalised scores.
__global__ void pool_stats_kernel(int G, double npairs, double unit,
                                  const PoolState* __restrict__ st,
                                  float* __restrict__ head_stats) {
  const int grp = blockIdx.x * blockDim.x + threadIdx.x;
  if (grp >= G) return;
  const PoolState& S = st[grp];
  float* hs = head_stats + size_t(grp) * 4;
  if (S.select_all) {
    hs[0] = float(npairs);
    hs[2] = 1.0f;
    hs[3] = 0.0f;
  } else {
    const double z = double(S.Z);
    const unsigned long long e1 = S.tie_mass / S.tie_cnt;
    hs[0] = float(S.above_cnt + S.take);
    hs[2] = float(double(S.above_mass + e1 * S.take) / z);
    hs[3] = float(double(e1) / z);
  }
  hs[1] = float(S.nnz);
}

__global__ void pool_norm_kernel(int N, double unit, const float* __restrict__ scores,
                                 const PoolState* __restrict__ st, float* __restrict__ out) {
  const int grp = blockIdx.y;
  const float m = key_to_float(st[grp].mkey);
  const float inv_z = float(unit / double(st[grp].Z));
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    out[size_t(grp) * N + i] = expf(scores[size_t(grp) * N + i] - m) * inv_z;
}

// Workspace of a pool selection, in this order (256-byte aligned): scores fp32
// [G][rows][N_b], PoolState [G], histogram counts u32 [G][256], masses u64 [G][256],
// per-chunk tie counts u32 [G][chunks], union bitmap u32 [G][N_b][W] (token rows only).
struct PoolWs {
  float* scores;
  PoolState* state;
  uint32_t* hcnt;
  unsigned long long* hmass;
  uint32_t* chunkcnt;
  uint32_t* qbits;
  size_t bytes;
};

static PoolWs pool_ws(void* ws, int G, int rows, int Nb, int rpc, bool tokrows) {
  const size_t W = (size_t(Nb) + 31) / 32;
  const size_t chunks = (size_t(rows) + rpc - 1) / rpc;
  PoolWs w{};
  unsigned char* p = static_cast<unsigned char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.scores = reinterpret_cast<float*>(take(size_t(G) * rows * Nb * 4));
  w.state = reinterpret_cast<PoolState*>(take(size_t(G) * sizeof(PoolState)));
  w.hcnt = reinterpret_cast<uint32_t*>(take(size_t(G) * 256 * 4));
  w.hmass = reinterpret_cast<unsigned long long*>(take(size_t(G) * 256 * 8));
  w.chunkcnt = reinterpret_cast<uint32_t*>(take(size_t(G) * chunks * 4));
  w.qbits = reinterpret_cast<uint32_t*>(take(tokrows ? size_t(G) * Nb * W * 4 : 0));
  w.bytes = off;
  return w;
}

// Histogram passes, tie ranks and the row bitmap of a pool whose scores and maximum are
// in place (state zeroed before the scores).
template <bool TOKROWS>
static int run_pool(const Geom& g, const PoolWs& w, int rows, int rpc, float tau, int topk,
                    uint32_t* rowbits, hipStream_t st) {
  const int G = g.B * g.Hh;
  const int chunks = (rows + rpc - 1) / rpc;
  const double npairs = double(rows) * g.Nb;
  const double unit = pool_unit(npairs);
  const dim3 cgrid(chunks, G);
  for (int pass = 0; pass < 4; ++pass) {
    pool_hist_kernel<<<cgrid, 256, 0, st>>>(rows, g.Nb, rpc, 24 - 8 * pass, unit, w.scores,
                                            w.state, w.hcnt, w.hmass);
    pool_step_kernel<<<G, 64, 0, st>>>(pass, tau, topk, npairs, w.state, w.hcnt, w.hmass);
  }
  pool_ties_count_kernel<<<cgrid, 256, 0, st>>>(rows, g.Nb, rpc, w.scores, w.state,
                                                w.chunkcnt);
  pool_ties_scan_kernel<<<G, 256, 0, st>>>(chunks, w.state, w.chunkcnt);
  pool_emit_kernel<TOKROWS><<<cgrid, 256, 0, st>>>(g, rows, rpc, w.scores, w.state,
                                                   w.chunkcnt, rowbits, w.qbits);
  return launch_status();
}

template <bool TOPK>
static int launch_local(const Geom& g, float tau, int topk, const float* scores,
                        uint32_t* bitmap, float* rowstats, float* norm_scores, hipStream_t st) {
  const int groups = g.B * g.Hh;
  const dim3 grid((g.Nb + 3) / 4, groups);
  const int U = (g.Nb + 63) / 64;
  if (U <= 1)
    select_local_kernel<TOPK, 1><<<grid, 256, 0, st>>>(g.Nb, tau, topk, scores, bitmap, rowstats, norm_scores);
  else if (U <= 2)
    select_local_kernel<TOPK, 2><<<grid, 256, 0, st>>>(g.Nb, tau, topk, scores, bitmap, rowstats, norm_scores);
  else if (U <= 4)
    select_local_kernel<TOPK, 4><<<grid, 256, 0, st>>>(g.Nb, tau, topk, scores, bitmap, rowstats, norm_scores);
  else if (U <= 8)
    select_local_kernel<TOPK, 8><<<grid, 256, 0, st>>>(g.Nb, tau, topk, scores, bitmap, rowstats, norm_scores);
  else
    select_local_kernel<TOPK, 16><<<grid, 256, 0, st>>>(g.Nb, tau, topk, scores, bitmap, rowstats, norm_scores);
  return launch_status();
}

// Rows per chunk of the block pool's passes (one query-block row per wave).
constexpr int kBlockRpc = 4;
// Block counts up to which the global strategies run in one workgroup per head group.
constexpr int kSingleSelectBlocks = 128;
// Rows per chunk of the token pool's passes.
constexpr int kTokenRpc = 64;

// Workspace of vmoba_select / vmoba_select_mode: the global strategies use the pool
// tables and a row bitmap behind them; the local ones the scores, a row bitmap and three
// floats per row.  Scores come first in both.
size_t select_ws(const Geom& g) {
  const int G = g.B * g.Hh;
  const size_t W = (size_t(g.Nb) + 31) / 32;
  const size_t bitmap = align256(size_t(G) * g.Nb * W * 4);
  const size_t global = pool_ws(nullptr, G, g.Nb, g.Nb, kBlockRpc, false).bytes + bitmap;
  const size_t local = align256(size_t(G) * g.Nb * g.Nb * 4) + bitmap +
                       align256(size_t(G) * g.Nb * 3 * 4);
  return std::max(global, local);
}

int launch_select(const Geom& g, const float* q_pool, const float* k_pool, int mode, float tau,
                  int topk, int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr,
                  int32_t* row_idx, float* head_stats, float* norm_scores, void* ws,
                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int groups = g.B * g.Hh;
  const size_t nb2 = size_t(g.Nb) * g.Nb;
  float* scores = static_cast<float*>(ws);
  const float scale = 1.0f / sqrtf(float(g.D));
  dim3 sgrid((g.Nb + 31) / 32, (g.Nb + 31) / 32, groups);
  if (g.D == 128)
    block_scores_kernel<128><<<sgrid, 64, 0, st>>>(g.Nb, q_pool, k_pool, scores, scale);
  else
    block_scores_kernel<64><<<sgrid, 64, 0, st>>>(g.Nb, q_pool, k_pool, scores, scale);
  int stt = launch_status();
  if (stt) return stt;
  const int max_lds = int(size_t(kMaxBlocks) * kMaxBlocks / 8);
  const size_t W = (size_t(g.Nb) + 31) / 32;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(emit_lists_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) != hipSuccess)
    return VMOBA_ERR_HIP;
  const bool global = mode == VMOBA_SEL_THRESHOLD_GLOBAL || mode == VMOBA_SEL_TOPK_GLOBAL;
  if (global && g.Nb <= kSingleSelectBlocks) {
    const size_t words = ((nb2 + 1023) / 1024) * 32;  // whole 1024-pair chunks
    const bool tk = mode == VMOBA_SEL_TOPK_GLOBAL;
    const void* fn = tk ? reinterpret_cast<const void*>(single_select_kernel<true>)
                        : reinterpret_cast<const void*>(single_select_kernel<false>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) !=
        hipSuccess)
      return VMOBA_ERR_HIP;
    if (tk)
      single_select_kernel<true><<<groups, kSelThreads, words * sizeof(uint32_t), st>>>(
          g.Nb, tau, topk, scores, row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores);
    else
      single_select_kernel<false><<<groups, kSelThreads, words * sizeof(uint32_t), st>>>(
          g.Nb, tau, topk, scores, row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores);
    return launch_status();
  }
  if (global) {
    const PoolWs w = pool_ws(ws, groups, g.Nb, g.Nb, kBlockRpc, false);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(ws) + w.bytes);
    const size_t zero_words = (reinterpret_cast<unsigned char*>(w.chunkcnt) -
                               reinterpret_cast<unsigned char*>(w.state)) / 4;
    fill_zero_kernel<<<64, 256, 0, st>>>(reinterpret_cast<uint32_t*>(w.state), zero_words);
    const int N = int(nb2);
    pool_max_kernel<<<dim3(std::min(64, (N + 255) / 256), groups), 256, 0, st>>>(N, scores,
                                                                              w.state);
    const int k = mode == VMOBA_SEL_TOPK_GLOBAL ? topk : 0;
    if ((stt = run_pool<false>(g, w, g.Nb, kBlockRpc, tau, k, bitmap, st))) return stt;
    emit_lists_kernel<<<groups, kSelThreads, size_t(g.Nb) * W * 4, st>>>(
        g.Nb, bitmap, nullptr, row_ptr, col_idx, col_ptr, row_idx, nullptr);
    const double npairs = double(nb2);
    pool_stats_kernel<<<(groups + 63) / 64, 64, 0, st>>>(groups, npairs, pool_unit(npairs),
                                                        w.state, head_stats);
    if (norm_scores)
      pool_norm_kernel<<<dim3(std::min(64, (N + 255) / 256), groups), 256, 0, st>>>(
          N, pool_unit(npairs), scores, w.state, norm_scores);
    return launch_status();
  }
  // local strategies: bitmap and row statistics behind the scores in the workspace
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + align256(groups * nb2 * sizeof(float)));
  float* rowstats = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(bitmap) +
                                             align256(groups * size_t(g.Nb) * W * 4));
  stt = mode == VMOBA_SEL_TOPK_LOCAL
            ? launch_local<true>(g, tau, topk, scores, bitmap, rowstats, norm_scores, st)
            : launch_local<false>(g, tau, topk, scores, bitmap, rowstats, norm_scores, st);
  if (stt) return stt;
  emit_lists_kernel<<<groups, kSelThreads, size_t(g.Nb) * W * 4, st>>>(
      g.Nb, bitmap, rowstats, row_ptr, col_idx, col_ptr, row_idx, head_stats);
  return launch_status();
}

size_t token_select_ws(const Geom& g) {
  return pool_ws(nullptr, g.B * g.Hh, g.L, g.Nb, kTokenRpc, true).bytes;
}

int launch_select_tokens(const Geom& g, const void* q, const float* k_pool, float tau,
                         uint32_t* tokmask, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* col_ptr, int32_t* row_idx, float* head_stats, void* ws,
                         void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = g.B * g.Hh;
  const size_t W = (size_t(g.Nb) + 31) / 32;
  const PoolWs w = pool_ws(ws, G, g.L, g.Nb, kTokenRpc, true);
  // zero the state, the histograms and the union bitmap (fill kernels, not memsets)
  const size_t zero_words = (reinterpret_cast<unsigned char*>(w.chunkcnt) -
                             reinterpret_cast<unsigned char*>(w.state)) / 4;
  fill_zero_kernel<<<64, 256, 0, st>>>(reinterpret_cast<uint32_t*>(w.state), zero_words);
  fill_zero_kernel<<<1024, 256, 0, st>>>(w.qbits, size_t(G) * g.Nb * W);
  const float scale = 1.0f / sqrtf(float(g.D));
  const dim3 sgrid((g.L + 31) / 32, ((g.Nb + 31) / 32 + kScoreTiles - 1) / kScoreTiles, G);
  if (g.D == 128)
    token_scores_kernel<128, uint16_t><<<sgrid, 64, 0, st>>>(
        g, static_cast<const uint16_t*>(q), k_pool, w.scores, w.state, scale);
  else
    token_scores_kernel<64, uint16_t><<<sgrid, 64, 0, st>>>(
        g, static_cast<const uint16_t*>(q), k_pool, w.scores, w.state, scale);
  int stt = launch_status();
  if (stt) return stt;
  if ((stt = run_pool<true>(g, w, g.L, kTokenRpc, tau, 0, tokmask, st))) return stt;
  const int max_lds = int(size_t(kMaxBlocks) * kMaxBlocks / 8);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(emit_lists_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) != hipSuccess)
    return VMOBA_ERR_HIP;
  emit_lists_kernel<<<G, kSelThreads, size_t(g.Nb) * W * 4, st>>>(
      g.Nb, w.qbits, nullptr, row_ptr, col_idx, col_ptr, row_idx, nullptr);
  const double npairs = double(g.L) * g.Nb;
  pool_stats_kernel<<<(G + 63) / 64, 64, 0, st>>>(G, npairs, pool_unit(npairs), w.state,
                                                  head_stats);
  return launch_status();
}

}  // namespace vmoba
