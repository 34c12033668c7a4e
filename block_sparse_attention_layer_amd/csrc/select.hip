// Global block selection with the cumulative-mass threshold (papernotes 关键设计 2 and 3;
// paperlayer §3.3-§3.4).
//
// Stage 1, block_scores_kernel: s_ij = <Qbar_i, Kbar_j> / sqrt(d) for one 32 x 32 tile of
// one head group per wave, on the fp32 matrix cores (v_mfma_f32_32x32x2_f32), so the
// products and sums keep fp32 precision; the selection compares masses near tau.
//
// Stage 2, threshold_select_kernel: one 1024-thread workgroup per head group.
//   1. m = max s; each pair's mass e = exp(s - m) is held as a 64-bit fixed-point integer
//      (2^44 units), so every mass sum is exact and independent of summation order.
//   2. The cutoff pair is found without sorting: the fp32 scores are mapped to
//      order-preserving 32-bit keys, and four 8-bit radix passes build per-digit
//      (count, mass) histograms of the still-undecided keys, walking down from the
//      largest digit until the running mass reaches ceil(tau * sum e).  What remains is
//      the key of the k*-th pair; exact ties at that key are taken in ascending linear
//      index i*N_b + j, as many as the threshold needs.
//   3. Compaction in linear order marks the prefix plus the diagonal in an LDS bitmap
//      (wave ballots, one 64-bit word per wave), then row and column counts, an
//      exclusive scan and an ascending walk per row / column emit CSR and CSC.
//   With TOPK the same walk counts pairs instead of mass: the cutoff is the key of the
//   k-th pair (top-k + global, one of the strategies of the ablation, paperlayer §4.4).
//
// Local strategies (threshold + local, top-k + local): every query block's row of N_b
// scores is its own pool, normalised by a softmax over the row.  select_local_kernel
// gives each row one wave; a pair is kept iff the fixed-point mass (threshold) or the
// number (top-k) of the row's pairs that precede it in the order (higher score, or the
// same score at a lower key index) is below the target.  Each lane counts that for its
// pairs against the whole row staged in LDS.  The rows go to a bitmap, and
// emit_lists_kernel turns the bitmap into CSR and CSC as above.
#include <math.h>

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
constexpr double kMassUnit = 17592186044416.0;  // 2^44

__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t fixed_mass(float s, float m) {
  const float e = expf(s - m);
  return uint64_t(double(e) * kMassUnit + 0.5);
}

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
__device__ __forceinline__ void histogram_add(SelShared& sh, bool match, uint32_t dg,
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
      atomicAdd(&sh.cnt[ldg], uint32_t(__popcll(smask)));
      atomicAdd(&sh.mass[ldg], msum);
    }
    match = match && !same;
    active &= ~smask;
  }
  if (match) {
    atomicAdd(&sh.cnt[dg], 1u);
    atomicAdd(&sh.mass[dg], mass);
  }
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

template <bool TOPK>
__global__ __launch_bounds__(kSelThreads) void global_select_kernel(
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
// mean smallest prefix score} over the rows.
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
  for (int i = tid; i < Nb; i += kSelThreads) {
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
  if (mode == VMOBA_SEL_THRESHOLD_GLOBAL || mode == VMOBA_SEL_TOPK_GLOBAL) {
    const size_t words = ((nb2 + 1023) / 1024) * 32;  // whole 1024-pair chunks
    const bool tk = mode == VMOBA_SEL_TOPK_GLOBAL;
    const void* fn = tk ? reinterpret_cast<const void*>(global_select_kernel<true>)
                        : reinterpret_cast<const void*>(global_select_kernel<false>);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) !=
        hipSuccess)
      return VMOBA_ERR_HIP;
    if (tk)
      global_select_kernel<true><<<groups, kSelThreads, words * sizeof(uint32_t), st>>>(
          g.Nb, tau, topk, scores, row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores);
    else
      global_select_kernel<false><<<groups, kSelThreads, words * sizeof(uint32_t), st>>>(
          g.Nb, tau, topk, scores, row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores);
    return launch_status();
  }
  // local strategies: bitmap and row statistics behind the scores in the workspace
  const size_t W = (size_t(g.Nb) + 31) / 32;
  unsigned char* base = static_cast<unsigned char*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + align256(groups * nb2 * sizeof(float)));
  float* rowstats = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(bitmap) +
                                             align256(groups * size_t(g.Nb) * W * 4));
  stt = mode == VMOBA_SEL_TOPK_LOCAL
            ? launch_local<true>(g, tau, topk, scores, bitmap, rowstats, norm_scores, st)
            : launch_local<false>(g, tau, topk, scores, bitmap, rowstats, norm_scores, st);
  if (stt) return stt;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(emit_lists_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds) != hipSuccess)
    return VMOBA_ERR_HIP;
  emit_lists_kernel<<<groups, kSelThreads, size_t(g.Nb) * W * 4, st>>>(
      g.Nb, bitmap, rowstats, row_ptr, col_idx, col_ptr, row_idx, head_stats);
  return launch_status();
}

}  // namespace vmoba
