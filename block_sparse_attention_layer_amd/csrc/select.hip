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

__global__ __launch_bounds__(kSelThreads) void threshold_select_kernel(
    int Nb, float tau, const float* __restrict__ scores, int32_t* __restrict__ row_ptr,
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
    const double r = ceil(double(tau) * double(z));
    sh.R = (unsigned long long)r;
    sh.select_all = (tau >= 1.0f || sh.R > z) ? 1u : 0u;
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
          if (acc + sh.mass[dg] >= sh.R && sh.cnt[dg] > 0) break;
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
    const unsigned long long need = sh.R - sh.above_mass;
    unsigned long long t = e1 ? (need + e1 - 1) / e1 : 1;
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

int launch_select(const Geom& g, const float* q_pool, const float* k_pool, float tau,
                  int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr,
                  int32_t* row_idx, float* head_stats, float* norm_scores, void* ws,
                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int groups = g.B * g.Hh;
  float* scores = static_cast<float*>(ws);
  const float scale = 1.0f / sqrtf(float(g.D));
  dim3 sgrid((g.Nb + 31) / 32, (g.Nb + 31) / 32, groups);
  if (g.D == 128)
    block_scores_kernel<128><<<sgrid, 64, 0, st>>>(g.Nb, q_pool, k_pool, scores, scale);
  else
    block_scores_kernel<64><<<sgrid, 64, 0, st>>>(g.Nb, q_pool, k_pool, scores, scale);
  int stt = launch_status();
  if (stt) return stt;
  const size_t words = ((size_t(g.Nb) * g.Nb + 1023) / 1024) * 32;  // whole 1024-pair chunks
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(threshold_select_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          int(size_t(kMaxBlocks) * kMaxBlocks / 8)) != hipSuccess)
    return VMOBA_ERR_HIP;
  threshold_select_kernel<<<groups, kSelThreads, words * sizeof(uint32_t), st>>>(
      g.Nb, tau, scores, row_ptr, col_idx, col_ptr, row_idx, head_stats, norm_scores);
  return launch_status();
}

}  // namespace vmoba
