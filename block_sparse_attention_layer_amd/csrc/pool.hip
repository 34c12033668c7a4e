// Block-mean pooling of Q and K under the layer's partition (papernotes 关键设计 1:
// B = mean(K') over the rearranged keys; the query blocks use the same partition).
//
// One workgroup per (block, head, batch, Q-or-K).  The block's tokens are gathered by
// arithmetic from the (t, h, w) partition: each token contributes one contiguous
// d-element row of its head, read as 16-byte chunks by consecutive lanes, so a wave
// reads whole rows.  Token slots accumulate in fp32 registers, then an LDS tree adds
// the slots in a fixed order (the result does not depend on scheduling).
#include "device_common.h"

namespace vmoba {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(Geom g, const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ q_pool,
                                                   float* __restrict__ k_pool) {
  constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int CH = D / VEC;             // chunks per row
  constexpr int SLOTS = 256 / CH;         // token slots per pass
  __shared__ float part[SLOTS][D + 1];

  const int blk = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool is_k = blockIdx.z & 1;
  const T* src = is_k ? k : q;
  float* dst = is_k ? k_pool : q_pool;

  const int c = threadIdx.x % CH;
  const int slot = threadIdx.x / CH;
  const int32_t base = block_base(g, blk);
  const size_t row_stride = size_t(g.Hh) * D;
  const T* head0 = src + (size_t(b) * g.L * g.Hh + h) * D + c * VEC;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  constexpr int UNROLL = 4;
  int r = slot;
  for (; r + (UNROLL - 1) * SLOTS < g.S; r += UNROLL * SLOTS) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int32_t x = base + block_offset(g, r + u * SLOTS);
      v[u] = *reinterpret_cast<const u32x4*>(head0 + size_t(x) * row_stride);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_to_f32(v[u][e] & 0xffffu);
          acc[2 * e + 1] += bf16_to_f32(v[u][e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[u][e]);
      }
    }
  }
  for (; r < g.S; r += SLOTS) {
    const int32_t x = base + block_offset(g, r);
    u32x4 v = *reinterpret_cast<const u32x4*>(head0 + size_t(x) * row_stride);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32(v[e] & 0xffffu);
        acc[2 * e + 1] += bf16_to_f32(v[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[slot][c * VEC + e] = acc[e];
  __syncthreads();
  // fixed-order tree over the slots
  for (int half = SLOTS / 2; half > 0; half >>= 1) {
    for (int idx = threadIdx.x; idx < half * D; idx += 256) {
      const int s = idx / D, dd = idx % D;
      part[s][dd] += part[s + half][dd];
    }
    __syncthreads();
  }
  const float inv = 1.0f / float(g.S);
  for (int dd = threadIdx.x; dd < D; dd += 256)
    dst[((size_t(b) * g.Hh + h) * g.Nb + blk) * D + dd] = part[0][dd] * inv;
}

template <typename T, int D>
static void launch_pool_t(const Geom& g, const void* q, const void* k, float* qp,
                          float* kp, hipStream_t s) {
  dim3 grid(g.Nb, g.Hh, g.B * 2);
  pool_kernel<T, D><<<grid, 256, 0, s>>>(g, static_cast<const T*>(q),
                                         static_cast<const T*>(k), qp, kp);
}

int launch_pool(const Geom& g, const void* q, const void* k, float* q_pool,
                float* k_pool, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.dtype == VMOBA_BF16) {
    if (g.D == 128) launch_pool_t<uint16_t, 128>(g, q, k, q_pool, k_pool, s);
    else launch_pool_t<uint16_t, 64>(g, q, k, q_pool, k_pool, s);
  } else {
    if (g.D == 128) launch_pool_t<float, 128>(g, q, k, q_pool, k_pool, s);
    else launch_pool_t<float, 64>(g, q, k, q_pool, k_pool, s);
  }
  return launch_status();
}

}  // namespace vmoba
