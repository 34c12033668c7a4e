// vmoba_sparse_attn_bwd_noalloc: the block-sparse backward without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops).  The one buffer the backward needs beyond its inputs and outputs, delta =
// rowsum(dO * O) (fp32 [B][Hh][L]), lives in a file-scope device array of fixed size.
//
// Each GPU holds its own copy of the array for the life of the process.  Host code never
// passes the array's name to a kernel or a copy (on the host that name is only a stand-in,
// not a device address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and cached.
//
// All calls on one GPU share its array.  Every call rewrites all of delta before reading
// it, so nothing carries over between calls, but two calls that overlap in time on one GPU
// (on different streams) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/vmoba.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(VMOBA_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_init_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on `dev`, looked up on first use with `dev` current.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return VMOBA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_init_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return VMOBA_ERR_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return VMOBA_ERR_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return VMOBA_ERR_HIP;
      if (e != hipSuccess || !p) return VMOBA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return VMOBA_OK;
}

}  // namespace

extern "C" int vmoba_sparse_attn_bwd_noalloc(const vmoba_problem* p, const void* q,
                                             const void* k, const void* v, const void* o,
                                             const float* lse, const void* dout,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             const int32_t* col_ptr, const int32_t* row_idx,
                                             void* dq, void* dk, void* dv, void* stream) {
  using namespace vmoba;
  int st = validate_problem(p);
  if (st) return st;
  const Geom g = make_geom(p);
  if (g.Nb > kMaxBlocks) return VMOBA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !row_ptr || !col_idx || !col_ptr ||
      !row_idx || !dq || !dk || !dv)
    return VMOBA_ERR_NULL;
  if (size_t(g.B) * g.Hh * g.L * sizeof(float) > kScratchBytes) return VMOBA_ERR_SCRATCH;
  int dev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return VMOBA_ERR_HIP;
  void* base = nullptr;
  if ((st = scratch_on(dev, &base))) return st;
  float* delta = static_cast<float*>(base);
  if ((st = launch_bwd_delta(g, o, dout, delta, stream))) return st;
  if ((st = launch_bwd_dkdv(g, false, q, k, v, lse, delta, dout, col_ptr, row_idx, dk, dv,
                            stream)))
    return st;
  return launch_bwd_dq(g, false, q, k, v, lse, delta, dout, row_ptr, col_idx, dq, stream);
}
