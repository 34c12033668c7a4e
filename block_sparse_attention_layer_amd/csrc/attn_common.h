// Shared pieces of the attention kernels: parameters, head-group decoding, the
// gathered token stream of a block list, and list compaction into LDS.
//
// A query block i attends to the concatenated tokens of the key blocks in its list
// (papernotes 方法详解/整体框架: attention only on the selected blocks).  That concatenation
// is walked as one "token stream": position p is token p % S of the (p / S)-th listed
// block, so tiles of the stream cross block boundaries and only the stream's last tile
// is ragged.  The same stream, built from a column list, gives the query tokens that
// attend to one key block in the backward pass.
#pragma once

#include "device_common.h"

namespace vmoba {

struct AttnParams {
  Geom g;
  const void* q;
  const void* k;
  const void* v;
  const void* o;       // forward output (read by the backward)
  const void* dout;
  void* out;           // forward: O; unused in backward
  float* lse;          // [G][L]
  float* delta;        // [G][L] (backward)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  int32_t tiles;       // tiles per block row (query tiles fwd/dq, key tiles dkdv)
  float scale;         // 1/sqrt(d)
  float scale_log2;    // log2(e)/sqrt(d)
  // token-granular selection: per query token, bits over key blocks (tokmask) and over the
  // positions of its block's list (posmask); mwords = ceil(N_b/32) words per token
  const uint32_t* tokmask;
  const uint32_t* posmask;
  int32_t mwords;
  // sparse launches: take each head group's lists longest first (sparse_item)
  int32_t ordered;
};

// A query token's row of the list-position mask (bit li of word li >> 5: the li-th key
// block listed for its query block is attended).  A key tile covers fewer than 32 list
// positions (blocks of at least 4 tokens, tiles of at most 64 keys), so two cached words
// serve a tile; they are refetched when the tile's first position enters another word.
struct PosMask {
  const uint32_t* row;
  int W, wi;
  uint32_t w0, w1;
  __device__ __forceinline__ void init(const uint32_t* r, int words) {
    row = r;
    W = words;
    wi = -1;
    w0 = w1 = 0u;
  }
  __device__ __forceinline__ void fetch(int li0) {
    const int n = li0 >> 5;
    if (n != wi) {
      wi = n;
      w0 = n < W ? row[n] : 0u;
      w1 = n + 1 < W ? row[n + 1] : 0u;
    }
  }
  // positions past the cached pair (keys past the stream's end) read garbage bits; the
  // ragged-tile mask covers them
  __device__ __forceinline__ bool keep(int li) const {
    const int rel = li - 32 * wi;
    return (((rel < 32) ? w0 : w1) >> (rel & 31)) & 1u;
  }
};

// The dispatcher hands workgroup b to XCD b % 8, and each XCD has its own L2; all XCDs
// share the device-wide Infinity Cache.  Work items are numbered head group by head
// group, and inside a head group so that neighbouring items share K/V (the tiles of one
// query block, then neighbouring blocks).  The launch index is mapped so that the 8 XCDs
// advance through the head groups together (one head group's K/V in the shared cache at
// a time), each XCD taking one contiguous eighth of the current head group's items.
// Returns -1 for the padding workgroups of the rounded-up grid (they exit at once).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_item(int bid, int groups, int per_group) {
  const int chunk = (per_group + kXcds - 1) / kXcds;
  const int k = bid / kXcds, x = bid % kXcds;
  const int grp = k / chunk;
  const int local = x * chunk + k % chunk;
  return (grp < groups && local < per_group) ? grp * per_group + local : -1;
}

inline int xcd_grid(int groups, int per_group) {
  return groups * kXcds * ((per_group + kXcds - 1) / kXcds);
}

// Blocks of at most this many tokens get an LDS table of in-block token offsets.
constexpr int kOffsetTable = 2048;

__device__ __forceinline__ int xcd_item(int bid, int items) {
  const int per = (items + kXcds - 1) / kXcds;
  const int item = (bid % kXcds) * per + bid / kXcds;
  return item < items ? item : -1;
}

inline int xcd_grid(int items) { return ((items + kXcds - 1) / kXcds) * kXcds; }

// Element offset of token x of head group grp in a [B][L][Hh][D] tensor.
__device__ __forceinline__ int32_t row_offset(const Geom& g, int grp, int32_t x) {
  const int b = grp / g.Hh, h = grp - b * g.Hh;
  return ((b * g.L + x) * g.Hh + h) * g.D;
}

// Token of stream position p over the block list `lst` (already validated).
__device__ __forceinline__ int32_t stream_token(const Geom& g, const int32_t* lst,
                                                uint32_t p) {
  const uint32_t bi = fd_div(p, g.div_S);
  const uint32_t r = p - bi * uint32_t(g.S);
  return block_base(g, uint32_t(lst[bi])) + block_offset(g, r);
}

// Copy the entries of list[0, n) that lie in [0, Nb) into lds[], keeping their order;
// returns how many were kept.  All threads of the workgroup must call it.  `scratch`
// needs one int per wave.
template <int NT>
__device__ int compact_list(const int32_t* __restrict__ list, int n, int Nb, int32_t* lds,
                            int32_t* scratch) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int kept = 0;
  for (int base = 0; base < n; base += NT) {
    const int t = base + threadIdx.x;
    const int32_t j = t < n ? list[t] : -1;
    const bool ok = j >= 0 && j < Nb;
    const unsigned long long m = __ballot(ok);
    if (lane == 0) scratch[w] = __popcll(m);
    __syncthreads();
    int off = kept, tot = 0;
    for (int i = 0; i < NWV; ++i) {
      if (i < w) off += scratch[i];
      tot += scratch[i];
    }
    if (ok) lds[off + __popcll(m & ((1ull << lane) - 1ull))] = j;
    kept += tot;
    __syncthreads();
  }
  return kept;
}

// Validated [start, start + len) range of list `which` of head group grp.
__device__ __forceinline__ void list_range(const Geom& g, const int32_t* ptr, int grp,
                                           int row, int* start, int* len) {
  const int cap = g.Nb * g.Nb;
  const int32_t* rp = ptr + grp * (g.Nb + 1);
  int s = rp[row], e = rp[row + 1];
  s = min(max(s, 0), cap);
  e = min(max(e, s), min(cap, s + g.Nb));
  *start = s;
  *len = e - s;
}

// Work item of a sparse attention workgroup: head group, block (whose row or column
// list it walks) and tile of that block.  Workgroups start roughly in launch order and
// their cost grows with the length of their list, which varies several-fold between the
// blocks of a head under a global selection; taken in block order, the longest lists
// can start last and leave a tail in which most of the chip idles.  With `ordered`, the
// blocks of each head group are taken longest list first (ties by ascending block
// index), and launch index b goes to XCD x = b % 8, which takes the sorted positions
// p, p+8, p+16, ... of the current head group g, p = (x + g) mod 8, each with all of its
// tiles in a row (they share their stream in that XCD's L2).  Rotating p with g evens
// out the XCDs' shares when N_b is not a multiple of 8.  Head groups still follow each
// other (one or two heads' K/V in the shared cache at a time).
// The rank of every list is found inside the workgroup: list lengths into `lds` (room
// for N_b rounded up to 4), then a count over all pairs, O(N_b^2 / NT) steps a thread.
struct SparseItem {
  int grp, blk, tile;
};

inline int sparse_grid(int groups, int nb, int tiles) {
  return groups * kXcds * ((nb + kXcds - 1) / kXcds) * tiles;
}

// Lists are ranked inside the workgroups only up to this many blocks a head: the count
// over all pairs costs O(N_b^2 / NT) per workgroup, while the work of a workgroup shrinks
// as N_b grows (smaller blocks).
constexpr int kOrderedMaxBlocks = 512;

// Grid of a bf16 attention launch (a.tiles set); sets a.ordered for sparse launches.
template <bool DENSE>
inline int launch_grid(AttnParams& a, int rows) {
  if (DENSE) return xcd_grid(a.g.B * a.g.Hh, rows * a.tiles);
  a.ordered = a.g.Nb <= kOrderedMaxBlocks;
  return sparse_grid(a.g.B * a.g.Hh, a.g.Nb, a.tiles);
}

// Returns false for the padding workgroups of the grid (the whole workgroup alike).
template <int NT>
__device__ bool sparse_item(const Geom& g, const int32_t* ptr, int tiles, bool ordered,
                            int32_t* lds, int32_t* pick, SparseItem* it) {
  const int nb = g.Nb;
  const int chunk = ((nb + kXcds - 1) / kXcds) * tiles;
  const int k = blockIdx.x / kXcds, x = blockIdx.x % kXcds;
  const int grp = k / chunk, r = k - grp * chunk;
  const int pos = (r / tiles) * kXcds + ((x + grp) & (kXcds - 1));
  if (grp >= g.B * g.Hh || pos >= nb) return false;
  it->grp = grp;
  it->tile = r % tiles;
  it->blk = pos;
  if (!ordered) return true;
  const int nb4 = (nb + 3) & ~3;
  for (int i = threadIdx.x; i < nb4; i += NT) {
    int len = -1;   // padding: below every real length
    if (i < nb) {
      int s, l;
      list_range(g, ptr, grp, i, &s, &l);
      len = l;
    }
    lds[i] = len;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += NT) {
    const int lj = lds[j];
    int rank = 0;
    for (int i = 0; i < nb4; i += 4) {
      const int4 l4 = *reinterpret_cast<const int4*>(lds + i);
      rank += (l4.x > lj) + (l4.y > lj) + (l4.z > lj) + (l4.w > lj);
      rank += (l4.x == lj && i < j) + (l4.y == lj && i + 1 < j) + (l4.z == lj && i + 2 < j) +
              (l4.w == lj && i + 3 < j);
    }
    if (rank == pos) *pick = j;   // ranks are a permutation: exactly one thread writes
  }
  __syncthreads();
  it->blk = *pick;
  __syncthreads();   // lds and pick are the caller's to reuse
  return true;
}

// ---------------------------------------------------------------------------------
// Row-major bf16 tiles in LDS, filled by direct global->LDS loads.
//
// A tile row holds one token's D values (D*2 bytes, 16-byte chunks).  Chunk c of row r
// is stored at chunk position c ^ swz(r).  The swizzle permutes the chunks of every row
// so that (1) 16 consecutive rows read at one chunk position (MFMA operands via
// ds_read_b128) hit 16 different 4-bank groups, and (2) a 4-row x 4-chunk patch (the
// transposing ds_read_b64_tr_b16 of 16 lanes) also covers all 64 banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of chunk c of row r inside a tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + 16 * (c ^ swz<D>(r));
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// Direct global->LDS loads go through buffer instructions.  The flat-addressed form
// (global_load_lds) is one the compiler must assume may also touch LDS through the LDS
// counter, so while any is in flight it waits for all of a wave's LDS reads at the first
// use of any one of them; the buffer form is counted on the vector-memory counter only,
// and the LDS reads that feed the matrix cores keep their one-by-one waits.
typedef __amdgpu_buffer_rsrc_t BufRes;

// Word 3 of a CDNA buffer descriptor for raw addressing: 32-bit data format, no index
// stride and no swizzle, so a lane's offset is a plain byte offset from the base.
constexpr int kBufferWord3 = 0x00020000;

// Descriptor of the `bytes` bytes at `base` (reads past the end return zero).
__device__ __forceinline__ BufRes buffer_res(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes),
                                           kBufferWord3);
}

// One wave instruction copies 64 x 16 bytes straight into the LDS range
// [dst, dst + 1024): lane L's chunk comes from byte `off` of the buffer and lands at
// dst + 16 L.  `dst` must be uniform.
__device__ __forceinline__ void load_to_lds16(BufRes r, uint32_t off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)dst, 16, off, 0, 0, 0);
}

// As load_to_lds16 with 4 bytes per lane: lane L's word lands at dst + 4 L.
__device__ __forceinline__ void load_to_lds4(BufRes r, uint32_t off, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)dst, 4, off, 0, 0, 0);
}

// Transposing LDS read: the 16 lanes of a group each name 8 bytes (4 bf16); lane i of
// the group receives element i % 4 of the chunks named by lanes i/4, i/4 + 4, i/4 + 8
// and i/4 + 12 (in that order).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)p);
  return __builtin_bit_cast(u32x2, r);
}

// Wait until this wave's direct-to-LDS loads have landed.
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N of this wave's vector-memory operations are outstanding (the
// oldest complete first); the LDS and export counters are not waited on.  s_waitcnt
// immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most N of this wave's vector-memory operations are outstanding (they
// complete oldest first) and all of its LDS operations have completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier between the steps of a tile pipeline.  Every wave has already waited
// for its own loads of the tile about to be read and for its own LDS reads of the stage
// about to be refilled, so the barrier itself need not drain the direct-to-LDS loads
// still in flight into other stages (a release fence would wait for all of them).  The
// acquire fence keeps the LDS reads and the loads issued after the barrier behind it.
__device__ __forceinline__ void pipeline_barrier() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace vmoba
