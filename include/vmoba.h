/*
 * vmoba.h — C ABI of the VMoBA block-sparse attention layer for AMD MI355X (gfx950).
 *
 * One VMoBA attention layer (papernotes.org reading notes "VMoBA: Mixture-of-Block
 * Attention for Video Diffusion Models", 方法详解/整体框架; paperlayer.ai digest of
 * arXiv 2506.23858, §3.1 Fig. 2) runs as four stream-ordered calls:
 *
 *   vmoba_partition_pool   block means of Q and K under the layer's 1D/2D/3D partition
 *   vmoba_select           per-head global block selection with the cumulative mass tau
 *   vmoba_select_mode      the ablation's other selection strategies (top-k, local pools)
 *   vmoba_sparse_attn_fwd  attention restricted to the selected block pairs
 *   vmoba_sparse_attn_bwd  its gradient with the selection held constant
 *
 * and the token-granular reading of the selection (vmoba_select_tokens, with
 * vmoba_token_attn_fwd / _bwd under its per-token mask),
 * plus a dense flash-attention pair in the same library as the speed baseline.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named q, k, v, o, dout, dq, dk, dv, q_pool, k_pool, lse, row_ptr, col_idx,
 *   col_ptr, row_idx, head_stats, norm_scores and ws are DEVICE pointers; `p` and `bytes`
 *   / `nb` out-parameters are HOST pointers.  `stream` is a hipStream_t (NULL = the null
 *   stream).  Every GPU call only enqueues work on `stream` and returns; no call
 *   allocates or frees device memory or synchronises, and calls from several host
 *   threads are safe.  The library keeps two kinds of state: vmoba_sparse_attn_bwd's
 *   second stream (one per host thread and device, kept until the process ends) and
 *   vmoba_sparse_attn_bwd_noalloc's fixed scratch array (one per device).  The caller
 *   owns every buffer.
 * - Token layout: Q, K, V, O, dO, dQ, dK, dV are contiguous [B][L][Hh][d] with
 *   L = T*H*W and token (t, h, w) at index (t*H + h)*W + w (frame-first flattening).
 *   Element type is `dtype` (bf16 or fp32) for Q, K, V, O, dO and `grad_dtype` for
 *   dQ, dK, dV.
 * - Pooled tensors are fp32 [B][Hh][N_b][d]; lse is fp32 [B][Hh][L] (natural log).
 * - Blocks: N_b = (T/bt)*(H/bh)*(W/bw) blocks of S = bt*bh*bw tokens, numbered row-major
 *   over the block grid; tokens inside a block are row-major over (dt, dh, dw).
 * - Selection lists per (b, h) "head group" g = b*Hh + h, each with capacity N_b*N_b:
 *     row_ptr [G][N_b+1], col_idx [G][N_b*N_b]   rows = query blocks, ascending columns
 *     col_ptr [G][N_b+1], row_idx [G][N_b*N_b]   rows = key blocks, ascending rows
 *   Offsets in row_ptr / col_ptr are local to the head group (first entry 0).
 * - Errors: argument errors are detected on the host before anything is enqueued and
 *   leave every output untouched.  A failed kernel launch returns VMOBA_ERR_HIP.
 *   Faults inside kernels surface at the caller's next synchronisation.  The attention
 *   kernels skip list entries outside [0, N_b) and clamp list lengths to N_b, so a
 *   malformed caller-built list cannot make them read out of bounds.
 */
#ifndef VMOBA_H
#define VMOBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VMOBA_OK = 0,
  VMOBA_ERR_NULL = 1,       /* a required pointer is NULL                              */
  VMOBA_ERR_SHAPE = 2,      /* non-positive size, or block shape does not divide T,H,W */
  VMOBA_ERR_MODE = 3,       /* block shape inconsistent with layer_idx mod 3           */
  VMOBA_ERR_TAU = 4,        /* tau not in (0, 1] or not finite                         */
  VMOBA_ERR_DTYPE = 5,      /* dtype not VMOBA_BF16 / VMOBA_FP32                       */
  VMOBA_ERR_HEAD_DIM = 6,   /* head_dim not 64 or 128                                  */
  VMOBA_ERR_WORKSPACE = 7,  /* ws too small (see vmoba_workspace_size)                 */
  VMOBA_ERR_OVERFLOW = 8,   /* an index or element count exceeds the int32 range used  */
  VMOBA_ERR_HIP = 9,        /* the HIP runtime reported an error at launch             */
  VMOBA_ERR_OP = 10,        /* unknown op in vmoba_workspace_size                      */
  VMOBA_ERR_SELECT = 11,    /* unknown selection mode, or top-k count k < 1            */
  VMOBA_ERR_SCRATCH = 12    /* problem needs more than the fixed no-allocation scratch */
} vmoba_status;

typedef enum { VMOBA_BF16 = 0, VMOBA_FP32 = 1 } vmoba_dtype;

typedef enum {
  VMOBA_OP_POOL = 0,
  VMOBA_OP_SELECT = 1,
  VMOBA_OP_SPARSE_FWD = 2,
  VMOBA_OP_SPARSE_BWD = 3,
  VMOBA_OP_DENSE_FWD = 4,
  VMOBA_OP_DENSE_BWD = 5,
  VMOBA_OP_SELECT_TOKENS = 6,
  VMOBA_OP_TOKEN_FWD = 7,
  VMOBA_OP_TOKEN_BWD = 8
} vmoba_op;

/* Problem description (host struct, passed by pointer, read during the call only). */
typedef struct {
  int32_t batch, heads, head_dim; /* B, Hh, d (d in {64, 128})                          */
  int32_t T, H, W;                /* video latent extents; L = T*H*W                    */
  int32_t layer_idx;              /* >= 0; partition mode = layer_idx % 3               */
  int32_t bt, bh, bw;             /* block shape: 1D needs (bh,bw)=(H,W), 2D needs bt=T */
  int32_t dtype;                  /* vmoba_dtype of Q, K, V, O and dO                   */
  int32_t grad_dtype;             /* vmoba_dtype of dQ, dK, dV (fp32 = the fp32
                                     accumulators unrounded; fp32 inputs need fp32)     */
} vmoba_problem;

/* Library version string (static storage). */
const char* vmoba_version(void);

/* Name of a status code (static storage; "unknown status" for other values). */
const char* vmoba_status_string(int status);

/* Host-only checks of `p`: sizes, divisibility, the partition mode of papernotes
 * 关键设计 1 (l mod 3 = 0 -> 1D whole frames, 1 -> 2D across all frames, 2 -> 3D box),
 * dtype, head_dim and int32 ranges.  No HIP call. */
int vmoba_validate(const vmoba_problem* p);

/* Number of blocks N_b of the partition (host-only). */
int vmoba_num_blocks(const vmoba_problem* p, int32_t* nb);

/* Workspace bytes `op` needs for `p` (host-only; 0 is a valid answer). */
int vmoba_workspace_size(const vmoba_problem* p, int op, size_t* bytes);

/* Block-mean pooling (papernotes 关键设计 1, B = mean(K')): q_pool[b][h][i] is the mean of
 * Q over block i's tokens for head h, k_pool likewise for K; the query blocks use the
 * key partition.  Accumulation is fp32.  q, k: [B][L][Hh][d] dtype.  q_pool, k_pool:
 * fp32 [B][Hh][N_b][d], written in full. */
int vmoba_partition_pool(const vmoba_problem* p, const void* q, const void* k,
                         float* q_pool, float* k_pool, void* stream);

/* Global block selection with the threshold tau (papernotes 关键设计 2 and 3; paperlayer
 * §3.3-§3.4).  Per head group: s_ij = <q_pool_i, k_pool_j>/sqrt(d) (fp32), normalised
 * by a softmax over all N_b^2 pairs; the pairs are ranked in descending order (exact
 * ties by ascending i*N_b + j) and the shortest prefix whose normalised mass is >= tau
 * is kept; every query block also keeps its own key block (i, i).
 * Outputs: row_ptr/col_idx (CSR) and col_ptr/row_idx (CSC) as described above, entries
 * past the list length are left unwritten; head_stats fp32 [G][4] = {k*, nnz, mass of
 * the prefix, normalised score of the k*-th pair}; norm_scores (may be NULL) fp32
 * [G][N_b][N_b] normalised scores.  ws: vmoba_workspace_size(VMOBA_OP_SELECT) bytes. */
int vmoba_select(const vmoba_problem* p, const float* q_pool, const float* k_pool,
                 float tau, int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr,
                 int32_t* row_idx, float* head_stats, float* norm_scores, void* ws,
                 size_t ws_bytes, void* stream);

/* Selection strategies.  THRESHOLD_GLOBAL is vmoba_select.  The other three are the
 * strategies paperlayer §4.4 (Table 3) compares it with, each dropping one or both of its
 * two ingredients:
 *   TOPK_GLOBAL       the topk highest pairs of the head group's global pool;
 *   THRESHOLD_LOCAL   every query-block row is its own pool, normalised by a softmax over
 *                     the row; the shortest prefix of the row with mass >= tau;
 *   TOPK_LOCAL        the topk highest key blocks of every query-block row (MoBA's rule).
 * Order, ties (lower index first) and the forced diagonal are those of vmoba_select; a
 * topk at least the pool size keeps the whole pool. */
typedef enum {
  VMOBA_SEL_THRESHOLD_GLOBAL = 0,
  VMOBA_SEL_TOPK_GLOBAL = 1,
  VMOBA_SEL_THRESHOLD_LOCAL = 2,
  VMOBA_SEL_TOPK_LOCAL = 3
} vmoba_selection;

/* Block selection under `mode` (a vmoba_selection): tau is checked and used by the
 * threshold modes (0 < tau <= 1), topk by the top-k modes (topk >= 1, else
 * VMOBA_ERR_SELECT).  Outputs as vmoba_select; for the local modes head_stats = {sum
 * over rows of the prefix lengths, nnz, mean over rows of the prefix mass, mean over rows
 * of the smallest normalised score in the prefix} and norm_scores holds the
 * row-normalised scores.  ws: vmoba_workspace_size(VMOBA_OP_SELECT) bytes. */
int vmoba_select_mode(const vmoba_problem* p, const float* q_pool, const float* k_pool,
                      int mode, float tau, int32_t topk, int32_t* row_ptr, int32_t* col_idx,
                      int32_t* col_ptr, int32_t* row_idx, float* head_stats,
                      float* norm_scores, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention forward (papernotes 方法详解/整体框架; paperlayer §3.1): for every
 * query token x of query block i, O_x = softmax over the keys of the blocks listed in row
 * i of the CSR of q_x.k_y/sqrt(d), applied to V; lse_x = log-sum-exp of those logits.
 * Any CSR may be passed (e.g. one built from a caller's mask); every listed row must be
 * non-empty for its O rows to be defined.  o: [B][L][Hh][d] dtype; lse fp32 [B][Hh][L].
 * ws: vmoba_workspace_size(VMOBA_OP_SPARSE_FWD) bytes (may be 0 / NULL). */
int vmoba_sparse_attn_fwd(const vmoba_problem* p, const void* q, const void* k,
                          const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                          void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Gradient of vmoba_sparse_attn_fwd for upstream dout with the selection held constant:
 * dV = P^T dO, dS = P*(dO V^T - rowsum(dO*O)), dQ = dS K/sqrt(d), dK = dS^T Q/sqrt(d)
 * with P = exp(q.k/sqrt(d) - lse) on the selected pairs.  The CSC must describe the same
 * pairs as the CSR.  o, lse: outputs of the forward.  dq, dk, dv: [B][L][Hh][d]
 * grad_dtype, written in full (rows of key tokens no query attends to get zeros).  With
 * grad_dtype bf16 each gradient is the round-to-nearest-even of its fp32 value.
 * ws: vmoba_workspace_size(VMOBA_OP_SPARSE_BWD) bytes.  The dQ pass runs on a second
 * stream of the device (one per calling host thread, made on its first call there and
 * kept), forked from `stream` after delta and joined back before the call returns: work
 * queued on `stream` afterwards sees all three gradients, and the call may be captured
 * in a graph from `stream`.  If that stream cannot be made, or this thread's first call
 * comes while `stream` is being captured, the passes run one after the other on
 * `stream`. */
int vmoba_sparse_attn_bwd(const vmoba_problem* p, const void* q, const void* k,
                          const void* v, const void* o, const float* lse,
                          const void* dout, const int32_t* row_ptr,
                          const int32_t* col_idx, const int32_t* col_ptr,
                          const int32_t* row_idx, void* dq, void* dk, void* dv, void* ws,
                          size_t ws_bytes, void* stream);

/* The three kernels of vmoba_sparse_attn_bwd as separate calls, each enqueueing exactly
 * one kernel, for callers that schedule or time them individually.  delta is a caller
 * buffer, fp32 [B][Hh][L].  Run _delta first (delta_x = rowsum(dO_x * O_x)); _dkdv (walks
 * the column lists: dK and dV of every key block) and _dq (walks the row lists: dQ of
 * every query block) only read delta and may run in either order or concurrently. */
int vmoba_sparse_attn_bwd_delta(const vmoba_problem* p, const void* o, const void* dout,
                                float* delta, void* stream);

int vmoba_sparse_attn_bwd_dkdv(const vmoba_problem* p, const void* q, const void* k,
                               const void* v, const float* lse, const float* delta,
                               const void* dout, const int32_t* col_ptr,
                               const int32_t* row_idx, void* dk, void* dv, void* stream);

int vmoba_sparse_attn_bwd_dq(const vmoba_problem* p, const void* q, const void* k,
                             const void* v, const float* lse, const float* delta,
                             const void* dout, const int32_t* row_ptr,
                             const int32_t* col_idx, void* dq, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops that forbid hipMalloc): vmoba_sparse_attn_bwd with no workspace argument.  Same
 * arguments, results and kernels as vmoba_sparse_attn_bwd.  Its one scratch buffer, delta
 * (fp32 [B][Hh][L]), is a fixed device array of VMOBA_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends; the call allocates nothing.
 * B * Hh * L * 4 > VMOBA_NOALLOC_SCRATCH_BYTES is rejected with VMOBA_ERR_SCRATCH before
 * anything is enqueued (16 MiB: up to 4,194,304 rows, e.g. 12 heads at 349,525 tokens).
 * The first call on a device looks the array's device address up (a runtime query, with
 * that device made current for the lookup); the stream's device is the one used.  Every
 * call on one GPU shares that GPU's array: each call rewrites it in full before reading
 * it, but calls that overlap in time on one GPU (e.g. on two streams) race on it. */
#define VMOBA_NOALLOC_SCRATCH_BYTES (16u << 20)

int vmoba_sparse_attn_bwd_noalloc(const vmoba_problem* p, const void* q, const void* k,
                                  const void* v, const void* o, const float* lse,
                                  const void* dout, const int32_t* row_ptr,
                                  const int32_t* col_idx, const int32_t* col_ptr,
                                  const int32_t* row_idx, void* dq, void* dk, void* dv,
                                  void* stream);

/* Token-granular selection: papernotes 关键设计 2 read with q_i all of the head's query
 * tokens (s x d) instead of block means.  The pool of a head group is every (query token
 * x, key block j) pair, L * N_b of them, s_xj = <q_x, k_pool_j>/sqrt(d) (fp32), normalised
 * by a softmax over the whole pool; ranked descending (exact ties by ascending
 * x*N_b + j), the shortest prefix whose normalised mass is >= tau is kept, and every token
 * also keeps its own block.  q: [B][L][Hh][d] bf16 (fp32 problems are rejected with
 * VMOBA_ERR_DTYPE); k_pool: fp32 [B][Hh][N_b][d] from vmoba_partition_pool.
 * Outputs:
 *   token_mask uint32 [G][L][W], W = ceil(N_b/32): bit (j & 31) of word (j >> 5) of token
 *              x is set iff x attends to key block j (written in full);
 *   row_ptr/col_idx, col_ptr/row_idx: CSR/CSC of the union over each query block's tokens
 *              (query block i lists key block j iff some token of i selected j);
 *   head_stats fp32 [G][4] = {k*, number of selected (token, block) pairs, prefix mass,
 *              normalised score of the k*-th pair}.
 * Needs L * N_b * G < 2^31 (VMOBA_ERR_OVERFLOW) and N_b <= 1024 (VMOBA_ERR_SHAPE).
 * ws: vmoba_workspace_size(VMOBA_OP_SELECT_TOKENS) bytes (4 L N_b G bytes of scores and
 * small tables). */
int vmoba_select_tokens(const vmoba_problem* p, const void* q, const float* k_pool, float tau,
                        uint32_t* token_mask, int32_t* row_ptr, int32_t* col_idx,
                        int32_t* col_ptr, int32_t* row_idx, float* head_stats, void* ws,
                        size_t ws_bytes, void* stream);

/* Attention under a token mask: query token x of query block i attends to the keys of the
 * blocks j listed in CSR row i whose bit j is set in x's token_mask row (layout as
 * vmoba_select_tokens).  A token with no such key gets O = 0 and lse = -inf.  bf16 only,
 * blocks of at least 4 tokens (VMOBA_ERR_SHAPE otherwise).  ws:
 * vmoba_workspace_size(VMOBA_OP_TOKEN_FWD) bytes (the mask re-indexed by list position,
 * 4 G L ceil(N_b/32) bytes). */
int vmoba_token_attn_fwd(const vmoba_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const uint32_t* token_mask, void* o, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/* Gradient of vmoba_token_attn_fwd with the selection held constant (formulas of
 * vmoba_sparse_attn_bwd over the masked pairs).  The CSC must list the same block pairs as
 * the CSR.  ws: vmoba_workspace_size(VMOBA_OP_TOKEN_BWD) bytes. */
int vmoba_token_attn_bwd(const vmoba_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* col_ptr, const int32_t* row_idx,
                         const uint32_t* token_mask, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream);

/* Dense flash attention over all L x L pairs in natural token order (the baseline the
 * sparse layer replaces).  Shapes as the sparse calls; the block shape is ignored apart
 * from validation. */
int vmoba_dense_attn_fwd(const vmoba_problem* p, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

int vmoba_dense_attn_bwd(const vmoba_problem* p, const void* q, const void* k,
                         const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, void* ws,
                         size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VMOBA_H */
