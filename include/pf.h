/*
 * pf.h — C ABI of the prefix/suffix attention library (gfx950 / MI355X).
 *
 * The library computes the attention work of one rollout group trained with
 * a training-time KV cache, as described in "PrefixFlow: Training-Time KV
 * Caching for Schedule-Level Prefix Reuse in LLM RL Training":
 *
 *   Phase A  pf_prefix_fwd             causal attention over the shared prefix,
 *                                      run once per group (§3.1, "Phase A").
 *   Phase B  pf_suffix_attn_fwd        suffix queries over the cached prefix
 *            pf_suffix_attn_bwd_accum  K/V plus their own causal suffix, and its
 *                                      backward, which ADDS the prefix-side
 *                                      gradients gK/gV into fp32 accumulators
 *                                      (§3.1 "Phase B", §3.3, §4.1, §4.2).
 *   Phase C  pf_prefix_bwd_inject      the delayed prefix backward, with the
 *                                      accumulated gK/gV added to the prefix
 *                                      K/V gradients (§3.1 "Phase C", §4.1).
 *   Trees    pf_tree_attn_fwd/bwd      compact rollout-tree rows under an
 *                                      ancestor mask ("HARTS: A Prefix-Sharing
 *                                      Training System for Agentic RL with
 *                                      Hybrid-Attention Models", §2.1, §2.2, §3.4).
 *   Logprob  pf_compact_logprob_fwd/bwd  per-position log-probabilities from
 *                                      compact-row logits (HARTS §3.5).
 *   Windows  pf_tree_suffix_attn_fwd,  a window of rollout trees over a cached
 *            pf_tree_suffix_attn_bwd_accum  prefix, with the prefix-side
 *                                      gradients accumulated (HARTS §3.4,
 *                                      window-scoped reuse and backward);
 *            ..._ranges variants       the cached rows as row ranges of a
 *                                      producer tree (its ancestor rows), and
 *            pf_tree_attn_bwd_inject   the producer tree's backward with the
 *                                      accumulated gradients injected.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors of rows are [tokens, heads, head_dim] with head_dim contiguous,
 *    described by pf_tensor (element strides).  Device pointers, 16-byte
 *    aligned; strides multiples of 8 elements (bf16) or 4 (fp32).  One
 *    tensor's rows (rows x stride_tok elements) must span less than 2 GiB
 *    (PF_ERR_UNSUPPORTED otherwise): the kernels address a head's rows
 *    through 32-bit buffer offsets.
 *  - LSE arrays are fp32 [num_q_heads, rows], contiguous, natural log.
 *  - gK/gV accumulators are fp32 [prefix_len, num_kv_heads, head_dim],
 *    contiguous.
 *  - Suffix and tree structure (cu_seqlens, node_off, parent) are HOST
 *    arrays.  They are validated on the host and passed to the kernels by
 *    value, so no call reads host memory after it returns.
 *  - The caller allocates every device buffer, including the workspace,
 *    sized by pf_workspace_size().  The library allocates nothing, keeps no
 *    state between calls, never synchronises and never frees.  The one
 *    exception is pf_suffix_attn_bwd_accum_noalloc, which takes no workspace:
 *    it runs in a static device array of the library and remembers that
 *    array's address per device.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *    and is asynchronous: a return of PF_OK means "launched".
 *  - Every argument is validated before anything is launched.  On an error
 *    return no HIP call has been made (except PF_ERR_HIP) and no output has
 *    been touched; pf_last_error() gives a message (thread-local).  No C++
 *    exception leaves an entry point.
 *  - Results are bitwise identical from run to run for the same inputs,
 *    call sequence and device; there are no floating-point atomics.
 *  - Calls on different streams may run concurrently unless they write the
 *    same buffers; calls that add into one gK/gV accumulator must be ordered
 *    (the same stream, or events).
 */
#ifndef PF_H_
#define PF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PF_ABI_VERSION 1
/* Suffixes per Phase-B call, or nodes per tree. */
#define PF_MAX_SEGMENTS 256
/* Query heads per call. */
#define PF_MAX_HEADS 256

typedef enum {
  PF_OK = 0,
  PF_ERR_INVALID_ARG = 1,  /* a shape, pointer, stride or structure is invalid   */
  PF_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels implement      */
  PF_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than pf_workspace_size() */
  PF_ERR_HIP = 4           /* a HIP launch failed; see pf_last_error()           */
} pf_status;

typedef enum { PF_F32 = 0, PF_BF16 = 1 } pf_dtype;

typedef enum {
  PF_OP_PREFIX_FWD = 0,
  PF_OP_SUFFIX_FWD = 1,
  PF_OP_SUFFIX_BWD = 2,
  PF_OP_PREFIX_BWD = 3,
  PF_OP_TREE_FWD = 4,
  PF_OP_TREE_BWD = 5,
  PF_OP_TREE_SUFFIX_FWD = 6,
  PF_OP_TREE_SUFFIX_BWD = 7
} pf_op;

/* Attention head configuration of one layer (the caller's local head shard). */
typedef struct {
  int32_t num_q_heads;     /* Hq >= 1                                             */
  int32_t num_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0                             */
  int32_t head_dim;        /* bf16: 128; fp32: 64 or 128                          */
  int32_t dtype;           /* pf_dtype of Q, K, V, O, dO, dQ, dK, dV              */
  float softmax_scale;     /* > 0, or <= 0 for 1/sqrt(head_dim)                   */
  const int32_t* q_to_kv;  /* host [Hq]: KV head read by each query head, every KV
                              head read by exactly Hq/Hkv query heads; or NULL for
                              contiguous groups (query head h reads h / (Hq/Hkv)) */
} pf_attn_desc;

/* A [tokens, heads, head_dim] device tensor; head_dim is contiguous. */
typedef struct {
  void* data;
  int64_t stride_tok;      /* elements between consecutive tokens */
  int64_t stride_head;     /* elements between consecutive heads  */
} pf_tensor;

/* Bytes of device workspace `op` needs.  rows = prefix_len for the prefix
 * ops, the total packed suffix rows for the suffix ops and the compact rows
 * for the tree and tree-window ops.  Pure host arithmetic; never fails (0 for bad args). */
size_t pf_workspace_size(int32_t op, const pf_attn_desc* desc, int32_t prefix_len, int32_t rows);

/* The smallest workspace `op` accepts (same arguments).  For the backward
 * ops, pf_workspace_size() adds a buffer for dS (num_q_heads x
 * (ceil256(prefix_len) + ceil256(rows)) x ceil256(rows) values of the input
 * dtype, bf16 or fp32; prefix_len counts as 0 for Phase C and trees): with it
 * the backward stores dS once and forms dQ from it instead of recomputing S
 * and dP.  The buffer is used only while one query head's share stays below
 * 2 GiB.  A workspace of at least this size but smaller than
 * pf_workspace_size() runs the recompute path.
 * Results agree to rounding; each path is deterministic.  Forward ops: equal
 * to pf_workspace_size(). */
size_t pf_workspace_size_min(int32_t op, const pf_attn_desc* desc, int32_t prefix_len,
                             int32_t rows);

/* Phase A (PrefixFlow §3.1 "Phase A: prefix forward"): causal attention of
 * the prefix over itself.
 *   q_p [P, Hq, d], k_p, v_p [P, Hkv, d]  in
 *   o_p [P, Hq, d]                        out (overwritten)
 *   lse_p [Hq, P] fp32                    out (overwritten)              */
pf_status pf_prefix_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor q_p,
                        pf_tensor k_p, pf_tensor v_p, pf_tensor o_p, float* lse_p,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Phase B forward (PrefixFlow §4.1: each suffix query sees every prefix
 * token and its own suffix causally, never another suffix; §4.2: packed
 * suffixes read the cached prefix K/V as one shared read-only block).  The
 * prefix K/V are read in place; nothing is concatenated.
 *   k_p, v_p [P, Hkv, d]                  in  (the cached prefix; P >= 0)
 *   cu_seqlens host [n_suffix + 1]        in  (0 = cu[0] <= cu[1] <= ...; rows = cu[n])
 *   q_s [rows, Hq, d], k_s, v_s [rows, Hkv, d]  in
 *   o_s [rows, Hq, d]                     out
 *   lse_s [Hq, rows] fp32                 out                            */
pf_status pf_suffix_attn_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor k_p,
                             pf_tensor v_p, int32_t n_suffix, const int32_t* cu_seqlens,
                             pf_tensor q_s, pf_tensor k_s, pf_tensor v_s, pf_tensor o_s,
                             float* lse_s, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Phase B backward (PrefixFlow §3.3: prefix backward is linear in the
 * adjoints at the K/V boundary, so per-suffix gK/gV may be summed; §4.1: the
 * cached leaves accumulate them across suffix waves).
 *   (forward arguments as above), o_s, lse_s from pf_suffix_attn_fwd,
 *   do_s [rows, Hq, d]                    in
 *   dq_s [rows, Hq, d]                    out (overwritten)
 *   dk_s, dv_s [rows, Hkv, d]             out (overwritten; own-suffix part only)
 *   gk_acc, gv_acc fp32 [P, Hkv, d]       in/out: this call's prefix-side
 *                                         gradients are ADDED.  The caller zeroes
 *                                         them once per group; replaying a call
 *                                         adds twice.                          */
pf_status pf_suffix_attn_bwd_accum(const pf_attn_desc* desc, int32_t prefix_len,
                                   pf_tensor k_p, pf_tensor v_p, int32_t n_suffix,
                                   const int32_t* cu_seqlens, pf_tensor q_s, pf_tensor k_s,
                                   pf_tensor v_s, pf_tensor o_s, const float* lse_s,
                                   pf_tensor do_s, pf_tensor dq_s, pf_tensor dk_s,
                                   pf_tensor dv_s, float* gk_acc, float* gv_acc,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* The Phase-B backward of pf_suffix_attn_bwd_accum for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation): same arguments and results, without
 * the workspace.  It allocates nothing and calls no allocating routine; its
 * device scratch is a static array of PF_NOALLOC_SCRATCH_BYTES in the
 * library, one per GPU, held until the process ends, on the calling thread's
 * current device (the stream must belong to that device).
 *   Scratch need: about 4 x rows + 8 x Hq x rows bytes (the per-row
 *   visibility tables, D and LSE); a call that needs more returns
 *   PF_ERR_UNSUPPORTED with nothing launched.
 *   It runs the recompute dQ path with every key block whole, so results
 *   agree with pf_suffix_attn_bwd_accum to rounding (fp32 sums in another
 *   order), and are bitwise identical run to run.
 *   Every call on a GPU shares that GPU's scratch: calls that overlap in time
 *   on one GPU (other streams, other threads) race and must be ordered by
 *   the caller.  Nothing in the scratch needs to start at zero; each call
 *   writes what it reads.                                                  */
#define PF_NOALLOC_SCRATCH_BYTES (16u << 20)
pf_status pf_suffix_attn_bwd_accum_noalloc(const pf_attn_desc* desc, int32_t prefix_len,
                                           pf_tensor k_p, pf_tensor v_p, int32_t n_suffix,
                                           const int32_t* cu_seqlens, pf_tensor q_s,
                                           pf_tensor k_s, pf_tensor v_s, pf_tensor o_s,
                                           const float* lse_s, pf_tensor do_s, pf_tensor dq_s,
                                           pf_tensor dk_s, pf_tensor dv_s, float* gk_acc,
                                           float* gv_acc, void* stream);

/* Phase C (PrefixFlow §3.1 "Phase C: prefix backward", §4.1): the causal
 * prefix backward, with the accumulated gK/gV added in fp32 before the one
 * rounding of dK_P/dV_P.
 *   q_p, k_p, v_p, o_p, lse_p             in  (Phase A inputs and outputs)
 *   do_p [P, Hq, d]                       in; do_p.data == NULL means a zero
 *                                         upstream (dQ_P = 0, dK_P = gK_acc)
 *   gk_acc, gv_acc fp32 [P, Hkv, d]       in
 *   dq_p [P, Hq, d] (desc dtype)          out
 *   dk_p, dv_p [P, Hkv, d] (dkv_dtype)    out; dkv_dtype is PF_F32 or desc dtype */
pf_status pf_prefix_bwd_inject(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor q_p,
                               pf_tensor k_p, pf_tensor v_p, pf_tensor o_p, const float* lse_p,
                               pf_tensor do_p, const float* gk_acc, const float* gv_acc,
                               pf_tensor dq_p, pf_tensor dk_p, pf_tensor dv_p, int32_t dkv_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Tree forward (HARTS §2.1: positions with equal token prefixes share one
 * compact row; §2.2: full attention reads ancestor K/V through a tree mask).
 * Nodes are numbered in DFS preorder: parent[0] = -1, parent[i] < i, and a
 * node's subtree occupies consecutive node numbers.  A later node with
 * parent -1 starts another tree of a forest; rows of different trees never
 * see each other (several rollout trees in one call).  Node i owns compact
 * rows [node_off[i], node_off[i+1]).  A row sees the rows of every strict
 * ancestor of its node and the rows of its own node up to itself.
 *   node_off host [n_nodes + 1], parent host [n_nodes]   in
 *   q [C, Hq, d], k, v [C, Hkv, d]        in  (C = node_off[n_nodes])
 *   o [C, Hq, d], lse [Hq, C] fp32        out                            */
pf_status pf_tree_attn_fwd(const pf_attn_desc* desc, int32_t n_nodes, const int32_t* node_off,
                           const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
                           pf_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Tree backward (HARTS §3.4: the backward of a gather of ancestor K/V sums the
 * gradients into the shared compact rows).  dK/dV of a row sum over every
 * descendant row that reads it, and over the query heads of its KV head.
 *   o, lse from pf_tree_attn_fwd; dout [C, Hq, d]    in
 *   dq [C, Hq, d], dk, dv [C, Hkv, d]                out (overwritten)   */
pf_status pf_tree_attn_bwd(const pf_attn_desc* desc, int32_t n_nodes, const int32_t* node_off,
                           const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
                           pf_tensor o, const float* lse, pf_tensor dout, pf_tensor dq,
                           pf_tensor dk, pf_tensor dv, void* workspace, size_t workspace_bytes,
                           void* stream);

/* A sharing window of rollout trees over a cached prefix ("HARTS", §3.4,
 * window-scoped reuse and backward: a producer forward caches the ancestor
 * K/V once; the consumers of a window run only their uncached tokens, and
 * their backward passes accumulate the gradients at that interface before
 * the one producer backward).  The window's rows are compact tree rows as for
 * pf_tree_attn_fwd (DFS preorder, node_off, parent); every row also sees all
 * prefix_len cached prefix rows, which precede the tree root in every
 * trajectory.  The prefix K/V are read in place.  A chain of nodes is one
 * Phase-B suffix; a window per call, several calls adding into one gK/gV,
 * then pf_prefix_bwd_inject is the producer backward.
 *   k_p, v_p [P, Hkv, d]                  in  (the cached prefix; P >= 0)
 *   node_off host [n_nodes + 1], parent host [n_nodes]   in
 *   q [C, Hq, d], k, v [C, Hkv, d]        in  (C = node_off[n_nodes])
 *   o [C, Hq, d], lse [Hq, C] fp32        out                            */
pf_status pf_tree_suffix_attn_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor k_p,
                                  pf_tensor v_p, int32_t n_nodes, const int32_t* node_off,
                                  const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
                                  pf_tensor o, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Backward of a tree window over a cached prefix: dQ of the window rows, dK/dV
 * of the window rows (summed over the descendant rows and query heads that
 * read them), and the window's prefix-side gradients ADDED into gK/gV.
 *   (forward arguments as above), o, lse from pf_tree_suffix_attn_fwd,
 *   dout [C, Hq, d]                       in
 *   dq [C, Hq, d], dk, dv [C, Hkv, d]     out (overwritten)
 *   gk_acc, gv_acc fp32 [P, Hkv, d]       in/out: added into, as in
 *                                         pf_suffix_attn_bwd_accum          */
pf_status pf_tree_suffix_attn_bwd_accum(const pf_attn_desc* desc, int32_t prefix_len,
                                        pf_tensor k_p, pf_tensor v_p, int32_t n_nodes,
                                        const int32_t* node_off, const int32_t* parent,
                                        pf_tensor q, pf_tensor k, pf_tensor v, pf_tensor o,
                                        const float* lse, pf_tensor dout, pf_tensor dq,
                                        pf_tensor dk, pf_tensor dv, float* gk_acc, float* gv_acc,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* A sharing window whose cached rows are row ranges of a producer's compact
 * rows, read in place ("HARTS", §3.4, window-scoped reuse: each internal node
 * of a rollout tree can carry the K/V cache of its ancestor rows, so a
 * consumer window attached under node u reads the rows of u and of every
 * ancestor of u, and its backward adds the interface gradients into exactly
 * those rows before the one producer backward).  Same as
 * pf_tree_suffix_attn_fwd, except that the cached rows are, in trajectory
 * order, the ranges [range_start[i], range_start[i] + range_len[i]) of k_c
 * and v_c instead of one prefix block; nothing is gathered or copied.
 *   k_c, v_c [c_rows, Hkv, d]             in  (the producer's compact K/V)
 *   n_ranges <= PF_MAX_SEGMENTS; range_start, range_len host [n_ranges]  in
 *     (inside [0, c_rows), pairwise disjoint: PF_ERR_INVALID_ARG otherwise;
 *     empty ranges are ignored)
 *   (tree and window tensors as for pf_tree_suffix_attn_fwd)
 * Workspace: pf_workspace_size(PF_OP_TREE_SUFFIX_FWD, desc, prefix_len, C)
 * with prefix_len = pf_ranges_cached_keys(n_ranges, range_len).          */
pf_status pf_tree_suffix_attn_fwd_ranges(const pf_attn_desc* desc, int32_t c_rows, pf_tensor k_c,
                                         pf_tensor v_c, int32_t n_ranges,
                                         const int32_t* range_start, const int32_t* range_len,
                                         int32_t n_nodes, const int32_t* node_off,
                                         const int32_t* parent, pf_tensor q, pf_tensor k,
                                         pf_tensor v, pf_tensor o, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Backward of pf_tree_suffix_attn_fwd_ranges: dQ, dK, dV of the window rows
 * (overwritten) and the window's gradients of the cached rows ADDED into
 * rows of gk_acc, gv_acc fp32 [c_rows, Hkv, d]: cached row r of range i
 * adds into row r, so windows under different nodes of one producer add into
 * the shared ancestor rows.  Workspace as for the forward, with
 * PF_OP_TREE_SUFFIX_BWD.                                                    */
pf_status pf_tree_suffix_attn_bwd_accum_ranges(
    const pf_attn_desc* desc, int32_t c_rows, pf_tensor k_c, pf_tensor v_c, int32_t n_ranges,
    const int32_t* range_start, const int32_t* range_len, int32_t n_nodes,
    const int32_t* node_off, const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
    pf_tensor o, const float* lse, pf_tensor dout, pf_tensor dq, pf_tensor dk, pf_tensor dv,
    float* gk_acc, float* gv_acc, void* workspace, size_t workspace_bytes, void* stream);

/* The padded cached-key count of a ranges call: the sum over ranges of
 * range_len rounded up to 32 (the prefix_len that sizes its workspace);
 * -1 for invalid arguments.  Host arithmetic only.                          */
int32_t pf_ranges_cached_keys(int32_t n_ranges, const int32_t* range_len);

/* The producer backward of a rollout tree whose rows were read by consumer
 * windows ("HARTS", §3.4: the consumers' interface gradients are accumulated
 * before the one producer backward): pf_tree_attn_bwd with gk_acc, gv_acc
 * fp32 [C, Hkv, d] added to the rows' K/V gradients in fp32 before the one
 * rounding, as pf_prefix_bwd_inject does for a flat prefix.
 *   dout.data == NULL means a zero upstream (dQ = 0, dK = gK, dV = gV)
 *   dq [C, Hq, d] (desc dtype); dk, dv [C, Hkv, d] (dkv_dtype: PF_F32 or
 *   the desc dtype)                                          out (overwritten) */
pf_status pf_tree_attn_bwd_inject(const pf_attn_desc* desc, int32_t n_nodes,
                                  const int32_t* node_off, const int32_t* parent, pf_tensor q,
                                  pf_tensor k, pf_tensor v, pf_tensor o, const float* lse,
                                  pf_tensor dout, const float* gk_acc, const float* gv_acc,
                                  pf_tensor dq, pf_tensor dk, pf_tensor dv, int32_t dkv_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Compact log-probability recovery ("HARTS" §3.5): logits exist once per
 * compact row; each semantic position s reads its row m(s) and target y_s,
 *   logp_s = z[m(s), y_s] - log sum_v exp z[m(s), v],
 * so neither direction forms S x V logits or gradients.  Positions are given
 * grouped by row: the positions of row c are pos[row_ptr[c] .. row_ptr[c+1]).
 *   z [n_rows, vocab] (dtype PF_BF16 or PF_F32), row stride z_stride elements
 *     (>= vocab, a multiple of 16 bytes), 16-byte aligned      in
 *   row_ptr device int32 [n_rows + 1], pos device int32 [n_pos],
 *   y device int32 [n_pos] (the target of position s is y[s])    in
 *   lse fp32 [n_rows]                                            out
 *   logp fp32 [n_pos], indexed by position                      out
 * The index arrays are read on the device: an index outside its range is
 * skipped (a position whose target is outside [0, vocab) gets NaN); positions
 * that no row lists are not written.                                        */
pf_status pf_compact_logprob_fwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride,
                                 int32_t dtype, const int32_t* row_ptr, const int32_t* pos,
                                 const int32_t* y, int32_t n_pos, float* lse, float* logp,
                                 void* stream);

/* Backward of the compact log-probabilities: every position adds its own term
 * to its row (HARTS §3.5: the backward sums each position's gradient into its
 * compact row rather than scaling one gradient by a reuse count),
 *   dz[c, v] = sum over positions s of row c of dlogp_s (1[v = y_s] - softmax(z_c)[v]).
 *   (forward arguments), lse from pf_compact_logprob_fwd, dlogp fp32 [n_pos]  in
 *   dz [n_rows, vocab] (dtype of z), row stride dz_stride elements,
 *     16-byte aligned                                            out (overwritten) */
pf_status pf_compact_logprob_bwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride,
                                 int32_t dtype, const float* lse, const int32_t* row_ptr,
                                 const int32_t* pos, const int32_t* y, int32_t n_pos,
                                 const float* dlogp, void* dz, int64_t dz_stride, void* stream);

/* Host-only helper: the end row of each node's subtree (exclusive), the
 * bound of the rows that can read that node's keys.  Validates the tree.
 * Used by the tree entry points; exposed for testing without a GPU.     */
pf_status pf_tree_subtree_end(int32_t n_nodes, const int32_t* node_off, const int32_t* parent,
                              int32_t* subtree_end);

/* Profiling aid: when a hook is set, the library calls it on the host right
 * before (end = 0) and right after (end = 1) enqueuing each kernel, with a
 * short kernel label and the stream the kernel goes to, so a caller can
 * record timing events on that stream around each kernel.  NULL removes the
 * hook.  The hook is process-wide; set it while no other thread launches. */
typedef void (*pf_launch_hook)(const char* kernel, void* stream, int32_t end, void* user);
void pf_set_launch_hook(pf_launch_hook hook, void* user);

const char* pf_status_string(pf_status status);
const char* pf_last_error(void);
int32_t pf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PF_H_ */
