// Internal declarations shared by the kernels and the host entry points.
//
// Every attention call in this library is one instance of a single problem:
// a set of query rows, an optional block of "external" keys that every query
// row sees (the cached prefix K/V in Phase B), and a set of "own" keys that
// are indexed like the query rows.  Own key k is visible to query q iff
//
//        k <= q   and   q < kend[k]
//
// where kend[k] is the end of the row range that may read key k.  With rows
// in DFS preorder this one rule covers:
//   - Phase A / Phase C (causal prefix):     kend[k] = P;
//   - Phase B own suffix keys:               kend[k] = end of k's suffix, so a
//     suffix never sees another suffix (PrefixFlow §4.1);
//   - trees:                                  kend[k] = end of the subtree of
//     k's node, i.e. the rows of the node and its descendants (HARTS §2.1,
//     §2.2).
// kend[] and per-block summaries of it are built on the device from the
// segment table by the prep kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pf.h"

namespace pf {

constexpr int kWave = 64;
constexpr int kKeyBlockSummary = 32;   // granularity of the kend min/max summaries

// Segment table passed by value to the prep kernel: segment i covers rows
// [start[i], start[i+1]); keys in it are visible up to row vis_end[i].
struct SegTable {
  int32_t n;
  int32_t start[PF_MAX_SEGMENTS + 1];
  int32_t vis_end[PF_MAX_SEGMENTS];
};

// Row ranges of a larger K/V tensor that form the external keys of a call
// (host side, by value to the tile kernel): range i is rows [start[i],
// start[i] + len[i]), padded to a multiple of 32 virtual keys starting at
// virtual tile vt0[i]; vt0[n] is the number of tiles.
struct RangeTable {
  int32_t n;
  int32_t start[PF_MAX_SEGMENTS];
  int32_t len[PF_MAX_SEGMENTS];
  int32_t vt0[PF_MAX_SEGMENTS + 1];
};

// Per-row visibility data and the head table, in the workspace.
struct RowInfo {
  int32_t* kend;      // [rows]
  int32_t* bmax;      // [ceil(rows/32)]: max kend over each 32-key block
  int32_t* bmin;      // [ceil(rows/32)]: min kend over the valid keys of the block
  int32_t* qhead;     // [Hq]: qhead[g * G + j] is the j-th query head of KV head g
};

// Query heads grouped by the KV head they read (host side; the prep kernel
// copies it into RowInfo::qhead so attention kernels index device memory,
// not their argument block).
struct HeadTable {
  int32_t n;
  int16_t qhead[PF_MAX_HEADS];
};

// Arguments of every attention kernel (passed by value).
struct AttnArgs {
  // query side, [rows, Hq, d]
  const void* q;  int64_t q_st, q_sh;
  const void* o;  int64_t o_st, o_sh;     // forward output (read by backward)
  const void* dout; int64_t do_st, do_sh; // upstream gradient
  void* out; int64_t out_st, out_sh;      // O (forward) or dQ (backward)
  float* lse;                             // [Hq, rows]
  float* neg_dsum;                        // [Hq, rows] -D = -rowsum(dO * O), workspace (negated:
                                          //   the dK/dV kernels start their dP sums from it)
  float* lse2;                            // [Hq, rows] LSE log2(e) (+inf for rows that see no key),
                                          //   written by the dQ pass for the dK/dV pass, workspace
  // external keys (every query row sees all of them), [n_ext, Hkv, d]
  const void* k_ext; int64_t kx_st, kx_sh;
  const void* v_ext; int64_t vx_st, vx_sh;
  int32_t n_ext;
  // External keys read from row ranges of a larger tensor (the cached rows of
  // a producer tree): ext_tiles[t] = (first row, valid rows) of virtual
  // external keys [32 t, 32 t + 32), so external key 32 t + i (i < valid) is
  // row first + i of k_ext / v_ext and of gk_acc / gv_acc; keys past `valid`
  // are padding (read as zero, never visible, never written).  Null: external
  // key e is row e.  n_ext then counts the padded virtual keys.
  const int2* ext_tiles;
  int32_t ext_rows;                       // rows of k_ext / v_ext (and gk_acc) with ext_tiles
  // own keys, indexed like the query rows, [rows, Hkv, d]
  const void* k_own; int64_t ko_st, ko_sh;
  const void* v_own; int64_t vo_st, vo_sh;
  // dK/dV outputs of the own keys, [rows, Hkv, d]
  void* dk_own; int64_t dko_st, dko_sh;
  void* dv_own; int64_t dvo_st, dvo_sh;
  int32_t dkv_f32;                        // dK/dV own outputs are fp32 (else input dtype)
  const float* gk_init;                   // optional fp32 [rows, Hkv, d] added into own dK
  const float* gv_init;                   //   and dV before the rounding (Phase C)
  // external-key gradient destination: fp32 [n_ext, Hkv, d]
  float* gk_acc; float* gv_acc;           // accumulators (RMW when n_chunks == 1)
  float* gk_part; float* gv_part;         // partials of chunks 1.. [n_chunks - 1, n_ext, Hkv, d]
  int32_t n_chunks;                       // query chunks per external key block
  // own-key gradient partials when own key blocks are split over query
  // chunks: fp32 [n_chunks_own, rows, Hkv, d], finished by launch_partial_sums
  float* dk_part; float* dv_part;
  int32_t n_chunks_own;
  // A backward with a dS buffer: the dK/dV pass stores dS of every key block
  // it processes (bf16 for bf16 inputs, fp32 for fp32 ones, where ds_ext is
  // read as float*; external keys at key indices [0, ds_own0), own keys from
  // ds_own0; ds_keys keys and ds_rows rows in all, layout in the kernels) and
  // dQ is then formed from it instead of by recomputing S, dP.
  __bf16* ds_ext; int32_t ds_keys, ds_rows, ds_own0;
  RowInfo ri;
  int32_t rows;
  int32_t hq, hkv, group;                 // group = Hq / Hkv
  float scale;                            // softmax scale
  float scale_log2;                       // scale * log2(e)
};

// Calls the caller's launch hook (if any) around one kernel launch.
void launch_hook(const char* kernel, hipStream_t stream, int end);

#define PF_LAUNCH(label, kernel, grid, block, stream, ...)                    \
  do {                                                                        \
    ::pf::launch_hook(label, stream, 0);                                      \
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);          \
    ::pf::launch_hook(label, stream, 1);                                      \
  } while (0)

// Launchers (return hipSuccess or the launch error).
hipError_t launch_prep(const SegTable& seg, const HeadTable& heads, RowInfo ri, hipStream_t stream);
// launch_prep's work and, in the same launch, D = rowsum(dO * O) and LSE
// log2(e) (+inf for rows that see no key) of every (row, query head) into
// a.neg_dsum (as -D) / a.lse2 (bf16 inputs).
hipError_t launch_prep_dsum_bf16(const SegTable& seg, const HeadTable& heads, const AttnArgs& a,
                                 hipStream_t stream);
// the same for fp32 inputs (head_dim 64 or 128)
hipError_t launch_prep_dsum_f32(const SegTable& seg, const HeadTable& heads, const AttnArgs& a,
                                int32_t head_dim, hipStream_t stream);
// ext_tiles[0 .. rt.vt0[rt.n]) from the range table
hipError_t launch_ext_tiles(const RangeTable& rt, int2* tiles, hipStream_t stream);
hipError_t launch_fill_zero(void* dst, int64_t rows, int32_t heads, int32_t d, int64_t st,
                            int64_t sh, int32_t elem_bytes, hipStream_t stream);
// One own-key gradient (dK or dV) to finish: dst = convert(init + sum of the
// chunk partials); part and init are contiguous [rows, heads, d] fp32 (init
// may be null), dst is strided (elements).
struct OwnFinish {
  const float4* part;
  const float4* init;
  char* dst;
  int64_t st, sh;
};
// The split key blocks' partials of one backward call, summed in a fixed
// pairwise order ((p0 + p1) + (p2 + p3)) + ...:
//   external: acc += sum of ext_planes planes (the first chunk already added
//             itself), K and V, ext_n4 float4 each;
//   own:      dst = convert(init + sum of own_planes planes), dK and dV.
// A part with zero planes is skipped; both run in one launch.
struct PartialSums {
  int32_t ext_planes;
  int64_t ext_n4;
  const int2* ext_tiles;                  // virtual external rows -> accumulator rows (or null)
  int32_t ext_row4;                       // float4 values per external row (Hkv d / 4)
  const float4* part_k;
  const float4* part_v;
  float4* acc_k;
  float4* acc_v;
  int32_t own_planes;
  OwnFinish fk, fv;
  int64_t rows;
  int32_t heads, d, dst_f32;
};
hipError_t launch_partial_sums(const PartialSums& ps, hipStream_t stream);
// the dQ-from-dS pass, followed in the same launch by the partial sums `ps`
// (which may be empty)
hipError_t launch_bwd_dq_ds_bf16(const AttnArgs& a, const PartialSums& ps, int32_t head_dim,
                                 hipStream_t stream);
hipError_t launch_convert_acc(const float* src, void* dst, int64_t rows, int32_t heads, int32_t d,
                              int64_t st, int64_t sh, int32_t dst_f32, hipStream_t stream);

hipError_t launch_fwd_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream);
// Order in which the KV-stationary backward's workgroups of one KV head take
// their items (key block x query chunk): item[i] is the item of the i-th
// workgroup.  Workgroups are dispatched in index order to whichever CU frees
// up first, so items sorted longest first make that a longest-first list
// schedule; n == 0 keeps the natural order (external blocks, then own).
constexpr int kMaxOrderedItems = 512;
struct ItemOrder {
  int32_t n;
  uint16_t item[kMaxOrderedItems];
};
// Fills `ord` for the bf16 KV-stationary backward of `a`; the own-key query
// ranges come from the segment table (the same visibility ends the prep
// kernel writes).  Host only; leaves n = 0 when the items do not fit.
void dkv_item_order(const AttnArgs& a, const SegTable& seg, ItemOrder& ord);
hipError_t launch_bwd_dkv_bf16(const AttnArgs& a, const ItemOrder& ord, int32_t head_dim,
                               hipStream_t stream);


hipError_t launch_fwd_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream);
hipError_t launch_bwd_dq_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream);
hipError_t launch_bwd_dkv_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream);
// keys one workgroup of the fp32 KV-stationary backward holds
int32_t dkv_keys_per_workgroup_f32();
// fp32 dQ from the dS buffer the fp32 dK/dV pass stored (then the partial sums
// `ps`, which may be empty, in a launch of their own)
hipError_t launch_bwd_dq_ds_f32(const AttnArgs& a, const PartialSums& ps, int32_t head_dim,
                                hipStream_t stream);

// Compact log-probabilities (pf_logprob.hip); strides in bytes, bf16 != 0
// selects bf16 logits (else fp32)
hipError_t launch_logprob_fwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride_b,
                              int32_t bf16, const int32_t* row_ptr, const int32_t* pos,
                              const int32_t* y, int32_t n_pos, float* lse, float* logp,
                              hipStream_t stream);
hipError_t launch_logprob_bwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride_b,
                              int32_t bf16, const float* lse, const int32_t* row_ptr,
                              const int32_t* pos, const int32_t* y, int32_t n_pos,
                              const float* dlogp, void* dz, int64_t dz_stride_b,
                              hipStream_t stream);

// Number of query chunks the KV-stationary backward splits the external
// (prefix) key blocks and the own key blocks into.  Functions of the shapes
// only, so results do not depend on the device.
int32_t ext_chunks(int32_t n_ext, int32_t rows, int32_t hq, int32_t hkv, int32_t head_dim,
                   int32_t dtype);
int32_t own_chunks(int32_t op, int32_t n_ext, int32_t rows, int32_t hq, int32_t hkv,
                   int32_t head_dim, int32_t dtype);
// keys per workgroup of the bf16 KV-stationary kernel
int32_t dkv_keys_per_workgroup_bf16();

}  // namespace pf
