// Host side of the C ABI declared in include/pf.h: argument validation,
// workspace layout, and the launch sequence of each entry point.  No entry
// point allocates or synchronises, and every check runs before the first HIP
// call.  The only state is the optional launch hook and, per device, the
// address of the static scratch of pf_suffix_attn_bwd_accum_noalloc.  No C++
// exception can leave an entry point: nothing here allocates on the heap or
// takes a lock (the error text is a fixed thread-local buffer).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "pf_internal.h"

namespace {

thread_local char g_last_error[512];

pf_status fail(pf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

pf_status hip_fail(hipError_t e, const char* where) {
  return fail(PF_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int32_t dtype) { return dtype == PF_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- validation

struct Desc {
  int hq, hkv, group, d, dtype;
  float scale;
  pf::HeadTable heads;
};

pf_status check_desc(const pf_attn_desc* desc, Desc* out) {
  if (!desc) return fail(PF_ERR_INVALID_ARG, "desc is NULL");
  const int hq = desc->num_q_heads, hkv = desc->num_kv_heads, d = desc->head_dim;
  if (hq < 1 || hkv < 1) return fail(PF_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d Hkv=%d)", hq, hkv);
  if (hq % hkv) return fail(PF_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", hq, hkv);
  if (hq > PF_MAX_HEADS) return fail(PF_ERR_UNSUPPORTED, "num_q_heads %d exceeds %d", hq, PF_MAX_HEADS);
  if (desc->dtype != PF_F32 && desc->dtype != PF_BF16)
    return fail(PF_ERR_INVALID_ARG, "dtype %d is not PF_F32 or PF_BF16", desc->dtype);
  if (desc->dtype == PF_BF16 && d != 128)
    return fail(PF_ERR_UNSUPPORTED, "bf16 kernels need head_dim 128 (got %d)", d);
  if (desc->dtype == PF_F32 && d != 64 && d != 128)
    return fail(PF_ERR_UNSUPPORTED, "fp32 kernels need head_dim 64 or 128 (got %d)", d);
  if (!isfinite(desc->softmax_scale)) return fail(PF_ERR_INVALID_ARG, "softmax_scale is not finite");
  const int group = hq / hkv;
  if (group > 256) return fail(PF_ERR_UNSUPPORTED, "more than 256 query heads per KV head");
  out->hq = hq;
  out->hkv = hkv;
  out->group = group;
  out->d = d;
  out->dtype = desc->dtype;
  out->scale = desc->softmax_scale > 0.f ? desc->softmax_scale : 1.0f / sqrtf((float)d);
  int fill[PF_MAX_HEADS];
  for (int g = 0; g < hkv; ++g) fill[g] = 0;
  for (int h = 0; h < hq; ++h) {
    const int g = desc->q_to_kv ? desc->q_to_kv[h] : h / group;
    if (g < 0 || g >= hkv) return fail(PF_ERR_INVALID_ARG, "q_to_kv[%d] = %d is out of range", h, g);
    if (fill[g] >= group)
      return fail(PF_ERR_INVALID_ARG, "KV head %d is read by more than %d query heads", g, group);
    out->heads.qhead[g * group + fill[g]++] = (int16_t)h;
  }
  out->heads.n = hq;
  return PF_OK;
}

pf_status check_tensor(const char* name, const pf_tensor& t, int64_t rows, int heads, const Desc& d,
                       int dtype) {
  if (rows == 0) return PF_OK;
  if (!t.data) return fail(PF_ERR_INVALID_ARG, "%s.data is NULL", name);
  if ((uintptr_t)t.data % 16) return fail(PF_ERR_INVALID_ARG, "%s.data is not 16-byte aligned", name);
  const int align = 16 / elem_bytes(dtype);
  if (t.stride_tok < 0 || t.stride_head < 0)
    return fail(PF_ERR_INVALID_ARG, "%s has a negative stride", name);
  if (t.stride_tok % align || t.stride_head % align)
    return fail(PF_ERR_INVALID_ARG, "%s strides must be multiples of %d elements", name, align);
  if (heads > 1 && t.stride_head < d.d)
    return fail(PF_ERR_INVALID_ARG, "%s.stride_head (%lld) < head_dim", name, (long long)t.stride_head);
  if (rows > 1 && t.stride_tok < (int64_t)(heads - 1) * t.stride_head + d.d)
    return fail(PF_ERR_INVALID_ARG, "%s.stride_tok (%lld) makes rows overlap", name,
                (long long)t.stride_tok);
  // the bf16 kernels address one head's rows through 32-bit buffer offsets
  if (rows * t.stride_tok * (int64_t)elem_bytes(dtype) >= ((int64_t)1 << 31))
    return fail(PF_ERR_UNSUPPORTED, "%s spans 2 GiB or more along the token axis", name);
  return PF_OK;
}

pf_status check_ptr(const char* name, const void* p, size_t align) {
  if (!p) return fail(PF_ERR_INVALID_ARG, "%s is NULL", name);
  if ((uintptr_t)p % align) return fail(PF_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return PF_OK;
}

pf_status check_cu(int32_t n, const int32_t* cu, int32_t* rows) {
  if (n < 0) return fail(PF_ERR_INVALID_ARG, "n_suffix is negative");
  if (n > PF_MAX_SEGMENTS) return fail(PF_ERR_UNSUPPORTED, "more than %d suffixes in one call", PF_MAX_SEGMENTS);
  if (n == 0) {
    *rows = 0;
    return PF_OK;
  }
  if (!cu) return fail(PF_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (cu[0] != 0) return fail(PF_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  for (int i = 0; i < n; ++i)
    if (cu[i + 1] < cu[i]) return fail(PF_ERR_INVALID_ARG, "cu_seqlens decreases at %d", i + 1);
  *rows = cu[n];
  return PF_OK;
}

pf_status check_tree(int32_t n, const int32_t* node_off, const int32_t* parent, int32_t* subtree_end) {
  if (n < 1) return fail(PF_ERR_INVALID_ARG, "a tree needs at least one node");
  if (n > PF_MAX_SEGMENTS) return fail(PF_ERR_UNSUPPORTED, "more than %d tree nodes", PF_MAX_SEGMENTS);
  if (!node_off || !parent) return fail(PF_ERR_INVALID_ARG, "node_off or parent is NULL");
  if (node_off[0] != 0) return fail(PF_ERR_INVALID_ARG, "node_off[0] must be 0");
  for (int i = 0; i < n; ++i)
    if (node_off[i + 1] < node_off[i]) return fail(PF_ERR_INVALID_ARG, "node_off decreases at %d", i + 1);
  if (parent[0] != -1) return fail(PF_ERR_INVALID_ARG, "parent[0] must be -1 (node 0 is a root)");
  for (int i = 1; i < n; ++i) {
    if (parent[i] == -1) continue;   // the root of the next tree of a forest
    if (parent[i] < 0 || parent[i] >= i)
      return fail(PF_ERR_INVALID_ARG, "parent[%d] = %d: nodes must be numbered in preorder", i, parent[i]);
    // preorder: the parent of node i is node i-1 or one of its ancestors
    int u = i - 1;
    while (u >= 0 && u != parent[i]) u = parent[u];
    if (u != parent[i])
      return fail(PF_ERR_INVALID_ARG, "node %d breaks DFS preorder (parent %d is not on the path to node %d)",
                  i, parent[i], i - 1);
  }
  for (int i = 0; i < n; ++i) subtree_end[i] = node_off[i + 1];
  for (int i = n - 1; i >= 1; --i)
    if (parent[i] >= 0 && subtree_end[i] > subtree_end[parent[i]])
      subtree_end[parent[i]] = subtree_end[i];
  return PF_OK;
}

// Row ranges of a producer tensor of c_rows rows as the external keys of a
// window call: empty ranges are dropped, the rest padded to whole 32-key
// tiles; *n_virtual is the padded key count (the prefix_len that sizes the
// call's workspace).
pf_status check_ranges(int32_t n, const int32_t* start, const int32_t* len, int32_t c_rows,
                       pf::RangeTable* rt, int32_t* n_virtual) {
  if (n < 0) return fail(PF_ERR_INVALID_ARG, "n_ranges is negative");
  if (n > PF_MAX_SEGMENTS) return fail(PF_ERR_UNSUPPORTED, "more than %d cached row ranges", PF_MAX_SEGMENTS);
  if (n > 0 && (!start || !len)) return fail(PF_ERR_INVALID_ARG, "range_start or range_len is NULL");
  if (c_rows < 0) return fail(PF_ERR_INVALID_ARG, "c_rows is negative");
  rt->n = 0;
  rt->vt0[0] = 0;
  for (int i = 0; i < n; ++i) {
    if (start[i] < 0 || len[i] < 0 || (int64_t)start[i] + len[i] > c_rows)
      return fail(PF_ERR_INVALID_ARG, "range %d = [%d, %d + %d) is outside the %d producer rows", i,
                  start[i], start[i], len[i], c_rows);
    if (len[i] == 0) continue;
    // every cached row is one key: overlapping ranges would also make two
    // workgroups add into the same gK/gV rows
    for (int j = 0; j < rt->n; ++j)
      if (start[i] < rt->start[j] + rt->len[j] && rt->start[j] < start[i] + len[i])
        return fail(PF_ERR_INVALID_ARG, "range %d = [%d, %d + %d) overlaps an earlier range", i,
                    start[i], start[i], len[i]);
    const int j = rt->n++;
    rt->start[j] = start[i];
    rt->len[j] = len[i];
    rt->vt0[j + 1] = rt->vt0[j] + (len[i] + 31) / 32;
  }
  const int64_t nv = 32 * (int64_t)rt->vt0[rt->n];
  if (nv >= ((int64_t)1 << 30)) return fail(PF_ERR_UNSUPPORTED, "too many cached rows");
  *n_virtual = (int32_t)nv;
  return PF_OK;
}

pf_status check_stream_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return PF_OK;
  if (!ws) return fail(PF_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if ((uintptr_t)ws % 16) return fail(PF_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(PF_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return PF_OK;
}

// ------------------------------------------------------------- static scratch

// Device memory of pf_suffix_attn_bwd_accum_noalloc, which cannot take a
// workspace from its caller.  Each GPU the library runs on holds one copy of
// this array until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = PF_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
// hipGetSymbolAddress returns the same address every time on a device, so
// two threads that both look it up store the same value
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The device address of `scratch` on the calling thread's current device.
pf_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PF_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch tracks", dev,
                kMaxDevices);
  void* known = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!known) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256)
      return fail(PF_ERR_HIP, "hipGetSymbolAddress(scratch) returned an unaligned address");
    g_scratch_addr[dev].store(p, std::memory_order_release);
    known = p;
  }
  *out = known;
  return PF_OK;
}

// ------------------------------------------------------------- workspace

struct WsLayout {
  size_t kend = 0, bmax = 0, bmin = 0, qhead = 0, neg_dsum = 0, lse2 = 0, gk_part = 0, gv_part = 0;
  size_t ext_tiles = 0;   // window ops: (first row, valid rows) per 32 cached keys
  size_t total = 0;
  size_t dk_part = 0, dv_part = 0;
  int32_t n_chunks = 1, n_chunks_own = 1;
  // Phase-B dS buffer (external keys, then own keys)
  bool use_ds = false;
  size_t ds_ext = 0;
  int32_t ds_keys = 0, ds_rows = 0, ds_own0 = 0;
};

// A backward keeps dS when the workspace allows it (Phase B, Phase C and
// trees): the buffer holds Hq x (ceil256(n_ext) + ceil256(rows)) keys x
// ceil256(rows) rows in the input dtype (bf16 or fp32), of which only the
// visible tiles are written and read (one head's share must stay below 2 GiB
// for 32-bit buffer offsets).
bool ds_eligible(int32_t op, const Desc& d, int32_t n_ext, int32_t rows) {
  if (op != PF_OP_SUFFIX_BWD && op != PF_OP_PREFIX_BWD && op != PF_OP_TREE_BWD &&
      op != PF_OP_TREE_SUFFIX_BWD)
    return false;
  if (rows <= 0) return false;
  const int64_t r = ((int64_t)rows + 255) / 256 * 256;
  const int64_t keys = ((int64_t)n_ext + 255) / 256 * 256 + r;
  return keys * r * elem_bytes(d.dtype) < ((int64_t)1 << 31);
}

WsLayout layout(int32_t op, const Desc& d, int32_t n_ext, int32_t rows, bool want_ds = false,
                bool split = true) {
  WsLayout w;
  size_t off = 0;
  const size_t nb = (size_t)((rows + 31) / 32);
  w.kend = off; off += align_up((size_t)rows * 4);
  w.bmax = off; off += align_up(nb * 4);
  w.bmin = off; off += align_up(nb * 4);
  w.qhead = off; off += align_up((size_t)d.hq * 4);
  if (op == PF_OP_TREE_SUFFIX_FWD || op == PF_OP_TREE_SUFFIX_BWD) {
    w.ext_tiles = off;
    off += align_up((size_t)(n_ext + 31) / 32 * 8);
  }
  const bool bwd = op == PF_OP_SUFFIX_BWD || op == PF_OP_PREFIX_BWD || op == PF_OP_TREE_BWD ||
                   op == PF_OP_TREE_SUFFIX_BWD;
  if (bwd) {
    w.neg_dsum = off;   // -D per (query head, row)
    off += align_up((size_t)d.hq * rows * 4);
    w.lse2 = off;
    off += align_up((size_t)d.hq * rows * 4);
  }
  if (split && (op == PF_OP_SUFFIX_BWD || op == PF_OP_TREE_SUFFIX_BWD)) {
    w.n_chunks = pf::ext_chunks(n_ext, rows, d.hq, d.hkv, d.d, d.dtype);
    if (w.n_chunks > 1) {
      const size_t part = (size_t)(w.n_chunks - 1) * n_ext * d.hkv * d.d * 4;
      w.gk_part = off; off += align_up(part);
      w.gv_part = off; off += align_up(part);
    }
  }
  if (bwd && split) {
    w.n_chunks_own = pf::own_chunks(op, n_ext, rows, d.hq, d.hkv, d.d, d.dtype);
    if (w.n_chunks_own > 1) {
      const size_t part = (size_t)w.n_chunks_own * rows * d.hkv * d.d * 4;
      w.dk_part = off; off += align_up(part);
      w.dv_part = off; off += align_up(part);
    }
  }
  if (want_ds && ds_eligible(op, d, n_ext, rows)) {
    w.use_ds = true;
    w.ds_rows = (rows + 255) / 256 * 256;
    w.ds_own0 = (n_ext + 255) / 256 * 256;
    w.ds_keys = w.ds_own0 + w.ds_rows;
    w.ds_ext = off;
    off += align_up((size_t)d.hq * w.ds_keys * w.ds_rows * elem_bytes(d.dtype));
  }
  w.total = rows > 0 ? off : 0;
  return w;
}

pf::RowInfo row_info(void* ws, const WsLayout& w) {
  char* b = (char*)ws;
  pf::RowInfo ri;
  ri.kend = (int32_t*)(b + w.kend);
  ri.bmax = (int32_t*)(b + w.bmax);
  ri.bmin = (int32_t*)(b + w.bmin);
  ri.qhead = (int32_t*)(b + w.qhead);
  return ri;
}

// the dS^T buffer of a layout that has one
void set_ds(pf::AttnArgs& a, void* ws, const WsLayout& w) {
  if (!w.use_ds) return;
  a.ds_ext = (__bf16*)((char*)ws + w.ds_ext);
  a.ds_keys = w.ds_keys;
  a.ds_rows = w.ds_rows;
  a.ds_own0 = w.ds_own0;
}

// the tile table of a call whose external keys are row ranges
void set_tiles(pf::AttnArgs& a, void* ws, const WsLayout& w, const pf::RangeTable* rt,
               int32_t c_rows) {
  if (!rt) return;
  a.ext_tiles = (const int2*)((char*)ws + w.ext_tiles);
  a.ext_rows = c_rows;
}

// the full layout (with the dS^T buffer) when the workspace holds it, else
// the minimal one; `w_min` has already been checked against the workspace
WsLayout pick_layout(int32_t op, const Desc& d, int32_t n_ext, int32_t rows, size_t ws_bytes,
                     const WsLayout& w_min) {
  const WsLayout w_ds = layout(op, d, n_ext, rows, true);
  return (w_ds.use_ds && ws_bytes >= w_ds.total) ? w_ds : w_min;
}

void set_own_parts(pf::AttnArgs& a, void* ws, const WsLayout& w) {
  a.n_chunks_own = w.n_chunks_own;
  if (w.n_chunks_own > 1) {
    a.dk_part = (float*)((char*)ws + w.dk_part);
    a.dv_part = (float*)((char*)ws + w.dv_part);
  }
}

pf::AttnArgs base_args(const Desc& d, int32_t rows) {
  pf::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.rows = rows;
  a.hq = d.hq;
  a.hkv = d.hkv;
  a.group = d.group;
  a.scale = d.scale;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  a.n_chunks = 1;
  a.n_chunks_own = 1;
  return a;
}

void set_q(pf::AttnArgs& a, const pf_tensor& t) { a.q = t.data; a.q_st = t.stride_tok; a.q_sh = t.stride_head; }
void set_o(pf::AttnArgs& a, const pf_tensor& t) { a.o = t.data; a.o_st = t.stride_tok; a.o_sh = t.stride_head; }
void set_do(pf::AttnArgs& a, const pf_tensor& t) { a.dout = t.data; a.do_st = t.stride_tok; a.do_sh = t.stride_head; }
void set_out(pf::AttnArgs& a, const pf_tensor& t) { a.out = t.data; a.out_st = t.stride_tok; a.out_sh = t.stride_head; }
void set_ext(pf::AttnArgs& a, const pf_tensor& k, const pf_tensor& v, int32_t n) {
  a.k_ext = k.data; a.kx_st = k.stride_tok; a.kx_sh = k.stride_head;
  a.v_ext = v.data; a.vx_st = v.stride_tok; a.vx_sh = v.stride_head;
  a.n_ext = n;
}
void set_own(pf::AttnArgs& a, const pf_tensor& k, const pf_tensor& v) {
  a.k_own = k.data; a.ko_st = k.stride_tok; a.ko_sh = k.stride_head;
  a.v_own = v.data; a.vo_st = v.stride_tok; a.vo_sh = v.stride_head;
}
void set_dkv(pf::AttnArgs& a, const pf_tensor& dk, const pf_tensor& dv) {
  a.dk_own = dk.data; a.dko_st = dk.stride_tok; a.dko_sh = dk.stride_head;
  a.dv_own = dv.data; a.dvo_st = dv.stride_tok; a.dvo_sh = dv.stride_head;
}

pf::SegTable flat_segments(int32_t n, const int32_t* cu) {
  pf::SegTable s;
  memset(&s, 0, sizeof(s));
  s.n = n;
  for (int i = 0; i <= n; ++i) s.start[i] = cu[i];
  for (int i = 0; i < n; ++i) s.vis_end[i] = cu[i + 1];
  return s;
}

pf::SegTable causal_segment(int32_t rows) {
  pf::SegTable s;
  memset(&s, 0, sizeof(s));
  s.n = 1;
  s.start[0] = 0;
  s.start[1] = rows;
  s.vis_end[0] = rows;
  return s;
}

pf::SegTable tree_segments(int32_t n, const int32_t* node_off, const int32_t* subtree_end) {
  pf::SegTable s;
  memset(&s, 0, sizeof(s));
  s.n = n;
  for (int i = 0; i <= n; ++i) s.start[i] = node_off[i];
  for (int i = 0; i < n; ++i) s.vis_end[i] = subtree_end[i];
  return s;
}

// ------------------------------------------------------------- launches

// the tile table of a call whose external keys are row ranges (no-op otherwise)
pf_status run_tiles(const pf::RangeTable* rt, const pf::AttnArgs& a, hipStream_t st) {
  if (!rt || !a.ext_tiles) return PF_OK;
  const hipError_t e = pf::launch_ext_tiles(*rt, const_cast<int2*>(a.ext_tiles), st);
  return e == hipSuccess ? PF_OK : hip_fail(e, "ext_tiles");
}

pf_status run_fwd(const Desc& d, const pf::AttnArgs& a, const pf::SegTable& seg, hipStream_t st,
                  const pf::RangeTable* rt = nullptr) {
  pf_status s = run_tiles(rt, a, st);
  if (s != PF_OK) return s;
  hipError_t e = pf::launch_prep(seg, d.heads, a.ri, st);
  if (e != hipSuccess) return hip_fail(e, "prep");
  e = d.dtype == PF_BF16 ? pf::launch_fwd_bf16(a, d.d, st) : pf::launch_fwd_f32(a, d.d, st);
  if (e != hipSuccess) return hip_fail(e, "forward");
  return PF_OK;
}

// the split key blocks' partial sums of a backward call (empty when no block
// is split)
pf::PartialSums partial_sums_of(const Desc& d, const pf::AttnArgs& a) {
  pf::PartialSums ps;
  memset(&ps, 0, sizeof(ps));
  if (a.n_chunks > 1 && a.n_ext > 0) {
    ps.ext_planes = a.n_chunks - 1;
    ps.ext_n4 = (int64_t)a.n_ext * d.hkv * d.d / 4;
    ps.part_k = (const float4*)a.gk_part;
    ps.part_v = (const float4*)a.gv_part;
    ps.acc_k = (float4*)a.gk_acc;
    ps.acc_v = (float4*)a.gv_acc;
    ps.ext_tiles = a.ext_tiles;
    ps.ext_row4 = d.hkv * d.d / 4;
  }
  if (a.n_chunks_own > 1) {
    ps.own_planes = a.n_chunks_own;
    ps.fk = pf::OwnFinish{(const float4*)a.dk_part, (const float4*)a.gk_init, (char*)a.dk_own,
                          a.dko_st, a.dko_sh};
    ps.fv = pf::OwnFinish{(const float4*)a.dv_part, (const float4*)a.gv_init, (char*)a.dv_own,
                          a.dvo_st, a.dvo_sh};
    ps.rows = a.rows;
    ps.heads = d.hkv;
    ps.d = d.d;
    ps.dst_f32 = a.dkv_f32;
  }
  return ps;
}

pf_status run_bwd(const Desc& d, const pf::AttnArgs& a, const pf::SegTable& seg, hipStream_t st,
                  const pf::RangeTable* rt = nullptr) {
  const pf_status s = run_tiles(rt, a, st);
  if (s != PF_OK) return s;
  hipError_t e;
  // longest-first order of the KV-stationary items (a host-side plan; no
  // device work)
  pf::ItemOrder ord;
  ord.n = 0;
  if (d.dtype == PF_BF16) pf::dkv_item_order(a, seg, ord);
  const pf::PartialSums ps = partial_sums_of(d, a);
  if (a.ds_ext) {
    // prep with D and LSE first; the dK/dV pass stores dS, then dQ is read
    // from it, followed by the split blocks' partial sums (bf16: in the same
    // launch)
    const bool bf16 = d.dtype == PF_BF16;
    e = bf16 ? pf::launch_prep_dsum_bf16(seg, d.heads, a, st)
             : pf::launch_prep_dsum_f32(seg, d.heads, a, d.d, st);
    if (e != hipSuccess) return hip_fail(e, "prep");
    e = bf16 ? pf::launch_bwd_dkv_bf16(a, ord, d.d, st) : pf::launch_bwd_dkv_f32(a, d.d, st);
    if (e != hipSuccess) return hip_fail(e, "dkv");
    e = bf16 ? pf::launch_bwd_dq_ds_bf16(a, ps, d.d, st) : pf::launch_bwd_dq_ds_f32(a, ps, d.d, st);
    if (e != hipSuccess) return hip_fail(e, "dq_ds");
    return PF_OK;
  }
  e = pf::launch_prep(seg, d.heads, a.ri, st);
  if (e != hipSuccess) return hip_fail(e, "prep");
  e = d.dtype == PF_BF16 ? pf::launch_bwd_dq_bf16(a, d.d, st) : pf::launch_bwd_dq_f32(a, d.d, st);
  if (e != hipSuccess) return hip_fail(e, "dq");
  e = d.dtype == PF_BF16 ? pf::launch_bwd_dkv_bf16(a, ord, d.d, st) : pf::launch_bwd_dkv_f32(a, d.d, st);
  if (e != hipSuccess) return hip_fail(e, "dkv");
  // the split blocks' partials: gK/gV += later chunks, own dK/dV = init +
  // chunks, in one launch
  e = pf::launch_partial_sums(ps, st);
  if (e != hipSuccess) return hip_fail(e, "partials");
  return PF_OK;
}

}  // namespace

namespace pf {

namespace {
// the user pointer is stored before the hook and read after it, so a launch
// that sees a hook sees its user pointer
std::atomic<pf_launch_hook> g_hook{nullptr};
std::atomic<void*> g_hook_user{nullptr};
}  // namespace

void launch_hook(const char* kernel, hipStream_t stream, int end) {
  const pf_launch_hook h = g_hook.load(std::memory_order_acquire);
  if (h) h(kernel, (void*)stream, end, g_hook_user.load(std::memory_order_relaxed));
}

// Workgroups of the KV-stationary backward that run at once on the chip: one
// per CU for the bf16 kernel (its LDS), two for the fp32 one.
int64_t dkv_slots(int32_t dtype) { return dtype == PF_BF16 ? 256 : 512; }

// External key blocks are split into query chunks until there is about one
// workgroup per slot while each chunk keeps at least 32 query steps of 32
// rows; the own key blocks (and any second round) fill in behind them in
// longest-first order.  Fewer chunks means fewer fp32 partials to write and
// reduce.
int32_t ext_chunks(int32_t n_ext, int32_t rows, int32_t hq, int32_t hkv, int32_t head_dim,
                   int32_t dtype) {
  (void)head_dim;
  if (n_ext <= 0 || rows <= 0) return 1;
  const int kb = dtype == PF_BF16 ? dkv_keys_per_workgroup_bf16() : dkv_keys_per_workgroup_f32();
  const int64_t wgs = (int64_t)((n_ext + kb - 1) / kb) * hkv;
  const int64_t steps = (int64_t)((rows + 31) / 32) * (hq / hkv);
  int32_t nc = 1;
  while (nc < 8 && wgs * nc < dkv_slots(dtype) && steps / (2 * nc) >= 32) nc *= 2;
  return nc;
}

// Own keys: a causal prefix (Phase C) or a tree has key blocks whose query
// ranges average about half the rows, split like the external blocks.  In
// Phase B a suffix key block sees at most its own suffix, a fraction of what
// an external block sees; after the external items fill every CU the own
// items form the tail of the launch, so with a prefix they are halved to
// shorten that tail (their partials are summed by the finishing pass).
int32_t own_chunks(int32_t op, int32_t n_ext, int32_t rows, int32_t hq, int32_t hkv,
                   int32_t head_dim, int32_t dtype) {
  (void)head_dim;
  if (rows <= 0) return 1;
  if (op == PF_OP_SUFFIX_BWD) return (n_ext > 0 && rows >= 512) ? 2 : 1;
  if (op != PF_OP_PREFIX_BWD && op != PF_OP_TREE_BWD && op != PF_OP_TREE_SUFFIX_BWD) return 1;
  const int kb = dtype == PF_BF16 ? dkv_keys_per_workgroup_bf16() : dkv_keys_per_workgroup_f32();
  const int64_t wgs = (int64_t)((rows + kb - 1) / kb) * hkv;
  const int64_t steps = (int64_t)((rows / 2 + 31) / 32) * (hq / hkv);
  int32_t nc = 1;
  while (nc < 8 && wgs * nc < 2 * dkv_slots(dtype) && steps / (2 * nc) >= 32) nc *= 2;
  return nc;
}

}  // namespace pf

extern "C" {

int32_t pf_abi_version(void) { return PF_ABI_VERSION; }

void pf_set_launch_hook(pf_launch_hook hook, void* user) {
  pf::g_hook_user.store(user, std::memory_order_relaxed);
  pf::g_hook.store(hook, std::memory_order_release);
}

const char* pf_last_error(void) { return g_last_error; }

const char* pf_status_string(pf_status s) {
  switch (s) {
    case PF_OK: return "PF_OK";
    case PF_ERR_INVALID_ARG: return "PF_ERR_INVALID_ARG";
    case PF_ERR_UNSUPPORTED: return "PF_ERR_UNSUPPORTED";
    case PF_ERR_WORKSPACE: return "PF_ERR_WORKSPACE";
    case PF_ERR_HIP: return "PF_ERR_HIP";
  }
  return "unknown pf_status";
}

size_t pf_workspace_size(int32_t op, const pf_attn_desc* desc, int32_t prefix_len, int32_t rows) {
  Desc d;
  if (check_desc(desc, &d) != PF_OK || rows < 0 || prefix_len < 0) return 0;
  if (op == PF_OP_PREFIX_FWD || op == PF_OP_PREFIX_BWD) rows = prefix_len;
  const int32_t n_ext = (op == PF_OP_SUFFIX_FWD || op == PF_OP_SUFFIX_BWD ||
                         op == PF_OP_TREE_SUFFIX_FWD || op == PF_OP_TREE_SUFFIX_BWD)
                            ? prefix_len
                            : 0;
  if (op < PF_OP_PREFIX_FWD || op > PF_OP_TREE_SUFFIX_BWD) return 0;
  return layout(op, d, n_ext, rows, true).total;
}

size_t pf_workspace_size_min(int32_t op, const pf_attn_desc* desc, int32_t prefix_len,
                             int32_t rows) {
  Desc d;
  if (check_desc(desc, &d) != PF_OK || rows < 0 || prefix_len < 0) return 0;
  if (op == PF_OP_PREFIX_FWD || op == PF_OP_PREFIX_BWD) rows = prefix_len;
  const int32_t n_ext = (op == PF_OP_SUFFIX_FWD || op == PF_OP_SUFFIX_BWD ||
                         op == PF_OP_TREE_SUFFIX_FWD || op == PF_OP_TREE_SUFFIX_BWD)
                            ? prefix_len
                            : 0;
  if (op < PF_OP_PREFIX_FWD || op > PF_OP_TREE_SUFFIX_BWD) return 0;
  return layout(op, d, n_ext, rows, false).total;
}

pf_status pf_tree_subtree_end(int32_t n_nodes, const int32_t* node_off, const int32_t* parent,
                              int32_t* subtree_end) {
  if (!subtree_end) return fail(PF_ERR_INVALID_ARG, "subtree_end is NULL");
  int32_t tmp[PF_MAX_SEGMENTS];
  const pf_status s = check_tree(n_nodes, node_off, parent, tmp);
  if (s != PF_OK) return s;
  for (int i = 0; i < n_nodes; ++i) subtree_end[i] = tmp[i];
  return PF_OK;
}

pf_status pf_prefix_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor q_p, pf_tensor k_p,
                        pf_tensor v_p, pf_tensor o_p, float* lse_p, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  if ((s = check_tensor("q_p", q_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("k_p", k_p, prefix_len, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v_p", v_p, prefix_len, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("o_p", o_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
  if (prefix_len > 0 && (s = check_ptr("lse_p", lse_p, 4)) != PF_OK) return s;
  const WsLayout w = layout(PF_OP_PREFIX_FWD, d, 0, prefix_len);
  if ((s = check_stream_ws(workspace, workspace_bytes, w.total)) != PF_OK) return s;
  if (prefix_len == 0) return PF_OK;
  pf::AttnArgs a = base_args(d, prefix_len);
  set_q(a, q_p);
  set_out(a, o_p);
  set_own(a, k_p, v_p);
  a.lse = lse_p;
  a.ri = row_info(workspace, w);
  return run_fwd(d, a, causal_segment(prefix_len), (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Phase B forward over a cached prefix for rows whose own-key visibility is
// the segment table `seg` (flat suffixes or a tree window); `rows` and the
// structure are already validated.
// With `rt`, the external keys are the row ranges rt of k_p / v_p, which hold
// c_rows rows, and prefix_len is the padded key count of check_ranges.
pf_status suffix_fwd_impl(int32_t op, const Desc& d, int32_t prefix_len, pf_tensor k_p,
                          pf_tensor v_p, int32_t rows, const pf::SegTable& seg, pf_tensor q_s,
                          pf_tensor k_s, pf_tensor v_s, pf_tensor o_s, float* lse_s,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const pf::RangeTable* rt = nullptr, int32_t c_rows = 0) {
  pf_status s;
  const int32_t x_rows = rt ? c_rows : prefix_len;
  if ((s = check_tensor("k_p", k_p, x_rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v_p", v_p, x_rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("q_s", q_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("k_s", k_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v_s", v_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("o_s", o_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if (rows > 0 && (s = check_ptr("lse_s", lse_s, 4)) != PF_OK) return s;
  const WsLayout w = layout(op, d, prefix_len, rows);
  if ((s = check_stream_ws(workspace, workspace_bytes, w.total)) != PF_OK) return s;
  if (rows == 0) return PF_OK;
  pf::AttnArgs a = base_args(d, rows);
  set_q(a, q_s);
  set_out(a, o_s);
  set_ext(a, k_p, v_p, prefix_len);
  set_tiles(a, workspace, w, rt, c_rows);
  set_own(a, k_s, v_s);
  a.lse = lse_s;
  a.ri = row_info(workspace, w);
  return run_fwd(d, a, seg, (hipStream_t)stream, rt);
}

// Phase B backward with gK/gV accumulation, for the same two row structures.
// With use_scratch the call runs in this library's static device scratch
// instead of a workspace argument (workspace and workspace_bytes are
// ignored): the recompute dQ path with no key block split, so the scratch
// holds only the per-row tables and D / LSE.
pf_status suffix_bwd_impl(int32_t op, const Desc& d, int32_t prefix_len, pf_tensor k_p,
                          pf_tensor v_p, int32_t rows, const pf::SegTable& seg, pf_tensor q_s,
                          pf_tensor k_s, pf_tensor v_s, pf_tensor o_s, const float* lse_s,
                          pf_tensor do_s, pf_tensor dq_s, pf_tensor dk_s, pf_tensor dv_s,
                          float* gk_acc, float* gv_acc, void* workspace, size_t workspace_bytes,
                          void* stream, bool use_scratch = false,
                          const pf::RangeTable* rt = nullptr, int32_t c_rows = 0) {
  pf_status s;
  const int32_t x_rows = rt ? c_rows : prefix_len;
  if ((s = check_tensor("k_p", k_p, x_rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v_p", v_p, x_rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("q_s", q_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("k_s", k_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v_s", v_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("o_s", o_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("do_s", do_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("dq_s", dq_s, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("dk_s", dk_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("dv_s", dv_s, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if (rows > 0 && (s = check_ptr("lse_s", lse_s, 4)) != PF_OK) return s;
  if (rows > 0 && prefix_len > 0) {
    if ((s = check_ptr("gk_acc", gk_acc, 16)) != PF_OK) return s;
    if ((s = check_ptr("gv_acc", gv_acc, 16)) != PF_OK) return s;
  }
  WsLayout w;
  if (use_scratch) {
    w = layout(op, d, prefix_len, rows, false, false);
    if (w.total > kScratchBytes)
      return fail(PF_ERR_UNSUPPORTED,
                  "this call needs %zu bytes of scratch; the static scratch holds %zu "
                  "(PF_NOALLOC_SCRATCH_BYTES)", w.total, kScratchBytes);
    if (rows == 0) return PF_OK;
    if ((s = scratch_of_current_device(&workspace)) != PF_OK) return s;
    workspace_bytes = kScratchBytes;
  } else {
    const WsLayout w_min = layout(op, d, prefix_len, rows, false);
    if ((s = check_stream_ws(workspace, workspace_bytes, w_min.total)) != PF_OK) return s;
    w = pick_layout(op, d, prefix_len, rows, workspace_bytes, w_min);
  }
  if (rows == 0) return PF_OK;
  pf::AttnArgs a = base_args(d, rows);
  set_q(a, q_s);
  set_o(a, o_s);
  set_do(a, do_s);
  set_out(a, dq_s);
  set_ext(a, k_p, v_p, prefix_len);
  set_own(a, k_s, v_s);
  set_dkv(a, dk_s, dv_s);
  a.dkv_f32 = d.dtype == PF_F32;
  a.lse = const_cast<float*>(lse_s);
  a.gk_acc = gk_acc;
  a.gv_acc = gv_acc;
  a.n_chunks = w.n_chunks;
  if (w.n_chunks > 1) {
    a.gk_part = (float*)((char*)workspace + w.gk_part);
    a.gv_part = (float*)((char*)workspace + w.gv_part);
  }
  a.neg_dsum = (float*)((char*)workspace + w.neg_dsum);
  a.lse2 = (float*)((char*)workspace + w.lse2);
  set_ds(a, workspace, w);
  set_own_parts(a, workspace, w);
  set_tiles(a, workspace, w, rt, c_rows);
  a.ri = row_info(workspace, w);
  return run_bwd(d, a, seg, (hipStream_t)stream, rt);
}

}  // namespace

extern "C" {

pf_status pf_suffix_attn_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor k_p,
                             pf_tensor v_p, int32_t n_suffix, const int32_t* cu_seqlens,
                             pf_tensor q_s, pf_tensor k_s, pf_tensor v_s, pf_tensor o_s,
                             float* lse_s, void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  int32_t rows = 0;
  if ((s = check_cu(n_suffix, cu_seqlens, &rows)) != PF_OK) return s;
  return suffix_fwd_impl(PF_OP_SUFFIX_FWD, d, prefix_len, k_p, v_p, rows,
                         flat_segments(n_suffix, cu_seqlens), q_s, k_s, v_s, o_s, lse_s,
                         workspace, workspace_bytes, stream);
}

pf_status pf_suffix_attn_bwd_accum(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor k_p,
                                   pf_tensor v_p, int32_t n_suffix, const int32_t* cu_seqlens,
                                   pf_tensor q_s, pf_tensor k_s, pf_tensor v_s, pf_tensor o_s,
                                   const float* lse_s, pf_tensor do_s, pf_tensor dq_s,
                                   pf_tensor dk_s, pf_tensor dv_s, float* gk_acc, float* gv_acc,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  int32_t rows = 0;
  if ((s = check_cu(n_suffix, cu_seqlens, &rows)) != PF_OK) return s;
  return suffix_bwd_impl(PF_OP_SUFFIX_BWD, d, prefix_len, k_p, v_p, rows,
                         flat_segments(n_suffix, cu_seqlens), q_s, k_s, v_s, o_s, lse_s, do_s,
                         dq_s, dk_s, dv_s, gk_acc, gv_acc, workspace, workspace_bytes, stream);
}

pf_status pf_suffix_attn_bwd_accum_noalloc(const pf_attn_desc* desc, int32_t prefix_len,
                                           pf_tensor k_p, pf_tensor v_p, int32_t n_suffix,
                                           const int32_t* cu_seqlens, pf_tensor q_s,
                                           pf_tensor k_s, pf_tensor v_s, pf_tensor o_s,
                                           const float* lse_s, pf_tensor do_s, pf_tensor dq_s,
                                           pf_tensor dk_s, pf_tensor dv_s, float* gk_acc,
                                           float* gv_acc, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  int32_t rows = 0;
  if ((s = check_cu(n_suffix, cu_seqlens, &rows)) != PF_OK) return s;
  return suffix_bwd_impl(PF_OP_SUFFIX_BWD, d, prefix_len, k_p, v_p, rows,
                         flat_segments(n_suffix, cu_seqlens), q_s, k_s, v_s, o_s, lse_s, do_s,
                         dq_s, dk_s, dv_s, gk_acc, gv_acc, nullptr, 0, stream, true);
}

pf_status pf_tree_suffix_attn_fwd(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor k_p,
                                  pf_tensor v_p, int32_t n_nodes, const int32_t* node_off,
                                  const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
                                  pf_tensor o, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  return suffix_fwd_impl(PF_OP_TREE_SUFFIX_FWD, d, prefix_len, k_p, v_p, node_off[n_nodes],
                         tree_segments(n_nodes, node_off, send), q, k, v, o, lse, workspace,
                         workspace_bytes, stream);
}

pf_status pf_tree_suffix_attn_bwd_accum(const pf_attn_desc* desc, int32_t prefix_len,
                                        pf_tensor k_p, pf_tensor v_p, int32_t n_nodes,
                                        const int32_t* node_off, const int32_t* parent,
                                        pf_tensor q, pf_tensor k, pf_tensor v, pf_tensor o,
                                        const float* lse, pf_tensor dout, pf_tensor dq,
                                        pf_tensor dk, pf_tensor dv, float* gk_acc, float* gv_acc,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  return suffix_bwd_impl(PF_OP_TREE_SUFFIX_BWD, d, prefix_len, k_p, v_p, node_off[n_nodes],
                         tree_segments(n_nodes, node_off, send), q, k, v, o, lse, dout, dq, dk,
                         dv, gk_acc, gv_acc, workspace, workspace_bytes, stream);
}

pf_status pf_tree_suffix_attn_fwd_ranges(const pf_attn_desc* desc, int32_t c_rows, pf_tensor k_c,
                                         pf_tensor v_c, int32_t n_ranges,
                                         const int32_t* range_start, const int32_t* range_len,
                                         int32_t n_nodes, const int32_t* node_off,
                                         const int32_t* parent, pf_tensor q, pf_tensor k,
                                         pf_tensor v, pf_tensor o, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  pf::RangeTable rt;
  int32_t n_virtual = 0;
  if ((s = check_ranges(n_ranges, range_start, range_len, c_rows, &rt, &n_virtual)) != PF_OK)
    return s;
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  return suffix_fwd_impl(PF_OP_TREE_SUFFIX_FWD, d, n_virtual, k_c, v_c, node_off[n_nodes],
                         tree_segments(n_nodes, node_off, send), q, k, v, o, lse, workspace,
                         workspace_bytes, stream, &rt, c_rows);
}

pf_status pf_tree_suffix_attn_bwd_accum_ranges(
    const pf_attn_desc* desc, int32_t c_rows, pf_tensor k_c, pf_tensor v_c, int32_t n_ranges,
    const int32_t* range_start, const int32_t* range_len, int32_t n_nodes,
    const int32_t* node_off, const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v,
    pf_tensor o, const float* lse, pf_tensor dout, pf_tensor dq, pf_tensor dk, pf_tensor dv,
    float* gk_acc, float* gv_acc, void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  pf::RangeTable rt;
  int32_t n_virtual = 0;
  if ((s = check_ranges(n_ranges, range_start, range_len, c_rows, &rt, &n_virtual)) != PF_OK)
    return s;
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  return suffix_bwd_impl(PF_OP_TREE_SUFFIX_BWD, d, n_virtual, k_c, v_c, node_off[n_nodes],
                         tree_segments(n_nodes, node_off, send), q, k, v, o, lse, dout, dq, dk,
                         dv, gk_acc, gv_acc, workspace, workspace_bytes, stream, false, &rt,
                         c_rows);
}

int32_t pf_ranges_cached_keys(int32_t n_ranges, const int32_t* range_len) {
  if (n_ranges < 0 || n_ranges > PF_MAX_SEGMENTS || (n_ranges > 0 && !range_len)) return -1;
  int64_t n = 0;
  for (int i = 0; i < n_ranges; ++i) {
    if (range_len[i] < 0) return -1;
    n += (range_len[i] + 31) / 32 * 32;
  }
  return n < ((int64_t)1 << 30) ? (int32_t)n : -1;
}

pf_status pf_prefix_bwd_inject(const pf_attn_desc* desc, int32_t prefix_len, pf_tensor q_p,
                               pf_tensor k_p, pf_tensor v_p, pf_tensor o_p, const float* lse_p,
                               pf_tensor do_p, const float* gk_acc, const float* gv_acc,
                               pf_tensor dq_p, pf_tensor dk_p, pf_tensor dv_p, int32_t dkv_dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (prefix_len < 0) return fail(PF_ERR_INVALID_ARG, "prefix_len is negative");
  if (dkv_dtype != PF_F32 && dkv_dtype != d.dtype)
    return fail(PF_ERR_INVALID_ARG, "dkv_dtype must be PF_F32 or the input dtype");
  const bool has_do = do_p.data != nullptr;
  if (has_do) {
    if ((s = check_tensor("q_p", q_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("k_p", k_p, prefix_len, d.hkv, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("v_p", v_p, prefix_len, d.hkv, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("o_p", o_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("do_p", do_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
    if (prefix_len > 0 && (s = check_ptr("lse_p", lse_p, 4)) != PF_OK) return s;
  }
  if ((s = check_tensor("dq_p", dq_p, prefix_len, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("dk_p", dk_p, prefix_len, d.hkv, d, dkv_dtype)) != PF_OK) return s;
  if ((s = check_tensor("dv_p", dv_p, prefix_len, d.hkv, d, dkv_dtype)) != PF_OK) return s;
  if (prefix_len > 0) {
    if ((s = check_ptr("gk_acc", gk_acc, 16)) != PF_OK) return s;
    if ((s = check_ptr("gv_acc", gv_acc, 16)) != PF_OK) return s;
  }
  const WsLayout w_min = layout(PF_OP_PREFIX_BWD, d, 0, prefix_len);
  if (has_do && (s = check_stream_ws(workspace, workspace_bytes, w_min.total)) != PF_OK) return s;
  const WsLayout w = has_do ? pick_layout(PF_OP_PREFIX_BWD, d, 0, prefix_len, workspace_bytes, w_min)
                            : w_min;
  if (prefix_len == 0) return PF_OK;
  hipStream_t st = (hipStream_t)stream;
  if (!has_do) {
    // zero upstream: dQ_P = 0 and the prefix K/V gradients are the accumulators
    const int eb = elem_bytes(d.dtype);
    hipError_t e = pf::launch_fill_zero(dq_p.data, prefix_len, d.hq, d.d, dq_p.stride_tok,
                                        dq_p.stride_head, eb, st);
    if (e == hipSuccess)
      e = pf::launch_convert_acc(gk_acc, dk_p.data, prefix_len, d.hkv, d.d, dk_p.stride_tok,
                                 dk_p.stride_head, dkv_dtype == PF_F32, st);
    if (e == hipSuccess)
      e = pf::launch_convert_acc(gv_acc, dv_p.data, prefix_len, d.hkv, d.d, dv_p.stride_tok,
                                 dv_p.stride_head, dkv_dtype == PF_F32, st);
    if (e != hipSuccess) return hip_fail(e, "inject");
    return PF_OK;
  }
  pf::AttnArgs a = base_args(d, prefix_len);
  set_q(a, q_p);
  set_o(a, o_p);
  set_do(a, do_p);
  set_out(a, dq_p);
  set_own(a, k_p, v_p);
  set_dkv(a, dk_p, dv_p);
  a.dkv_f32 = dkv_dtype == PF_F32;
  a.gk_init = gk_acc;
  a.gv_init = gv_acc;
  a.lse = const_cast<float*>(lse_p);
  a.neg_dsum = (float*)((char*)workspace + w.neg_dsum);
  a.lse2 = (float*)((char*)workspace + w.lse2);
  set_ds(a, workspace, w);
  set_own_parts(a, workspace, w);
  a.ri = row_info(workspace, w);
  return run_bwd(d, a, causal_segment(prefix_len), st);
}

pf_status pf_tree_attn_fwd(const pf_attn_desc* desc, int32_t n_nodes, const int32_t* node_off,
                           const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v, pf_tensor o,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  const int32_t rows = node_off[n_nodes];
  if ((s = check_tensor("q", q, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("k", k, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("v", v, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("o", o, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if (rows > 0 && (s = check_ptr("lse", lse, 4)) != PF_OK) return s;
  const WsLayout w = layout(PF_OP_TREE_FWD, d, 0, rows);
  if ((s = check_stream_ws(workspace, workspace_bytes, w.total)) != PF_OK) return s;
  if (rows == 0) return PF_OK;
  pf::AttnArgs a = base_args(d, rows);
  set_q(a, q);
  set_out(a, o);
  set_own(a, k, v);
  a.lse = lse;
  a.ri = row_info(workspace, w);
  return run_fwd(d, a, tree_segments(n_nodes, node_off, send), (hipStream_t)stream);
}

}  // extern "C"

namespace {

// The tree backward; with gk_acc / gv_acc (fp32 [C, Hkv, d]) they are added
// to dK / dV before the one rounding (the producer backward of HARTS §3.4),
// in dkv_dtype.  A NULL dout.data with injection means a zero upstream.
pf_status tree_bwd_impl(const Desc& d, int32_t n_nodes, const int32_t* node_off,
                        const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v, pf_tensor o,
                        const float* lse, pf_tensor dout, const float* gk_acc,
                        const float* gv_acc, pf_tensor dq, pf_tensor dk, pf_tensor dv,
                        int32_t dkv_dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  pf_status s;
  int32_t send[PF_MAX_SEGMENTS];
  if ((s = check_tree(n_nodes, node_off, parent, send)) != PF_OK) return s;
  const int32_t rows = node_off[n_nodes];
  const bool inject = gk_acc != nullptr || gv_acc != nullptr;
  const bool has_do = dout.data != nullptr || !inject;
  if (dkv_dtype != PF_F32 && dkv_dtype != d.dtype)
    return fail(PF_ERR_INVALID_ARG, "dkv_dtype must be PF_F32 or the input dtype");
  if (has_do) {
    if ((s = check_tensor("q", q, rows, d.hq, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("k", k, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("v", v, rows, d.hkv, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("o", o, rows, d.hq, d, d.dtype)) != PF_OK) return s;
    if ((s = check_tensor("dout", dout, rows, d.hq, d, d.dtype)) != PF_OK) return s;
    if (rows > 0 && (s = check_ptr("lse", lse, 4)) != PF_OK) return s;
  }
  if ((s = check_tensor("dq", dq, rows, d.hq, d, d.dtype)) != PF_OK) return s;
  if ((s = check_tensor("dk", dk, rows, d.hkv, d, dkv_dtype)) != PF_OK) return s;
  if ((s = check_tensor("dv", dv, rows, d.hkv, d, dkv_dtype)) != PF_OK) return s;
  if (inject && rows > 0) {
    if ((s = check_ptr("gk_acc", gk_acc, 16)) != PF_OK) return s;
    if ((s = check_ptr("gv_acc", gv_acc, 16)) != PF_OK) return s;
  }
  const WsLayout w_min = layout(PF_OP_TREE_BWD, d, 0, rows);
  if (has_do && (s = check_stream_ws(workspace, workspace_bytes, w_min.total)) != PF_OK) return s;
  if (rows == 0) return PF_OK;
  hipStream_t st = (hipStream_t)stream;
  if (!has_do) {
    // zero upstream: dQ = 0 and the K/V gradients are the accumulators
    hipError_t e = pf::launch_fill_zero(dq.data, rows, d.hq, d.d, dq.stride_tok, dq.stride_head,
                                        elem_bytes(d.dtype), st);
    if (e == hipSuccess)
      e = pf::launch_convert_acc(gk_acc, dk.data, rows, d.hkv, d.d, dk.stride_tok,
                                 dk.stride_head, dkv_dtype == PF_F32, st);
    if (e == hipSuccess)
      e = pf::launch_convert_acc(gv_acc, dv.data, rows, d.hkv, d.d, dv.stride_tok,
                                 dv.stride_head, dkv_dtype == PF_F32, st);
    if (e != hipSuccess) return hip_fail(e, "inject");
    return PF_OK;
  }
  const WsLayout w = pick_layout(PF_OP_TREE_BWD, d, 0, rows, workspace_bytes, w_min);
  pf::AttnArgs a = base_args(d, rows);
  set_q(a, q);
  set_o(a, o);
  set_do(a, dout);
  set_out(a, dq);
  set_own(a, k, v);
  set_dkv(a, dk, dv);
  a.dkv_f32 = dkv_dtype == PF_F32;
  a.gk_init = gk_acc;
  a.gv_init = gv_acc;
  a.lse = const_cast<float*>(lse);
  a.neg_dsum = (float*)((char*)workspace + w.neg_dsum);
  a.lse2 = (float*)((char*)workspace + w.lse2);
  set_ds(a, workspace, w);
  set_own_parts(a, workspace, w);
  a.ri = row_info(workspace, w);
  return run_bwd(d, a, tree_segments(n_nodes, node_off, send), st);
}

}  // namespace

extern "C" {

pf_status pf_tree_attn_bwd(const pf_attn_desc* desc, int32_t n_nodes, const int32_t* node_off,
                           const int32_t* parent, pf_tensor q, pf_tensor k, pf_tensor v, pf_tensor o,
                           const float* lse, pf_tensor dout, pf_tensor dq, pf_tensor dk,
                           pf_tensor dv, void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  return tree_bwd_impl(d, n_nodes, node_off, parent, q, k, v, o, lse, dout, nullptr, nullptr, dq,
                       dk, dv, d.dtype, workspace, workspace_bytes, stream);
}

pf_status pf_tree_attn_bwd_inject(const pf_attn_desc* desc, int32_t n_nodes,
                                  const int32_t* node_off, const int32_t* parent, pf_tensor q,
                                  pf_tensor k, pf_tensor v, pf_tensor o, const float* lse,
                                  pf_tensor dout, const float* gk_acc, const float* gv_acc,
                                  pf_tensor dq, pf_tensor dk, pf_tensor dv, int32_t dkv_dtype,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  Desc d;
  pf_status s = check_desc(desc, &d);
  if (s != PF_OK) return s;
  if (!gk_acc || !gv_acc) return fail(PF_ERR_INVALID_ARG, "gk_acc or gv_acc is NULL");
  return tree_bwd_impl(d, n_nodes, node_off, parent, q, k, v, o, lse, dout, gk_acc, gv_acc, dq,
                       dk, dv, dkv_dtype, workspace, workspace_bytes, stream);
}

// ------------------------------------------------- compact log-probabilities

namespace {

pf_status check_logprob(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride,
                        int32_t dtype, const int32_t* row_ptr, const int32_t* pos,
                        const int32_t* y, int32_t n_pos) {
  if (dtype != PF_BF16 && dtype != PF_F32) return fail(PF_ERR_INVALID_ARG, "dtype must be PF_BF16 or PF_F32");
  if (n_rows < 0 || n_pos < 0) return fail(PF_ERR_INVALID_ARG, "n_rows and n_pos must be >= 0");
  if (vocab < 1) return fail(PF_ERR_INVALID_ARG, "vocab must be >= 1");
  if (n_rows == 0) return PF_OK;
  const int64_t eb = dtype == PF_BF16 ? 2 : 4;
  if (!z || (uintptr_t)z % 16) return fail(PF_ERR_INVALID_ARG, "z is NULL or not 16-byte aligned");
  if (z_stride < vocab || (z_stride * eb) % 16)
    return fail(PF_ERR_INVALID_ARG, "z row stride must be >= vocab and a multiple of 16 bytes");
  if (!row_ptr) return fail(PF_ERR_INVALID_ARG, "row_ptr is NULL");
  if (n_pos > 0 && (!pos || !y)) return fail(PF_ERR_INVALID_ARG, "pos or y is NULL");
  return PF_OK;
}

}  // namespace

pf_status pf_compact_logprob_fwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride,
                                 int32_t dtype, const int32_t* row_ptr, const int32_t* pos,
                                 const int32_t* y, int32_t n_pos, float* lse, float* logp,
                                 void* stream) {
  pf_status s = check_logprob(n_rows, vocab, z, z_stride, dtype, row_ptr, pos, y, n_pos);
  if (s != PF_OK) return s;
  if (n_rows == 0) return PF_OK;
  if (!lse) return fail(PF_ERR_INVALID_ARG, "lse is NULL");
  if (n_pos > 0 && !logp) return fail(PF_ERR_INVALID_ARG, "logp is NULL");
  const int64_t eb = dtype == PF_BF16 ? 2 : 4;
  const hipError_t e = pf::launch_logprob_fwd(n_rows, vocab, z, z_stride * eb, dtype == PF_BF16,
                                              row_ptr, pos, y, n_pos, lse, logp,
                                              (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "logprob_fwd");
}

pf_status pf_compact_logprob_bwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride,
                                 int32_t dtype, const float* lse, const int32_t* row_ptr,
                                 const int32_t* pos, const int32_t* y, int32_t n_pos,
                                 const float* dlogp, void* dz, int64_t dz_stride, void* stream) {
  pf_status s = check_logprob(n_rows, vocab, z, z_stride, dtype, row_ptr, pos, y, n_pos);
  if (s != PF_OK) return s;
  if (n_rows == 0) return PF_OK;
  const int64_t eb = dtype == PF_BF16 ? 2 : 4;
  if (!lse) return fail(PF_ERR_INVALID_ARG, "lse is NULL");
  if (n_pos > 0 && !dlogp) return fail(PF_ERR_INVALID_ARG, "dlogp is NULL");
  if (!dz || (uintptr_t)dz % 16) return fail(PF_ERR_INVALID_ARG, "dz is NULL or not 16-byte aligned");
  if (dz_stride < vocab || (dz_stride * eb) % 16)
    return fail(PF_ERR_INVALID_ARG, "dz row stride must be >= vocab and a multiple of 16 bytes");
  const hipError_t e = pf::launch_logprob_bwd(n_rows, vocab, z, z_stride * eb, dtype == PF_BF16, lse,
                                              row_ptr, pos, y, n_pos, dlogp, dz, dz_stride * eb,
                                              (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "logprob_bwd");
}

}  // extern "C"
