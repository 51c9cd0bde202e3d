// bf16 attention kernels for gfx950 (CDNA4), head_dim 128, fp32 accumulation.
//
// Three kernels cover every phase (see pf_internal.h for the visibility rule):
//   fwd_kernel      Q-stationary forward with online softmax: the Phase-B
//                   suffix forward over the cached prefix (read in place),
//                   Phase A (causal prefix) and the tree forward.
//   bwd_dq_kernel   Q-stationary backward: D = rowsum(dO * O) and dQ.
//   bwd_dkv_kernel  KV-stationary backward: dK, dV of a key block summed over
//                   the query rows of its range and every query head of its KV
//                   head.  For the prefix ("external") keys of Phase B that sum
//                   is the group's prefix-side gradient gK/gV (PrefixFlow §3.3,
//                   §4.1), added to the fp32 accumulator by the one workgroup
//                   that owns the block, or written as a per-chunk partial and
//                   reduced in a fixed order: no atomics, no races.
//
// Matrix cores: every product is v_mfma_f32_32x32x16_bf16,
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8 (l / 32) + e][l % 32]
//   C (32 x 32): lane l holds C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i = 0..15
// A C tile is reused directly as the B operand of the next product: its 16
// values per lane are two 8-value k-steps whose contraction index runs over
// rows {16 s + 8 (e / 4) + 4 (l / 32) + e % 4}.  The matching A operand is read
// from a row-major tile with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16), whose per-lane row addresses implement that order, so
// no tile is ever stored transposed.
//
// LDS tiles hold rows of 128 bf16 (256 B) without padding; the 16-byte chunk
// c of row r is stored at chunk c ^ swz(r).  swz spreads 16 consecutive rows
// read at one chunk (the 16-byte fragment reads) and 4 consecutive rows read
// across 4 chunks (the transposing reads) over all 64 banks.
//
// Each wave owns 64 rows of its stationary operand (queries in the forward
// and dQ kernels, keys in the dK/dV kernel), so every fragment read from LDS
// feeds two MFMAs and LDS traffic stays near half of its bandwidth at full
// MFMA rate.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "pf_internal.h"
#include "pf_partials.h"

namespace pf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kD = 128;            // head_dim of this kernel family
constexpr int kThreads = 256;      // 4 waves
constexpr int kRowB = 2 * kD;      // bytes of one LDS tile row
constexpr int kRowsPerWg = 256;    // query rows (token x head) per Q-stationary workgroup
constexpr float kRescale = 8.0f;   // lazy rescale threshold (log2 units)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulating product with the accumulator held in AGPRs (acc += A B).  The
// compiler keeps MFMA results it feeds to VALU code in VGPRs; the long-lived
// accumulators of the PV, dQ and dK/dV products go to the AGPR file through
// this form so the two files together hold a wave's working set.
// The compiler inserts wait states around builtin MFMAs but not around asm:
//   - operands written by VALU code (packed P or dS fragments, fragments
//     assembled from two transposing reads) need 2 wait states before an
//     MFMA reads them; every asm product carries them itself (s_nop 1);
//   - back-to-back accumulation into the same registers needs none;
//   - accumulators pass through fence_acc() between the last product and
//     VALU reads of them, and between VALU writes (rescaling) and the next
//     product;
//   - nothing else may touch an accumulator within a product's latency.  The
//     compiler only moves AGPR values when it runs short of registers, so
//     the kernels stay below the register files' size, and the build checks
//     the generated assembly for any such access (asm_check.py).
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void fence_acc(f32x16 (&x)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0][0]), "+a"(x[0][1]), "+a"(x[1][0]), "+a"(x[1][1]), "+a"(x[2][0]),
                 "+a"(x[2][1]), "+a"(x[3][0]), "+a"(x[3][1]));
}

__device__ __forceinline__ void fence_acc(f32x16 (&x)[4][2], f32x16 (&y)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0][0]), "+a"(x[0][1]), "+a"(x[1][0]), "+a"(x[1][1]), "+a"(x[2][0]),
                 "+a"(x[2][1]), "+a"(x[3][0]), "+a"(x[3][1]), "+a"(y[0][0]), "+a"(y[0][1]),
                 "+a"(y[1][0]), "+a"(y[1][1]), "+a"(y[2][0]), "+a"(y[2][1]), "+a"(y[3][0]),
                 "+a"(y[3][1]));
}

// keep a stationary fragment in the AGPR file; MFMAs read it from there
__device__ __forceinline__ void pin_agpr(bf16x8& x) { asm("" : "+a"(x)); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 load8(const __bf16* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.f;
  return z;
}

// 8 bf16 values from a C-tile half (values [8 half, 8 half + 8))
__device__ __forceinline__ bf16x8 pack_half(const f32x16& c, int half) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)c[8 * half + i];
  return r;
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.  Every kernel keeps its tiles in one __shared__ byte
// array at compile-time offsets; a fragment read is one per-lane offset from
// the Frag table plus an immediate (tile, buffer, row block).
__device__ __forceinline__ uint32_t swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// byte offset of element (r, col) of a tile
__device__ __forceinline__ uint32_t toff(int r, int col) {
  return (uint32_t)r * kRowB + ((((uint32_t)col >> 3) ^ swz(r)) << 4) + (((uint32_t)col & 7) << 1);
}

// Per-lane offsets of the two fragment shapes (swz depends on the row mod 16
// only, so whole 16-row blocks are immediates):
//   row8[ds]    16-byte fragment (row l % 32, columns 16 ds + 8 (l / 32) ..+7):
//               the A/B operand layout along the contraction over head_dim;
//               add 32 rows (8192 B) per further 32-row tile.
//   tr[dt][hi]  transposing read for the A operand (32 m x 16 k) from a
//               row-major [k][m] tile, m-tile dt (columns 32 dt ..), rows
//               4 (l / 32) + (l % 16) / 4 + 8 hi; add 4096 B per 16-row k-step.
//               Element e of the fragment is tile[16 s + 8 (e / 4) + 4 (l / 32)
//               + e % 4][32 dt + l % 32], the contraction order of a C tile
//               reused as a B operand: within each 16-lane group the
//               transposing read hands lane i element (i & 3) of the 8 bytes
//               addressed by lane 4 k + (i >> 2), for k = 0..3.
struct Frag {
  uint32_t row8[kD / 16];
  uint32_t tr[kD / 32][2];
};

__device__ __forceinline__ void frag_init(Frag& f, int lane) {
  const int col = lane & 31, h = lane >> 5, i = lane & 15;
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) f.row8[ds] = toff(col, ds * 16 + 8 * h);
  const int r0 = 4 * h + (i >> 2);
  const int c0 = 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) {
    f.tr[dt][0] = toff(r0, dt * 32 + c0);
    f.tr[dt][1] = toff(r0 + 8, dt * 32 + c0);
  }
}

// The same offsets derived from three registers: row8[ds] = row8[0] ^ 32 ds
// and tr[dt][hi] = tr[0][hi] ^ 64 dt, because the terms differ only in chunk
// bits that the swizzle XORs.  fresh() hides the bases from loop-invariant
// hoisting, so a kernel short of registers recomputes each offset with one
// XOR instead of holding sixteen.
struct FragC {
  uint32_t row8_0;
  uint32_t tr0[2];
  __device__ void init(const Frag& f) {
    row8_0 = f.row8[0];
    tr0[0] = f.tr[0][0];
    tr0[1] = f.tr[0][1];
  }
  __device__ void fresh() { asm volatile("" : "+v"(row8_0), "+v"(tr0[0]), "+v"(tr0[1])); }
  __device__ uint32_t row8(int ds) const { return row8_0 ^ (uint32_t)(ds << 5); }
  __device__ uint32_t tr(int dt, int hi) const { return tr0[hi] ^ (uint32_t)(dt << 6); }
};

__device__ __forceinline__ bf16x8 ld_row8(const lds_t* p) { return *(const lds_bf16x8*)p; }

__device__ __forceinline__ bf16x8 ld_tr(const lds_t* lo, const lds_t* hi) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lo);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void st16(lds_t* p, u32x4 v) { *(lds_u32x4*)p = v; }

__device__ __forceinline__ u32x4 load16(const __bf16* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }


template <int B> using Buf = std::integral_constant<int, B>;

// f(integral_constant<I>) for I in [I0, N): loop indices that must be
// compile-time constants (asm operand selection)
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>());
    static_for<I0 + 1, N>(f);
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (buffer loads with the LDS destination).  A
// buffer resource covers one block of rows; reads past its end return zero,
// so ragged tails need no masking of the load.  Each wave moves four 256-byte
// rows per instruction, lane l landing at byte 16 l of them: lane l of wave w
// fetches the logical chunk (l & 15) ^ swz(r) of row r = 4 w + l / 16 (plus 16
// rows per further pass), which puts every chunk at its swizzled position.
//
// The loads are issued from inline asm.  The compiler treats a staging load
// as a write to any LDS address, so it would wait for every staging load in
// flight before the next LDS read, which defeats staging ahead; here every
// wait is explicit (dma_wait*).  The statement sets M0 (the LDS base of the
// load) itself; the build checks that no other instruction reads or writes
// M0.  Resources are plain SGPR quads: base, stride 0, size in bytes, and
// the raw-buffer format word.
typedef __attribute__((address_space(3))) void lds_void;
typedef u32x4 Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  Rsrc r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const lds_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// 16 bytes per lane into dst + 16 lane
__device__ __forceinline__ void lds_dma16(Rsrc r, const lds_t* dst, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr(dst)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

// 4 bytes per lane into dst + 4 lane
__device__ __forceinline__ void lds_dma4(Rsrc r, const lds_t* dst, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr(dst)), "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

__device__ __forceinline__ Rsrc row_rsrc(const void* base, int nvalid, uint32_t st_b) {
  return make_rsrc(base, nvalid > 0 ? (uint32_t)(nvalid - 1) * st_b + kRowB : 0u);
}

__device__ __forceinline__ uint32_t dma_lane_off(int wave, int lane, uint32_t st_b) {
  const int r = 4 * wave + (lane >> 4);
  return (uint32_t)r * st_b + ((((uint32_t)lane & 15) ^ swz(r)) << 4);
}

// ROWS rows into `tile`, issued by every one of the group's WAVES waves (each
// moves 4 rows per load)
template <int ROWS, int WAVES = 4>
__device__ __forceinline__ void dma_rows(Rsrc res, uint32_t lane_off, uint32_t st_b, lds_t* tile,
                                         int wave) {
  static_assert(ROWS % (4 * WAVES) == 0, "rows must cover every wave");
#pragma unroll
  for (int i = 0; i < ROWS / (4 * WAVES); ++i)
    lds_dma16(res, tile + (4 * WAVES * i + 4 * wave) * kRowB, lane_off, i * 4 * WAVES * st_b);
}

// completes this wave's staging loads (a barrier then publishes them)
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup -> (KV head, item) with XCD awareness: workgroups are dispatched
// round-robin over the 8 XCDs, so when Hkv is a multiple of 8 every XCD gets
// the items of its own KV heads (their K/V or Q/dO stay in that XCD's L2),
// and when Hkv divides 8 every KV head gets 8 / Hkv XCDs of its own.  Padding
// workgroups of the second form get g = Hkv (the kernels return at once).
__device__ __forceinline__ void map_block(int bid, int hkv, int items, int& g, int& item) {
  if ((hkv & 7) == 0) {
    const int xcd = bid & 7, pos = bid >> 3;
    const int hh = pos / items;
    item = pos - hh * items;
    g = xcd + 8 * hh;
  } else if ((8 % hkv) == 0) {
    const int xpg = 8 / hkv, xcd = bid & 7;
    g = xcd / xpg;
    item = (bid >> 3) * xpg + (xcd - g * xpg);
    if (item >= items) g = hkv;
  } else {
    g = bid / items;
    item = bid - g * items;
  }
}

// ---------------------------------------------------------------------------
// Query-row bookkeeping shared by the Q-stationary kernels.  A workgroup owns
// tq tokens x G query heads of one KV head; row r of the tile is head
// j = r / tq, token t0 + r % tq.  Wave w owns rows [64 w, 64 w + 64) as two
// 32-row column tiles.
struct QCol {
  int tok;
  int head;
  bool valid;
};

__device__ __forceinline__ QCol qcol(const AttnArgs& a, int g, int t0, int tq, int r) {
  QCol c;
  const int j = r / tq;
  c.tok = t0 + (r - j * tq);
  c.valid = (j < a.group) && (c.tok < a.rows);
  c.head = c.valid ? a.ri.qhead[g * a.group + j] : 0;
  if (!c.valid) c.tok = 0;
  return c;
}

// Uniform reads of tables the kernel never writes (key-block summaries) as
// scalar loads: through the constant address space the compiler may use the
// scalar cache, so reading them does not wait on the vector memory counter
// that the staging loads use.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((const_i32*)p)[i]; }

// Iteration over key blocks of a Q-stationary tile: external blocks first,
// then own blocks that hold at least one key visible to some query of the
// tile (bmax > t0), stopping at the tile's last token.
template <int BN>
struct KeyWalk {
  int n_ext_blocks;
  int t0, t1;             // token range [t0, t1) of the tile
  const int32_t* bmax;
  const int32_t* bmin;
  int rows;
  const int2* tiles;      // external keys as row ranges (padding needs a mask), or null

  __device__ int own_block_max(int kb) const {
    int m = -1;
#pragma unroll
    for (int s = 0; s < BN / kKeyBlockSummary; ++s) {
      const int b = kb * (BN / kKeyBlockSummary) + s;
      if (b * kKeyBlockSummary < rows) m = max(m, ld_uniform(bmax, b));
    }
    return m;
  }
  __device__ int own_block_min(int kb) const {
    int m = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < BN / kKeyBlockSummary; ++s) {
      const int b = kb * (BN / kKeyBlockSummary) + s;
      if (b * kKeyBlockSummary < rows) m = min(m, ld_uniform(bmin, b));
    }
    return m;
  }
  // next block index >= i (ext blocks are [0, n_ext_blocks), own block kb is
  // index n_ext_blocks + kb); returns -1 when done
  __device__ int next(int i) const {
    if (i < n_ext_blocks) return i;
    for (int kb = i - n_ext_blocks; kb * BN < t1; ++kb) {
      if (own_block_max(kb) > t0) return n_ext_blocks + kb;
    }
    return -1;
  }
  // does the block need an element mask
  __device__ bool masked(int i, int n_ext) const {
    if (i < n_ext_blocks) {
      if ((i + 1) * BN > n_ext) return true;
      if (!tiles) return false;
      int m = 32;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
        m = min(m, ld_uniform((const int32_t*)tiles, 2 * ((i * BN) / 32 + kt) + 1));
      return m < 32;
    }
    const int kb = i - n_ext_blocks;
    const int k0 = kb * BN;
    if (k0 + BN > rows) return true;
    if (k0 + BN - 1 > t0) return true;
    return own_block_min(kb) < t1;
  }
};

// The rows of one KV head in a key source (the cached prefix or the call's
// own rows) as one buffer resource over all of them: a block is selected by
// the scalar offset, which the hardware range check includes, so rows past
// the last one read zero.  Built once per workgroup; staging a block is then
// scalar arithmetic plus the loads.
struct RowSrc {
  Rsrc res;
  const char* base;    // row 0
  int nrows;           // rows the resource covers
  uint32_t st_b;       // bytes per row
  uint32_t lane_off;   // this lane's byte offset within a 4-row pass
  __device__ void init(const void* base_, int nrows_, int64_t st_elems, int wave, int lane) {
    base = (const char*)base_;
    nrows = nrows_;
    st_b = 2u * (uint32_t)st_elems;
    res = row_rsrc(base_, nrows_, st_b);
    lane_off = dma_lane_off(wave, lane, st_b);
  }
  // the same for the virtual external keys [r0, r0 + ROWS) of a call whose
  // external keys are row ranges (tile table `tiles`, n_ext virtual keys):
  // each pass of 4 WAVES rows lies in one 32-key tile and is read from that
  // tile's rows; padding and keys past n_ext read zero
  template <int ROWS, int WAVES = 4>
  __device__ void stage_tiled(const int2* tiles, int n_ext, int r0, lds_t* tile, int wave) const {
    constexpr int RS = 4 * WAVES;
    static_assert(32 % RS == 0 && ROWS % RS == 0, "a pass lies in one tile");
#pragma unroll
    for (int i = 0; i < ROWS / RS; ++i) {
      const int vr = r0 + RS * i;
      int first = 0, valid = 0;
      if (vr < n_ext) {
        first = ld_uniform((const int32_t*)tiles, 2 * (vr >> 5));
        valid = ld_uniform((const int32_t*)tiles, 2 * (vr >> 5) + 1) - (vr & 31);
        first += vr & 31;
      }
      lds_dma16(row_rsrc(base + (int64_t)first * st_b, valid, st_b),
                tile + (RS * i + 4 * wave) * kRowB, lane_off, 0u);
    }
  }
  // rows [r0, r0 + ROWS) into `tile`, issued by every one of the group's
  // WAVES waves (each moves 4 rows per load)
  template <int ROWS, int WAVES = 4>
  __device__ void stage(int r0, lds_t* tile, int wave) const {
    static_assert(ROWS % (4 * WAVES) == 0, "rows per stage must cover every wave");
#pragma unroll
    for (int i = 0; i < ROWS / (4 * WAVES); ++i)
      lds_dma16(res, tile + (4 * WAVES * i + 4 * wave) * kRowB, lane_off,
                (uint32_t)(r0 + 4 * WAVES * i) * st_b);
  }
};

// The key blocks a Q-stationary tile visits, in order (see KeyWalk): block b
// < n_ext_blocks is prefix block b, later ones are own blocks.
template <int BN>
struct BlockSrc {
  int n_ext_blocks;
  const int2* tiles;   // external keys as row ranges (or null)
  int n_ext;
  RowSrc kx, vx, ko, vo;
  __device__ void init(const AttnArgs& a, int g, int n_ext_blk, int wave, int lane) {
    n_ext_blocks = n_ext_blk;
    tiles = a.ext_tiles;
    n_ext = a.n_ext;
    const int xrows = a.ext_tiles ? a.ext_rows : a.n_ext;
    kx.init((const __bf16*)a.k_ext + (int64_t)g * a.kx_sh, xrows, a.kx_st, wave, lane);
    vx.init((const __bf16*)a.v_ext + (int64_t)g * a.vx_sh, xrows, a.vx_st, wave, lane);
    ko.init((const __bf16*)a.k_own + (int64_t)g * a.ko_sh, a.rows, a.ko_st, wave, lane);
    vo.init((const __bf16*)a.v_own + (int64_t)g * a.vo_sh, a.rows, a.vo_st, wave, lane);
  }
  __device__ bool ext(int b) const { return b < n_ext_blocks; }
  __device__ int k0(int b) const { return (ext(b) ? b : b - n_ext_blocks) * BN; }
  // stage the K or V rows of block b into an LDS tile (rows past the end
  // read 0), issued by all WAVES waves of the group
  template <int WAVES = 4>
  __device__ void dma_k(int b, lds_t* tile, int wave, int /*lane*/) const {
    if (ext(b)) {
      if (tiles)
        kx.stage_tiled<BN, WAVES>(tiles, n_ext, k0(b), tile, wave);
      else
        kx.stage<BN, WAVES>(k0(b), tile, wave);
    } else {
      ko.stage<BN, WAVES>(k0(b), tile, wave);
    }
  }
  template <int WAVES = 4>
  __device__ void dma_v(int b, lds_t* tile, int wave, int /*lane*/) const {
    if (ext(b)) {
      if (tiles)
        vx.stage_tiled<BN, WAVES>(tiles, n_ext, k0(b), tile, wave);
      else
        vx.stage<BN, WAVES>(k0(b), tile, wave);
    } else {
      vo.stage<BN, WAVES>(k0(b), tile, wave);
    }
  }
  // valid keys of the external 32-key tiles of block b (b external)
  __device__ void ext_valid(int b, int (&v)[BN / 32]) const {
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt) {
      const int vk = b * BN + 32 * kt;
      if (tiles)
        v[kt] = vk < n_ext ? ld_uniform((const int32_t*)tiles, 2 * (vk >> 5) + 1) : 0;
      else
        v[kt] = min(32, max(0, n_ext - vk));
    }
  }
};

// kend of the own keys of block b (thread tid < BN holds key k0 + tid)
template <int BN>
__device__ __forceinline__ int load_kend(const AttnArgs& a, const BlockSrc<BN>& src, int b, int tid) {
  if (src.ext(b) || tid >= BN) return -1;
  const int kk = src.k0(b) + tid;
  return kk < a.rows ? a.ri.kend[kk] : -1;
}

// Mask of an S^T tile set (BN keys x NT query columns, C layout: rows are
// keys): invisible entries become -inf.  Branch-free per element; the kend
// values are read four keys at a time, one group after another, so the mask
// holds few registers beside the tiles.  tok[nt] is the lane's query token of
// column tile nt.
// evalid[kt] is the number of valid keys of external key tile kt (padding of
// row ranges, or the end of the external keys); own keys use klim.
template <int BN, int NT>
__device__ __forceinline__ void mask_st(f32x16 (&s)[BN / 32][NT], bool ext, int k0, int klim,
                                        const int32_t* kend, const int (&tok)[NT], int h32,
                                        const int (&evalid)[BN / 32]) {
#pragma unroll
  for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int kl0 = kt * 32 + 8 * jj + 4 * h32;
      int ke4[4];
      if (!ext) {
        const int4 v = *(const int4*)&kend[kl0];
        ke4[0] = v.x; ke4[1] = v.y; ke4[2] = v.z; ke4[3] = v.w;
      } else {
        ke4[0] = ke4[1] = ke4[2] = ke4[3] = 0x7fffffff;
      }
      // bitwise, not short-circuit, tests: one select per element, no branch
      const int ext_i = ext ? 1 : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * jj + r;
        const int kk = k0 + kl0 + r;
        const int in = ext ? ((8 * jj + 4 * h32 + r) < evalid[kt] ? 1 : 0) : (kk < klim ? 1 : 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int own = (kk <= tok[nt] ? 1 : 0) & (tok[nt] < ke4[r] ? 1 : 0);
          s[kt][nt][i] = (in & (ext_i | own)) ? s[kt][nt][i] : -INFINITY;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Forward.
//
// A workgroup holds kRowsPerWg query rows; each wave holds NT column tiles of
// 32 rows, so there are 8 / NT waves.  With NT = 1 (the build's choice) the
// eight waves run two per SIMD: while one issues matrix-core products the
// other's softmax arithmetic, LDS reads and waits proceed, which a single
// wave per SIMD cannot overlap with its own products.  Each key block j (64
// keys) runs in two matrix-core phases:
//   A  S^T of block j + 1 (K Q^T) on the matrix cores while the VALU finishes
//      P_j = exp2(S_j c - m), packs it to bf16 and adds its row sums;
//   B  O^T += V_j^T P_j^T on the matrix cores while the VALU takes the row
//      maxima of S_{j+1} and moves the running maxima (lazy rescale).
// K and V rotate through three LDS buffers each: iteration j stages K of
// block j + 3 and V of block j + 2, so every staging load has a whole
// iteration to land before the wait that precedes its use.  One barrier per
// block.  Two register sets for S alternate with the buffers (unrolled x6).
constexpr int kFwdBN = 64;
constexpr int kFwdTile = kFwdBN * kRowB;            // one K or V block
constexpr int kFwdK = 0, kFwdV = 3 * kFwdTile;      // three K buffers, then three V buffers
constexpr int kFwdNT = 1;                           // 32-row query tiles per wave

// max(x[l], x[l ^ 32]) in every lane, without LDS
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// waits for all but the `n` most recent staging loads of this wave
template <int N>
__device__ __forceinline__ void dma_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// workgroup barrier for LDS hand-offs: this wave's LDS accesses complete,
// then all waves meet.  Unlike __syncthreads() it does not wait for global
// memory operations, so staging loads issued ahead stay in flight (their
// own waits are explicit).  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Register placement of the forward's accumulators.  With one wave per SIMD
// (NT = 2) the wave has 512 registers and the long-lived O accumulators and Q
// fragments go to the AGPR file through the asm product; with two waves per
// SIMD (NT = 1) a wave has 256, and a kernel that uses any AGPR gets only half
// of them as VGPRs, so everything stays in VGPRs and the builtin product
// (whose hazards the compiler handles) is used.
template <int NT>
__device__ __forceinline__ void fence_acc_nt(f32x16 (&x)[kD / 32][NT]) {
  if constexpr (NT == 2) fence_acc(x);
}
template <int NT>
__device__ __forceinline__ void mfma_acc_nt(f32x16& acc, bf16x8 a, bf16x8 b) {
  if constexpr (NT == 2)
    mfma_acc(acc, a, b);
  else
    acc = mfma(a, b, acc);
}

template <int NT>
__global__ __launch_bounds__(64 * 8 / NT, 1) void fwd_kernel(AttnArgs a) {
  constexpr int BN = kFwdBN;
  constexpr int WAVES = 8 / NT;
  constexpr int kDma = BN / (4 * WAVES);     // staging loads per wave per K or V tile
  constexpr int VPS = 4 * NT;                // P (or maxima) values per lane per step
  constexpr int KPD = NT == 1 ? 2 : 1;       // K fragment prefetch distance (steps)
  constexpr int VPD = NT == 1 ? 3 : 2;       // V fragment prefetch distance (products)
  __shared__ __attribute__((aligned(16))) char smem[6 * kFwdTile];
  __shared__ __attribute__((aligned(16))) int32_t kend_s[3][BN];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;

  int g, item;
  map_block(blockIdx.x, a.hkv, n_qt, g, item);
  if (g >= a.hkv) return;
  const int qt = n_qt - 1 - item;            // later tiles (more own keys) first
  const int t0 = qt * tq;
  const int t1 = min(t0 + tq, a.rows);

  // this lane's query columns and their Q fragments (B operand of K Q^T,
  // kept in AGPRs)
  QCol qc[NT];
  int tok[NT];
  bf16x8 qf[NT][kD / 16];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    qc[nt] = qcol(a, g, t0, tq, wave * 32 * NT + nt * 32 + col);
    tok[nt] = qc[nt].tok;
    const __bf16* qp = (const __bf16*)a.q + (int64_t)qc[nt].tok * a.q_st +
                       (int64_t)qc[nt].head * a.q_sh + 8 * h32;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) qf[nt][ds] = load8(qp + ds * 16);   // row 0 if invalid
  }
  // all loads in flight before the first use
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      if (!qc[nt].valid) qf[nt][ds] = zero8();
      if constexpr (NT == 2) pin_agpr(qf[nt][ds]);
    }

  KeyWalk<BN> walk;
  walk.n_ext_blocks = (a.n_ext + BN - 1) / BN;
  walk.t0 = t0;
  walk.t1 = t1;
  walk.bmax = a.ri.bmax;
  walk.bmin = a.ri.bmin;
  walk.rows = a.rows;
  walk.tiles = a.ext_tiles;
  BlockSrc<BN> src;
  src.init(a, g, walk.n_ext_blocks, wave, lane);

  FragC f;
  {
    Frag ff;
    frag_init(ff, lane);
    f.init(ff);
  }
  // V reads (the only users of the transposed offsets here): the V region's
  // base folded into the lane offsets (it only sets bits above the swizzled
  // ones), so buffer and slice offsets fit the LDS instructions' 16-bit
  // immediate and need no address add
  f.tr0[0] += (uint32_t)kFwdV;
  f.tr0[1] += (uint32_t)kFwdV;
  const float c = a.scale_log2;
  float mrow[NT], lrow[NT];                 // running max (log2 units) in use; row-sum share
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    mrow[nt] = -INFINITY;
    lrow[nt] = 0.f;
  }
  f32x16 acc[kD / 32][NT];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[dt][nt] = zero16();
  fence_acc_nt<NT>(acc);

  // S^T tile of the K block in `kt_s`: 64 keys x this wave's query columns
  auto s_tile = [&](const lds_t* kt_s, f32x16 (&s)[BN / 32][NT]) {
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[kt][nt] = zero16();
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
        const bf16x8 af = ld_row8(kt_s + kt * 32 * kRowB + f.row8(ds));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[kt][nt] = mfma(af, qf[nt][ds], s[kt][nt]);
      }
    }
  };
  // key blocks in walk order, with whether they need an element mask (found
  // when the block is first reached, so the mask test reads no memory later)
  struct Blk {
    int id;
    bool masked;
  };
  auto blk = [&](int b) { return Blk{b, b >= 0 && walk.masked(b, a.n_ext)}; };
  auto nxt = [&](Blk b) { return blk(b.id >= 0 ? walk.next(b.id + 1) : -1); };
  auto mask_if = [&](f32x16 (&s)[BN / 32][NT], Blk b, const int32_t* kend) {
    if (b.masked) {
      int ev[BN / 32] = {};
      if (src.ext(b.id)) src.ext_valid(b.id, ev);
      mask_st<BN, NT>(s, src.ext(b.id), src.k0(b.id), src.ext(b.id) ? a.n_ext : a.rows, kend,
                      tok, h32, ev);
    }
  };
  // the lazy move of the running maxima to the block maxima mx (valid when
  // `live`): only when a block exceeds them by more than kRescale, so
  // probabilities stay below 2^kRescale.  Returns the factors the
  // accumulators must be scaled by.
  auto move_max = [&](const float (&mx)[NT], bool live, float (&alpha)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mh = max_halves(mx[nt]) * c;
      const float m = live ? mh : -INFINITY;
      const bool grow = m > mrow[nt] + kRescale;
      const float mnew = grow ? m : mrow[nt];
      alpha[nt] = fast_exp2(grow ? mrow[nt] - mnew : 0.f);
      lrow[nt] *= alpha[nt];
      mrow[nt] = mnew;
    }
  };
  auto rescale = [&](const float (&alpha)[NT]) {
    bool any = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) any = any || alpha[nt] != 1.f;
    if (__builtin_amdgcn_ballot_w64(any) != 0) {
      fence_acc_nt<NT>(acc);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) acc[dt][nt] *= alpha[nt];
      fence_acc_nt<NT>(acc);
    }
  };
  auto stage_k = [&](int b, int buf) {
    src.template dma_k<WAVES>(b, sb + kFwdK + buf * kFwdTile, wave, lane);
  };
  auto stage_v = [&](int b, int buf) {
    src.template dma_v<WAVES>(b, sb + kFwdV + buf * kFwdTile, wave, lane);
  };
  // visibility ends of an own block's keys into kend_s[buf], by one staging
  // load of wave 0 (keys past the end read 0: invisible)
  auto stage_kend = [&](int b, int buf) {
    if (src.ext(b) || wave != 0) return;
    const int k0 = src.k0(b);
    lds_dma4(make_rsrc(a.ri.kend + k0, 4u * (uint32_t)(a.rows - k0)), (const lds_t*)&kend_s[buf][0],
             4u * lane, 0u);
  };

  // prologue: K and V of blocks 0 and 1, K of block 2; S of block 0
  const Blk b0 = blk(walk.next(0));
  const Blk b1 = nxt(b0);
  const Blk b2 = nxt(b1);
  if (b0.id >= 0) {
    stage_kend(b0.id, 0);
    if (b1.id >= 0) stage_kend(b1.id, 1);
    if (b2.id >= 0) stage_kend(b2.id, 2);
    stage_k(b0.id, 0);
    stage_v(b0.id, 0);
    if (b1.id >= 0) {
      stage_k(b1.id, 1);
      stage_v(b1.id, 1);
    }
    if (b2.id >= 0) stage_k(b2.id, 2);
  }
  dma_wait();
  __syncthreads();
  f32x16 sA[BN / 32][NT], sB[BN / 32][NT];
  if (b0.id >= 0) {
    s_tile(sb + kFwdK, sA);
    mask_if(sA, b0, kend_s[0]);
    float mx[NT], alpha[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mx[nt] = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx[nt] = fmaxf(mx[nt], sA[kt][nt][i]);
    }
    move_max(mx, true, alpha);
  }

  // iteration j: block j's S in sc (maxima applied), its V in V buffer B, K
  // of block j + 1 (n1) in K buffer B + 1.  Stages K of n3 into K buffer B
  // and V of n2 into V buffer B + 2.
  auto iter = [&](auto bc, f32x16 (&sc)[BN / 32][NT], f32x16 (&sn)[BN / 32][NT], Blk n1, Blk n2,
                  Blk n3) {
    constexpr int B = decltype(bc)::value;
    constexpr int B1 = (B + 1) % 3, B2 = (B + 2) % 3;
    f.fresh();
    // wave 0 stages n3's kend before the tiles, so the waits below (which
    // leave this iteration's tile loads in flight) cover it
    if (n3.id >= 0) stage_kend(n3.id, B);
    if (n3.id >= 0) stage_k(n3.id, B);
    if (n2.id >= 0) stage_v(n2.id, B2);

    // phase A: S^T of block j + 1 while P_j is completed and packed.  Eight
    // steps, one per 16-wide slice of head_dim: each issues the K fragments
    // KPD steps ahead, its products and one eighth of the P work; the
    // scheduling fences keep that order.
    const lds_t* kt_s = sb + kFwdK + B1 * kFwdTile;
    bf16x8 kfr[KPD + 1][BN / 32];
    auto ldk = [&](int ds, bf16x8 (&dst)[BN / 32]) {
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) dst[kt] = ld_row8(kt_s + kt * 32 * kRowB + f.row8(ds));
    };
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sn[kt][nt] = zero16();
    bf16x8 pb[NT][BN / 16];
    float ls[NT], muse[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ls[nt] = 0.f;
      muse[nt] = (mrow[nt] == -INFINITY) ? 0.f : mrow[nt];
    }
#pragma unroll
    for (int d0 = 0; d0 < KPD; ++d0) ldk(d0, kfr[d0]);
    static_for<0, kD / 16>([&](auto dsc) {
      constexpr int ds = decltype(dsc)::value;
      if constexpr (ds + KPD < kD / 16) ldk(ds + KPD, kfr[(ds + KPD) % (KPD + 1)]);
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          sn[kt][nt] = mfma(kfr[ds % (KPD + 1)][kt], qf[nt][ds], sn[kt][nt]);
      // P values ds * VPS .. ds * VPS + VPS - 1 in (column, key tile, value) order
#pragma unroll
      for (int e = 0; e < VPS; ++e) {
        const int lin = ds * VPS + e, nt = lin >> 5, kt = (lin >> 4) & 1, i = lin & 15;
        const float p = fast_exp2(fmaf(sc[kt][nt][i], c, -muse[nt]));
        sc[kt][nt][i] = p;
        ls[nt] += p;
        if ((i & 7) == 7) {
          pb[nt][2 * kt + (i >> 3)] = pack_half(sc[kt][nt], i >> 3);
          // the half is formed here, not sunk towards its use in phase B
          asm volatile("" : "+v"(pb[nt][2 * kt + (i >> 3)]));
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(ls[nt]));
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lrow[nt] += ls[nt];
    mask_if(sn, n1, kend_s[B1]);

    // phase B: O^T += V_j^T P_j^T while the maxima of S_{j+1} are taken.
    // Sixteen steps, one per V fragment (fetched VPD steps ahead), each with
    // NT products and a sixteenth of that VALU work.
    const lds_t* vt_s = sb + B * kFwdTile;   // kFwdV is in fv's offsets
    auto ldv = [&](int fi) {
      const int dt = fi >> 2, ks = fi & 3;
      const lds_t* vb = vt_s + ks * 16 * kRowB;
      return ld_tr(vb + f.tr(dt, 0), vb + f.tr(dt, 1));
    };
    bf16x8 vfr[VPD + 1];
#pragma unroll
    for (int f0 = 0; f0 < VPD; ++f0) vfr[f0] = ldv(f0);
    float mx[NT], alpha[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mx[nt] = -INFINITY;
      alpha[nt] = 1.f;
    }
    const bool live = n1.id >= 0;
    static_for<0, kD / 32 * BN / 16>([&](auto fic) {
      constexpr int fi = decltype(fic)::value;
      constexpr int dt = fi >> 2, ks = fi & 3;
      if constexpr (fi + VPD < kD / 32 * BN / 16) vfr[(fi + VPD) % (VPD + 1)] = ldv(fi + VPD);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mfma_acc_nt<NT>(acc[dt][nt], vfr[fi % (VPD + 1)], pb[nt][ks]);
      if constexpr (fi < 8) {
        // maxima: values fi * VPS .. in (column, key tile, value) order
#pragma unroll
        for (int e = 0; e < VPS; ++e) {
          const int lin = fi * VPS + e, nt = lin >> 5, kt = (lin >> 4) & 1, i = lin & 15;
          mx[nt] = fmaxf(mx[nt], sn[kt][nt][i]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(mx[nt]));
      } else if constexpr (fi == 8) {
        move_max(mx, live, alpha);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(lrow[nt]), "+v"(mrow[nt]));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    rescale(alpha);

    if (n3.id >= 0) {
      dma_wait_n<2 * kDma>();
    } else if (n2.id >= 0) {
      dma_wait_n<kDma>();
    } else {
      dma_wait();
    }
    lds_barrier();
  };

  Blk cur = b0, n1 = b1, n2 = b2;
  while (cur.id >= 0) {
    Blk n3 = nxt(n2);
    iter(Buf<0>(), sA, sB, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(Buf<1>(), sB, sA, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(Buf<2>(), sA, sB, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(Buf<0>(), sB, sA, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(Buf<1>(), sA, sB, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(Buf<2>(), sB, sA, n1, n2, n3);
    cur = n1; n1 = n2; n2 = n3;
  }

  // finalize: O = acc / l, LSE = (m + log2 l) ln 2
  fence_acc_nt<NT>(acc);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = sum_halves(lrow[nt]);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    if (!qc[nt].valid) continue;
    __bf16* op = (__bf16*)a.out + (int64_t)qc[nt].tok * a.out_st + (int64_t)qc[nt].head * a.out_sh;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[dt][nt][4 * j + r] * inv);
        *(bf16x4*)(op + dt * 32 + 8 * j + 4 * h32) = w;
      }
    if (h32 == 0)
      a.lse[(int64_t)qc[nt].head * a.rows + qc[nt].tok] =
          (l > 0.f) ? (mrow[nt] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Backward, Q-stationary: D and dQ.
//
// Per key block j (32 keys): S^T = K Q^T and dP^T = V dO^T (matrix cores),
// dS^T = P^T (dP^T - D) with P^T = exp2(S^T c - LSE log2 e) (VALU), and
// dQ^T += K^T dS^T (matrix cores).  Software-pipelined in two phases:
//   A  S^T, dP^T of block j + 1   with  dS of block j (first 22 values)
//   B  dQ from block j - 1        with  dS of block j (last 10 values)
// so the dQ product trails one block and both phases carry VALU work.  K/V
// blocks rotate through five LDS buffers (block j - 1 is still read by phase
// B while block j + 3 is staged); the buffer of a block is a runtime index.
constexpr int kDqBN = 32;
constexpr int kDqTile = kDqBN * kRowB;
constexpr int kDqBufs = 5;
constexpr int kDqK = 0, kDqV = kDqBufs * kDqTile;   // five K buffers, then five V buffers
constexpr int kDqDma = 2 * (kDqBN / 16);            // staging loads per wave per block
constexpr int kDqSplit = 22;                        // dS values formed in phase A

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(AttnArgs a) {
  constexpr int BN = kDqBN;
  __shared__ __attribute__((aligned(16))) char smem[2 * kDqBufs * kDqTile];
  __shared__ __attribute__((aligned(16))) int32_t kend_s[kDqBufs][BN];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;

  int g, item;
  map_block(blockIdx.x, a.hkv, n_qt, g, item);
  if (g >= a.hkv) return;
  const int qt = n_qt - 1 - item;
  const int t0 = qt * tq;
  const int t1 = min(t0 + tq, a.rows);

  // stationary Q and dO fragments (AGPRs), D = rowsum(dO * O) and LSE (log2)
  // per query column; -D and LSE (log2) are also written for the dK/dV pass
  QCol qc[2];
  bf16x8 qf[2][kD / 16], df[2][kD / 16];
  float lse2[2], dsum[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    qc[nt] = qcol(a, g, t0, tq, wave * 64 + nt * 32 + col);
    const int64_t qo = (int64_t)qc[nt].tok * a.q_st + (int64_t)qc[nt].head * a.q_sh + 8 * h32;
    const int64_t doo = (int64_t)qc[nt].tok * a.do_st + (int64_t)qc[nt].head * a.do_sh + 8 * h32;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      qf[nt][ds] = load8((const __bf16*)a.q + qo + ds * 16);          // row 0 if invalid
      df[nt][ds] = load8((const __bf16*)a.dout + doo + ds * 16);
    }
  }
  {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int64_t oo = (int64_t)qc[nt].tok * a.o_st + (int64_t)qc[nt].head * a.o_sh + 8 * h32;
      float dot = 0.f;
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) {
        const bf16x8 ov = load8((const __bf16*)a.o + oo + ds * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf((float)df[nt][ds][e], (float)ov[e], dot);
      }
      dot = sum_halves(dot);
      if (!qc[nt].valid) dot = 0.f;
      dsum[nt] = dot;
      const float l = qc[nt].valid ? a.lse[(int64_t)qc[nt].head * a.rows + qc[nt].tok] : 0.f;
      lse2[nt] = (l == -INFINITY) ? INFINITY : l * kLog2e;
      if (qc[nt].valid && h32 == 0) {
        a.neg_dsum[(int64_t)qc[nt].head * a.rows + qc[nt].tok] = -dot;
        a.lse2[(int64_t)qc[nt].head * a.rows + qc[nt].tok] = lse2[nt];
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      if (!qc[nt].valid) {
        qf[nt][ds] = zero8();
        df[nt][ds] = zero8();
      }
      pin_agpr(qf[nt][ds]);
      pin_agpr(df[nt][ds]);
    }

  const int toks[2] = {qc[0].tok, qc[1].tok};
  KeyWalk<BN> walk;
  walk.n_ext_blocks = (a.n_ext + BN - 1) / BN;
  walk.t0 = t0;
  walk.t1 = t1;
  walk.bmax = a.ri.bmax;
  walk.bmin = a.ri.bmin;
  walk.rows = a.rows;
  walk.tiles = a.ext_tiles;
  BlockSrc<BN> src;
  src.init(a, g, walk.n_ext_blocks, wave, lane);

  FragC f;
  {
    Frag ff;
    frag_init(ff, lane);
    f.init(ff);
  }
  const float c = a.scale_log2;
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();
  fence_acc(acc);

  struct Blk {
    int id;
    bool masked;
  };
  auto blk = [&](int b) { return Blk{b, b >= 0 && walk.masked(b, a.n_ext)}; };
  auto nxt = [&](Blk b) { return blk(b.id >= 0 ? walk.next(b.id + 1) : -1); };
  // K and V of block b into buffer buf (a block that does not exist reads
  // zeros: its rows are past the end of the resource)
  auto stage = [&](Blk b, int buf) {
    lds_t* kt_s = sb + kDqK + buf * kDqTile;
    lds_t* vt_s = sb + kDqV + buf * kDqTile;
    if (b.id >= 0) {
      src.dma_k(b.id, kt_s, wave, lane);
      src.dma_v(b.id, vt_s, wave, lane);
      if (!src.ext(b.id) && wave == 0) {
        const int k0 = src.k0(b.id);
        lds_dma4(make_rsrc(a.ri.kend + k0, 4u * (uint32_t)(a.rows - k0)),
                 (const lds_t*)&kend_s[buf][0], 4u * lane, 0u);
      }
    } else {
      src.kx.stage<BN>(src.kx.nrows + BN, kt_s, wave);   // past the end: zeros
      src.vx.stage<BN>(src.vx.nrows + BN, vt_s, wave);
    }
  };

  // per-lane elements: (nt, i) is query column nt, key 8 (i / 4) + 4 h32 + i % 4
  f32x16 sA[1][2], dpA[2], sB[1][2], dpB[2];   // S^T as one key tile for mask_st
  bf16x8 dsA[2][2], dsB[2][2];    // packed dS^T [column][key half]
  // S^T, dP^T of the block in buffer buf into (s, dp); fragments one d-step
  // ahead; `work(ds)` is VALU work placed beside d-step ds
  auto sdp = [&](int buf, f32x16 (&s)[1][2], f32x16 (&dp)[2], auto&& work) {
    const uint32_t kb = f.row8_0 + kDqK + buf * kDqTile;
    const uint32_t vb = f.row8_0 + kDqV + buf * kDqTile;
    bf16x8 ka[2], va[2];
    ka[0] = ld_row8(sb + kb);
    va[0] = ld_row8(sb + vb);
    s[0][0] = zero16(); s[0][1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
    static_for<0, kD / 16>([&](auto dsc) {
      constexpr int ds = decltype(dsc)::value;
      if constexpr (ds + 1 < kD / 16) {
        ka[(ds + 1) & 1] = ld_row8(sb + (kb ^ (uint32_t)((ds + 1) << 5)));
        va[(ds + 1) & 1] = ld_row8(sb + (vb ^ (uint32_t)((ds + 1) << 5)));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s[0][nt] = mfma(ka[ds & 1], qf[nt][ds], s[0][nt]);
        dp[nt] = mfma(va[ds & 1], df[nt][ds], dp[nt]);
      }
      work(dsc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // dS value e (0..31) of (s, dp) into ds; e = 16 nt + i
  auto ds_elem = [&](f32x16 (&s)[1][2], f32x16 (&dp)[2], bf16x8 (&dsb)[2][2], auto ec) {
    constexpr int e = decltype(ec)::value;
    constexpr int nt = e >> 4, i = e & 15;
    const float p = fast_exp2(fmaf(s[0][nt][i], c, -lse2[nt]));
    s[0][nt][i] = p * (dp[nt][i] - dsum[nt]);
    asm volatile("" : "+v"(s[0][nt][i]));
    if constexpr ((i & 7) == 7) {
      dsb[nt][i >> 3] = pack_half(s[0][nt], i >> 3);
      asm volatile("" : "+v"(dsb[nt][i >> 3]));
    }
  };
  // dQ^T += K^T dS^T for the block whose K is in buffer buf (transposed K
  // fragments two ahead), with `work(k)` beside product pair k
  auto dq_prod = [&](int buf, const bf16x8 (&dsb)[2][2], auto&& work) {
    const uint32_t t0b = f.tr0[0] + kDqK + buf * kDqTile;
    const uint32_t t1b = f.tr0[1] + kDqK + buf * kDqTile;
    auto ldk = [&](int k) {
      const int dt = k >> 1, ks = k & 1;
      const uint32_t o = ks * 16 * kRowB;
      return ld_tr(sb + (t0b ^ (uint32_t)(dt << 6)) + o, sb + (t1b ^ (uint32_t)(dt << 6)) + o);
    };
    bf16x8 kfr[3];
    kfr[0] = ldk(0);
    kfr[1] = ldk(1);
    static_for<0, 2 * kD / 32>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int dt = k >> 1, ks = k & 1;
      if constexpr (k + 2 < 2 * kD / 32) kfr[(k + 2) % 3] = ldk(k + 2);
      mfma_acc(acc[dt][0], kfr[k % 3], dsb[0][ks]);
      mfma_acc(acc[dt][1], kfr[k % 3], dsb[1][ks]);
      work(kc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // prologue: blocks 0..2 staged into buffers 0..2, zeros into buffer 4 (the
  // "block -1" whose dQ product the first iteration runs, with dS = 0)
  const Blk b0 = blk(walk.next(0));
  const Blk b1 = nxt(b0);
  const Blk b2 = nxt(b1);
  stage(b0, 0);
  stage(b1, 1);
  stage(b2, 2);
  stage(Blk{-1, false}, kDqBufs - 1);
  dma_wait();
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int k = 0; k < 2; ++k) dsB[nt][k] = zero8();
  if (b0.id >= 0) {
    sdp(0, sA, dpA, [&](auto) {});
    if (b0.masked) {
      int ev[BN / 32] = {};
      if (src.ext(b0.id)) src.ext_valid(b0.id, ev);
      mask_st<BN, 2>(sA, src.ext(b0.id), src.k0(b0.id),
                     src.ext(b0.id) ? a.n_ext : a.rows, kend_s[0], toks, h32, ev);
    }
  }

  // iteration for block j in buffer bj with (sc, dpc) = its S^T, dP^T and
  // (sn, dpn) receiving block j + 1's; dsp holds dS of block j - 1 (buffer
  // bp), dsc receives block j's.  Stages block j + 3.
  auto iter = [&](f32x16 (&sc)[1][2], f32x16 (&dpc)[2], f32x16 (&sn)[1][2], f32x16 (&dpn)[2],
                  bf16x8 (&dsc)[2][2], const bf16x8 (&dsp)[2][2], int bj, Blk n1, Blk n3) {
    const int b1i = bj + 1 == kDqBufs ? 0 : bj + 1;
    const int b3i = bj + 3 >= kDqBufs ? bj + 3 - kDqBufs : bj + 3;
    const int bpi = bj == 0 ? kDqBufs - 1 : bj - 1;
    f.fresh();
    stage(n3, b3i);
    // phase A
    sdp(b1i, sn, dpn, [&](auto dsc_) {
      constexpr int ds = decltype(dsc_)::value;
      static_for<0, 3>([&](auto uc) {
        constexpr int e = 3 * ds + decltype(uc)::value;
        if constexpr (e < kDqSplit) ds_elem(sc, dpc, dsc, std::integral_constant<int, e>());
      });
    });
    if (n1.masked) {
      int ev[BN / 32] = {};
      if (src.ext(n1.id)) src.ext_valid(n1.id, ev);
      mask_st<BN, 2>(sn, src.ext(n1.id), src.k0(n1.id),
                     src.ext(n1.id) ? a.n_ext : a.rows, kend_s[b1i], toks, h32, ev);
    }
    // phase B
    dq_prod(bpi, dsp, [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      static_for<0, 2>([&](auto uc) {
        constexpr int e = kDqSplit + 2 * k + decltype(uc)::value;
        if constexpr (e < 32) ds_elem(sc, dpc, dsc, std::integral_constant<int, e>());
      });
    });
    // every iteration stages kDqDma tile loads per wave (zeros for a block
    // that does not exist), and wave 0 one kend load for an own block; at
    // most kDqDma outstanding means every load of earlier iterations landed
    dma_wait_n<kDqDma>();
    lds_barrier();
  };

  Blk cur = b0, n1 = b1, n2 = b2;
  int bj = 0, last = 0;
  bool last_in_a = true;   // whether the last block's dS went to dsA
  while (cur.id >= 0) {
    Blk n3 = nxt(n2);
    iter(sA, dpA, sB, dpB, dsA, dsB, bj, n1, n3);
    last = bj;
    last_in_a = true;
    bj = bj + 1 == kDqBufs ? 0 : bj + 1;
    cur = n1; n1 = n2; n2 = n3;
    if (cur.id < 0) break;
    n3 = nxt(n2);
    iter(sB, dpB, sA, dpA, dsB, dsA, bj, n1, n3);
    last = bj;
    last_in_a = false;
    bj = bj + 1 == kDqBufs ? 0 : bj + 1;
    cur = n1; n1 = n2; n2 = n3;
  }
  // the dQ product of the last block (one call site: the accumulators must
  // not be merged from two paths, which would copy them right after a product)
  if (b0.id >= 0) {
    bf16x8 dsl[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // select values, not array addresses (which would put both arrays in memory)
        bf16x8 xa = dsA[nt][k], xb = dsB[nt][k];
        asm volatile("" : "+v"(xa), "+v"(xb));
        dsl[nt][k] = last_in_a ? xa : xb;
      }
    dq_prod(last, dsl, [&](auto) {});
  }

  fence_acc(acc);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!qc[nt].valid) continue;
    __bf16* op = (__bf16*)a.out + (int64_t)qc[nt].tok * a.out_st + (int64_t)qc[nt].head * a.out_sh;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[dt][nt][4 * j + r] * a.scale);
        *(bf16x4*)(op + dt * 32 + 8 * j + 4 * h32) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Backward, dQ from the stored dS^T (Phase B).
//
// dQ^T [d x q] = s K^T [d x k] dS^T [k x q] over every key a query sees, with
// both operands read from memory: the K rows and the dS^T the dK/dV pass
// stored (so S and dP are not computed a second time).  A workgroup owns 256
// tokens of one query head, 64 per wave as two 32-column tiles, and walks the
// external key blocks and the own key blocks its tokens can see (32 keys
// each); per block it stages K (32 x 256 B) and dS^T (32 keys x 256 tokens, as
// two 128-token tiles) and each wave runs 16 products.  Two workgroups share a
// CU (72 KiB of LDS each).
//
// dS^T is stored as [query head][32-key block][32-row step][half][key][16
// values], so a block's eight steps of one workgroup are 16 contiguous KiB and
// each dK/dV store instruction writes one contiguous KiB (a half of 32 keys).
// The 32 values of a (step, key) are in the dK/dV pass's register order: value
// p is row 16 (p / 16) + 8 ((p % 8) / 4) + 4 ((p / 8) % 2) + p % 4 of the step,
// and half h holds values 16 h .. 16 h + 15.  The
// dK/dV pass writes an own key block's steps from its 256-key workgroup block
// on to its last visible row; other steps of that block hold no values and
// are read as zero here.
constexpr int kDsStep = 32;                       // query rows per stored dS^T step
// cache-policy operand of a buffer load: non-temporal (each dS^T value is
// read once; streaming it measured 6 % off the Phase-B backward at config 2,
// with the streaming store on the dK/dV side)
constexpr int kCachePolicyNT = 2;
constexpr int kDxBN = 32;
constexpr int kDxTok = 256;
constexpr int kDxTile = kDxBN * kRowB;
constexpr int kDxBufBytes = 3 * kDxTile;          // K tile, then two dS^T tiles
constexpr int kDxBufs = 3;
constexpr int kDxDma = 3 * (kDxBN / 16);          // K staging + dS^T loads per wave per block

__device__ __forceinline__ int ds_col_row(int p) {
  return 16 * (p >> 4) + 8 * ((p & 7) >> 2) + 4 * ((p >> 3) & 1) + (p & 3);
}

// The dQ pass's grid (n_dq workgroups) is followed by the split key blocks'
// partial sums (PartialSums, nbx blocks per array from array y0 on): the two
// read disjoint data, and one launch saves the gap between two.
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_ds_kernel(AttnArgs a, PartialSums ps,
                                                                int n_dq, int ps_nbx, int ps_y0) {
  if ((int)blockIdx.x >= n_dq) {
    const int pb = (int)blockIdx.x - n_dq;
    partial_sums_block(ps, ps_y0 + pb / ps_nbx, pb % ps_nbx, ps_nbx);
    return;
  }
  constexpr int BN = kDxBN;
  __shared__ __attribute__((aligned(16))) char smem[kDxBufs * kDxBufBytes];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int n_tt = (a.rows + kDxTok - 1) / kDxTok;
  int g, item;
  map_block(blockIdx.x, a.hkv, a.group * n_tt, g, item);
  if (g >= a.hkv) return;
  // later token tiles first: under a causal or tree mask they see the most keys
  const int j = item / n_tt, tt = n_tt - 1 - (item - j * n_tt);
  const int head = ld_uniform(a.ri.qhead, g * a.group + j);
  const int t0 = tt * kDxTok;

  KeyWalk<BN> walk;
  walk.n_ext_blocks = (a.n_ext + BN - 1) / BN;
  walk.t0 = t0;
  walk.t1 = min(t0 + kDxTok, a.rows);
  walk.bmax = a.ri.bmax;
  walk.bmin = a.ri.bmin;
  walk.rows = a.rows;
  walk.tiles = a.ext_tiles;
  BlockSrc<BN> src;
  src.init(a, g, walk.n_ext_blocks, wave, lane);

  // dS^T of this head for the tile's 8 steps.  LDS dS^T tile d (0, 1) is [32
  // keys][128 tokens] with 256-byte rows: logical chunk c of row r is values
  // 8 (c % 4) .. of step 4 d + c / 4.  Each lane's chunk and row within a
  // staging pass are fixed, so its offset is fixed; the key block and the
  // pass move the scalar offset.
  const int n_steps = a.ds_rows / kDsStep, nkb = a.ds_keys / 32, s0 = t0 / kDsStep;
  const __bf16* dbase = a.ds_ext + ((int64_t)head * nkb * n_steps + s0) * 32 * kDsStep;
  const __amdgpu_buffer_rsrc_t dres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)dbase, (short)0, (nkb * n_steps - s0) * 32 * kDsStep * 2, 0x00020000);
  uint32_t d_loff;
  {
    const int r = 4 * wave + (lane >> 4);
    const int lc = (lane & 15) ^ (int)swz(r);
    d_loff = (uint32_t)((lc >> 2) * 32 * kDsStep + ((lc & 3) >> 1) * 16 * 32 + r * 16 +
                        8 * (lc & 1)) * 2u;
  }
  // key block b of the walk -> its 32-key block in the dS^T store
  auto ds_block = [&](int b) {
    return src.ext(b) ? b : a.ds_own0 / 32 + (b - walk.n_ext_blocks);
  };
  // Block b's K rows go to LDS buffer `buf` by staging loads; its dS^T goes
  // through registers (plain loads, two blocks ahead in one of two register
  // stages) and is written to the buffer one block later, so the staging
  // path carries only K (mostly L2 hits) and the dS^T stream, the HBM-bound
  // part, has two blocks of time to arrive.
  u32x4 dsr[2][2][BN / 16];   // [register stage][dS^T tile][16-key pass]
  auto stage = [&](int b, int buf, u32x4 (&r)[2][BN / 16]) {
    lds_t* base = sb + buf * kDxBufBytes;
    if (b >= 0) {
      src.dma_k(b, base, wave, lane);
    } else {
      // keep the per-wave load count uniform: K rows past the end
      src.kx.stage<BN>(src.kx.nrows + BN, base, wave);
    }
    // past the last block: offsets past the resource, which read zero (the
    // values are never used; every block issues the same loads)
    const int kbs = b >= 0 ? ds_block(b) : nkb;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < BN / 16; ++i)
        r[d][i] = __builtin_amdgcn_raw_buffer_load_b128(
            dres, (int)d_loff, ((kbs * n_steps + 4 * d) * 32 * kDsStep + 16 * i * 16) * 2,
            kCachePolicyNT);
  };
  auto commit = [&](int buf, const u32x4 (&r)[2][BN / 16]) {
    lds_t* base = sb + buf * kDxBufBytes;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < BN / 16; ++i)
        st16(base + (1 + d) * kDxTile + (16 * i + 4 * wave) * kRowB + 16 * lane, r[d][i]);
  };
  // steps of own block b the dK/dV pass wrote: from its 256-key workgroup
  // block's first row to the last row any of those keys is visible to
  auto own_steps = [&](int b, int& lo, int& hi) {
    const int kb = b - walk.n_ext_blocks;
    const int k0 = (kb * BN) / 256 * 256;
    int m = -1;
    for (int q = k0 / kKeyBlockSummary; q * kKeyBlockSummary < min(k0 + 256, a.rows); ++q)
      m = max(m, ld_uniform(a.ri.bmax, q));
    const int qhi = min(m, a.rows);
    lo = k0 / kDsStep;
    hi = qhi > k0 ? (qhi + kDsStep - 1) / kDsStep : lo;
  };

  FragC f;
  {
    Frag ff;
    frag_init(ff, lane);
    f.init(ff);
  }
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();
  fence_acc(acc);

  // this wave's dS^T tile, its two column tiles in it and their steps
  const int dtile = 1 + (wave >> 1);
  const int ct0 = 2 * (wave & 1);
  const int step0 = s0 + 4 * (wave >> 1) + ct0;
  // cur is the block in buffer `buf`, n1 the next (its dS^T in register
  // stage RS ^ 1), n2 the one after (staged during this block into stage RS)
  int cur = walk.next(0);
  int n1 = cur >= 0 ? walk.next(cur + 1) : -1;
  stage(cur, 0, dsr[0]);
  stage(n1, 1, dsr[1]);
  dma_wait();
  commit(0, dsr[0]);
  __syncthreads();
  int buf = 0;
  auto block = [&](auto rsc) {
    constexpr int RS = decltype(rsc)::value;
    const int n2 = n1 >= 0 ? walk.next(n1 + 1) : -1;
    f.fresh();
    stage(n2, buf == 0 ? 2 : buf - 1, dsr[RS]);
    // column tiles of steps this block holds no values for read as zero
    bool live0 = true, live1 = true;
    if (!src.ext(cur)) {
      int lo, hi;
      own_steps(cur, lo, hi);
      live0 = step0 >= lo && step0 < hi;
      live1 = step0 + 1 >= lo && step0 + 1 < hi;
    }
    const lds_t* kt_s = sb + buf * kDxBufBytes;
    const lds_t* ds_s = kt_s + dtile * kDxTile;
    // per 16-key slice: two dS^T fragments (B, one per column tile) and four
    // K^T fragments (A, one per d tile), fetched one slice ahead
    auto ldb = [&](int ks, int nt) {
      const lds_t* p = ds_s + ks * 16 * kRowB;
      const bf16x8 v = ld_tr(p + f.tr(ct0 + nt, 0), p + f.tr(ct0 + nt, 1));
      return (nt ? live1 : live0) ? v : zero8();
    };
    auto lda = [&](int ks, int dt) {
      const lds_t* p = kt_s + ks * 16 * kRowB;
      return ld_tr(p + f.tr(dt, 0), p + f.tr(dt, 1));
    };
    bf16x8 bf[2][2], af[2][kD / 32];
    bf[0][0] = ldb(0, 0);
    bf[0][1] = ldb(0, 1);
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) af[0][dt] = lda(0, dt);
    static_for<0, BN / 16>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int cs = ks & 1, ns = cs ^ 1;
      if constexpr (ks + 1 < BN / 16) {
        bf[ns][0] = ldb(ks + 1, 0);
        bf[ns][1] = ldb(ks + 1, 1);
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) af[ns][dt] = lda(ks + 1, dt);
      }
      static_for<0, kD / 32>([&](auto dtc) {
        constexpr int dt = decltype(dtc)::value;
        mfma_acc(acc[dt][0], af[cs][dt], bf[cs][0]);
        mfma_acc(acc[dt][1], af[cs][dt], bf[cs][1]);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // the next block's K and dS^T have landed (this block's loads stay in
    // flight): its dS^T goes to its buffer
    dma_wait_n<kDxDma>();
    commit(buf == 2 ? 0 : buf + 1, dsr[RS ^ 1]);
    lds_barrier();
    cur = n1;
    n1 = n2;
    buf = buf == 2 ? 0 : buf + 1;
  };
  while (cur >= 0) {
    block(std::integral_constant<int, 0>());
    if (cur < 0) break;
    block(std::integral_constant<int, 1>());
  }
  dma_wait();

  fence_acc(acc);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int tok = t0 + 128 * (wave >> 1) + 32 * (ct0 + nt) + ds_col_row(col);
    if (tok >= a.rows) continue;
    __bf16* op = (__bf16*)a.out + (int64_t)tok * a.out_st + (int64_t)head * a.out_sh;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[dt][nt][4 * jj + r] * a.scale);
        *(bf16x4*)(op + dt * 32 + 8 * jj + 4 * h32) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Backward, KV-stationary: dK, dV.
//
// A workgroup owns 256 keys of one KV head and walks query steps of 32 tokens
// x one query head over every head of the group.  Each wave owns KT 32-key
// column tiles: four waves of 64 keys (one per SIMD, 512 registers each, every
// Q/dO fragment read from LDS feeding two products), or eight waves of 32 keys
// (two per SIMD, 128 VGPRs and the 128 AGPRs of their dK/dV accumulators).  The query range of a key block is [0, rows) for external
// keys and [k0, max kend) for own keys; it is split into chunks of the
// (query tile, head) index space when the grid needs more workgroups, and each
// chunk writes an fp32 partial that a fixed-order reduce sums.  K fragments
// stay in registers; the workgroup's V rows stay in LDS.
//
// Per step t the work is S = Q K^T, dP = dO V^T (matrix cores), P =
// exp2(S c - LSE log2 e), dS = P (dP - D) (VALU), dV^T += dO^T P and dK^T +=
// Q^T dS (matrix cores).  The steps are software-pipelined so the VALU work
// of one step runs beside the products of another (the four runs of MFMA
// pairs described at `step` below).  dS reads P back from its packed bf16
// form, so one set of S/dP registers serves every step.  Q/dO tiles and the steps' LSE (log2 units) and -D rotate
// through four LDS buffers; step t + 3 is staged during step t, one staging
// load per M1 product pair.
constexpr int kQStep = 32;
static_assert(kQStep == kDsStep, "the dS^T store and the dQ pass share the step");
constexpr int kKeysPerWg = 256;
// 32-key tiles per wave: two (four waves, one per SIMD) when a call has
// external keys, one (eight waves, two per SIMD) otherwise.  Measured on one
// box at config 2: the eight-wave form takes the same time for Phase B's
// dK/dV (0.658-0.664 ms against 0.651-0.660) and 6 % less for Phase C's
// (0.330-0.334 against 0.350-0.355 ms).
constexpr int kDkvKTExt = 2, kDkvKTOwn = 1;
constexpr int kStepTile = kQStep * kRowB;
constexpr int kDkvBufs = 4;
constexpr int kDkvQ = 0;                                  // Q step buffers
constexpr int kDkvO = kDkvBufs * kStepTile;               // dO step buffers
constexpr int kDkvV = 2 * kDkvBufs * kStepTile;           // V rows of the workgroup
constexpr int kDkvL = kDkvV + kKeysPerWg * kRowB;         // per buffer: 64 LSE values (log2)
constexpr int kDkvD = kDkvL + kDkvBufs * 256;             // per buffer: 64 -D values
constexpr int kDkvBytes = kDkvD + kDkvBufs * 256;

// value k of a packed bf16 fragment, as fp32
__device__ __forceinline__ float unpack_bf16(const bf16x8& v, int k) { return (float)v[k]; }

// One workgroup's key block: external (prefix) keys, which every query row
// sees unmasked, or own keys; the two are separate instantiations so the
// external path carries no masking code.
// The dK/dV accumulators stay in AGPRs for any KT: with two waves per SIMD
// (KT = 1) the compiler gives a wave that uses AGPRs 128 of each file, and the
// 32 keys' dK and dV accumulators are exactly 128 registers.
template <int KT>
__device__ __forceinline__ void fence_dkv(f32x16 (&x)[kD / 32][KT], f32x16 (&y)[kD / 32][KT]) {
  if constexpr (KT == 2) {
    fence_acc(x, y);
  } else {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(x[0][0]), "+a"(x[1][0]), "+a"(x[2][0]), "+a"(x[3][0]), "+a"(y[0][0]),
                   "+a"(y[1][0]), "+a"(y[2][0]), "+a"(y[3][0]));
  }
}

template <bool EXT, int KT>
__device__ __forceinline__ void dkv_block(const AttnArgs& a, int g, int kb, int chunk, int nch,
                                          char* smem) {
  constexpr bool ext = EXT;
  constexpr int WAVES = 8 / KT;                   // waves of the workgroup
  constexpr int KPW = 32 * KT;                    // keys per wave
  constexpr int NQL = kQStep / (4 * WAVES);       // Q (and dO) staging loads per wave per step
  constexpr int kDma = 2 * NQL + 2;               // staging loads per wave per step
  constexpr int NE = 16 * KT;                     // P (or dS) values per lane per step
  constexpr int RING = KT == 2 ? 3 : 2;           // fragment ring slots (read RING - 1 pairs ahead)
  static_assert(WAVES * KPW == kKeysPerWg, "a workgroup holds kKeysPerWg keys");
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int k0 = kb * kKeysPerWg;
  const int klim = ext ? a.n_ext : a.rows;
  const int kw0 = k0 + wave * KPW;               // this wave's first key

  // query range (tokens) and the (tile, head) index range of this workgroup
  int qlo, qhi;
  if (ext) {
    qlo = 0;
    qhi = a.rows;
  } else {
    qlo = k0;
    int m = -1;
    for (int b = k0 / kKeyBlockSummary; b * kKeyBlockSummary < min(k0 + kKeysPerWg, a.rows); ++b)
      m = max(m, ld_uniform(a.ri.bmax, b));
    qhi = min(m, a.rows);
  }
  const int qt_lo = qlo / kQStep;
  const int qt_hi = (qhi > qlo) ? (qhi + kQStep - 1) / kQStep : qt_lo;
  const int n_it = (qt_hi - qt_lo) * a.group;
  int it_lo = 0, it_hi = n_it;
  if (nch > 1) {
    const int per = (n_it + nch - 1) / nch;
    it_lo = min(n_it, chunk * per);
    it_hi = min(n_it, it_lo + per);
  }

  // V rows of the workgroup into LDS; K fragments (B operand of Q K^T) of the
  // wave's two 32-key tiles into registers; visibility bounds of the keys.
  // Keys past the end get zero K/V; their (discarded) gradients are the only
  // values they influence, so they need no mask.
  bf16x8 kf[KT][kD / 16];
  int kend_k[KT];
  bool kvalid[KT];
  int krow[KT];       // row of the lane's key in k/v (and gK/gV for external keys)
  int wave_kend_min = 0x7fffffff;
  // external keys as row ranges of a larger tensor (tile table), or not
  const int2* tiles = ext ? a.ext_tiles : nullptr;
  {
    const __bf16* kbase = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vbase = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    {
      const uint32_t st_b = 2u * (uint32_t)vst;
      const uint32_t loff = dma_lane_off(wave, lane, st_b);
      if (tiles) {
        // passes of 4 WAVES rows, each inside one 32-key tile and read from its rows
        const __bf16* vg = vbase + (int64_t)g * vsh;
        constexpr int VRS = 4 * WAVES;
#pragma unroll
        for (int i = 0; i < kKeysPerWg / VRS; ++i) {
          const int vr = k0 + VRS * i;
          int first = 0, valid = 0;
          if (vr < klim) {
            first = ld_uniform((const int32_t*)tiles, 2 * (vr >> 5)) + (vr & 31);
            valid = ld_uniform((const int32_t*)tiles, 2 * (vr >> 5) + 1) - (vr & 31);
          }
          lds_dma16(row_rsrc(vg + (int64_t)first * vst, valid, st_b),
                    sb + kDkvV + (VRS * i + 4 * wave) * kRowB, loff, 0u);
        }
      } else {
        dma_rows<kKeysPerWg, WAVES>(
            row_rsrc(vbase + (int64_t)k0 * vst + (int64_t)g * vsh, klim - k0, st_b), loff, st_b,
            sb + kDkvV, wave);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int kk = kw0 + kt * 32 + col;
      kvalid[kt] = kk < klim;
      krow[kt] = kk;
      if (tiles && kvalid[kt]) {
        const int vt = (kw0 + kt * 32) >> 5;
        krow[kt] = ld_uniform((const int32_t*)tiles, 2 * vt) + col;
        kvalid[kt] = col < ld_uniform((const int32_t*)tiles, 2 * vt + 1);
      }
      const __bf16* kp = kbase + (int64_t)(kvalid[kt] ? krow[kt] : 0) * kst + (int64_t)g * ksh + 8 * h32;
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) kf[kt][ds] = load8(kp + ds * 16);
      kend_k[kt] = (!ext && kvalid[kt]) ? a.ri.kend[kk] : (ext ? 0x7fffffff : -1);
      if (kvalid[kt]) wave_kend_min = min(wave_kend_min, kend_k[kt]);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds)
        if (!kvalid[kt]) kf[kt][ds] = zero8();
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    wave_kend_min = min(wave_kend_min, __shfl_xor(wave_kend_min, off));
  const int wave_khi = min(kw0 + KPW, klim) - 1;   // last valid key of the wave

  FragC f;
  {
    Frag ff;
    frag_init(ff, lane);
    f.init(ff);
  }
  // this wave's V fragments: rows 64 wave + l % 32 (+ 32 per tile); the base
  // is a multiple of 256 bytes, so the XOR form applies to it as well
  uint32_t vrow0 = kDkvV + wave * KPW * kRowB + f.row8_0;

  // staging sources: Q and dO rows of every query head (a step selects one
  // head and 32 tokens by the scalar offset; rows past the end read zero),
  // and the steps' LSE (log2) and -D values, 64 per step (the 32 of the step
  // and 32 that are not used), every wave loading the same values
  const uint32_t q_st_b = 2u * (uint32_t)a.q_st, do_st_b = 2u * (uint32_t)a.do_st;
  const uint32_t q_bytes = (uint32_t)(((int64_t)(a.rows - 1) * a.q_st + (int64_t)(a.hq - 1) * a.q_sh) * 2 + kRowB);
  const uint32_t do_bytes = (uint32_t)(((int64_t)(a.rows - 1) * a.do_st + (int64_t)(a.hq - 1) * a.do_sh) * 2 + kRowB);
  const uint32_t l_bytes = (uint32_t)a.hq * (uint32_t)a.rows * 4u;
  const Rsrc q_res = make_rsrc(a.q, q_bytes);
  const Rsrc do_res = make_rsrc(a.dout, do_bytes);
  const Rsrc l_res = make_rsrc(a.lse2, l_bytes);
  const Rsrc d_res = make_rsrc(a.neg_dsum, l_bytes);
  const uint32_t q_loff = dma_lane_off(wave, lane, q_st_b);
  const uint32_t do_loff = dma_lane_off(wave, lane, do_st_b);

  // the step the next staging call loads (steps past it_hi read zeros)
  int iss_it = it_lo, iss_qt = qt_lo + it_lo / a.group, iss_j = it_lo % a.group;
  uint32_t st_q = 0, st_do = 0, st_l = 0;   // scalar offsets of the step being staged
  auto stage_begin = [&]() {
    if (iss_it < it_hi) {
      const int head = ld_uniform(a.ri.qhead, g * a.group + iss_j);
      const int tbase = iss_qt * kQStep;
      st_q = (uint32_t)(((int64_t)tbase * a.q_st + (int64_t)head * a.q_sh) * 2);
      st_do = (uint32_t)(((int64_t)tbase * a.do_st + (int64_t)head * a.do_sh) * 2);
      st_l = ((uint32_t)head * (uint32_t)a.rows + (uint32_t)tbase) * 4u;
    } else {
      st_q = q_bytes;
      st_do = do_bytes;
      st_l = l_bytes;
    }
    ++iss_it;
    if (++iss_j == a.group) {
      iss_j = 0;
      ++iss_qt;
    }
  };
  // staging load k (0..kDma-1) of the current step into buffer B: NQL loads
  // of Q rows, NQL of dO rows (each wave moves 4 rows per load), then LSE, -D
  auto stage_load = [&](auto bc, int k) {
    constexpr int B = decltype(bc)::value;
    constexpr int RS = 4 * WAVES;                 // rows one load moves over the group
    if (k < NQL) {
      lds_dma16(q_res, sb + kDkvQ + B * kStepTile + (RS * k + 4 * wave) * kRowB, q_loff,
                st_q + (uint32_t)(RS * k) * q_st_b);
    } else if (k < 2 * NQL) {
      lds_dma16(do_res, sb + kDkvO + B * kStepTile + (RS * (k - NQL) + 4 * wave) * kRowB,
                do_loff, st_do + (uint32_t)(RS * (k - NQL)) * do_st_b);
    } else if (k == 2 * NQL) {
      lds_dma4(l_res, sb + kDkvL + B * 256, 4u * lane, st_l);
    } else {
      lds_dma4(d_res, sb + kDkvD + B * 256, 4u * lane, st_l);
    }
  };
  auto stage_all = [&](auto bc) {
    stage_begin();
#pragma unroll
    for (int k = 0; k < kDma; ++k) stage_load(bc, k);
  };

  const float c = a.scale_log2;
  f32x16 dk[kD / 32][KT], dv[kD / 32][KT];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      dk[dt][kt] = zero16();
      dv[dt][kt] = zero16();
    }
  fence_dkv<KT>(dk, dv);

  // Per-lane elements of a step's 32 x 32 tiles (C layout): element (kt, i)
  // is query row 8 (i / 4) + 4 h32 + i % 4 of the step, key kw0 + 32 kt + col.
  f32x16 s[KT], dp[KT];        // S then P (fp32) / dP then dS of a step
  bf16x8 pb[KT][2], db[KT][2]; // packed P and dS: [key tile][query half]

  // LSE (log2) of one 4-row group of a step (rows 8 (k & 3) + 4 h32 + r of
  // group k = 0..7, the same rows for both key tiles), double-buffered: each
  // group's values are read from LDS while the group before it is in use
  f32x4 lg[2];
  auto ld_l = [&](auto blc, auto kc) {
    constexpr int BL = decltype(blc)::value, k = decltype(kc)::value;
    lg[k & 1] = *(const lds_f32x4*)(sb + kDkvL + BL * 256 + 4 * (8 * (k & 3) + 4 * h32));
  };
  // -D of a step's rows in C layout (element i: row 8 (i / 4) + 4 h32 + i % 4),
  // the starting value of both key tiles' dP sums, which so end as dP - D;
  // quarter q is elements 4q .. 4q + 3
  f32x16 nd;
  auto ld_nd = [&](auto bdc, auto qc) {
    constexpr int BD = decltype(bdc)::value, q = decltype(qc)::value;
    const f32x4 v = *(const lds_f32x4*)(sb + kDkvD + BD * 256 + 4 * (8 * q + 4 * h32));
#pragma unroll
    for (int r = 0; r < 4; ++r) nd[4 * q + r] = v[r];
  };

  // P element e of the step whose LSE is in buffer BL (in place in s); group
  // 0's LSE must have been read (ld_l) beforehand
  auto p_elem = [&](auto blc, auto ec) {
    constexpr int e = decltype(ec)::value;
    constexpr int kt = e >> 4, i = e & 15, k = e >> 2, r = i & 3;
    if constexpr (r == 0 && k + 1 < 4 * KT) ld_l(blc, std::integral_constant<int, k + 1>());
    s[kt][i] = fast_exp2(fmaf(s[kt][i], c, -lg[k & 1][r]));
    // formed here, beside this step's products (not moved to its first use)
    asm volatile("" : "+v"(s[kt][i]));
    if constexpr ((i & 7) == 7) {
      pb[kt][i >> 3] = pack_half(s[kt], i >> 3);
      asm volatile("" : "+v"(pb[kt][i >> 3]));
    }
  };
  // dS element e of a step (in place in dp, which holds dP - D)
  auto ds_elem = [&](auto ec) {
    constexpr int e = decltype(ec)::value;
    constexpr int kt = e >> 4, i = e & 15;
    dp[kt][i] = unpack_bf16(pb[kt][i >> 3], i & 7) * dp[kt][i];
    asm volatile("" : "+v"(dp[kt][i]));
    if constexpr ((i & 7) == 7) {
      db[kt][i >> 3] = pack_half(dp[kt], i >> 3);
      asm volatile("" : "+v"(db[kt][i >> 3]));
    }
  };
  // invisible entries of a step's S (own keys) become -inf
  auto mask_s = [&](int t0) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int kk = kw0 + kt * 32 + col;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tq = t0 + 8 * (i >> 2) + 4 * h32 + (i & 3);
        const int vis = (kk <= tq ? 1 : 0) & (tq < kend_k[kt] ? 1 : 0);
        s[kt][i] = vis ? s[kt][i] : -INFINITY;
      }
    }
  };
  auto step_needs_mask = [&](int t0) {
    return !ext && !(t0 >= wave_khi && t0 + kQStep - 1 < wave_kend_min);
  };

  // One step t (buffer B; step t + 1 in B + 1) is 32 MFMA pairs in four runs
  // of 8, each run paired with VALU work of another step:
  //   pairs  0-7   S of step t + 1        with  dS of step t (first half)
  //   pairs  8-15  dV^T += dO^T P, step t  with  dS of step t (second half)
  //   pairs 16-23  dK^T += Q^T dS, step t  with  P of step t + 1 (first half)
  //   pairs 24-31  dP of step t + 1        with  P of step t + 1 (second half)
  // Every pair's A fragment (and the two V fragments of a dP pair) is read
  // from LDS two pairs ahead through a three-slot ring, across the runs.
  bf16x8 fr[RING], vr[RING][KT];
  auto frag = [&](auto bc, auto pc) {
    constexpr int B = decltype(bc)::value, B1 = (B + 1) % kDkvBufs;
    constexpr int p = decltype(pc)::value, run = p >> 3, idx = p & 7, sl = p % RING;
    if constexpr (run == 0) {
      fr[sl] = ld_row8(sb + kDkvQ + B1 * kStepTile + f.row8(idx));
    } else if constexpr (run == 1 || run == 2) {
      const lds_t* t = sb + (run == 1 ? kDkvO : kDkvQ) + B * kStepTile + (idx >> 2) * 16 * kRowB;
      fr[sl] = ld_tr(t + f.tr(idx & 3, 0), t + f.tr(idx & 3, 1));
    } else {
      fr[sl] = ld_row8(sb + kDkvO + B1 * kStepTile + f.row8(idx));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        vr[sl][kt] = ld_row8(sb + kt * 32 * kRowB + (vrow0 ^ (uint32_t)(idx << 5)));
    }
  };
  auto step = [&](auto bc, __bf16* ds_dst, int t0n) {
    constexpr int B = decltype(bc)::value;
    constexpr int B1 = (B + 1) % kDkvBufs, B3 = (B + 3) % kDkvBufs;
    static_for<0, RING - 1>([&](auto pc) { frag(bc, pc); });
    static_for<0, 32>([&](auto pc) {
      constexpr int p = decltype(pc)::value, run = p >> 3, idx = p & 7, sl = p % RING;
      constexpr int hf = idx >> 2, dt = idx & 3;
      if constexpr (p + RING - 1 < 32) frag(bc, std::integral_constant<int, p + RING - 1>());
      // this pair's share of the step's NE P or dS values: KT of them, from `base`
      auto elems = [&](auto&& fn, auto base) {
        static_for<0, KT>([&](auto jc) {
          fn(std::integral_constant<int, decltype(base)::value + KT * idx + decltype(jc)::value>());
        });
      };
      if constexpr (run == 0) {
        if constexpr (idx == 0) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) s[kt] = zero16();
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) s[kt] = mfma(fr[sl], kf[kt][idx], s[kt]);
        elems([&](auto ec) { ds_elem(ec); }, std::integral_constant<int, 0>());
        if constexpr (idx < kDma) stage_load(Buf<B3>(), idx);
      } else if constexpr (run == 1) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) mfma_acc(dv[dt][kt], fr[sl], pb[kt][hf]);
        elems([&](auto ec) { ds_elem(ec); }, std::integral_constant<int, NE / 2>());
        // group 0 of the LSE of step t + 1 (lg[0] is free from here)
        if constexpr (idx == 4) ld_l(Buf<B1>(), std::integral_constant<int, 0>());
      } else if constexpr (run == 2) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) mfma_acc(dk[dt][kt], fr[sl], db[kt][hf]);
        if constexpr (idx == 0) {
          if (step_needs_mask(t0n)) mask_s(t0n);
        }
        elems([&](auto ec) { p_elem(Buf<B1>(), ec); }, std::integral_constant<int, 0>());
        if constexpr (idx < 2 * KT) {
          // dS^T of this step for the dQ pass: key tile idx / 2, query half idx
          // % 2; a streaming store (read once, by the dQ pass, long after)
          if (ds_dst)
            __builtin_nontemporal_store(
                db[idx >> 1][idx & 1],
                (bf16x8*)(ds_dst + (int64_t)(idx >> 1) * (a.ds_rows / kQStep) * 32 * kQStep +
                          16 * 32 * (idx & 1)));
        }
        // -D of step t + 1, a quarter per pair, for its dP sums (this step's
        // dS, formed in runs 0-1, no longer needs dp)
        if constexpr (idx >= 4) ld_nd(Buf<B1>(), std::integral_constant<int, idx - 4>());
      } else {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          dp[kt] = mfma(fr[sl], vr[sl][kt], idx == 0 ? nd : dp[kt]);
        elems([&](auto ec) { p_elem(Buf<B1>(), ec); }, std::integral_constant<int, NE / 2>());
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // S, P and dP - D of the step in buffer BQ without overlap (pipeline fill)
  auto fill = [&](auto bqc, int t0) {
    constexpr int BQ = decltype(bqc)::value;
    const lds_t* q_s = sb + kDkvQ + BQ * kStepTile;
    const lds_t* d_s = sb + kDkvO + BQ * kStepTile;
    ld_l(bqc, std::integral_constant<int, 0>());
    static_for<0, 4>([&](auto qc) { ld_nd(bqc, qc); });
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = zero16();
      dp[kt] = nd;
    }
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 qa = ld_row8(q_s + f.row8(ds));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] = mfma(qa, kf[kt][ds], s[kt]);
      const bf16x8 da = ld_row8(d_s + f.row8(ds));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        dp[kt] = mfma(da, ld_row8(sb + kt * 32 * kRowB + (vrow0 ^ (uint32_t)(ds << 5))), dp[kt]);
    }
    if (step_needs_mask(t0)) mask_s(t0);
    static_for<0, NE>([&](auto ec) { p_elem(bqc, ec); });
  };

  if (it_lo < it_hi) {
    stage_all(Buf<0>());
    stage_all(Buf<1>());
    stage_all(Buf<2>());
  }
  dma_wait();
  __syncthreads();
  if (it_lo < it_hi) {
    // query tile of step t + 1, advanced per step
    int nqt = qt_lo + it_lo / a.group, nj = it_lo % a.group;
    int cqt = nqt, cj = nj;   // step t
    fill(Buf<0>(), nqt * kQStep);
    auto advance = [&]() {
      if (++nj == a.group) {
        nj = 0;
        ++nqt;
      }
    };
    advance();
    // step t in buffer B: step t + 1 in B + 1, staging of step t + 3 into B + 3
    auto iter = [&](auto bc) {
      f.fresh();
      asm volatile("" : "+v"(vrow0));
      stage_begin();
      // this lane's dS^T destination for step t: key kw0 + col (the next key
      // tile is the next 32-key block), positions 8 h32 .. 8 h32 + 7 of each
      // 16-position half of the step's 32 values
      __bf16* ds_dst = nullptr;
      if (a.ds_ext) {
        const int head = ld_uniform(a.ri.qhead, g * a.group + cj);
        const int64_t n_steps = a.ds_rows / kQStep, nkb = a.ds_keys / 32;
        const int kbs = ((EXT ? 0 : a.ds_own0) + kw0) / 32;
        ds_dst = a.ds_ext + (((int64_t)head * nkb + kbs) * n_steps + cqt) * 32 * kQStep + 16 * col +
                 8 * h32;
      }
      step(bc, ds_dst, nqt * kQStep);
      cqt = nqt;
      cj = nj;
      advance();
      // the vector memory counter also counts the dS^T stores issued after
      // this iteration's staging loads: leave both in flight
      if (ds_dst)
        dma_wait_n<kDma + 2 * KT>();
      else
        dma_wait_n<kDma>();
      lds_barrier();
    };
    for (int it = it_lo; it < it_hi; it += kDkvBufs) {
      iter(Buf<0>());
      if (it + 1 >= it_hi) break;
      iter(Buf<1>());
      if (it + 2 >= it_hi) break;
      iter(Buf<2>());
      if (it + 3 >= it_hi) break;
      iter(Buf<3>());
    }
  }
  dma_wait();

  // lane holds key kw0 + 32 kt + col, d = 32 dt + 8 j + 4 h32 + r.  One
  // (key tile, d tile) at a time, so the epilogue reads 32 accumulators at once.
  fence_dkv<KT>(dk, dv);
  // destination: 0 add into gK/gV, 1 external partial, 2 own partial, 3 own output.
  // The first query chunk of a split external block adds into gK/gV itself
  // (no other workgroup touches those elements during the launch); chunks
  // 1.. write partial planes 0.. that the finishing pass adds afterwards, so
  // every element is acc + c0 + (c1 + c2 + ...), a fixed order.
  const int mode = ext ? ((nch == 1 || chunk == 0) ? 0 : 1) : (nch > 1 ? 2 : 3);
  static_for<0, KT>([&](auto ktc) {
    constexpr int kt = decltype(ktc)::value;
    const int kk = kw0 + kt * 32 + col;
    const int64_t base = ((int64_t)kk * a.hkv + g) * kD;         // partial planes: virtual keys
    const int64_t abase = ((int64_t)krow[kt] * a.hkv + g) * kD;  // gK/gV: accumulator rows
    static_for<0, kD / 32>([&](auto dtc) {
      constexpr int dt = decltype(dtc)::value;
      if (kvalid[kt]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = dt * 32 + 8 * j + 4 * h32;
          f32x4 vk, vv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            vk[r] = dk[dt][kt][4 * j + r] * a.scale;
            vv[r] = dv[dt][kt][4 * j + r];
          }
          if (mode == 0) {
            *(f32x4*)(a.gk_acc + abase + d) += vk;
            *(f32x4*)(a.gv_acc + abase + d) += vv;
          } else if (mode == 1) {
            const int64_t pb = (int64_t)(chunk - 1) * a.n_ext * a.hkv * kD + base;
            *(f32x4*)(a.gk_part + pb + d) = vk;
            *(f32x4*)(a.gv_part + pb + d) = vv;
          } else if (mode == 2) {
            // own keys split over query chunks: fp32 partials, finished by a reduce
            const int64_t pb = (int64_t)chunk * a.rows * a.hkv * kD + base;
            *(f32x4*)(a.dk_part + pb + d) = vk;
            *(f32x4*)(a.dv_part + pb + d) = vv;
          } else {
            if (a.gk_init) {
              vk += *(const f32x4*)(a.gk_init + base + d);
              vv += *(const f32x4*)(a.gv_init + base + d);
            }
            const int64_t ko = (int64_t)kk * a.dko_st + (int64_t)g * a.dko_sh + d;
            const int64_t vo = (int64_t)kk * a.dvo_st + (int64_t)g * a.dvo_sh + d;
            if (a.dkv_f32) {
              *(f32x4*)((float*)a.dk_own + ko) = vk;
              *(f32x4*)((float*)a.dv_own + vo) = vv;
            } else {
              bf16x4 wk, wv;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                wk[r] = (__bf16)vk[r];
                wv[r] = (__bf16)vv[r];
              }
              *(bf16x4*)((__bf16*)a.dk_own + ko) = wk;
              *(bf16x4*)((__bf16*)a.dv_own + vo) = wv;
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

template <int KT>
__global__ __launch_bounds__(64 * 8 / KT, 1) void bwd_dkv_kernel(AttnArgs a, ItemOrder ord) {
  __shared__ __attribute__((aligned(16))) char smem[kDkvBytes];
  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb * a.n_chunks_own;   // per KV head
  int g, item;
  map_block(blockIdx.x, a.hkv, items, g, item);
  if (g >= a.hkv) return;
  if (ord.n == items) item = ord.item[item];
  if (item < n_ext_kb * a.n_chunks) {
    const int kb = item / a.n_chunks;
    dkv_block<true, KT>(a, g, kb, item - kb * a.n_chunks, a.n_chunks, smem);
  } else {
    const int oi = item - n_ext_kb * a.n_chunks;
    const int kb = oi / a.n_chunks_own;
    dkv_block<false, KT>(a, g, kb, oi - kb * a.n_chunks_own, a.n_chunks_own, smem);
  }
}

// grid size: per-KV-head items, padded so the XCD mapping covers every item
int grid_for(int hkv, int items) {
  if ((hkv & 7) == 0) return 8 * ((hkv / 8) * items);
  if ((8 % hkv) == 0) {
    const int xpg = 8 / hkv;
    return 8 * ((items + xpg - 1) / xpg);
  }
  return hkv * items;
}

}  // namespace

hipError_t launch_fwd_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  if (a.rows <= 0) return hipSuccess;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;
  PF_LAUNCH("pf_fwd_bf16", fwd_kernel<kFwdNT>, dim3(grid_for(a.hkv, n_qt)),
            dim3(64 * 8 / kFwdNT), stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  if (a.rows <= 0) return hipSuccess;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;
  PF_LAUNCH("pf_bwd_dq_bf16", bwd_dq_kernel, dim3(grid_for(a.hkv, n_qt)), dim3(kThreads),
            stream, a);
  return hipGetLastError();
}

// Query steps of item (key block kb, chunk c of nch) as dkv_block counts them,
// with the own keys' visibility ends taken from the segment table.
static int dkv_item_steps(const AttnArgs& a, const SegTable& seg, bool ext, int kb, int c, int nch) {
  int n_it;
  if (ext) {
    n_it = (a.rows + kQStep - 1) / kQStep * a.group;
  } else {
    const int k0 = kb * kKeysPerWg, k1 = std::min(k0 + kKeysPerWg, a.rows);
    int m = -1;
    for (int i = 0; i < seg.n; ++i)
      if (seg.start[i] < k1 && seg.start[i + 1] > k0) m = std::max(m, seg.vis_end[i]);
    const int qhi = std::min(m, a.rows);
    const int qt_lo = k0 / kQStep;
    const int qt_hi = (qhi > k0) ? (qhi + kQStep - 1) / kQStep : qt_lo;
    n_it = (qt_hi - qt_lo) * a.group;
  }
  if (nch <= 1) return n_it;
  const int per = (n_it + nch - 1) / nch;
  const int lo = std::min(n_it, c * per);
  return std::min(n_it, lo + per) - lo;
}

void dkv_item_order(const AttnArgs& a, const SegTable& seg, ItemOrder& ord) {
  ord.n = 0;
  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int n_ext_items = n_ext_kb * a.n_chunks;
  const int items = n_ext_items + n_own_kb * a.n_chunks_own;
  if (items <= 0 || items > kMaxOrderedItems) return;
  // cost = query steps plus a fixed start-up (K/V loads, pipeline fill and
  // drain, the result write) of about four steps
  int cost[kMaxOrderedItems];
  for (int i = 0; i < items; ++i) {
    const bool ext = i < n_ext_items;
    const int j = ext ? i : i - n_ext_items;
    const int nch = ext ? a.n_chunks : a.n_chunks_own;
    cost[i] = 4 + dkv_item_steps(a, seg, ext, j / nch, j % nch, nch);
  }
  for (int i = 0; i < items; ++i) ord.item[i] = (uint16_t)i;
  std::stable_sort(ord.item, ord.item + items,
                   [&](uint16_t x, uint16_t y) { return cost[x] > cost[y]; });
  ord.n = items;
}

hipError_t launch_bwd_dkv_bf16(const AttnArgs& a, const ItemOrder& ord, int32_t head_dim,
                               hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb * a.n_chunks_own;
  if (items <= 0) return hipSuccess;
  if (ord.n != 0 && ord.n != items) return hipErrorInvalidValue;
  if (a.n_ext > 0)
    PF_LAUNCH("pf_bwd_dkv_bf16", bwd_dkv_kernel<kDkvKTExt>, dim3(grid_for(a.hkv, items)),
              dim3(64 * 8 / kDkvKTExt), stream, a, ord);
  else
    PF_LAUNCH("pf_bwd_dkv_bf16", bwd_dkv_kernel<kDkvKTOwn>, dim3(grid_for(a.hkv, items)),
              dim3(64 * 8 / kDkvKTOwn), stream, a, ord);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds_bf16(const AttnArgs& a, const PartialSums& ps, int32_t head_dim,
                                 hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  if (a.rows <= 0) return launch_partial_sums(ps, stream);
  const int n_tt = (a.rows + kDxTok - 1) / kDxTok;
  const int n_dq = grid_for(a.hkv, a.group * n_tt);
  int nbx, ny, y0;
  partial_sums_grid(ps, nbx, ny, y0);
  PF_LAUNCH("pf_bwd_dq_ds_bf16", bwd_dq_ds_kernel, dim3(n_dq + nbx * ny), dim3(kThreads), stream,
            a, ps, n_dq, nbx > 0 ? nbx : 1, y0);
  return hipGetLastError();
}

int32_t dkv_keys_per_workgroup_bf16() { return kKeysPerWg; }

}  // namespace pf
