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

#include <type_traits>

#include "pf_internal.h"

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
// this form so the two files together hold a wave's working set.  Back-to-back
// accumulation into the same registers needs no wait states; VALU reads of an
// accumulator after its last product are separated by acc_fence().
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// wait states between the last accumulating product and VALU reads of it
__device__ __forceinline__ void acc_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

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

__device__ __forceinline__ bf16x8 ld_row8(const lds_t* p) { return *(const lds_bf16x8*)p; }

__device__ __forceinline__ bf16x8 ld_tr(const lds_t* lo, const lds_t* hi) {
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lo);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void st16(lds_t* p, u32x4 v) { *(lds_u32x4*)p = v; }

__device__ __forceinline__ u32x4 load16(const __bf16* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

// Staging offset of thread t: chunk (t & 15) of row t / 16 (+ 16 rows =
// + 4096 B per further pass of 256 threads).
__device__ __forceinline__ uint32_t stage_off(int t) { return toff(t >> 4, (t & 15) * 8); }

template <int B> using Buf = std::integral_constant<int, B>;

// Workgroup -> (KV head, item) with XCD awareness: workgroups are dispatched
// round-robin over the 8 XCDs, so when Hkv is a multiple of 8 every XCD gets
// the items of its own KV heads (their K/V or Q/dO stay in that XCD's L2).
__device__ __forceinline__ void map_block(int bid, int hkv, int items, int& g, int& item) {
  if ((hkv & 7) == 0) {
    const int xcd = bid & 7, pos = bid >> 3;
    const int hh = pos / items;
    item = pos - hh * items;
    g = xcd + 8 * hh;
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

  __device__ int own_block_max(int kb) const {
    int m = -1;
#pragma unroll
    for (int s = 0; s < BN / kKeyBlockSummary; ++s) {
      const int b = kb * (BN / kKeyBlockSummary) + s;
      if (b * kKeyBlockSummary < rows) m = max(m, bmax[b]);
    }
    return m;
  }
  __device__ int own_block_min(int kb) const {
    int m = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < BN / kKeyBlockSummary; ++s) {
      const int b = kb * (BN / kKeyBlockSummary) + s;
      if (b * kKeyBlockSummary < rows) m = min(m, bmin[b]);
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
    if (i < n_ext_blocks) return (i + 1) * BN > n_ext;
    const int kb = i - n_ext_blocks;
    const int k0 = kb * BN;
    if (k0 + BN > rows) return true;
    if (k0 + BN - 1 > t0) return true;
    return own_block_min(kb) < t1;
  }
};

// Key/value block staging for the Q-stationary kernels: BN rows of K and V
// (128 bf16 each) from global memory through registers into swizzled LDS.
template <int BN>
struct KvStage {
  static constexpr int kPer = BN * 16 / kThreads;   // 16-byte chunks per thread per tensor
  u32x4 kreg[kPer], vreg[kPer];
  int kendreg;

  __device__ void issue(const AttnArgs& a, int g, bool ext, int k0, int tid) {
    const int klim = ext ? a.n_ext : a.rows;
    const __bf16* kb = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vb = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + kThreads * i;
      const int kk = k0 + (c >> 4), ch = c & 15;
      const bool ok = kk < klim;
      kreg[i] = ok ? load16(kb + (int64_t)kk * kst + (int64_t)g * ksh + ch * 8) : zero_u4();
      vreg[i] = ok ? load16(vb + (int64_t)kk * vst + (int64_t)g * vsh + ch * 8) : zero_u4();
    }
    if (!ext && tid < BN) {
      const int kk = k0 + tid;
      kendreg = (kk < a.rows) ? a.ri.kend[kk] : -1;
    }
  }
  __device__ void stash(lds_t* kt, lds_t* vt, int32_t* kend, bool ext, int tid, uint32_t so) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      st16(kt + so + i * 16 * kRowB, kreg[i]);
      st16(vt + so + i * 16 * kRowB, vreg[i]);
    }
    if (!ext && tid < BN) kend[tid] = kendreg;
  }
};

// ---------------------------------------------------------------------------
// Forward.
constexpr int kFwdBN = 64;
constexpr int kFwdTile = kFwdBN * kRowB;            // one K or V block
constexpr int kFwdK = 0, kFwdV = 2 * kFwdTile;      // two K buffers, then two V buffers

__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(AttnArgs a) {
  constexpr int BN = kFwdBN;
  __shared__ __attribute__((aligned(16))) char smem[4 * kFwdTile];
  __shared__ int32_t kend_s[2][BN];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;

  int g, item;
  map_block(blockIdx.x, a.hkv, n_qt, g, item);
  if (g >= a.hkv) return;
  const int qt = n_qt - 1 - item;            // later tiles (more own keys) first
  const int t0 = qt * tq;
  const int t1 = min(t0 + tq, a.rows);

  // this lane's two query columns and their Q fragments (B operand of K Q^T)
  QCol qc[2];
  bf16x8 qf[2][kD / 16];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    qc[nt] = qcol(a, g, t0, tq, wave * 64 + nt * 32 + col);
    const __bf16* qp = (const __bf16*)a.q + (int64_t)qc[nt].tok * a.q_st +
                       (int64_t)qc[nt].head * a.q_sh + 8 * h32;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) qf[nt][ds] = qc[nt].valid ? load8(qp + ds * 16) : zero8();
  }

  KeyWalk<BN> walk;
  walk.n_ext_blocks = (a.n_ext + BN - 1) / BN;
  walk.t0 = t0;
  walk.t1 = t1;
  walk.bmax = a.ri.bmax;
  walk.bmin = a.ri.bmin;
  walk.rows = a.rows;

  Frag f;
  frag_init(f, lane);
  const uint32_t so = stage_off(tid);
  KvStage<BN> st;
  const float c = a.scale_log2;
  float mrow[2] = {-INFINITY, -INFINITY};   // running max (log2 units) in use
  float lrow[2] = {0.f, 0.f};
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();

  auto blk_k0 = [&](int b) { return (b < walk.n_ext_blocks ? b : b - walk.n_ext_blocks) * BN; };

  // one key block held in buffer B; stages block nxt into the other buffer
  auto block = [&](auto bc, int blk, int nxt) {
    constexpr int B = decltype(bc)::value;
    const lds_t* kt_s = sb + kFwdK + B * kFwdTile;
    const lds_t* vt_s = sb + kFwdV + B * kFwdTile;
    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = blk_k0(blk);
    const bool msk = walk.masked(blk, a.n_ext);

    // S^T = K Q^T for BN keys x 64 queries
    f32x16 s[BN / 32][2];
#pragma unroll
    for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) s[kt][nt] = zero16();
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
        const bf16x8 af = ld_row8(kt_s + kt * 32 * kRowB + f.row8[ds]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s[kt][nt] = mfma(af, qf[nt][ds], s[kt][nt]);
      }
    }
    if (msk) {
      const int klim = ext ? a.n_ext : a.rows;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kt * 32 + 8 * (i >> 2) + 4 * h32 + (i & 3);
          const int kk = k0 + kl;
          bool vis0 = kk < klim, vis1 = kk < klim;
          if (!ext) {
            const int ke = kend_s[B][kl];
            vis0 = vis0 && kk <= qc[0].tok && qc[0].tok < ke;
            vis1 = vis1 && kk <= qc[1].tok && qc[1].tok < ke;
          }
          if (!vis0) s[kt][0][i] = -INFINITY;
          if (!vis1) s[kt][1][i] = -INFINITY;
        }
    }
    // online softmax (log2 domain), per query column, with lazy rescaling:
    // the running maximum in use only moves when a block exceeds it by more
    // than kRescale, so probabilities stay below 2^kRescale
    float mx[2];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, s[kt][nt][i]);
      m = fmaxf(m, __shfl_xor(m, 32)) * c;
      mx[nt] = m;
      grow = grow || (m > mrow[nt] + kRescale);
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      acc_fence();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mnew = fmaxf(mrow[nt], mx[nt]);
        const float alpha = (mnew > mrow[nt]) ? fast_exp2(mrow[nt] - mnew) : 1.f;
        lrow[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) acc[dt][nt] *= alpha;
        mrow[nt] = mnew;
      }
      acc_fence();
    }
    bf16x8 pb[2][BN / 16];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float muse = (mrow[nt] == -INFINITY) ? 0.f : mrow[nt];
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[kt][nt][i], c, -muse));
          s[kt][nt][i] = p;
          lsum += p;
        }
        pb[nt][2 * kt] = pack_half(s[kt][nt], 0);
        pb[nt][2 * kt + 1] = pack_half(s[kt][nt], 1);
      }
      lrow[nt] += lsum;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const lds_t* vb = vt_s + ks * 16 * kRowB;
        const bf16x8 af = ld_tr(vb + f.tr[dt][0], vb + f.tr[dt][1]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) mfma_acc(acc[dt][nt], af, pb[nt][ks]);
      }
    }
    if (nxt >= 0)
      st.stash(sb + kFwdK + (1 - B) * kFwdTile, sb + kFwdV + (1 - B) * kFwdTile, kend_s[1 - B],
               nxt < walk.n_ext_blocks, tid, so);
    __syncthreads();
  };

  int blk = walk.next(0);
  if (blk >= 0) {
    const bool ext = blk < walk.n_ext_blocks;
    st.issue(a, g, ext, blk_k0(blk), tid);
    st.stash(sb + kFwdK, sb + kFwdV, kend_s[0], ext, tid, so);
  }
  __syncthreads();
  while (blk >= 0) {
    int nxt = walk.next(blk + 1);
    if (nxt >= 0) st.issue(a, g, nxt < walk.n_ext_blocks, blk_k0(nxt), tid);
    block(Buf<0>(), blk, nxt);
    blk = nxt;
    if (blk < 0) break;
    nxt = walk.next(blk + 1);
    if (nxt >= 0) st.issue(a, g, nxt < walk.n_ext_blocks, blk_k0(nxt), tid);
    block(Buf<1>(), blk, nxt);
    blk = nxt;
  }

  // finalize: O = acc / l, LSE = (m + log2 l) ln 2
  acc_fence();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = lrow[nt] + __shfl_xor(lrow[nt], 32);
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
constexpr int kDqBN = 32;
constexpr int kDqTile = kDqBN * kRowB;
constexpr int kDqK = 0, kDqV = 2 * kDqTile;

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(AttnArgs a) {
  constexpr int BN = kDqBN;
  __shared__ __attribute__((aligned(16))) char smem[4 * kDqTile];
  __shared__ int32_t kend_s[2][BN];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;

  int g, item;
  map_block(blockIdx.x, a.hkv, n_qt, g, item);
  if (g >= a.hkv) return;
  const int qt = n_qt - 1 - item;
  const int t0 = qt * tq;
  const int t1 = min(t0 + tq, a.rows);

  QCol qc[2];
  bf16x8 qf[2][kD / 16], df[2][kD / 16];
  float lse2[2], dsum[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    qc[nt] = qcol(a, g, t0, tq, wave * 64 + nt * 32 + col);
    const int64_t qo = (int64_t)qc[nt].tok * a.q_st + (int64_t)qc[nt].head * a.q_sh + 8 * h32;
    const int64_t doo = (int64_t)qc[nt].tok * a.do_st + (int64_t)qc[nt].head * a.do_sh + 8 * h32;
    const int64_t oo = (int64_t)qc[nt].tok * a.o_st + (int64_t)qc[nt].head * a.o_sh + 8 * h32;
    float dot = 0.f;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      qf[nt][ds] = qc[nt].valid ? load8((const __bf16*)a.q + qo + ds * 16) : zero8();
      df[nt][ds] = qc[nt].valid ? load8((const __bf16*)a.dout + doo + ds * 16) : zero8();
      const bf16x8 ov = qc[nt].valid ? load8((const __bf16*)a.o + oo + ds * 16) : zero8();
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf((float)df[nt][ds][e], (float)ov[e], dot);
    }
    dot += __shfl_xor(dot, 32);
    dsum[nt] = dot;
    float l = qc[nt].valid ? a.lse[(int64_t)qc[nt].head * a.rows + qc[nt].tok] : 0.f;
    lse2[nt] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    if (qc[nt].valid && h32 == 0) a.dsum[(int64_t)qc[nt].head * a.rows + qc[nt].tok] = dot;
  }

  KeyWalk<BN> walk;
  walk.n_ext_blocks = (a.n_ext + BN - 1) / BN;
  walk.t0 = t0;
  walk.t1 = t1;
  walk.bmax = a.ri.bmax;
  walk.bmin = a.ri.bmin;
  walk.rows = a.rows;

  Frag f;
  frag_init(f, lane);
  const uint32_t so = stage_off(tid);
  KvStage<BN> st;
  const float c = a.scale_log2;
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();

  auto blk_k0 = [&](int b) { return (b < walk.n_ext_blocks ? b : b - walk.n_ext_blocks) * BN; };

  auto block = [&](auto bc, int blk, int nxt) {
    constexpr int B = decltype(bc)::value;
    const lds_t* kt_s = sb + kDqK + B * kDqTile;
    const lds_t* vt_s = sb + kDqV + B * kDqTile;
    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = blk_k0(blk);
    const bool msk = walk.masked(blk, a.n_ext);

    // S^T = K Q^T and dP^T = V dO^T: 32 keys x 64 queries
    f32x16 s[2], dp[2];
    s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 ka = ld_row8(kt_s + f.row8[ds]);
      const bf16x8 va = ld_row8(vt_s + f.row8[ds]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s[nt] = mfma(ka, qf[nt][ds], s[nt]);
        dp[nt] = mfma(va, df[nt][ds], dp[nt]);
      }
    }
    bf16x8 dsb[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s[nt][i], c, -lse2[nt]));
        if (msk) {
          const int kl = 8 * (i >> 2) + 4 * h32 + (i & 3);
          const int kk = k0 + kl;
          bool vis = kk < (ext ? a.n_ext : a.rows);
          if (!ext) vis = vis && kk <= qc[nt].tok && qc[nt].tok < kend_s[B][kl];
          if (!vis) p = 0.f;
        }
        s[nt][i] = p * (dp[nt][i] - dsum[nt]);
      }
      dsb[nt][0] = pack_half(s[nt], 0);
      dsb[nt][1] = pack_half(s[nt], 1);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const lds_t* kb = kt_s + ks * 16 * kRowB;
        const bf16x8 af = ld_tr(kb + f.tr[dt][0], kb + f.tr[dt][1]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) mfma_acc(acc[dt][nt], af, dsb[nt][ks]);
      }
    }
    if (nxt >= 0)
      st.stash(sb + kDqK + (1 - B) * kDqTile, sb + kDqV + (1 - B) * kDqTile, kend_s[1 - B],
               nxt < walk.n_ext_blocks, tid, so);
    __syncthreads();
  };

  int blk = walk.next(0);
  if (blk >= 0) {
    const bool ext = blk < walk.n_ext_blocks;
    st.issue(a, g, ext, blk_k0(blk), tid);
    st.stash(sb + kDqK, sb + kDqV, kend_s[0], ext, tid, so);
  }
  __syncthreads();
  while (blk >= 0) {
    int nxt = walk.next(blk + 1);
    if (nxt >= 0) st.issue(a, g, nxt < walk.n_ext_blocks, blk_k0(nxt), tid);
    block(Buf<0>(), blk, nxt);
    blk = nxt;
    if (blk < 0) break;
    nxt = walk.next(blk + 1);
    if (nxt >= 0) st.issue(a, g, nxt < walk.n_ext_blocks, blk_k0(nxt), tid);
    block(Buf<1>(), blk, nxt);
    blk = nxt;
  }

  acc_fence();
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
// Backward, KV-stationary: dK, dV.
//
// A workgroup owns 256 keys of one KV head (64 per wave, as two 32-key column
// tiles) and walks query steps of 32 tokens x one query head over every head
// of the group.  The query range of a key block is [0, rows) for external
// keys and [k0, max kend) for own keys; it is split into chunks of the
// (query tile, head) index space when the grid needs more workgroups, and each
// chunk writes an fp32 partial that a fixed-order reduce sums.  K fragments
// stay in registers; the workgroup's V rows stay in LDS.
constexpr int kQStep = 32;
constexpr int kKeysPerWave = 64;
constexpr int kKeysPerWg = 4 * kKeysPerWave;
constexpr int kStepTile = kQStep * kRowB;
constexpr int kDkvV = 0;                                  // V rows of the workgroup
constexpr int kDkvQ = kKeysPerWg * kRowB;                 // two Q step buffers
constexpr int kDkvO = kDkvQ + 2 * kStepTile;              // two dO step buffers
constexpr int kDkvBytes = kDkvO + 2 * kStepTile;

__global__ __launch_bounds__(kThreads, 1) void bwd_dkv_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kDkvBytes];
  __shared__ __attribute__((aligned(16))) float lse_s[2][kQStep];
  __shared__ __attribute__((aligned(16))) float dsum_s[2][kQStep];
  lds_t* const sb = (lds_t*)smem;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;

  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb * a.n_chunks_own;   // per KV head
  int g, item;
  map_block(blockIdx.x, a.hkv, items, g, item);
  if (g >= a.hkv) return;

  const bool ext = item < n_ext_kb * a.n_chunks;
  int kb, chunk, nch;
  if (ext) {
    kb = item / a.n_chunks;
    chunk = item - kb * a.n_chunks;
    nch = a.n_chunks;
  } else {
    const int oi = item - n_ext_kb * a.n_chunks;
    kb = oi / a.n_chunks_own;
    chunk = oi - kb * a.n_chunks_own;
    nch = a.n_chunks_own;
  }
  const int k0 = kb * kKeysPerWg;
  const int klim = ext ? a.n_ext : a.rows;
  const int kw0 = k0 + wave * kKeysPerWave;      // this wave's first key

  // query range (tokens) and the (tile, head) index range of this workgroup
  int qlo, qhi;
  if (ext) {
    qlo = 0;
    qhi = a.rows;
  } else {
    qlo = k0;
    int m = -1;
    for (int b = k0 / kKeyBlockSummary; b * kKeyBlockSummary < min(k0 + kKeysPerWg, a.rows); ++b)
      m = max(m, a.ri.bmax[b]);
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

  const uint32_t so = stage_off(tid);
  // V rows of the workgroup into LDS; K fragments (B operand of Q K^T) of the
  // wave's two 32-key tiles into registers; visibility bounds of the keys
  bf16x8 kf[2][kD / 16];
  int kend_k[2];
  bool kvalid[2];
  int wave_qlo = 0x7fffffff, wave_kend_min = 0x7fffffff, wave_kend_max = -1;
  {
    const __bf16* kbase = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vbase = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
#pragma unroll 4
    for (int i = 0; i < kKeysPerWg / 16; ++i) {
      const int kk = k0 + 16 * i + (tid >> 4);
      const u32x4 v = kk < klim ? load16(vbase + (int64_t)kk * vst + (int64_t)g * vsh + (tid & 15) * 8)
                                : zero_u4();
      st16(sb + kDkvV + so + i * 16 * kRowB, v);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = kw0 + kt * 32 + col;
      kvalid[kt] = kk < klim;
      const __bf16* kp = kbase + (int64_t)kk * kst + (int64_t)g * ksh + 8 * h32;
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) kf[kt][ds] = kvalid[kt] ? load8(kp + ds * 16) : zero8();
      kend_k[kt] = (!ext && kvalid[kt]) ? a.ri.kend[kk] : (ext ? 0x7fffffff : -1);
      if (kvalid[kt]) {
        wave_qlo = min(wave_qlo, kk);
        wave_kend_min = min(wave_kend_min, kend_k[kt]);
        wave_kend_max = max(wave_kend_max, kend_k[kt]);
      }
    }
  }
  // wave-wide bounds: the wave's keys are read by tokens in [wave_qlo, wave_kend_max)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wave_qlo = min(wave_qlo, __shfl_xor(wave_qlo, off));
    wave_kend_min = min(wave_kend_min, __shfl_xor(wave_kend_min, off));
    wave_kend_max = max(wave_kend_max, __shfl_xor(wave_kend_max, off));
  }
  const int wave_khi = min(kw0 + kKeysPerWave, klim) - 1;   // last valid key of the wave

  Frag f;
  frag_init(f, lane);
  uint32_t vrow[kD / 16];   // this wave's V fragments: rows 64 wave + l % 32 (+ 32 per tile)
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds) vrow[ds] = f.row8[ds] + wave * kKeysPerWave * kRowB;

  // staging of one query step: Q and dO rows (32 tokens x 128 d each)
  u32x4 qreg[2], dreg[2];
  float lreg = 0.f, dsreg = 0.f;
  auto issue = [&](int it) {
    const int qt = qt_lo + it / a.group;
    const int j = it % a.group;
    const int head = a.ri.qhead[g * a.group + j];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = qt * kQStep + 16 * i + (tid >> 4);
      const int ch = tid & 15;
      const bool ok = tok < a.rows;
      qreg[i] = ok ? load16((const __bf16*)a.q + (int64_t)tok * a.q_st + (int64_t)head * a.q_sh +
                            ch * 8)
                   : zero_u4();
      dreg[i] = ok ? load16((const __bf16*)a.dout + (int64_t)tok * a.do_st +
                            (int64_t)head * a.do_sh + ch * 8)
                   : zero_u4();
    }
    if (tid < kQStep) {
      const int tok = qt * kQStep + tid;
      if (tok < a.rows) {
        const float l = a.lse[(int64_t)head * a.rows + tok];
        lreg = (l == -INFINITY) ? INFINITY : l * kLog2e;
        dsreg = a.dsum[(int64_t)head * a.rows + tok];
      } else {
        lreg = INFINITY;   // exp2(s - inf) = 0: padded rows contribute nothing
        dsreg = 0.f;
      }
    }
  };
  auto stash = [&](auto bc) {
    constexpr int B = decltype(bc)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      st16(sb + kDkvQ + B * kStepTile + so + i * 16 * kRowB, qreg[i]);
      st16(sb + kDkvO + B * kStepTile + so + i * 16 * kRowB, dreg[i]);
    }
    if (tid < kQStep) {
      lse_s[B][tid] = lreg;
      dsum_s[B][tid] = dsreg;
    }
  };

  const float c = a.scale_log2;
  f32x16 dk[kD / 32][2], dv[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      dk[dt][kt] = zero16();
      dv[dt][kt] = zero16();
    }

  // one query step held in buffer B; stages step it + 1 into the other buffer
  auto step = [&](auto bc, int it) {
    constexpr int B = decltype(bc)::value;
    const bool more = it + 1 < it_hi;
    if (more) issue(it + 1);
    const int qt = qt_lo + it / a.group;
    const int tq0 = qt * kQStep;
    // skip steps none of the wave's keys is visible to (wave-uniform)
    const bool live = ext || (tq0 + kQStep - 1 >= wave_qlo && tq0 < wave_kend_max);
    if (live) {
      const lds_t* q_s = sb + kDkvQ + B * kStepTile;
      const lds_t* d_s = sb + kDkvO + B * kStepTile;
      // S = Q K^T and dP = dO V^T: 32 queries x the wave's 64 keys
      f32x16 s[2], dp[2];
      s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
#pragma unroll
      for (int ds = 0; ds < kD / 16; ++ds) {
        const bf16x8 qa = ld_row8(q_s + f.row8[ds]);
        const bf16x8 da = ld_row8(d_s + f.row8[ds]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 vb = ld_row8(sb + kDkvV + kt * 32 * kRowB + vrow[ds]);
          s[kt] = mfma(qa, kf[kt][ds], s[kt]);
          dp[kt] = mfma(da, vb, dp[kt]);
        }
      }
      // P and dS; the C rows are queries 8 (i/4) + 4 h32 + i%4
      const bool need_mask =
          !ext && !(tq0 >= wave_khi && tq0 + kQStep - 1 < wave_kend_min);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int qr = 8 * jj + 4 * h32;
        const f32x4 l4 = *(const f32x4*)&lse_s[B][qr];
        const f32x4 d4 = *(const f32x4*)&dsum_s[B][qr];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * jj + r;
            float p = fast_exp2(fmaf(s[kt][i], c, -l4[r]));
            if (need_mask) {
              const int tq = tq0 + qr + r;
              const int kk = kw0 + kt * 32 + col;
              if (!(kk <= tq && tq < kend_k[kt])) p = 0.f;
            }
            if (!kvalid[kt]) p = 0.f;
            s[kt][i] = p;
            dp[kt][i] = p * (dp[kt][i] - d4[r]);
          }
      }
      bf16x8 pb[2][2], db[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        pb[kt][0] = pack_half(s[kt], 0);
        pb[kt][1] = pack_half(s[kt], 1);
        db[kt][0] = pack_half(dp[kt], 0);
        db[kt][1] = pack_half(dp[kt], 1);
      }
      // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const lds_t* ob = d_s + hf * 16 * kRowB;
          const lds_t* qb = q_s + hf * 16 * kRowB;
          const bf16x8 oa = ld_tr(ob + f.tr[dt][0], ob + f.tr[dt][1]);
          const bf16x8 qa = ld_tr(qb + f.tr[dt][0], qb + f.tr[dt][1]);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            mfma_acc(dv[dt][kt], oa, pb[kt][hf]);
            mfma_acc(dk[dt][kt], qa, db[kt][hf]);
          }
        }
      }
    }
    if (more) stash(Buf<1 - B>());
    __syncthreads();
  };

  if (it_lo < it_hi) {
    issue(it_lo);
    stash(Buf<0>());
  }
  __syncthreads();
  for (int it = it_lo; it < it_hi; it += 2) {
    step(Buf<0>(), it);
    if (it + 1 < it_hi) step(Buf<1>(), it + 1);
  }

  // lane holds key kw0 + 32 kt + col, d = 32 dt + 8 j + 4 h32 + r
  acc_fence();
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (!kvalid[kt]) continue;
    const int kk = kw0 + kt * 32 + col;
    const int64_t base = ((int64_t)kk * a.hkv + g) * kD;
    if (ext) {
      if (nch == 1) {
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = dt * 32 + 8 * j + 4 * h32;
            f32x4 gk = *(f32x4*)(a.gk_acc + base + d);
            f32x4 gv = *(f32x4*)(a.gv_acc + base + d);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              gk[r] += dk[dt][kt][4 * j + r] * a.scale;
              gv[r] += dv[dt][kt][4 * j + r];
            }
            *(f32x4*)(a.gk_acc + base + d) = gk;
            *(f32x4*)(a.gv_acc + base + d) = gv;
          }
      } else {
        const int64_t pbase = (int64_t)chunk * a.n_ext * a.hkv * kD + base;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = dt * 32 + 8 * j + 4 * h32;
            f32x4 gk, gv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              gk[r] = dk[dt][kt][4 * j + r] * a.scale;
              gv[r] = dv[dt][kt][4 * j + r];
            }
            *(f32x4*)(a.gk_part + pbase + d) = gk;
            *(f32x4*)(a.gv_part + pbase + d) = gv;
          }
      }
      continue;
    }
    if (nch > 1) {
      // own keys split over query chunks: fp32 partials, finished by a reduce
      const int64_t pbase = (int64_t)chunk * a.rows * a.hkv * kD + base;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = dt * 32 + 8 * j + 4 * h32;
          f32x4 gk, gv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gk[r] = dk[dt][kt][4 * j + r] * a.scale;
            gv[r] = dv[dt][kt][4 * j + r];
          }
          *(f32x4*)(a.dk_part + pbase + d) = gk;
          *(f32x4*)(a.dv_part + pbase + d) = gv;
        }
      continue;
    }
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = dt * 32 + 8 * j + 4 * h32;
        f32x4 vk, vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          vk[r] = dk[dt][kt][4 * j + r] * a.scale;
          vv[r] = dv[dt][kt][4 * j + r];
        }
        if (a.gk_init) {
          const f32x4 ik = *(const f32x4*)(a.gk_init + base + d);
          const f32x4 iv = *(const f32x4*)(a.gv_init + base + d);
          vk += ik;
          vv += iv;
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

// grid size: per-KV-head items, padded so the XCD mapping covers every item
int grid_for(int hkv, int items) {
  if ((hkv & 7) == 0) return 8 * ((hkv / 8) * items);
  return hkv * items;
}

}  // namespace

hipError_t launch_fwd_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  if (a.rows <= 0) return hipSuccess;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;
  PF_LAUNCH("pf_fwd_bf16", fwd_kernel, dim3(grid_for(a.hkv, n_qt)), dim3(kThreads), stream, a);
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

hipError_t launch_bwd_dkv_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb * a.n_chunks_own;
  if (items <= 0) return hipSuccess;
  PF_LAUNCH("pf_bwd_dkv_bf16", bwd_dkv_kernel, dim3(grid_for(a.hkv, items)), dim3(kThreads),
            stream, a);
  return hipGetLastError();
}

int32_t dkv_keys_per_workgroup_bf16() { return kKeysPerWg; }

}  // namespace pf
