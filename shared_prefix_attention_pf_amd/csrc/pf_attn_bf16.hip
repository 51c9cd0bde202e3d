// bf16 attention kernels for gfx950 (CDNA4), head_dim 128, fp32 accumulation.
//
// Three kernels cover every phase (see pf_internal.h for the visibility rule):
//   fwd_kernel      Q-stationary forward with online softmax: the Phase-B
//                   suffix forward over the cached prefix (read in place),
//                   Phase A (causal prefix) and the tree forward.
//   bwd_dq_kernel   Q-stationary backward: D = rowsum(dO * O) and dQ.
//   bwd_dkv_kernel  KV-stationary backward: dK, dV of one key block summed over
//                   every query row and every query head of its KV head.  For
//                   the prefix ("external") keys of Phase B that sum is the
//                   group's prefix-side gradient gK/gV (PrefixFlow §3.3, §4.1),
//                   added to the fp32 accumulator by the one workgroup that
//                   owns the block (or written as a per-chunk partial and
//                   reduced in fixed order): no atomics, no races.
//
// Matrix-core layout.  All contractions use v_mfma_f32_32x32x16_bf16:
//   A (32 x 16): lane l holds A[l % 32][8 (l / 32) + i], i = 0..7
//   B (16 x 32): lane l holds B[8 (l / 32) + i][l % 32]
//   C (32 x 32): lane l holds C[8 (i / 4) + 4 (l / 32) + (i % 4)][l % 32], i = 0..15
// The forward and dQ kernels compute S^T = K Q^T, so a lane owns one query
// (column) and the softmax statistics are per lane.  A C tile of P^T (or
// dS^T) is reused directly as the B operand of the next product: its 16
// values per lane are two 8-value k-steps whose contraction index runs over
// keys {16s + 8(i/4) + 4(l/32) + i%4}.  The matching A operands (V^T, K^T) are
// staged in LDS with keys permuted the same way inside every 16-key group
// (offsets 4..7 and 8..11 swapped), so each A fragment is one 16-byte read.
// The dK/dV kernel computes S = Q K^T (a lane owns one key) and reuses P and
// dS as B operands the same way, with Q^T and dO^T staged permuted in LDS.
#include <math.h>

#include "pf_internal.h"

namespace pf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kD = 128;           // head_dim of this kernel family
constexpr int kDP = kD + 8;       // LDS row pitch (elements) of [row][d] tiles
constexpr int kThreads = 256;     // 4 waves
constexpr int kRowsPerWg = 256;   // query rows (token x head) per Q-stationary workgroup

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// position of key offset o (0..15) inside a permuted 16-key group
__device__ __forceinline__ int perm16(int o) { return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1); }

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
  c.head = c.valid ? a.heads.qhead[g * a.group + j] : 0;
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

// ---------------------------------------------------------------------------
// Forward.
//
// LDS per stage: K [BN][kDP] and V^T [kD][BN + 8] (keys permuted), kend [BN].
template <int BN>
struct FwdSmem {
  __bf16 k[2][BN][kDP];
  __bf16 vt[2][kD][BN + 8];
  int32_t kend[2][BN];
};

template <int BN>
__global__ __launch_bounds__(kThreads) void fwd_kernel(AttnArgs a) {
  static_assert(BN == 64, "staging below assumes 64-key blocks");
  __shared__ FwdSmem<BN> sm;
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

  // staging registers: K rows (4 x 16 B per thread) and V (4 keys x 8 d)
  uint4 kreg[4], vreg[4];
  int kendreg = 0;
  const int v_kg = tid & 15, v_dc = tid >> 4;   // V: keys 4 v_kg..+3, d 8 v_dc..+7

  auto issue = [&](int blk) {
    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = (ext ? blk : blk - walk.n_ext_blocks) * BN;
    const int klim = ext ? a.n_ext : a.rows;
    const __bf16* kb = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vb = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int key = c >> 4, dch = c & 15;
      const int kk = k0 + key;
      kreg[i] = (kk < klim) ? *(const uint4*)(kb + (int64_t)kk * kst + (int64_t)g * ksh + dch * 8)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = k0 + 4 * v_kg + r;
      vreg[r] = (kk < klim) ? *(const uint4*)(vb + (int64_t)kk * vst + (int64_t)g * vsh + v_dc * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    if (!ext && tid < BN) {
      const int kk = k0 + tid;
      kendreg = (kk < a.rows) ? a.ri.kend[kk] : -1;
    }
  };
  auto stash = [&](int buf, int blk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      *(uint4*)&sm.k[buf][c >> 4][(c & 15) * 8] = kreg[i];
    }
    // transpose V: for each of the 8 d values, 4 consecutive keys
    const __bf16* v16[4] = {(const __bf16*)&vreg[0], (const __bf16*)&vreg[1],
                            (const __bf16*)&vreg[2], (const __bf16*)&vreg[3]};
    const int kpos = (4 * v_kg & ~15) + perm16((4 * v_kg) & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 w;
      w[0] = v16[0][e]; w[1] = v16[1][e]; w[2] = v16[2][e]; w[3] = v16[3][e];
      *(bf16x4*)&sm.vt[buf][v_dc * 8 + e][kpos] = w;
    }
    if (blk >= walk.n_ext_blocks && tid < BN) sm.kend[buf][tid] = kendreg;
  };

  const float c = a.scale_log2;
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();

  int blk = walk.next(0);
  if (blk >= 0) {
    issue(blk);
    stash(0, blk);
  }
  __syncthreads();
  int buf = 0;
  while (blk >= 0) {
    const int nxt = walk.next(blk + 1);
    if (nxt >= 0) issue(nxt);

    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = (ext ? blk : blk - walk.n_ext_blocks) * BN;
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
        const bf16x8 af = load8(&sm.k[buf][kt * 32 + col][ds * 16 + 8 * h32]);
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
            const int ke = sm.kend[buf][kl];
            vis0 = vis0 && kk <= qc[0].tok && qc[0].tok < ke;
            vis1 = vis1 && kk <= qc[1].tok && qc[1].tok < ke;
          }
          if (!vis0) s[kt][0][i] = -INFINITY;
          if (!vis1) s[kt][1][i] = -INFINITY;
        }
    }
    // online softmax (log2 domain), per query column
    bf16x8 pb[2][BN / 16];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BN / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][nt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[nt], mx * c);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(mrow[nt] - muse);
      mrow[nt] = mnew;
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
      lrow[nt] = lrow[nt] * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) acc[dt][nt] *= alpha;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const bf16x8 af = load8(&sm.vt[buf][dt * 32 + col][ks * 16 + 8 * h32]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = mfma(af, pb[nt][ks], acc[dt][nt]);
      }
    }
    if (nxt >= 0) stash(buf ^ 1, nxt);
    __syncthreads();
    buf ^= 1;
    blk = nxt;
  }

  // finalize: O = acc / l, LSE = (m + log2 l) ln 2
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
//
// LDS per stage: K [BN][kDP], V [BN][kDP], K^T [kD][BN + 8] (keys permuted).
template <int BN>
struct DqSmem {
  __bf16 k[2][BN][kDP];
  __bf16 v[2][BN][kDP];
  __bf16 kt[2][kD][BN + 8];
  int32_t kend[2][BN];
};

template <int BN>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(AttnArgs a) {
  static_assert(BN == 32, "staging below assumes 32-key blocks");
  __shared__ DqSmem<BN> sm;
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

  // staging: K and V rows (2 x 16 B each per thread); K^T from the K registers
  uint4 kreg[2], vreg[2];
  int kendreg = 0;
  auto issue = [&](int blk) {
    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = (ext ? blk : blk - walk.n_ext_blocks) * BN;
    const int klim = ext ? a.n_ext : a.rows;
    const __bf16* kb = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vb = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    // thread -> (key = 4 * (tid & 7) + i, d chunk = tid >> 3), i = 0..1 pairs of
    // consecutive keys (0/1 or 2/3) so the transposed store writes 4 keys at once
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = 4 * (tid & 7) + 2 * (tid >> 7) + i;   // tid >> 7 in {0, 1}
      const int dch = (tid >> 3) & 15;
      const int kk = k0 + key;
      kreg[i] = (kk < klim) ? *(const uint4*)(kb + (int64_t)kk * kst + (int64_t)g * ksh + dch * 8)
                            : make_uint4(0, 0, 0, 0);
      vreg[i] = (kk < klim) ? *(const uint4*)(vb + (int64_t)kk * vst + (int64_t)g * vsh + dch * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    if (!ext && tid < BN) {
      const int kk = k0 + tid;
      kendreg = (kk < a.rows) ? a.ri.kend[kk] : -1;
    }
  };
  auto stash = [&](int buf, int blk) {
    const int kg = tid & 7, half = tid >> 7, dch = (tid >> 3) & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = 4 * kg + 2 * half + i;
      *(uint4*)&sm.k[buf][key][dch * 8] = kreg[i];
      *(uint4*)&sm.v[buf][key][dch * 8] = vreg[i];
    }
    // K^T: 2 consecutive keys per d value (keys 4 kg + 2 half + {0, 1})
    const __bf16* k16[2] = {(const __bf16*)&kreg[0], (const __bf16*)&kreg[1]};
    const int o = 4 * kg + 2 * half;
    const int kpos = (o & ~15) + perm16(o & 15);    // o & 3 in {0, 2}: stays contiguous
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 w[2] = {k16[0][e], k16[1][e]};
      *(uint32_t*)&sm.kt[buf][dch * 8 + e][kpos] = *(uint32_t*)w;
    }
    if (blk >= walk.n_ext_blocks && tid < BN) sm.kend[buf][tid] = kendreg;
  };

  const float c = a.scale_log2;
  f32x16 acc[kD / 32][2];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = zero16();

  int blk = walk.next(0);
  if (blk >= 0) {
    issue(blk);
    stash(0, blk);
  }
  __syncthreads();
  int buf = 0;
  while (blk >= 0) {
    const int nxt = walk.next(blk + 1);
    if (nxt >= 0) issue(nxt);
    const bool ext = blk < walk.n_ext_blocks;
    const int k0 = (ext ? blk : blk - walk.n_ext_blocks) * BN;
    const bool msk = walk.masked(blk, a.n_ext);

    f32x16 s[2], dp[2];
    s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 ka = load8(&sm.k[buf][col][ds * 16 + 8 * h32]);
      const bf16x8 va = load8(&sm.v[buf][col][ds * 16 + 8 * h32]);
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
          if (!ext) vis = vis && kk <= qc[nt].tok && qc[nt].tok < sm.kend[buf][kl];
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
        const bf16x8 af = load8(&sm.kt[buf][dt * 32 + col][ks * 16 + 8 * h32]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = mfma(af, dsb[nt][ks], acc[dt][nt]);
      }
    }
    if (nxt >= 0) stash(buf ^ 1, nxt);
    __syncthreads();
    buf ^= 1;
    blk = nxt;
  }

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
// A workgroup owns 128 keys (32 per wave) of one KV head and walks query
// steps of 32 tokens x one query head, over every head of the group.
// External key blocks walk all rows (split into n_chunks contiguous ranges of
// the (query tile, head) index space); own key blocks walk the rows that can
// see them: [k0, max kend).
constexpr int kQStep = 32;
constexpr int kKeysPerWg = 128;
constexpr int kQTP = kQStep + 8;   // LDS pitch of the transposed [d][query] tiles

struct DkvSmem {
  __bf16 q[2][kQStep][kDP];
  __bf16 dO[2][kQStep][kDP];
  __bf16 qt[2][kD][kQTP];
  __bf16 dOt[2][kD][kQTP];
  float lse2[2][kQStep];
  float dsum[2][kQStep];
};

__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(AttnArgs a) {
  __shared__ DkvSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, h32 = lane >> 5;

  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb;   // per KV head
  int g, item;
  map_block(blockIdx.x, a.hkv, items, g, item);
  if (g >= a.hkv) return;

  const bool ext = item < n_ext_kb * a.n_chunks;
  int kb, chunk = 0;
  if (ext) {
    kb = item / a.n_chunks;
    chunk = item - kb * a.n_chunks;
  } else {
    kb = item - n_ext_kb * a.n_chunks;
  }
  const int k0 = kb * kKeysPerWg;
  const int klim = ext ? a.n_ext : a.rows;
  const int kk = k0 + wave * 32 + col;   // this lane's key
  const bool kvalid = kk < klim;

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
  if (ext && a.n_chunks > 1) {
    const int per = (n_it + a.n_chunks - 1) / a.n_chunks;
    it_lo = min(n_it, chunk * per);
    it_hi = min(n_it, it_lo + per);
  }

  // stationary K^T and V^T fragments (B operands of Q K^T and dO V^T)
  bf16x8 kf[kD / 16], vf[kD / 16];
  {
    const __bf16* kbase = (const __bf16*)(ext ? a.k_ext : a.k_own);
    const __bf16* vbase = (const __bf16*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    const __bf16* kp = kbase + (int64_t)kk * kst + (int64_t)g * ksh + 8 * h32;
    const __bf16* vp = vbase + (int64_t)kk * vst + (int64_t)g * vsh + 8 * h32;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      kf[ds] = kvalid ? load8(kp + ds * 16) : zero8();
      vf[ds] = kvalid ? load8(vp + ds * 16) : zero8();
    }
  }
  const int kend_k = (!ext && kvalid) ? a.ri.kend[kk] : 0;

  // staging of one query step: Q and dO rows (32 tokens x 128 d each)
  uint4 qreg[2], dreg[2];
  float lreg = 0.f, dsreg = 0.f;
  // thread -> token 4 * (tid & 7) + 2 * (tid >> 7) + i, d chunk (tid >> 3) & 15
  auto issue = [&](int it) {
    const int qt = qt_lo + it / a.group;
    const int j = it % a.group;
    const int head = a.heads.qhead[g * a.group + j];
    const int dch = (tid >> 3) & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = qt * kQStep + 4 * (tid & 7) + 2 * (tid >> 7) + i;
      const bool ok = tok < a.rows;
      qreg[i] = ok ? *(const uint4*)((const __bf16*)a.q + (int64_t)tok * a.q_st +
                                     (int64_t)head * a.q_sh + dch * 8)
                   : make_uint4(0, 0, 0, 0);
      dreg[i] = ok ? *(const uint4*)((const __bf16*)a.dout + (int64_t)tok * a.do_st +
                                     (int64_t)head * a.do_sh + dch * 8)
                   : make_uint4(0, 0, 0, 0);
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
  auto stash = [&](int buf) {
    const int kg = tid & 7, half = tid >> 7, dch = (tid >> 3) & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 4 * kg + 2 * half + i;
      *(uint4*)&sm.q[buf][t][dch * 8] = qreg[i];
      *(uint4*)&sm.dO[buf][t][dch * 8] = dreg[i];
    }
    const __bf16* q16[2] = {(const __bf16*)&qreg[0], (const __bf16*)&qreg[1]};
    const __bf16* d16[2] = {(const __bf16*)&dreg[0], (const __bf16*)&dreg[1]};
    const int o = 4 * kg + 2 * half;
    const int tpos = (o & ~15) + perm16(o & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 w[2] = {q16[0][e], q16[1][e]};
      __bf16 x[2] = {d16[0][e], d16[1][e]};
      *(uint32_t*)&sm.qt[buf][dch * 8 + e][tpos] = *(uint32_t*)w;
      *(uint32_t*)&sm.dOt[buf][dch * 8 + e][tpos] = *(uint32_t*)x;
    }
    if (tid < kQStep) {
      sm.lse2[buf][tid] = lreg;
      sm.dsum[buf][tid] = dsreg;
    }
  };

  const float c = a.scale_log2;
  f32x16 dk[kD / 32], dv[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  if (it_lo < it_hi) {
    issue(it_lo);
    stash(0);
  }
  __syncthreads();
  int buf = 0;
  for (int it = it_lo; it < it_hi; ++it) {
    if (it + 1 < it_hi) issue(it + 1);
    const int qt = qt_lo + it / a.group;
    const int tq0 = qt * kQStep;

    // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 qa = load8(&sm.q[buf][col][ds * 16 + 8 * h32]);
      const bf16x8 da = load8(&sm.dO[buf][col][ds * 16 + 8 * h32]);
      s = mfma(qa, kf[ds], s);
      dp = mfma(da, vf[ds], dp);
    }
    // P and dS; the C rows are queries 8 (i/4) + 4 h32 + i%4
    const bool need_mask = !ext && !(tq0 + kQStep - 1 < kend_k && tq0 >= k0 + kKeysPerWg);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int qr = 8 * jj + 4 * h32;
      const f32x4 l4 = *(const f32x4*)&sm.lse2[buf][qr];
      const f32x4 d4 = *(const f32x4*)&sm.dsum[buf][qr];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * jj + r;
        float p = fast_exp2(fmaf(s[i], c, -l4[r]));
        if (need_mask) {
          const int tq = tq0 + qr + r;
          if (!(kk <= tq && tq < kend_k)) p = 0.f;
        }
        if (!kvalid) p = 0.f;
        s[i] = p;
        dp[i] = p * (dp[i] - d4[r]);
      }
    }
    const bf16x8 pb0 = pack_half(s, 0), pb1 = pack_half(s, 1);
    const bf16x8 db0 = pack_half(dp, 0), db1 = pack_half(dp, 1);
    // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
      const bf16x8 oa0 = load8(&sm.dOt[buf][dt * 32 + col][8 * h32]);
      const bf16x8 oa1 = load8(&sm.dOt[buf][dt * 32 + col][16 + 8 * h32]);
      const bf16x8 qa0 = load8(&sm.qt[buf][dt * 32 + col][8 * h32]);
      const bf16x8 qa1 = load8(&sm.qt[buf][dt * 32 + col][16 + 8 * h32]);
      dv[dt] = mfma(oa0, pb0, dv[dt]);
      dv[dt] = mfma(oa1, pb1, dv[dt]);
      dk[dt] = mfma(qa0, db0, dk[dt]);
      dk[dt] = mfma(qa1, db1, dk[dt]);
    }
    if (it + 1 < it_hi) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (!kvalid) return;
  // lane holds key kk, d = 32 dt + 8 j + 4 h32 + r
  if (ext) {
    const int64_t base = ((int64_t)kk * a.hkv + g) * kD;
    if (a.n_chunks == 1) {
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = dt * 32 + 8 * j + 4 * h32;
          f32x4 gk = *(f32x4*)(a.gk_acc + base + d);
          f32x4 gv = *(f32x4*)(a.gv_acc + base + d);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gk[r] += dk[dt][4 * j + r] * a.scale;
            gv[r] += dv[dt][4 * j + r];
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
            gk[r] = dk[dt][4 * j + r] * a.scale;
            gv[r] = dv[dt][4 * j + r];
          }
          *(f32x4*)(a.gk_part + pbase + d) = gk;
          *(f32x4*)(a.gv_part + pbase + d) = gv;
        }
    }
    return;
  }
  const int64_t ibase = ((int64_t)kk * a.hkv + g) * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = dt * 32 + 8 * j + 4 * h32;
      f32x4 vk, vv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vk[r] = dk[dt][4 * j + r] * a.scale;
        vv[r] = dv[dt][4 * j + r];
      }
      if (a.gk_init) {
        const f32x4 ik = *(const f32x4*)(a.gk_init + ibase + d);
        const f32x4 iv = *(const f32x4*)(a.gv_init + ibase + d);
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
  PF_LAUNCH("pf_fwd_bf16", fwd_kernel<64>, dim3(grid_for(a.hkv, n_qt)), dim3(kThreads), stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  if (a.rows <= 0) return hipSuccess;
  const int tq = kRowsPerWg / a.group;
  const int n_qt = (a.rows + tq - 1) / tq;
  PF_LAUNCH("pf_bwd_dq_bf16", bwd_dq_kernel<32>, dim3(grid_for(a.hkv, n_qt)), dim3(kThreads),
            stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv_bf16(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int n_ext_kb = (a.n_ext + kKeysPerWg - 1) / kKeysPerWg;
  const int n_own_kb = (a.rows + kKeysPerWg - 1) / kKeysPerWg;
  const int items = n_ext_kb * a.n_chunks + n_own_kb;
  if (items <= 0) return hipSuccess;
  PF_LAUNCH("pf_bwd_dkv_bf16", bwd_dkv_kernel, dim3(grid_for(a.hkv, items)), dim3(kThreads), stream, a);
  return hipGetLastError();
}

}  // namespace pf
