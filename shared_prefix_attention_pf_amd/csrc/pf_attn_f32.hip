// fp32 attention kernels (head_dim 64 or 128) on the matrix cores: every
// product is an fp32 MFMA with fp32 inputs and fp32 accumulation
// (v_mfma_f32_32x32x2_f32 in the forward and dQ kernels, v_mfma_f32_16x16x4_f32
// in dK/dV), so fp32 groups are never rounded to bf16.  The kernels compute
// what the bf16 family computes (forward; dQ with D = rowsum(dO o O), from a
// stored dS or recomputing S and dP; dK/dV, with the external keys' gradients
// added into the fp32 accumulators).
//
// Layout of one 32x32x2 product for lane l (half h = l / 32, column l % 32):
//   A operand: lane l supplies A[l % 32][h]; B operand: B[h][l % 32];
//   C register r holds C[crow(r, h)][l % 32], crow(r, h) = 8 (r / 4) + 4 h + r % 4.
// A product's contraction index may be taken in any order, so each one is
// ordered to fit what the wave already holds:
//   - over head_dim (S, dP): step s of lane half h takes d = (D / 2) h + s,
//     so a stationary operand is D / 2 consecutive values of the lane's row;
//   - over keys or queries (O, dQ, dK, dV): step s of lane half h takes index
//     crow(s, h), so the B operand of step s is C register s of the score
//     tile the lane already holds; nothing is transposed.
// Forward and dQ are Q-stationary and form S^T = K Q^T: one query per lane
// column, so its LSE and D are one value per lane.  dK/dV is KV-stationary
// and forms S = Q K^T: one key per lane column, whose P and dS then feed
// dV^T += dO^T P and dK^T += Q^T dS (the same ordering on 16x16 tiles; see
// dkv_f32_kernel).
// K/V (or Q/dO) tiles of 32 rows reach LDS through buffer-to-LDS loads,
// double buffered, with rows padded to D + 4 floats: the row-sliced reads
// (16 bytes of 32 rows) and the column-sliced ones (32 floats of a row) then
// both spread over the banks, and every read is a per-lane base plus a
// constant offset.
#include <math.h>

#include "pf_internal.h"

namespace pf {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
using Rsrc = __amdgpu_buffer_rsrc_t;

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kDkvKeys = 16 * kWaves;     // keys per KV-stationary workgroup
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mm(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 16x16x4 product: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
// C register r holds C[4 (l / 16) + r][l % 16].  Same rate as the 32x32x2
// form (32 cycles for half the work), on tiles a quarter the size.
__device__ __forceinline__ f32x4 mm16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__host__ __device__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// keep a stationary operand in the AGPR file; the products read it there
__device__ __forceinline__ void pin_agpr(float& x) { asm("" : "+a"(x)); }

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes > 0 ? bytes : 0), 0x00020000);
}

// rows [0, valid) of D floats each, row stride st floats, from `base`; loads
// of later rows fall outside the resource and read zero
template <int D>
__device__ __forceinline__ Rsrc rows_rsrc(const float* base, int valid, int64_t st) {
  return make_rsrc(base, valid > 0 ? (int64_t)(valid - 1) * st * 4 + D * 4 : 0);
}

// A 32-row LDS tile of D floats per row, rows padded to D + 4 floats.  A
// buffer-to-LDS load writes 64 consecutive 16-byte chunks (one per lane), so a
// tile takes kNi such loads; lanes whose chunk is padding, or past the last
// row, fetch from an offset past every resource's end and write zero.
template <int D>
struct Tile {
  static constexpr int kRs = D + 4;                  // row stride (floats)
  static constexpr int kCpr = kRs / 4;               // chunks per row, padding included
  static constexpr int kNi = (32 * kCpr + 63) / 64;  // loads per tile
  static constexpr int kFloats = 256 * kNi;          // floats the loads write
};

// The 32 rows of a tile (row r at byte r * st_b of the resource; rows past
// its end read zero) into a padded LDS tile, the loads dealt round the
// workgroup's waves.
template <int D>
__device__ __forceinline__ void dma_tile(Rsrc r, float* tile, uint32_t st_b, int wave, int lane) {
  using T = Tile<D>;
#pragma unroll
  for (int j = 0; j < (T::kNi + kWaves - 1) / kWaves; ++j) {
    const int i = wave + kWaves * j;
    if (i < T::kNi) {
      const int c = 64 * i + lane, row = c / T::kCpr, ch = c % T::kCpr;
      const uint32_t off =
          (row < 32 && ch < T::kCpr - 1) ? (uint32_t)row * st_b + 16u * (uint32_t)ch : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + 256 * i), 16, (int)off, 0, 0,
                                               0);
    }
  }
}

// 64 consecutive 4-byte values (past the resource's end: zero) into LDS
__device__ __forceinline__ void dma_vec(Rsrc r, void* dst, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, 4 * lane, 0, 0, 0);
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The Q-stationary kernels' share of the work: workgroup x of KV head g holds
// four consecutive (32-token tile, query head) pairs of that KV head, one per
// wave, pairs ordered tile-major and taken from the last; the tiles of keys it
// walks are the external ones, then the own ones that some of its rows may see.
struct QTiles {
  int g, head, t0, tok;
  bool active, tvalid;
  int wt_hi;                 // last token of the wave's tile
  int tmin;                  // first token of the workgroup
  int n_ext_t, n_t;          // external tiles; all tiles (external, then own)

  // block x: KV head x % Hkv, rank x / Hkv; rank 0 holds the last pairs of
  // its head.  Later tokens see more keys (causal prefix, trees) and
  // workgroups start in index order, so this is a longest-first schedule over
  // all heads; with 8 KV heads each head's workgroups share one XCD.  With
  // head_major (a 2-D grid, y the KV head) the heads go one after another.
  __device__ QTiles(const AttnArgs& a, int wave, int col, bool head_major = false) {
    g = head_major ? (int)blockIdx.y : (int)blockIdx.x % a.hkv;
    const int rank = head_major ? (int)blockIdx.x : (int)blockIdx.x / a.hkv;
    const int n_pairs = ((a.rows + 31) / 32) * a.group;
    const int p0 = ((n_pairs + kWaves - 1) / kWaves - 1 - rank) * kWaves;
    const int p = p0 + wave;
    active = p < n_pairs;
    const int j = active ? p % a.group : 0;
    t0 = active ? (p / a.group) * 32 : 0;
    head = a.ri.qhead[g * a.group + j];
    tok = t0 + col;
    tvalid = active && tok < a.rows;
    wt_hi = min(a.rows, t0 + 32) - 1;
    tmin = (p0 / a.group) * 32;
    const int tmax = min(a.rows, ((min(p0 + kWaves, n_pairs) - 1) / a.group) * 32 + 32) - 1;
    n_ext_t = (a.n_ext + 31) / 32;
    n_t = n_ext_t + tmax / 32 + 1;
  }
  // some row of the workgroup may see a key of tile i
  __device__ bool live(const AttnArgs& a, int i) const {
    return i < n_ext_t || a.ri.bmax[i - n_ext_t] > tmin;
  }
  __device__ int next(const AttnArgs& a, int i) const {
    for (++i; i < n_t; ++i)
      if (live(a, i)) return i;
    return -1;
  }
  // some row of this wave may see a key of tile i
  __device__ bool wave_sees(const AttnArgs& a, int i) const {
    if (!active) return false;
    if (i < n_ext_t) return true;
    const int b = i - n_ext_t;
    return 32 * b <= wt_hi && a.ri.bmax[b] > t0;
  }
  __device__ int key0(int i) const { return (i < n_ext_t ? i : i - n_ext_t) * 32; }
};

// External key tile t (32 keys): the row of its first key in k_ext / v_ext
// (and in gK/gV) and how many of its keys are real.  With a tile table the
// external keys are row ranges of a larger tensor, each padded to whole tiles;
// without one they are rows 0 .. n_ext - 1.  t is uniform over the wave.
__device__ __forceinline__ int2 ext_tile(const AttnArgs& a, int t) {
  if (a.ext_tiles) return a.ext_tiles[t];
  return int2{32 * t, min(32, a.n_ext - 32 * t)};
}

// Key tile i of a Q-stationary workgroup: the row of its first key in its
// tensor and how many of its keys are real
__device__ __forceinline__ int2 key_tile(const AttnArgs& a, const QTiles& w, int i) {
  if (i < w.n_ext_t) return ext_tile(a, i);
  const int k0 = w.key0(i);
  return int2{k0, a.rows - k0};
}

// K/V tile i of a Q-stationary workgroup (and the kend values of own keys)
// into LDS buffer b
template <int D>
__device__ __forceinline__ void stage_kv(const AttnArgs& a, const QTiles& w, int i, float* k_s,
                                         float* v_s, int32_t* kend_s, int wave, int lane) {
  const bool ext = i < w.n_ext_t;
  const int2 kt = key_tile(a, w, i);
  const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
  const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
  const float* kb =
      (const float*)(ext ? a.k_ext : a.k_own) + (int64_t)kt.x * kst + (int64_t)w.g * ksh;
  const float* vb =
      (const float*)(ext ? a.v_ext : a.v_own) + (int64_t)kt.x * vst + (int64_t)w.g * vsh;
  dma_tile<D>(rows_rsrc<D>(kb, kt.y, kst), k_s, 4u * (uint32_t)kst, wave, lane);
  dma_tile<D>(rows_rsrc<D>(vb, kt.y, vst), v_s, 4u * (uint32_t)vst, wave, lane);
  if (!ext && wave == kWaves - 1) dma_vec(make_rsrc(a.ri.kend + kt.x, 4LL * kt.y), kend_s, lane);
}

// The scores of key tile i against the wave's queries, in log2 units, with
// the keys the lane's query cannot see at -inf: register r is the tile's key
// crow(r, h).
template <int D>
__device__ __forceinline__ void visible_scores(const AttnArgs& a, const QTiles& w, int i, int h,
                                               const f32x16& s, const int32_t* kend_s,
                                               float (&x)[16]) {
  const float c = a.scale_log2;
  const int tok = w.tok;
  if (i < w.n_ext_t) {
    const int n_valid = ext_tile(a, i).y;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = crow(r, h) < n_valid ? s[r] * c : -INFINITY;
  } else {
    const int k0 = w.key0(i);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const i32x4 ke = *(const i32x4*)(kend_s + 8 * q4 + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e, kk = k0 + crow(r, h);
        x[r] = (kk <= tok && tok < ke[e]) ? s[r] * c : -INFINITY;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_f32_kernel(AttnArgs a) {
  constexpr int H = D / 2, NT = D / 32, RS = Tile<D>::kRs;
  __shared__ __attribute__((aligned(16))) float kv_s[2][2][Tile<D>::kFloats];
  __shared__ __attribute__((aligned(16))) int32_t kend_s[2][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const QTiles w(a, wave, col);

  // the lane's half of its query row: B operand of S^T = K Q^T
  float q[H];
  {
    const float* qp = (const float*)a.q + (int64_t)(w.tvalid ? w.tok : 0) * a.q_st +
                      (int64_t)w.head * a.q_sh + H * h;
#pragma unroll
    for (int u = 0; u < H / 4; ++u) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (w.tvalid) v = *(const f32x4*)(qp + 4 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[4 * u + e] = v[e];
    }
#pragma unroll
    for (int s = 0; s < H; ++s) pin_agpr(q[s]);
  }

  f32x16 o[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) o[dt] = zero16();
  float m = -INFINITY, lsum = 0.f;   // running max (log2 units) and this half's sum

  int cur = w.live(a, 0) ? 0 : w.next(a, 0);
  if (w.n_t <= 0) cur = -1;
  if (cur >= 0) stage_kv<D>(a, w, cur, kv_s[0][0], kv_s[0][1], kend_s[0], wave, lane);
  for (int b = 0; cur >= 0; b ^= 1) {
    const int nxt = w.next(a, cur);
    wait_dma();
    __syncthreads();
    if (nxt >= 0) stage_kv<D>(a, w, nxt, kv_s[b ^ 1][0], kv_s[b ^ 1][1], kend_s[b ^ 1], wave, lane);
    if (w.wave_sees(a, cur)) {
      const float* ks = kv_s[b][0];
      const float* vs = kv_s[b][1];
      f32x16 s = zero16();
#pragma unroll
      for (int u = 0; u < H / 4; ++u) {
        const f32x4 kv = *(const f32x4*)(ks + col * RS + H * h + 4 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) s = mm(kv[e], q[4 * u + e], s);
      }
      float x[16];
      visible_scores<D>(a, w, cur, h, s, kend_s[b], x);
      float mx = x[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2_(m - ms);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = exp2_(x[r] - ms);
        ps += x[r];
      }
      lsum = lsum * alpha + ps;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
          o[dt] = mm(vs[crow(s2, h) * RS + 32 * dt + col], x[s2], o[dt]);
      }
    }
    cur = nxt;
  }

  const float lt = lsum + __shfl_xor(lsum, 32);
  if (!w.tvalid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float* op = (float*)a.out + (int64_t)w.tok * a.out_st + (int64_t)w.head * a.out_sh;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * q4 + e] * inv;
      *(f32x4*)(op + 32 * dt + 8 * q4 + 4 * h) = v;
    }
  if (h == 0)
    a.lse[(int64_t)w.head * a.rows + w.tok] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dq_f32_kernel(AttnArgs a) {
  constexpr int H = D / 2, NT = D / 32, RS = Tile<D>::kRs;
  __shared__ __attribute__((aligned(16))) float kv_s[2][2][Tile<D>::kFloats];
  __shared__ __attribute__((aligned(16))) int32_t kend_s[2][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const QTiles w(a, wave, col);

  // the lane's halves of its Q and dO rows (B operands of S^T and dP^T) and
  // D = rowsum(dO o O) of its row
  float q[H], dov[H];
  float dsum;
  {
    const int64_t t = w.tvalid ? w.tok : 0;
    const float* qp = (const float*)a.q + t * a.q_st + (int64_t)w.head * a.q_sh + H * h;
    const float* dp = (const float*)a.dout + t * a.do_st + (int64_t)w.head * a.do_sh + H * h;
    const float* opp = (const float*)a.o + t * a.o_st + (int64_t)w.head * a.o_sh + H * h;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < H / 4; ++u) {
      f32x4 qv = {0.f, 0.f, 0.f, 0.f}, dv = qv, ov = qv;
      if (w.tvalid) {
        qv = *(const f32x4*)(qp + 4 * u);
        dv = *(const f32x4*)(dp + 4 * u);
        ov = *(const f32x4*)(opp + 4 * u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[4 * u + e] = qv[e];
        dov[4 * u + e] = dv[e];
        acc = fmaf(dv[e], ov[e], acc);
      }
    }
    dsum = acc + __shfl_xor(acc, 32);
#pragma unroll
    for (int s = 0; s < H; ++s) {
      pin_agpr(q[s]);
      pin_agpr(dov[s]);
    }
  }
  // -D for the dK/dV pass, which starts from the workspace's negated D
  if (w.tvalid && h == 0) a.neg_dsum[(int64_t)w.head * a.rows + w.tok] = -dsum;
  // LSE in log2 units; rows that see no key (LSE -inf) and rows past the end
  // take +inf, so every P of theirs is zero
  float lse2 = INFINITY;
  if (w.tvalid) {
    const float l = a.lse[(int64_t)w.head * a.rows + w.tok];
    if (l != -INFINITY) lse2 = l * kLog2e;
  }

  f32x16 dq[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) dq[dt] = zero16();

  int cur = w.live(a, 0) ? 0 : w.next(a, 0);
  if (w.n_t <= 0) cur = -1;
  if (cur >= 0) stage_kv<D>(a, w, cur, kv_s[0][0], kv_s[0][1], kend_s[0], wave, lane);
  for (int b = 0; cur >= 0; b ^= 1) {
    const int nxt = w.next(a, cur);
    wait_dma();
    __syncthreads();
    if (nxt >= 0) stage_kv<D>(a, w, nxt, kv_s[b ^ 1][0], kv_s[b ^ 1][1], kend_s[b ^ 1], wave, lane);
    if (w.wave_sees(a, cur)) {
      const float* ks = kv_s[b][0];
      const float* vs = kv_s[b][1];
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int u = 0; u < H / 4; ++u) {
        const f32x4 kv = *(const f32x4*)(ks + col * RS + H * h + 4 * u);
        const f32x4 vv = *(const f32x4*)(vs + col * RS + H * h + 4 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mm(kv[e], q[4 * u + e], s);
          dp = mm(vv[e], dov[4 * u + e], dp);
        }
      }
      float x[16];
      visible_scores<D>(a, w, cur, h, s, kend_s[b], x);
      // dS^T = P^T o (dP^T - D), P^T = 2^(x - LSE2); invisible entries are 0
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = x[r] == -INFINITY ? 0.f : exp2_(x[r] - lse2);
        x[r] = p * (dp[r] - dsum);
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
          dq[dt] = mm(ks[crow(s2, h) * RS + 32 * dt + col], x[s2], dq[dt]);
    }
    cur = nxt;
  }

  if (!w.tvalid) return;
  float* op = (float*)a.out + (int64_t)w.tok * a.out_st + (int64_t)w.head * a.out_sh;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = dq[dt][4 * q4 + e] * a.scale;
      *(f32x4*)(op + 32 * dt + 8 * q4 + 4 * h) = v;
    }
}

// KV-stationary: a workgroup holds 64 keys of KV head y, 16 per wave, and
// walks the (32-token tile, query head) steps whose rows may see them: all
// rows for external keys, rows from the block's first key to the largest
// visibility end of its keys for own keys.  A block's steps may be split into
// query chunks (a.n_chunks external, a.n_chunks_own own), one workgroup each;
// item x is (external block, chunk) pairs first, then (own block, chunk).
// The products are 16x16x4: a wave's 16 keys are the columns of its S and dP
// tiles (two 16-query halves of the step), so the lane holding P or dS of
// (query, key) supplies it as the B operand of dV^T += dO^T P and
// dK^T += Q^T dS; contraction step (half, r) of lane group g takes query
// 16 half + 4 g + r.  Everything stays in VGPRs (about 200 at head_dim 128),
// two workgroups per CU: two waves per SIMD cover each other's waits.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void dkv_f32_kernel(AttnArgs a) {
  constexpr int Q4 = D / 4, NTD = D / 16, RS = Tile<D>::kRs;
  __shared__ __attribute__((aligned(16))) float qd_s[2][2][Tile<D>::kFloats];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float ld_s[2][2][64];       // [buffer][LSE, -D]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, j16 = lane & 15, g4 = lane >> 4;
  // block x: KV head x % Hkv, item x / Hkv (the heads interleaved: external
  // items, the longest, start first on every head)
  const int g = (int)blockIdx.x % a.hkv;
  const int bx = (int)blockIdx.x / a.hkv;
  const int n_ext_b = (a.n_ext + kDkvKeys - 1) / kDkvKeys;
  const int n_ext_items = n_ext_b * a.n_chunks;
  const bool ext = bx < n_ext_items;
  const int nch = ext ? a.n_chunks : a.n_chunks_own;
  const int item = ext ? bx : bx - n_ext_items;
  const int chunk = item % nch;
  const int k0 = (item / nch) * kDkvKeys;
  const int kw0 = k0 + 16 * wave;
  const int kk = kw0 + j16;
  // the lane's key: its row in k/v (and in gK/gV for external keys), and
  // whether it is real (a wave's 16 keys lie in one 32-key tile)
  int krow = kk;
  bool kvalid = kk < a.rows;
  if (ext) {
    kvalid = false;
    if (kw0 < a.n_ext) {   // the last block's second tile may lie past the keys
      const int2 et = ext_tile(a, kw0 >> 5);
      krow = et.x + (kk & 31);
      kvalid = (kk & 31) < et.y;
    }
  }

  // the lane's quarter of its K and V rows (head_dim Q4 g .. Q4 g + Q4 - 1):
  // B operands of S = Q K^T and dP = dO V^T
  float kr[Q4], vr[Q4];
  {
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    const int64_t r = kvalid ? krow : 0;
    const float* kp =
        (const float*)(ext ? a.k_ext : a.k_own) + r * kst + (int64_t)g * ksh + Q4 * g4;
    const float* vp =
        (const float*)(ext ? a.v_ext : a.v_own) + r * vst + (int64_t)g * vsh + Q4 * g4;
#pragma unroll
    for (int u = 0; u < Q4 / 4; ++u) {
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = kv;
      if (kvalid) {
        kv = *(const f32x4*)(kp + 4 * u);
        vv = *(const f32x4*)(vp + 4 * u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kr[4 * u + e] = kv[e];
        vr[4 * u + e] = vv[e];
      }
    }
  }
  const int kend_k = (!ext && kvalid) ? a.ri.kend[kk] : -1;
  // rows that may see the wave's keys end before wave_hi (own keys; the
  // largest visibility end over the 32-key block holding them)
  const int wave_hi = (!ext && kw0 < a.rows) ? a.ri.bmax[kw0 / 32] : 0;

  int qlo = 0, qhi = a.rows;
  if (!ext) {
    qlo = k0;
    int mx = -1;
    for (int b = k0 / 32; b < (k0 + kDkvKeys) / 32 && b * 32 < a.rows; ++b)
      mx = max(mx, a.ri.bmax[b]);
    qhi = min(mx, a.rows);
  }
  const int qt_lo = qlo / 32;
  const int n_qt = qhi > qlo ? (qhi - 1) / 32 - qt_lo + 1 : 0;
  // this chunk's steps [it_lo, it_hi) of the block's n_qt * group
  int it_lo = 0, it_hi = n_qt * a.group;
  if (nch > 1) {
    const int per = (it_hi + nch - 1) / nch;
    it_lo = min(it_hi, chunk * per);
    it_hi = min(it_hi, it_lo + per);
  }

  auto stage = [&](int it, int b) {
    const int t0 = (qt_lo + it / a.group) * 32;
    const int head = a.ri.qhead[g * a.group + it % a.group];
    const int valid = a.rows - t0;
    const float* qb = (const float*)a.q + (int64_t)t0 * a.q_st + (int64_t)head * a.q_sh;
    const float* db = (const float*)a.dout + (int64_t)t0 * a.do_st + (int64_t)head * a.do_sh;
    dma_tile<D>(rows_rsrc<D>(qb, valid, a.q_st), qd_s[b][0], 4u * (uint32_t)a.q_st, wave, lane);
    dma_tile<D>(rows_rsrc<D>(db, valid, a.do_st), qd_s[b][1], 4u * (uint32_t)a.do_st, wave, lane);
    if (wave == kWaves - 1)
      dma_vec(make_rsrc(a.lse + (int64_t)head * a.rows + t0, 4LL * valid), ld_s[b][0], lane);
    if (wave == kWaves - 2)
      dma_vec(make_rsrc(a.neg_dsum + (int64_t)head * a.rows + t0, 4LL * valid), ld_s[b][1], lane);
  };

  f32x4 dk[NTD], dv[NTD];   // dK^T, dV^T: register r is head_dim 16 dt + 4 g + r
#pragma unroll
  for (int dt = 0; dt < NTD; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = dk[dt];
  }
  const float c = a.scale_log2;
  // the dS buffer (fp32): 32 x 32 tiles [query head][query step][key tile],
  // each row-major over (query, key); own keys from key tile ds_own0 / 32
  float* const dsb = (float*)a.ds_ext;
  const int ds_qt = a.ds_rows / 32, ds_kt = a.ds_keys / 32;
  const int ds_k0 = ext ? 0 : a.ds_own0 / 32;

  if (it_lo < it_hi) stage(it_lo, 0);
  for (int it = it_lo, b = 0; it < it_hi; ++it, b ^= 1) {
    wait_dma();
    __syncthreads();
    if (it + 1 < it_hi) stage(it + 1, b ^ 1);
    const int t0 = (qt_lo + it / a.group) * 32;
    // own keys: the step's rows may see some key of the wave
    if (!ext && (t0 + 31 < kw0 || t0 >= wave_hi)) continue;
    const float* qs = qd_s[b][0];
    const float* ds = qd_s[b][1];
    // S and dP of the two 16-query halves, four independent chains
    f32x4 s[2], dp[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      s[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[hf] = s[hf];
    }
#pragma unroll
    for (int u = 0; u < Q4 / 4; ++u) {
      f32x4 qv[2], dv4[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        qv[hf] = *(const f32x4*)(qs + (16 * hf + j16) * RS + Q4 * g4 + 4 * u);
        dv4[hf] = *(const f32x4*)(ds + (16 * hf + j16) * RS + Q4 * g4 + 4 * u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          s[hf] = mm16(qv[hf][e], kr[4 * u + e], s[hf]);
          dp[hf] = mm16(dv4[hf][e], vr[4 * u + e], dp[hf]);
        }
    }
    // register (hf, r): query row t0 + 16 hf + 4 g + r against the lane's
    // key; P in s, dS in dp
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 lv = *(const f32x4*)(ld_s[b][0] + 16 * hf + 4 * g4);
      const f32x4 ndv = *(const f32x4*)(ld_s[b][1] + 16 * hf + 4 * g4);   // -D
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tq = t0 + 16 * hf + 4 * g4 + r;
        const bool vis = tq < a.rows && kvalid && (ext || (kk <= tq && tq < kend_k));
        // a visible row sees at least this key, so its LSE is finite
        const float p = vis ? exp2_(s[hf][r] * c - lv[r] * kLog2e) : 0.f;
        s[hf][r] = p;
        dp[hf][r] = p * (dp[hf][r] + ndv[r]);
      }
    }
    if (dsb) {
      // this wave's 16 columns of the step's dS tile for the dQ pass: rows are
      // the step's queries, columns the tile's 32 keys (streaming stores, read
      // once later)
      const int head = a.ri.qhead[g * a.group + it % a.group];
      float* tile = dsb + ((int64_t)(head * ds_qt + t0 / 32) * ds_kt + ds_k0 + kw0 / 32) * 1024 +
                    (kw0 & 31) + j16;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_nontemporal_store(dp[hf][r], tile + (16 * hf + 4 * g4 + r) * 32);
    }
#pragma unroll
    for (int dt = 0; dt < NTD; ++dt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int at = (16 * hf + 4 * g4 + r) * RS + 16 * dt + j16;
          dv[dt] = mm16(ds[at], s[hf][r], dv[dt]);
          dk[dt] = mm16(qs[at], dp[hf][r], dk[dt]);
        }
  }

  if (!kvalid) return;
  // Destination: 0 add into gK/gV (an unsplit external block, or the first
  // chunk of a split one: no other workgroup touches those elements in the
  // launch), 1 external partial plane chunk - 1, 2 own partial plane chunk,
  // 3 own output (+ gk_init / gv_init).  The finishing pass adds the planes
  // in a fixed order, so every result is the same run to run.
  // The partial planes are indexed by the key's position among the external
  // keys; gK/gV by its row.
  const int mode = ext ? (chunk == 0 ? 0 : 1) : (nch > 1 ? 2 : 3);
  const int64_t base = ((int64_t)kk * a.hkv + g) * D;
  float* pk = nullptr;
  float* pv = nullptr;
  if (mode == 0) {
    const int64_t abase = ((int64_t)krow * a.hkv + g) * D;
    pk = a.gk_acc + abase;
    pv = a.gv_acc + abase;
  } else if (mode == 1) {
    const int64_t pb = (int64_t)(chunk - 1) * a.n_ext * a.hkv * D + base;
    pk = a.gk_part + pb;
    pv = a.gv_part + pb;
  } else if (mode == 2) {
    const int64_t pb = (int64_t)chunk * a.rows * a.hkv * D + base;
    pk = a.dk_part + pb;
    pv = a.dv_part + pb;
  } else {
    pk = (float*)a.dk_own + (int64_t)kk * a.dko_st + (int64_t)g * a.dko_sh;
    pv = (float*)a.dv_own + (int64_t)kk * a.dvo_st + (int64_t)g * a.dvo_sh;
  }
#pragma unroll
  for (int dt = 0; dt < NTD; ++dt) {
    const int d0 = 16 * dt + 4 * g4;
    f32x4 xk = dk[dt] * a.scale, xv = dv[dt];
    if (mode == 0) {
      xk += *(const f32x4*)(pk + d0);
      xv += *(const f32x4*)(pv + d0);
    } else if (mode == 3 && a.gk_init) {
      xk += *(const f32x4*)(a.gk_init + base + d0);
      xv += *(const f32x4*)(a.gv_init + base + d0);
    }
    *(f32x4*)(pk + d0) = xk;
    *(f32x4*)(pv + d0) = xv;
  }
}

// K tile i of a Q-stationary workgroup into LDS
template <int D>
__device__ __forceinline__ void stage_k(const AttnArgs& a, const QTiles& w, int i, float* k_s,
                                        int wave, int lane) {
  const bool ext = i < w.n_ext_t;
  const int2 kt = key_tile(a, w, i);
  const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
  const float* kb =
      (const float*)(ext ? a.k_ext : a.k_own) + (int64_t)kt.x * kst + (int64_t)w.g * ksh;
  dma_tile<D>(rows_rsrc<D>(kb, kt.y, kst), k_s, 4u * (uint32_t)kst, wave, lane);
}

// dQ from the stored dS: Q-stationary like dq_f32_kernel, over the same key
// tiles, with dQ^T += K^T dS^T and dS^T read from the buffer instead of
// recomputed.  A lane's 16 values of a tile (its query's row, keys crow(s, h))
// are four 16-byte loads, issued one tile ahead.  Every tile a wave reads is
// one the dK/dV pass wrote: both skip exactly the own tiles none of the wave's
// rows can see, and the entries of invisible pairs are zero.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void dq_ds_f32_kernel(AttnArgs a) {
  constexpr int NT = D / 32, RS = Tile<D>::kRs;
  __shared__ __attribute__((aligned(16))) float k_s[2][Tile<D>::kFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const QTiles w(a, wave, col, a.n_ext > 0);
  const float* const dsb = (const float*)a.ds_ext;
  const int64_t row_tiles = (int64_t)(w.head * (a.ds_rows / 32) + w.t0 / 32) * (a.ds_keys / 32);
  auto load_ds = [&](int i, f32x4 (&dst)[4]) {
    const int kt = i < w.n_ext_t ? i : a.ds_own0 / 32 + (i - w.n_ext_t);
    const float* t = dsb + (row_tiles + kt) * 1024 + col * 32 + 4 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = __builtin_nontemporal_load((const f32x4*)(t + 8 * j));
  };

  f32x16 dq[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) dq[dt] = zero16();
  f32x4 cur[4], nxt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cur[j] = nxt[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int ci = w.live(a, 0) ? 0 : w.next(a, 0);
  if (ci >= 0) {
    stage_k<D>(a, w, ci, k_s[0], wave, lane);
    if (w.wave_sees(a, ci)) load_ds(ci, cur);
  }
  for (int b = 0; ci >= 0; b ^= 1) {
    const int ni = w.next(a, ci);
    wait_dma();
    __syncthreads();
    if (ni >= 0) {
      stage_k<D>(a, w, ni, k_s[b ^ 1], wave, lane);
      if (w.wave_sees(a, ni)) load_ds(ni, nxt);
    }
    if (w.wave_sees(a, ci)) {
      const float* ks = k_s[b];
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
          dq[dt] = mm(ks[crow(s2, h) * RS + 32 * dt + col], cur[s2 >> 2][s2 & 3], dq[dt]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
    ci = ni;
  }

  if (!w.tvalid) return;
  float* op = (float*)a.out + (int64_t)w.tok * a.out_st + (int64_t)w.head * a.out_sh;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = dq[dt][4 * q4 + e] * a.scale;
      *(f32x4*)(op + 32 * dt + 8 * q4 + 4 * h) = v;
    }
}

// Q-stationary grid: per KV head, one workgroup per 4 (tile, query head) pairs,
// the heads interleaved (see QTiles)
dim3 q_grid(const AttnArgs& a) {
  const int pairs = ((a.rows + 31) / 32) * a.group;
  return dim3((unsigned)(((pairs + kWaves - 1) / kWaves) * a.hkv));
}

dim3 q_grid_head_major(const AttnArgs& a) {
  const int pairs = ((a.rows + 31) / 32) * a.group;
  return dim3((pairs + kWaves - 1) / kWaves, a.hkv);
}

}  // namespace

hipError_t launch_fwd_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (head_dim == 64)
    PF_LAUNCH("pf_fwd_f32", fwd_f32_kernel<64>, q_grid(a), dim3(kThreads), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_fwd_f32", fwd_f32_kernel<128>, q_grid(a), dim3(kThreads), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (head_dim == 64)
    PF_LAUNCH("pf_bwd_dq_f32", dq_f32_kernel<64>, q_grid(a), dim3(kThreads), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_bwd_dq_f32", dq_f32_kernel<128>, q_grid(a), dim3(kThreads), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds_f32(const AttnArgs& a, const PartialSums& ps, int32_t head_dim,
                                hipStream_t stream) {
  if (a.rows > 0) {
    // measured at the config-2 shape in fp32: with external keys (Phase B)
    // the heads one after another read the dS stream faster (1.25 against
    // 1.45 ms); without (Phase C) one head per XCD does (0.76 against 1.02)
    const dim3 grid = a.n_ext > 0 ? q_grid_head_major(a) : q_grid(a);
    if (head_dim == 64)
      PF_LAUNCH("pf_bwd_dq_ds_f32", dq_ds_f32_kernel<64>, grid, dim3(kThreads), stream, a);
    else if (head_dim == 128)
      PF_LAUNCH("pf_bwd_dq_ds_f32", dq_ds_f32_kernel<128>, grid, dim3(kThreads), stream, a);
    else
      return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_partial_sums(ps, stream);
}

int32_t dkv_keys_per_workgroup_f32() { return kDkvKeys; }

hipError_t launch_bwd_dkv_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  const int blocks = (a.n_ext + kDkvKeys - 1) / kDkvKeys * a.n_chunks +
                     (a.rows + kDkvKeys - 1) / kDkvKeys * a.n_chunks_own;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)(blocks * a.hkv));
  if (head_dim == 64)
    PF_LAUNCH("pf_bwd_dkv_f32", dkv_f32_kernel<64>, grid, dim3(kThreads), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_bwd_dkv_f32", dkv_f32_kernel<128>, grid, dim3(kThreads), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pf
