// Compact log-probability recovery ("HARTS: A Prefix-Sharing Training System
// for Agentic RL with Hybrid-Attention Models", §3.5, "Compact log-probability
// recovery").  Logits exist once per compact row (C x V); every semantic
// position s reads its row m(s) and target y_s:
//
//   forward   lse_c = log sum_v exp z[c, v];   logp_s = z[m(s), y_s] - lse_m(s)
//   backward  dz[c, v] = sum over s in row c of dlogp_s (1[v = y_s] - exp(z[c, v] - lse_c))
//
// so both directions stream C x V once or twice and never form S x V.
// Positions come grouped by row: pos[row_ptr[c] .. row_ptr[c + 1]) (device).
//
// Forward: one workgroup per compact row; backward: one per chunk of a row
// (the softmax needs only the row's lse and gradient sum); 256 threads,
// 16-byte loads, the HBM stream of the logits is the bound.  Index arrays live on the device, so the kernels
// check every index against its range and skip what falls outside (a position
// with an out-of-range target gets NaN); nothing is read or written out of
// bounds.  No atomics: the row sums are fixed-order reductions and each dz
// element is written by one thread (target columns are rewritten, by the
// workgroup of their chunk after a barrier, with their position terms added in
// position order).
#include <float.h>
#include <math.h>

#include "pf_internal.h"

namespace pf {
namespace {

constexpr int kLpThreads = 256;
// target 8-column vectors per backward workgroup.  Measured on 12288 rows of
// 151936 bf16 logits: 768 (three vectors a thread) streams 5.9 TB/s; 512 loses
// to each workgroup's set-up, 1024 to 8192 lose 2 to 10 % as fewer, longer
// workgroups spread their streams over more rows at once.
constexpr int kLpBwdChunkVec = 768;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// eight consecutive logits of a row as fp32 (16 bytes of bf16 or two 16-byte
// fp32 loads)
template <bool BF16>
__device__ __forceinline__ void load8(const char* row, int v0, float (&x)[8]) {
  if constexpr (BF16) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 w = *(const bf16x8*)(row + 2 * (int64_t)v0);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)w[e];
  } else {
    const float4 a = *(const float4*)(row + 4 * (int64_t)v0);
    const float4 b = *(const float4*)(row + 4 * (int64_t)v0 + 16);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// the 16 (bf16) or 32 (fp32) raw bytes of eight consecutive logits, loaded
// ahead of their use and converted later (raw keeps the bf16 form in 4 VGPRs).
// Streaming (non-temporal) loads: each logit is read once per kernel, and
// keeping the stream out of the caches' normal replacement measured 6.0 ->
// 6.8 TB/s for the forward on 12288 x 151936 bf16.
template <bool BF16>
struct Raw8 {
  uint4 w[BF16 ? 1 : 2];
};
__device__ __forceinline__ uint4 load16_nt(const char* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t[0], t[1], t[2], t[3]);
}
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const char* row, int v0) {
  Raw8<BF16> r;
  if constexpr (BF16) {
    r.w[0] = load16_nt(row + 2 * (int64_t)v0);
  } else {
    r.w[0] = load16_nt(row + 4 * (int64_t)v0);
    r.w[1] = load16_nt(row + 4 * (int64_t)v0 + 16);
  }
  return r;
}
// the U vectors v0 + u * kLpThreads (u < U) of a group, the ones at or past
// nvec left unloaded
template <bool BF16, int U>
__device__ __forceinline__ void load_group(const char* row, int v0, int nvec, Raw8<BF16> (&r)[U]);

template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float (&x)[8]) {
  if constexpr (BF16) {
    const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(u[k] << 16);
      x[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  } else {
    const uint4 a = r.w[0], b = r.w[1];
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
    x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
    x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  }
}

template <bool BF16, int U>
__device__ __forceinline__ void load_group(const char* row, int v0, int nvec, Raw8<BF16> (&r)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (v0 + u * kLpThreads < nvec) r[u] = load_raw8<BF16>(row, 8 * (v0 + u * kLpThreads));
}

template <bool BF16>
__device__ __forceinline__ float load1(const char* row, int v) {
  if constexpr (BF16) return (float)*(const __bf16*)(row + 2 * (int64_t)v);
  return *(const float*)(row + 4 * (int64_t)v);
}

template <bool BF16>
__device__ __forceinline__ void store1(char* row, int v, float x) {
  if constexpr (BF16) *(__bf16*)(row + 2 * (int64_t)v) = (__bf16)x;
  else *(float*)(row + 4 * (int64_t)v) = x;
}

// eight results as one streaming (non-temporal) store: dz is written once and
// not read again by this kernel
template <bool BF16>
__device__ __forceinline__ void store8_nt(char* row, int v0, const float (&x)[8]) {
  if constexpr (BF16) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (__bf16)x[e];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w), (u32x4*)(row + 2 * (int64_t)v0));
  } else {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4*)(row + 4 * (int64_t)v0));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]},
                                (f32x4*)(row + 4 * (int64_t)v0 + 16));
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(char* row, int v0, const float (&x)[8]) {
  if constexpr (BF16) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    bf16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (__bf16)x[e];
    *(bf16x8*)(row + 2 * (int64_t)v0) = w;
  } else {
    *(float4*)(row + 4 * (int64_t)v0) = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(row + 4 * (int64_t)v0 + 16) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// (m, l) of a running log-sum-exp in log2 units: the sum is l * 2^m
struct Lse2 {
  float m, l;
};
__device__ __forceinline__ Lse2 lse_merge(Lse2 a, Lse2 b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return Lse2{m, 0.f};
  return Lse2{m, a.l * fexp2(a.m - m) + b.l * fexp2(b.m - m)};
}

// Adds the U vectors r (valid: the first n_valid of them) to the running
// log-sum-exp acc of this thread (log2 units).  The running maximum moves
// only when a value exceeds it by more than kLpRescale (then the sum is
// rescaled once), so each logit costs one exponential, and every term stays
// below 2^kLpRescale.  The raw vectors are converted twice (once for the
// maximum, once for the sum) rather than held as U x 8 floats.
constexpr float kLpRescale = 8.0f;
template <bool BF16, int U>
__device__ __forceinline__ void lse_add(Lse2& acc, const Raw8<BF16> (&r)[U], int n_valid) {
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < n_valid) {
      float x[8];
      unpack8<BF16>(r[u], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, x[e]);
    }
  }
  m *= kLog2e;
  if (m > acc.m + kLpRescale) {
    acc.l *= fexp2(acc.m - m);   // 0 while acc.m is still -FLT_MAX
    acc.m = m;
  }
  float l = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < n_valid) {
      float x[8];
      unpack8<BF16>(r[u], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) l += fexp2(fmaf(x[e], kLog2e, -acc.m));
    }
  }
  acc.l += l;
}

// log-sum-exp (natural log) of one row, every thread of the workgroup
template <bool BF16>
__device__ float row_lse(const char* row, int vocab, float* red) {
  // -FLT_MAX, not -inf, so that a row of -inf logits sums to 0 without NaN
  Lse2 acc{-FLT_MAX, 0.f};
  const int nvec = vocab / 8;
  constexpr int U = 4;   // vectors per group; the next group's loads are issued first
  constexpr int G = U * kLpThreads;
  // two register sets in turn, each refilled with the group two ahead as
  // soon as its own group is summed
  auto add_group = [&](const Raw8<BF16>(&r)[U], int i) {
    lse_add<BF16, U>(acc, r, (nvec - i + kLpThreads - 1) / kLpThreads);
  };
  Raw8<BF16> ra[U], rb[U];
  load_group<BF16, U>(row, threadIdx.x, nvec, ra);
  load_group<BF16, U>(row, threadIdx.x + G, nvec, rb);
  for (int i = threadIdx.x; i < nvec; i += 2 * G) {
    add_group(ra, i);
    if (i + 2 * G < nvec) load_group<BF16, U>(row, i + 2 * G, nvec, ra);
    if (i + G < nvec) {
      add_group(rb, i + G);
      if (i + 3 * G < nvec) load_group<BF16, U>(row, i + 3 * G, nvec, rb);
    }
  }
  for (int v = 8 * nvec + threadIdx.x; v < vocab; v += kLpThreads) {
    const float m = load1<BF16>(row, v) * kLog2e;
    acc = lse_merge(acc, Lse2{m, 1.f});
  }
  // fixed-order reduction: within the wave, then the four waves in order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Lse2 o{__shfl_xor(acc.m, off), __shfl_xor(acc.l, off)};
    acc = lse_merge(acc, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[2 * wave] = acc.m;
    red[2 * wave + 1] = acc.l;
  }
  __syncthreads();
  Lse2 t = lse_merge(lse_merge(Lse2{red[0], red[1]}, Lse2{red[2], red[3]}),
                     lse_merge(Lse2{red[4], red[5]}, Lse2{red[6], red[7]}));
  __syncthreads();
  return (t.m + __log2f(t.l)) * kLn2;
}

struct LpArgs {
  int32_t n_rows, vocab, n_pos;
  const char* z;
  int64_t z_stride_b;      // bytes between rows of z
  char* dz;
  int64_t dz_stride_b;
  const int32_t* row_ptr;  // [n_rows + 1]
  const int32_t* pos;      // [n_pos]
  const int32_t* y;        // [n_pos], indexed by position
  float* lse;              // [n_rows]
  float* logp;             // [n_pos]
  const float* dlogp;      // [n_pos]
};

// this row's slice of pos[], clipped to the array
__device__ __forceinline__ void row_range(const LpArgs& a, int c, int& b, int& e) {
  b = min(max(a.row_ptr[c], 0), a.n_pos);
  e = min(max(a.row_ptr[c + 1], b), a.n_pos);
}

template <bool BF16>
__global__ __launch_bounds__(kLpThreads) void logprob_fwd_kernel(LpArgs a) {
  __shared__ float red[8];
  const int c = blockIdx.x;
  const char* row = a.z + (int64_t)c * a.z_stride_b;
  const float lse = row_lse<BF16>(row, a.vocab, red);
  if (threadIdx.x == 0) a.lse[c] = lse;
  int b, e;
  row_range(a, c, b, e);
  for (int i = b + threadIdx.x; i < e; i += kLpThreads) {
    const int p = a.pos[i];
    if (p < 0 || p >= a.n_pos) continue;
    const int t = a.y[p];
    a.logp[p] = (t >= 0 && t < a.vocab) ? load1<BF16>(row, t) - lse : NAN;
  }
}

// Backward, one workgroup per chunk of a row: chunk k of row c covers the
// 8-column vectors [k * chunk_vec, min(nvec, (k + 1) * chunk_vec)) (the last
// chunk also the columns past the last whole vector).  Chunks of one row are
// adjacent in dispatch order, so the workgroups in flight stream a window of
// consecutive rows, as a plain elementwise pass does.
template <bool BF16>
__global__ __launch_bounds__(kLpThreads) void logprob_bwd_kernel(LpArgs a, int32_t chunk_vec,
                                                                 int32_t n_chunks) {
  const int c = blockIdx.x / n_chunks;
  const int k = blockIdx.x - c * n_chunks;
  const char* row = a.z + (int64_t)c * a.z_stride_b;
  char* drow = a.dz + (int64_t)c * a.dz_stride_b;
  const int nvec = a.vocab / 8;
  const int v_lo = k * chunk_vec;
  const int v_hi = min(nvec, v_lo + chunk_vec);
  const bool last = k == n_chunks - 1;
  // the first two groups of logits are requested before anything else: they
  // do not depend on the position gradients
  constexpr int U = 4;
  constexpr int G = U * kLpThreads;
  Raw8<BF16> ra[U], rb[U];
  load_group<BF16, U>(row, v_lo + threadIdx.x, v_hi, ra);
  load_group<BF16, U>(row, v_lo + G + threadIdx.x, v_hi, rb);
  int b, e;
  row_range(a, c, b, e);
  // g = sum of the row's position gradients (valid positions and targets),
  // summed by every wave on its own in the same order: no barrier
  const int lane = threadIdx.x & 63;
  float part = 0.f;
  for (int i = b + lane; i < e; i += 64) {
    const int p = a.pos[i];
    if (p < 0 || p >= a.n_pos) continue;
    const int t = a.y[p];
    if (t >= 0 && t < a.vocab) part += a.dlogp[p];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  const float g = part;
  const float lse2 = a.lse[c] * kLog2e;
  // dense part: dz = -g softmax(z) in groups of U vectors per thread, two
  // register sets in turn: a set is refilled with the group two ahead as soon
  // as its own group is written, so the other set's loads stay in flight
  auto softmax_grad = [&](const Raw8<BF16>(&r)[U], int i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u * kLpThreads < v_hi) {
        float x[8];
        unpack8<BF16>(r[u], x);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = -g * fexp2(fmaf(x[q], kLog2e, -lse2));
        store8_nt<BF16>(drow, 8 * (i + u * kLpThreads), x);
      }
    }
  };
  for (int i = v_lo + threadIdx.x; i < v_hi; i += 2 * G) {
    softmax_grad(ra, i);
    if (i + 2 * G < v_hi) load_group<BF16, U>(row, i + 2 * G, v_hi, ra);
    if (i + G < v_hi) {
      softmax_grad(rb, i + G);
      if (i + 3 * G < v_hi) load_group<BF16, U>(row, i + 3 * G, v_hi, rb);
    }
  }
  if (last)
    for (int v = 8 * nvec + threadIdx.x; v < a.vocab; v += kLpThreads)
      store1<BF16>(drow, v, -g * fexp2(fmaf(load1<BF16>(row, v), kLog2e, -lse2)));
  __syncthreads();   // the dense stores above, then the target columns again
  // target columns of this chunk: the first position of each distinct target
  // rewrites it with every position term of that target added in position order
  const int col_lo = 8 * v_lo, col_hi = last ? a.vocab : 8 * v_hi;
  for (int i = b + threadIdx.x; i < e; i += kLpThreads) {
    const int p = a.pos[i];
    if (p < 0 || p >= a.n_pos) continue;
    const int t = a.y[p];
    if (t < col_lo || t >= col_hi) continue;
    bool first = true;
    for (int j = b; j < i && first; ++j) {
      const int pj = a.pos[j];
      if (pj >= 0 && pj < a.n_pos && a.y[pj] == t) first = false;
    }
    if (!first) continue;
    float val = -g * fexp2(fmaf(load1<BF16>(row, t), kLog2e, -lse2));
    for (int j = i; j < e; ++j) {
      const int pj = a.pos[j];
      if (pj >= 0 && pj < a.n_pos && a.y[pj] == t) val += a.dlogp[pj];
    }
    store1<BF16>(drow, t, val);
  }
}

}  // namespace

hipError_t launch_logprob_fwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride_b,
                              int32_t bf16, const int32_t* row_ptr, const int32_t* pos,
                              const int32_t* y, int32_t n_pos, float* lse, float* logp,
                              hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  LpArgs a{n_rows, vocab, n_pos, (const char*)z, z_stride_b, nullptr, 0, row_ptr, pos, y, lse,
           logp, nullptr};
  if (bf16)
    PF_LAUNCH("pf_logprob_fwd", logprob_fwd_kernel<true>, dim3(n_rows), dim3(kLpThreads), stream, a);
  else
    PF_LAUNCH("pf_logprob_fwd", logprob_fwd_kernel<false>, dim3(n_rows), dim3(kLpThreads), stream, a);
  return hipGetLastError();
}

hipError_t launch_logprob_bwd(int32_t n_rows, int32_t vocab, const void* z, int64_t z_stride_b,
                              int32_t bf16, const float* lse, const int32_t* row_ptr,
                              const int32_t* pos, const int32_t* y, int32_t n_pos,
                              const float* dlogp, void* dz, int64_t dz_stride_b,
                              hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  LpArgs a{n_rows, vocab, n_pos, (const char*)z, z_stride_b, (char*)dz, dz_stride_b, row_ptr, pos,
           y, const_cast<float*>(lse), nullptr, dlogp};
  // chunks of about kLpBwdChunkVec vectors (12 KB of bf16), equal in size and
  // a whole number of vectors per thread
  const int nvec = vocab / 8;
  const int n_chunks = max(1, (nvec + kLpBwdChunkVec - 1) / kLpBwdChunkVec);
  const int per = (nvec + n_chunks - 1) / n_chunks;
  const int chunk_vec = max(kLpThreads, (per + kLpThreads - 1) / kLpThreads * kLpThreads);
  const int64_t blocks = (int64_t)n_rows * n_chunks;
  if (blocks > INT32_MAX / kLpThreads) return hipErrorInvalidValue;
  if (bf16)
    PF_LAUNCH("pf_logprob_bwd", logprob_bwd_kernel<true>, dim3((uint32_t)blocks), dim3(kLpThreads),
              stream, a, chunk_vec, n_chunks);
  else
    PF_LAUNCH("pf_logprob_bwd", logprob_bwd_kernel<false>, dim3((uint32_t)blocks), dim3(kLpThreads),
              stream, a, chunk_vec, n_chunks);
  return hipGetLastError();
}

}  // namespace pf
