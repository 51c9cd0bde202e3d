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
// One workgroup per compact row, 256 threads, 16-byte loads; the HBM stream of
// the row is the bound.  Index arrays live on the device, so the kernels
// check every index against its range and skip what falls outside (a position
// with an out-of-range target gets NaN); nothing is read or written out of
// bounds.  No atomics: the row sums are fixed-order reductions and each dz
// element is written by one thread (target columns are rewritten, in the same
// workgroup after a barrier, with their position terms added in position
// order).
#include <math.h>

#include "pf_internal.h"

namespace pf {
namespace {

constexpr int kLpThreads = 256;
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

// the workgroup's sum of per-thread values, in a fixed order
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// log-sum-exp (natural log) of one row, every thread of the workgroup
template <bool BF16>
__device__ float row_lse(const char* row, int vocab, float* red) {
  Lse2 acc{-INFINITY, 0.f};
  const int nvec = vocab / 8;
  constexpr int U = 4;   // vectors in flight per thread
  int i = threadIdx.x;
  for (; i + (U - 1) * kLpThreads < nvec; i += U * kLpThreads) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load8<BF16>(row, 8 * (i + u * kLpThreads), x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float m = x[u][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, x[u][e]);
      m *= kLog2e;
      float l = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) l += fexp2(fmaf(x[u][e], kLog2e, -m));
      acc = lse_merge(acc, Lse2{m, l});
    }
  }
  for (; i < nvec; i += kLpThreads) {
    float x[8];
    load8<BF16>(row, 8 * i, x);
    float m = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, x[e]);
    m *= kLog2e;
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) l += fexp2(fmaf(x[e], kLog2e, -m));
    acc = lse_merge(acc, Lse2{m, l});
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

template <bool BF16>
__global__ __launch_bounds__(kLpThreads) void logprob_bwd_kernel(LpArgs a) {
  __shared__ float red[8];
  const int c = blockIdx.x;
  const char* row = a.z + (int64_t)c * a.z_stride_b;
  char* drow = a.dz + (int64_t)c * a.dz_stride_b;
  int b, e;
  row_range(a, c, b, e);
  // g = sum of the row's position gradients (valid positions and targets)
  float part = 0.f;
  for (int i = b + threadIdx.x; i < e; i += kLpThreads) {
    const int p = a.pos[i];
    if (p < 0 || p >= a.n_pos) continue;
    const int t = a.y[p];
    if (t >= 0 && t < a.vocab) part += a.dlogp[p];
  }
  const float g = block_sum(part, red);
  const float lse2 = a.lse[c] * kLog2e;
  // dense part: dz = -g softmax(z), four vectors in flight per thread
  const int nvec = a.vocab / 8;
  constexpr int U = 4;
  int i = threadIdx.x;
  for (; i + (U - 1) * kLpThreads < nvec; i += U * kLpThreads) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load8<BF16>(row, 8 * (i + u * kLpThreads), x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[u][k] = -g * fexp2(fmaf(x[u][k], kLog2e, -lse2));
      store8<BF16>(drow, 8 * (i + u * kLpThreads), x[u]);
    }
  }
  for (; i < nvec; i += kLpThreads) {
    float x[8];
    load8<BF16>(row, 8 * i, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = -g * fexp2(fmaf(x[k], kLog2e, -lse2));
    store8<BF16>(drow, 8 * i, x);
  }
  for (int v = 8 * nvec + threadIdx.x; v < a.vocab; v += kLpThreads)
    store1<BF16>(drow, v, -g * fexp2(fmaf(load1<BF16>(row, v), kLog2e, -lse2)));
  __syncthreads();   // the dense stores above, then the target columns again
  // target columns: the first position of each distinct target rewrites it
  // with every position term of that target added in position order
  for (int i = b + threadIdx.x; i < e; i += kLpThreads) {
    const int p = a.pos[i];
    if (p < 0 || p >= a.n_pos) continue;
    const int t = a.y[p];
    if (t < 0 || t >= a.vocab) continue;
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
  if (bf16)
    PF_LAUNCH("pf_logprob_bwd", logprob_bwd_kernel<true>, dim3(n_rows), dim3(kLpThreads), stream, a);
  else
    PF_LAUNCH("pf_logprob_bwd", logprob_bwd_kernel<false>, dim3(n_rows), dim3(kLpThreads), stream, a);
  return hipGetLastError();
}

}  // namespace pf
