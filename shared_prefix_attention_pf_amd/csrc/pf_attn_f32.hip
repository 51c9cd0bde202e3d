// fp32 attention kernels (head_dim 64 or 128): the same three kernels as the
// bf16 family with fp32 inputs, fp32 products and fp32 accumulation, so fp32
// groups are never rounded to bf16.  One thread owns one query row (forward,
// dQ) or one key row (dK/dV); K/V or Q/dO tiles of 64 rows are staged in LDS
// and read by broadcast.  These kernels serve small fp32 groups; the bf16
// MFMA kernels carry the large workloads.
#include <math.h>

#include "pf_internal.h"

namespace pf {
namespace {

constexpr int kT = 64;   // rows per tile, threads per workgroup

// key block kb (64 keys) of the own rows holds a key visible to a token >= t0
__device__ __forceinline__ bool own_block_live(const AttnArgs& a, int kb, int t0) {
  int m = -1;
  for (int b = 2 * kb; b < 2 * kb + 2 && b * 32 < a.rows; ++b) m = max(m, a.ri.bmax[b]);
  return m > t0;
}

template <int D>
__global__ __launch_bounds__(kT) void fwd_f32_kernel(AttnArgs a) {
  __shared__ float ks[kT][D + 1];
  __shared__ float vs[kT][D + 1];
  __shared__ int kend_s[kT];
  const int head = blockIdx.y;
  // KV head of this query head: position of `head` in the grouped table
  int kvh = 0;
  for (int i = 0; i < a.hq; ++i)
    if (a.ri.qhead[i] == head) kvh = i / a.group;
  const int t0 = blockIdx.x * kT;
  const int tok = t0 + threadIdx.x;
  const bool valid = tok < a.rows;
  const int t1 = min(t0 + kT, a.rows);

  float q[D], o[D];
  const float* qp = (const float*)a.q + (int64_t)tok * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int n_ext_b = (a.n_ext + kT - 1) / kT;
  const int n_own_b = (t1 + kT - 1) / kT;
  for (int blk = 0; blk < n_ext_b + n_own_b; ++blk) {
    const bool ext = blk < n_ext_b;
    const int k0 = (ext ? blk : blk - n_ext_b) * kT;
    if (!ext && !own_block_live(a, blk - n_ext_b, t0)) continue;
    const int klim = ext ? a.n_ext : a.rows;
    const float* kb = (const float*)(ext ? a.k_ext : a.k_own);
    const float* vb = (const float*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    __syncthreads();
    for (int e = threadIdx.x; e < kT * D; e += kT) {
      const int r = e / D, d = e % D, kk = k0 + r;
      ks[r][d] = kk < klim ? kb[(int64_t)kk * kst + (int64_t)kvh * ksh + d] : 0.f;
      vs[r][d] = kk < klim ? vb[(int64_t)kk * vst + (int64_t)kvh * vsh + d] : 0.f;
    }
    if (!ext) kend_s[threadIdx.x] = (k0 + threadIdx.x < a.rows) ? a.ri.kend[k0 + threadIdx.x] : -1;
    __syncthreads();
    for (int r = 0; r < kT; ++r) {
      const int kk = k0 + r;
      bool vis = kk < klim;
      if (!ext) vis = vis && kk <= tok && tok < kend_s[r];
      if (!vis) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[r][d], s);
      s *= a.scale;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);
      const float p = expf(s - mn);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, p * vs[r][d]);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = (float*)a.out + (int64_t)tok * a.out_st + (int64_t)head * a.out_sh;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  a.lse[(int64_t)head * a.rows + tok] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kT) void dq_f32_kernel(AttnArgs a) {
  __shared__ float ks[kT][D + 1];
  __shared__ float vs[kT][D + 1];
  __shared__ int kend_s[kT];
  const int head = blockIdx.y;
  int kvh = 0;
  for (int i = 0; i < a.hq; ++i)
    if (a.ri.qhead[i] == head) kvh = i / a.group;
  const int t0 = blockIdx.x * kT;
  const int tok = t0 + threadIdx.x;
  const bool valid = tok < a.rows;
  const int t1 = min(t0 + kT, a.rows);

  float q[D], dout[D], dq[D];
  float dsum = 0.f;
  const int64_t qo = (int64_t)tok * a.q_st + (int64_t)head * a.q_sh;
  const int64_t doo = (int64_t)tok * a.do_st + (int64_t)head * a.do_sh;
  const int64_t oo = (int64_t)tok * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? ((const float*)a.q)[qo + d] : 0.f;
    dout[d] = valid ? ((const float*)a.dout)[doo + d] : 0.f;
    const float ov = valid ? ((const float*)a.o)[oo + d] : 0.f;
    dsum = fmaf(dout[d], ov, dsum);
    dq[d] = 0.f;
  }
  const float lse = valid ? a.lse[(int64_t)head * a.rows + tok] : 0.f;
  if (valid) a.dsum[(int64_t)head * a.rows + tok] = dsum;

  const int n_ext_b = (a.n_ext + kT - 1) / kT;
  const int n_own_b = (t1 + kT - 1) / kT;
  for (int blk = 0; blk < n_ext_b + n_own_b; ++blk) {
    const bool ext = blk < n_ext_b;
    const int k0 = (ext ? blk : blk - n_ext_b) * kT;
    if (!ext && !own_block_live(a, blk - n_ext_b, t0)) continue;
    const int klim = ext ? a.n_ext : a.rows;
    const float* kb = (const float*)(ext ? a.k_ext : a.k_own);
    const float* vb = (const float*)(ext ? a.v_ext : a.v_own);
    const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
    const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;
    __syncthreads();
    for (int e = threadIdx.x; e < kT * D; e += kT) {
      const int r = e / D, d = e % D, kk = k0 + r;
      ks[r][d] = kk < klim ? kb[(int64_t)kk * kst + (int64_t)kvh * ksh + d] : 0.f;
      vs[r][d] = kk < klim ? vb[(int64_t)kk * vst + (int64_t)kvh * vsh + d] : 0.f;
    }
    if (!ext) kend_s[threadIdx.x] = (k0 + threadIdx.x < a.rows) ? a.ri.kend[k0 + threadIdx.x] : -1;
    __syncthreads();
    if (!valid) continue;
    for (int r = 0; r < kT; ++r) {
      const int kk = k0 + r;
      bool vis = kk < klim;
      if (!ext) vis = vis && kk <= tok && tok < kend_s[r];
      if (!vis) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], ks[r][d], s);
        dp = fmaf(dout[d], vs[r][d], dp);
      }
      const float p = expf(s * a.scale - lse);
      const float ds = p * (dp - dsum);
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, ks[r][d], dq[d]);
    }
  }
  if (!valid) return;
  float* op = (float*)a.out + (int64_t)tok * a.out_st + (int64_t)head * a.out_sh;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = dq[d] * a.scale;
}

// One thread per key of one KV head; external keys (blockIdx.x < n_ext
// blocks) walk every row, own keys the rows [k, kend[k]).
template <int D>
__global__ __launch_bounds__(kT) void dkv_f32_kernel(AttnArgs a) {
  __shared__ float qs[kT][D + 1];
  __shared__ float ds_s[kT][D + 1];
  __shared__ float lse_s[kT];
  __shared__ float dsum_s[kT];
  const int g = blockIdx.y;
  const int n_ext_b = (a.n_ext + kT - 1) / kT;
  const bool ext = (int)blockIdx.x < n_ext_b;
  const int k0 = (ext ? blockIdx.x : blockIdx.x - n_ext_b) * kT;
  const int kk = k0 + threadIdx.x;
  const int klim = ext ? a.n_ext : a.rows;
  const bool kvalid = kk < klim;
  const float* kb = (const float*)(ext ? a.k_ext : a.k_own);
  const float* vb = (const float*)(ext ? a.v_ext : a.v_own);
  const int64_t kst = ext ? a.kx_st : a.ko_st, ksh = ext ? a.kx_sh : a.ko_sh;
  const int64_t vst = ext ? a.vx_st : a.vo_st, vsh = ext ? a.vx_sh : a.vo_sh;

  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    k[d] = kvalid ? kb[(int64_t)kk * kst + (int64_t)g * ksh + d] : 0.f;
    v[d] = kvalid ? vb[(int64_t)kk * vst + (int64_t)g * vsh + d] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int kend = (!ext && kvalid) ? a.ri.kend[kk] : 0;
  int qlo = 0, qhi = a.rows;
  if (!ext) {
    qlo = k0;
    int m = -1;
    for (int b = k0 / 32; b * 32 < min(k0 + kT, a.rows); ++b) m = max(m, a.ri.bmax[b]);
    qhi = min(m, a.rows);
  }
  for (int j = 0; j < a.group; ++j) {
    const int head = a.ri.qhead[g * a.group + j];
    for (int t0 = qlo; t0 < qhi; t0 += kT) {
      __syncthreads();
      for (int e = threadIdx.x; e < kT * D; e += kT) {
        const int r = e / D, d = e % D, tok = t0 + r;
        const bool ok = tok < a.rows;
        qs[r][d] = ok ? ((const float*)a.q)[(int64_t)tok * a.q_st + (int64_t)head * a.q_sh + d]
                      : 0.f;
        ds_s[r][d] = ok ? ((const float*)a.dout)[(int64_t)tok * a.do_st +
                                                 (int64_t)head * a.do_sh + d]
                        : 0.f;
      }
      {
        const int tok = t0 + threadIdx.x;
        const bool ok = tok < a.rows;
        lse_s[threadIdx.x] = ok ? a.lse[(int64_t)head * a.rows + tok] : INFINITY;
        dsum_s[threadIdx.x] = ok ? a.dsum[(int64_t)head * a.rows + tok] : 0.f;
      }
      __syncthreads();
      if (!kvalid) continue;
      for (int r = 0; r < kT; ++r) {
        const int tok = t0 + r;
        if (tok >= a.rows) break;
        if (!ext && !(kk <= tok && tok < kend)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          s = fmaf(qs[r][d], k[d], s);
          dp = fmaf(ds_s[r][d], v[d], dp);
        }
        const float p = expf(s * a.scale - lse_s[r]);
        const float dsv = p * (dp - dsum_s[r]);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dv[d] = fmaf(p, ds_s[r][d], dv[d]);
          dk[d] = fmaf(dsv, qs[r][d], dk[d]);
        }
      }
    }
  }
  if (!kvalid) return;
  const int64_t base = ((int64_t)kk * a.hkv + g) * D;
  if (ext) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      a.gk_acc[base + d] += dk[d] * a.scale;
      a.gv_acc[base + d] += dv[d];
    }
    return;
  }
  float* dkp = (float*)a.dk_own + (int64_t)kk * a.dko_st + (int64_t)g * a.dko_sh;
  float* dvp = (float*)a.dv_own + (int64_t)kk * a.dvo_st + (int64_t)g * a.dvo_sh;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    float x = dk[d] * a.scale, y = dv[d];
    if (a.gk_init) {
      x += a.gk_init[base + d];
      y += a.gv_init[base + d];
    }
    dkp[d] = x;
    dvp[d] = y;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  dim3 grid((a.rows + kT - 1) / kT, a.hq);
  if (head_dim == 64)
    PF_LAUNCH("pf_fwd_f32", fwd_f32_kernel<64>, grid, dim3(kT), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_fwd_f32", fwd_f32_kernel<128>, grid, dim3(kT), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  dim3 grid((a.rows + kT - 1) / kT, a.hq);
  if (head_dim == 64)
    PF_LAUNCH("pf_bwd_dq_f32", dq_f32_kernel<64>, grid, dim3(kT), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_bwd_dq_f32", dq_f32_kernel<128>, grid, dim3(kT), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkv_f32(const AttnArgs& a, int32_t head_dim, hipStream_t stream) {
  const int blocks = (a.n_ext + kT - 1) / kT + (a.rows + kT - 1) / kT;
  if (blocks <= 0) return hipSuccess;
  dim3 grid(blocks, a.hkv);
  if (head_dim == 64)
    PF_LAUNCH("pf_bwd_dkv_f32", dkv_f32_kernel<64>, grid, dim3(kT), stream, a);
  else if (head_dim == 128)
    PF_LAUNCH("pf_bwd_dkv_f32", dkv_f32_kernel<128>, grid, dim3(kT), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pf
