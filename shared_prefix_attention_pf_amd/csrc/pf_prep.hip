// Small device kernels around the attention kernels:
//   - prep: per-row kend[] and its 32-key block min/max from the segment table;
//   - partial sums, one launch: gK/gV accumulator += the later query chunks'
//     partials of split prefix key blocks, in a fixed pairwise order
//     (contention-free and run-to-run deterministic; this is the per-suffix
//     accumulation of PrefixFlow §3.1 "Savings over the baseline", an
//     element-wise O(|P| d) add), and dK/dV of split own key blocks = init +
//     sum of their partials, converted to the output dtype;
//   - D = rowsum(dO * O), stored negated, and LSE in log2 units for the
//     backward passes;
//   - zero fill and fp32 -> output conversion for Phase C with no upstream.
#include <math.h>

#include "pf_internal.h"
#include "pf_partials.h"

namespace pf {

// thread t of the prep grid (block `blk`)
__device__ __forceinline__ void prep_body(const SegTable& seg, const HeadTable& heads,
                                          const RowInfo& ri, int blk) {
  const int rows = seg.start[seg.n];
  const int t = blk * blockDim.x + threadIdx.x;
  if (t < heads.n) ri.qhead[t] = heads.qhead[t];
  int kend = -1;          // rows past the end: ignored by both summaries
  if (t < rows) {
    // segment of row t: the last i with start[i] <= t (empty segments skipped)
    int lo = 0, hi = seg.n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg.start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    kend = seg.vis_end[lo];
    ri.kend[t] = kend;
  }
  // 32-key block summaries: lanes [32b, 32b+32) of the wave hold one block
  int mx = kend;
  int mn = (t < rows) ? kend : 0x7fffffff;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off, 32));
    mn = min(mn, __shfl_xor(mn, off, 32));
  }
  if ((threadIdx.x & 31) == 0 && t < rows) {
    ri.bmax[t >> 5] = mx;
    ri.bmin[t >> 5] = mn;
  }
}

__global__ __launch_bounds__(256) void prep_kernel(SegTable seg, HeadTable heads, RowInfo ri) {
  prep_body(seg, heads, ri, blockIdx.x);
}

static int prep_blocks(const SegTable& seg, const HeadTable& heads) {
  return (max(seg.start[seg.n], heads.n) + 255) / 256;
}

hipError_t launch_prep(const SegTable& seg, const HeadTable& heads, RowInfo ri,
                       hipStream_t stream) {
  const int rows = seg.start[seg.n];
  if (rows <= 0) return hipSuccess;
  PF_LAUNCH("pf_prep", prep_kernel, dim3(prep_blocks(seg, heads)), dim3(256), stream, seg, heads,
            ri);
  return hipGetLastError();
}

// One thread per virtual tile of 32 external keys: the range holding it (the
// last i with vt0[i] <= t) and, from the tile's offset in that range, its
// first row and valid rows.
__global__ __launch_bounds__(256) void ext_tiles_kernel(RangeTable rt, int2* tiles) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rt.vt0[rt.n]) return;
  int lo = 0, hi = rt.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rt.vt0[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int off = 32 * (t - rt.vt0[lo]);
  tiles[t] = make_int2(rt.start[lo] + off, min(32, rt.len[lo] - off));
}

hipError_t launch_ext_tiles(const RangeTable& rt, int2* tiles, hipStream_t stream) {
  const int n = rt.vt0[rt.n];
  if (n <= 0) return hipSuccess;
  PF_LAUNCH("pf_ext_tiles", ext_tiles_kernel, dim3((n + 255) / 256), dim3(256), stream, rt, tiles);
  return hipGetLastError();
}

// D and LSE (log2) per (row, query head): 16 lanes per pair, each lane
// reading D / 16 head_dim values of dO and O in 16-byte loads; a 16-lane group
// covers kDsumPairs consecutive pairs, all of whose loads are issued before
// the first product so that enough bytes are in flight to stream from HBM;
// block `blk` covers 16 kDsumPairs pairs.
constexpr int kDsumPairs = 4;
template <typename T, int D>
__device__ __forceinline__ void dsum_body(const AttnArgs& a, int blk) {
  constexpr int PER = D / 16;                  // values per lane
  constexpr int VEC = 16 / (int)sizeof(T);     // values per 16-byte load
  constexpr int NV = PER / VEC;                // loads per lane per tensor
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  static_assert(NV * VEC == PER, "head_dim / 16 values per lane in whole 16-byte loads");
  const int sub = threadIdx.x & 15;
  const int64_t n = (int64_t)a.rows * a.hq;
  const int64_t p0 = ((int64_t)blk * 16 + (threadIdx.x >> 4)) * kDsumPairs;
  vec_t dv[kDsumPairs][NV], ov[kDsumPairs][NV];
  int hh[kDsumPairs], tt[kDsumPairs];
#pragma unroll
  for (int u = 0; u < kDsumPairs; ++u) {
    const int64_t pc = p0 + u < n ? p0 + u : n - 1;
    hh[u] = (int)(pc / a.rows);
    tt[u] = (int)(pc - (int64_t)hh[u] * a.rows);
    const T* dp = (const T*)a.dout + (int64_t)tt[u] * a.do_st + (int64_t)hh[u] * a.do_sh + PER * sub;
    const T* op = (const T*)a.o + (int64_t)tt[u] * a.o_st + (int64_t)hh[u] * a.o_sh + PER * sub;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      dv[u][v] = *(const vec_t*)(dp + VEC * v);
      ov[u][v] = *(const vec_t*)(op + VEC * v);
    }
  }
#pragma unroll
  for (int u = 0; u < kDsumPairs; ++u) {
    float dot = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < VEC; ++e) dot = fmaf((float)dv[u][v][e], (float)ov[u][v][e], dot);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 16);
    if (sub == 0 && p0 + u < n) {
      const int64_t i = (int64_t)hh[u] * a.rows + tt[u];
      const float l = a.lse[i];
      a.neg_dsum[i] = -dot;
      a.lse2[i] = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
    }
  }
}

// the prep grid followed by the D/LSE grid, in one launch (neither reads
// what the other writes)
template <typename T, int D>
__global__ __launch_bounds__(256) void prep_dsum_kernel(SegTable seg, HeadTable heads, RowInfo ri,
                                                        AttnArgs a, int n_prep) {
  if ((int)blockIdx.x < n_prep)
    prep_body(seg, heads, ri, blockIdx.x);
  else
    dsum_body<T, D>(a, blockIdx.x - n_prep);
}

template <typename T, int D>
static hipError_t launch_prep_dsum(const SegTable& seg, const HeadTable& heads, const AttnArgs& a,
                                   hipStream_t stream) {
  const int64_t n = (int64_t)a.rows * a.hq;
  if (n <= 0) return hipSuccess;
  const int np = prep_blocks(seg, heads);
  const int64_t per_blk = 16 * kDsumPairs;
  PF_LAUNCH("pf_prep_dsum", (prep_dsum_kernel<T, D>),
            dim3((unsigned)(np + (n + per_blk - 1) / per_blk)), dim3(256), stream, seg, heads,
            a.ri, a, np);
  return hipGetLastError();
}

hipError_t launch_prep_dsum_bf16(const SegTable& seg, const HeadTable& heads, const AttnArgs& a,
                                 hipStream_t stream) {
  return launch_prep_dsum<__bf16, 128>(seg, heads, a, stream);
}

hipError_t launch_prep_dsum_f32(const SegTable& seg, const HeadTable& heads, const AttnArgs& a,
                                int32_t head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_prep_dsum<float, 64>(seg, heads, a, stream);
  if (head_dim == 128) return launch_prep_dsum<float, 128>(seg, heads, a, stream);
  return hipErrorInvalidValue;
}

// Sums of the split key blocks' partial planes (PartialSums); blockIdx.y + y0
// selects the array.
__global__ __launch_bounds__(256) void partial_sums_kernel(PartialSums ps, int y0) {
  partial_sums_block(ps, (int)blockIdx.y + y0, (int)blockIdx.x, (int)gridDim.x);
}

hipError_t launch_partial_sums(const PartialSums& ps, hipStream_t stream) {
  int nbx, ny, y0;
  partial_sums_grid(ps, nbx, ny, y0);
  if (ny == 0) return hipSuccess;
  PF_LAUNCH("pf_partials", partial_sums_kernel, dim3((unsigned)nbx, (unsigned)ny), dim3(256),
            stream, ps, y0);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(char* dst, int64_t rows, int heads,
                                                        int row_bytes, int64_t st_b,
                                                        int64_t sh_b) {
  // one thread per 16 bytes of one (row, head) vector
  const int per = row_bytes / 16;
  const int64_t total = rows * heads * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % per);
    const int64_t rh = i / per;
    const int h = (int)(rh % heads);
    const int64_t r = rh / heads;
    *(uint4*)(dst + r * st_b + h * sh_b + c * 16) = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_fill_zero(void* dst, int64_t rows, int32_t heads, int32_t d, int64_t st,
                            int64_t sh, int32_t elem_bytes, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t total = rows * heads * (d * elem_bytes / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  PF_LAUNCH("pf_fill_zero", fill_zero_kernel, dim3((unsigned)blocks), dim3(256), stream, (char*)dst,
                     rows, (int)heads, (int)(d * elem_bytes), st * elem_bytes, sh * elem_bytes);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void convert_acc_kernel(const float4* __restrict__ src,
                                                          char* dst, int64_t rows, int heads,
                                                          int d, int64_t st, int64_t sh,
                                                          int dst_f32) {
  const int per = d / 4;
  const int64_t total = rows * heads * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int c = (int)(i % per);
    const int64_t rh = i / per;
    const int h = (int)(rh % heads);
    const int64_t r = rh / heads;
    const float4 v = src[i];
    const int64_t off = r * st + (int64_t)h * sh + c * 4;   // elements
    if (dst_f32) {
      *(float4*)((float*)dst + off) = v;
    } else {
      __bf16* o = (__bf16*)dst + off;
      o[0] = (__bf16)v.x; o[1] = (__bf16)v.y; o[2] = (__bf16)v.z; o[3] = (__bf16)v.w;
    }
  }
}

hipError_t launch_convert_acc(const float* src, void* dst, int64_t rows, int32_t heads, int32_t d,
                              int64_t st, int64_t sh, int32_t dst_f32, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t total = rows * heads * (d / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  PF_LAUNCH("pf_convert_acc", convert_acc_kernel, dim3((unsigned)blocks), dim3(256), stream, (const float4*)src, (char*)dst, rows, (int)heads, (int)d, st, sh,
                     (int)dst_f32);
  return hipGetLastError();
}

}  // namespace pf
