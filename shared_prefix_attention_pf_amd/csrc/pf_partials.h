// Device code shared by the partial-sum launch and the dQ pass, which runs the
// same sums as extra workgroups of its own launch.
#pragma once

#include "pf_internal.h"

namespace pf {

// (((p0 + p1) + (p2 + p3)) + ...) over nc partial planes of n4 float4 each (planes past nc are zero).
template <int NC>
__device__ inline float4 tree_sum(const float4* part, int64_t n4, int64_t i, int nc) {
  float4 v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = (c < nc) ? part[c * n4 + i] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 1; w < NC; w <<= 1) {
#pragma unroll
    for (int c = 0; c + w < NC; c += 2 * w) {
      v[c].x += v[c + w].x; v[c].y += v[c + w].y; v[c].z += v[c + w].z; v[c].w += v[c + w].w;
    }
  }
  return v[0];
}

// One block of the sums of the split key blocks' partial planes
// (PartialSums): y selects the array, 0 / 1 external K / V (acc += planes),
// 2 / 3 own dK / dV (dst = convert(init + planes)); block bx of nbx walks
// that array with a grid stride.
__device__ inline void partial_sums_block(const PartialSums& ps, int y, int bx, int nbx) {
  const int64_t stride = (int64_t)nbx * blockDim.x;
  if (y < 2) {
    const float4* __restrict__ part = y ? ps.part_v : ps.part_k;
    float4* __restrict__ acc = y ? ps.acc_v : ps.acc_k;
    const int nc = ps.ext_planes;
    const int64_t n4 = ps.ext_n4;
    for (int64_t i = (int64_t)bx * blockDim.x + threadIdx.x; i < n4; i += stride) {
      float4 s;
      if (nc == 1) s = part[i];
      else if (nc <= 2) s = tree_sum<2>(part, n4, i, nc);
      else if (nc <= 4) s = tree_sum<4>(part, n4, i, nc);
      else s = tree_sum<8>(part, n4, i, nc);
      int64_t ai = i;
      if (ps.ext_tiles) {
        // virtual external row -> accumulator row; padding rows are skipped
        const int64_t vr = i / ps.ext_row4;
        const int2 t = ps.ext_tiles[vr >> 5];
        const int loc = (int)(vr & 31);
        if (loc >= t.y) continue;
        ai = (int64_t)(t.x + loc) * ps.ext_row4 + (i - vr * ps.ext_row4);
      }
      float4 a = acc[ai];
      a.x += s.x; a.y += s.y; a.z += s.z; a.w += s.w;
      acc[ai] = a;
    }
    return;
  }
  const OwnFinish& fo = (y == 3) ? ps.fv : ps.fk;
  const float4* __restrict__ part = fo.part;
  const float4* __restrict__ init = fo.init;
  char* dst = fo.dst;
  const int64_t st = fo.st, sh = fo.sh;
  const int nc = ps.own_planes, heads = ps.heads;
  const int per = ps.d / 4;
  const int64_t n4 = ps.rows * heads * per;
  for (int64_t i = (int64_t)bx * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 v;
    if (nc <= 2) v = tree_sum<2>(part, n4, i, nc);
    else if (nc <= 4) v = tree_sum<4>(part, n4, i, nc);
    else v = tree_sum<8>(part, n4, i, nc);
    if (init) {
      const float4 w = init[i];
      v.x = w.x + v.x; v.y = w.y + v.y; v.z = w.z + v.z; v.w = w.w + v.w;
    }
    const int c = (int)(i % per);
    const int64_t rh = i / per;
    const int h = (int)(rh % heads);
    const int64_t r = rh / heads;
    const int64_t off = r * st + (int64_t)h * sh + c * 4;   // elements
    if (ps.dst_f32) {
      *(float4*)((float*)dst + off) = v;
    } else {
      __bf16* o = (__bf16*)dst + off;
      o[0] = (__bf16)v.x; o[1] = (__bf16)v.y; o[2] = (__bf16)v.z; o[3] = (__bf16)v.w;
    }
  }
}

// blocks per array and number of arrays of a PartialSums launch (ny = 0 when
// there is nothing to sum); y0 is the first array
inline void partial_sums_grid(const PartialSums& ps, int& nbx, int& ny, int& y0) {
  const bool ext = ps.ext_planes > 0 && ps.ext_n4 > 0;
  const bool own = ps.own_planes > 1 && ps.rows > 0;
  nbx = ny = y0 = 0;
  if (!ext && !own) return;
  const int64_t own_n4 = own ? ps.rows * ps.heads * (ps.d / 4) : 0;
  const int64_t n4 = ext && ps.ext_n4 > own_n4 ? ps.ext_n4 : own_n4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  nbx = (int)blocks;
  y0 = ext ? 0 : 2;
  ny = (ext ? 2 : 0) + (own ? 2 : 0);
}

}  // namespace pf
