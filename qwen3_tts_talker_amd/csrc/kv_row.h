// K rows of the key cache (head_dim 128), formed the same way wherever they
// are written: the append kernel and the Q|K|V product's epilogue.
#pragma once

#include "common.h"

namespace qtalk {

// One K row of head_dim 128 formed by a row of 16 lanes: lane i holds dims
// 4i .. 4i+3 in x1 and their NEOX partners 64+4i .. in x2, the gains of
// those dims in g1 / g2 and the (cos, sin) pairs of rotation angles 4i ..
// 4i+3 in c01 (pairs 0, 1) and c23 (pairs 2, 3).  Per-head RMSNorm, gain,
// rotation (Qwen3 attention: RMSNorm on each key head, then RoPE on dim
// pairs (j, j + 64)); x1 / x2 receive the result.  Every operation is
// written out with contraction off, so each kernel that forms K rows this
// way produces the same bits.
__device__ __forceinline__ void k_row_norm_rope(float4& x1, float4& x2, const float4 g1, const float4 g2,
                                                const float4 c01, const float4 c23, float eps) {
#pragma clang fp contract(off)
  float ss = x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
  ss += x2.x * x2.x + x2.y * x2.y + x2.z * x2.z + x2.w * x2.w;
  ss = row16_sum(ss);
  const float inv = rsqrtf(ss / 128.0f + eps);
  const float a1[4] = {x1.x * inv * g1.x, x1.y * inv * g1.y, x1.z * inv * g1.z, x1.w * inv * g1.w};
  const float a2[4] = {x2.x * inv * g2.x, x2.y * inv * g2.y, x2.z * inv * g2.z, x2.w * inv * g2.w};
  const float c[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
  float y1[4], y2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y1[e] = a1[e] * c[e] - a2[e] * sn[e];
    y2[e] = a2[e] * c[e] + a1[e] * sn[e];
  }
  x1 = make_float4(y1[0], y1[1], y1[2], y1[3]);
  x2 = make_float4(y2[0], y2[1], y2[2], y2[3]);
}

}  // namespace qtalk
