// Shared device helpers for the Talker kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtalk {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef _Float16 f16_t;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int WAVE = 64;
constexpr int MAX_ROWS = 64;  // rows (tokens) described by one RowMeta

// Which (sequence, position) each activation row belongs to.  Prefill and
// extend rows are uniform (one sequence, consecutive positions from p0);
// a batched prefill stacks `per` such rows for each listed sequence;
// batched decode rows carry one (seq, pos) each.
struct RowMeta {
  int n;        // number of rows
  int uniform;  // 1: row t is (seq0, p0 + t); 2: (seq[t / per], p0 + t % per);
                // 0: (seq[t], pos[t])
  int seq0;
  int p0;
  int per;
  int seq[MAX_ROWS];
  int pos[MAX_ROWS];
};

__device__ __forceinline__ int row_seq(const RowMeta& r, int t) {
  return r.uniform == 1 ? r.seq0 : (r.uniform == 2 ? r.seq[t / r.per] : r.seq[t]);
}
__device__ __forceinline__ int row_pos(const RowMeta& r, int t) {
  return r.uniform == 1 ? r.p0 + t : (r.uniform == 2 ? r.p0 + t % r.per : r.pos[t]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Cross-lane reductions on DPP (VALU lane moves, a few cycles each) rather
// than ds_bpermute shuffles, which cost an LDS round trip per step.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum within each row of 16 lanes; every lane receives its row's sum
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0x128>(v);  // row_ror:8
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x122>(v);  // row_ror:2
  v += dpp_mov<0x121>(v);  // row_ror:1
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0x128>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x122>(v));
  v = fmaxf(v, dpp_mov<0x121>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// wave-wide sum / max, the same value in every lane
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// sum within aligned groups of 16 lanes (one DPP row)
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 16, "16-lane groups");
  return row16_sum(v);
}

// block-wide sum for blockDim.x == NT (multiple of 64); `red` holds NT/64 floats
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

// 16-byte streaming load (non-temporal: data read once per pass)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// 16 bytes of weights -> floats
__device__ __forceinline__ void unpack8_bf16(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

}  // namespace qtalk
