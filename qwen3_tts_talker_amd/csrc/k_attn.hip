// Attention-side kernels: per-head QK RMSNorm + NEOX RoPE + KV append, and
// split-KV causal GQA attention over the cache with a log-sum-exp merge.
//
// Semantics: "qwentts.cpp src/talker-forward.h", talker_layer_forward (QK
// norm over head_dim with one [head_dim] gain, NEOX rotate-half RoPE at the
// absolute position, set_rows of K/V into the cache, then attention over the
// cache window with scale 1/sqrt(head_dim) and the causal mask key <= pos);
// "transcribe.cpp src/causal_lm/causal_lm.cpp", block_prefill (query head h
// reads KV head h / (n_heads / n_kv_heads)).  An f32 or f16 cache is read
// after the write, so K/V pass through its storage type.  A Q8_0 cache gives
// the positions of earlier calls dequantised and the call's own rows as
// computed, unquantised ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
// forward_step_cached: the cached prefix cast to F32 joined with the current
// k/v; forward_prefill_cached: attention on the fresh k/v).
#include <type_traits>

#include "kernels.h"
#include "kv_row.h"

namespace qtalk {

// Cache rows: row (seq, kv head, pos) holds head_dim values.  Storage kinds:
// float32, float16, and Q8_0 (q8_t): head_dim int8 codes followed by one
// float16 scale per 32 codes, value = code * scale (blocks of 32 along
// head_dim; "rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
// TalkerKvStorage::TurboQuantQ8_0).  KVIO<T>::load<N>(row, d, f) reads
// values d .. d+N-1 (N divides 32, d a multiple of N) of one row.
struct q8_t {};

template <typename KVT>
struct KVIO;
template <>
struct KVIO<float> {
  static __host__ __device__ constexpr size_t row_bytes(int hd) { return (size_t)hd * 4; }
  template <int N>
  static __device__ __forceinline__ void load(const char* row, int d, float* f) {
    const float* p = reinterpret_cast<const float*>(row) + d;
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + i);
      f[i] = v.x;
      f[i + 1] = v.y;
      f[i + 2] = v.z;
      f[i + 3] = v.w;
    }
  }
};
template <>
struct KVIO<f16_t> {
  static __host__ __device__ constexpr size_t row_bytes(int hd) { return (size_t)hd * 2; }
  template <int N>
  static __device__ __forceinline__ void load(const char* row, int d, float* f) {
    const f16_t* p = reinterpret_cast<const f16_t*>(row) + d;
    if constexpr (N == 8) {
      const f16x8_t v = *reinterpret_cast<const f16x8_t*>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 h4;
        const h4 v = *reinterpret_cast<const h4*>(p + i);
        f[i] = (float)v[0];
        f[i + 1] = (float)v[1];
        f[i + 2] = (float)v[2];
        f[i + 3] = (float)v[3];
      }
    }
  }
};
template <>
struct KVIO<q8_t> {
  static __host__ __device__ constexpr size_t row_bytes(int hd) { return (size_t)hd + (size_t)hd / 16; }
  // values d .. d+N-1 of a row of hd values (the scales follow the codes)
  template <int N>
  static __device__ __forceinline__ void load_hd(const char* row, int hd, int d, float* f) {
    static_assert(N == 4 || N == 8, "4 or 8 codes per load");
    const float sc = (float)*reinterpret_cast<const f16_t*>(row + hd + (d >> 5) * 2);
    if constexpr (N == 8) {
      const uint2 c = *reinterpret_cast<const uint2*>(row + d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = (float)(int8_t)(c.x >> (8 * i)) * sc;
        f[i + 4] = (float)(int8_t)(c.y >> (8 * i)) * sc;
      }
    } else {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(row + d);
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = (float)(int8_t)(c >> (8 * i)) * sc;
    }
  }
};

// values d .. d+N-1 of cache row `row` (head_dim hd) as float
template <typename KVT, int N>
__device__ __forceinline__ void kv_load(const char* row, int hd, int d, float* f) {
  if constexpr (std::is_same<KVT, q8_t>::value) KVIO<q8_t>::template load_hd<N>(row, hd, d, f);
  else KVIO<KVT>::template load<N>(row, d, f);
}

// v[l ^ 16] and v[l ^ 32] combined with v[l] by v_permlane16_swap (odd
// 16-lane rows of one operand with the even rows of the other) and
// v_permlane32_swap (upper half with lower half)
__device__ __forceinline__ float half_xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of each 16-lane row)
__device__ __forceinline__ float xor_sum4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max over each aligned 32-lane half of the wave (DPP inside 16-lane rows,
// then v_permlane16_swap across the row pair)
__device__ __forceinline__ float half32_max(float v) {
  v = row16_max(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// QK-norm + RoPE + append.  grid (rows, n_heads + 2 n_kv), one wave per head.
// Lane i < hd/2 holds the NEOX pair (x_i, x_{i+hd/2}).

template <int HD, typename KVT>
__global__ __launch_bounds__(256) void k_qk_rope_append(QkArgs a) {
  constexpr int HALF = HD / 2;
  // one wave per (row, head) unit, four units per block (a one-wave block per
  // unit left the dispatcher, not memory, setting the pace)
  const int nh = (a.skip_q ? 0 : a.n_heads) + 2 * a.n_kv_heads;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (unit >= a.rows.n * nh) return;  // whole waves: only wave-level reductions below
  const int t = unit / nh, hh = unit % nh + (a.skip_q ? a.n_heads : 0);
  const int nq = a.n_heads, nkv = a.n_kv_heads;
  float* row = a.qkv + (size_t)t * a.ldqkv;
  const int seq = row_seq(a.rows, t), pos = row_pos(a.rows, t);
  int kind, kvh = 0;
  float* x;
  const float* g = nullptr;
  if (hh < nq) {
    kind = 0;
    x = row + hh * HD;
    g = a.g_q;
  } else if (hh < nq + nkv) {
    kind = 1;
    kvh = hh - nq;
    x = row + (nq + kvh) * HD;
    g = a.g_k;
  } else {
    kind = 2;
    kvh = hh - nq - nkv;
    x = row + (nq + nkv + kvh) * HD;
  }
  const bool act = lane < HALF;
  float x1 = act ? x[lane] : 0.f;
  float x2 = act ? x[lane + HALF] : 0.f;
  constexpr bool Q8 = std::is_same<KVT, q8_t>::value;
  if (kind < 2) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float inv = rsqrtf(ss / (float)HD + a.eps);
    if (act) {
      x1 = x1 * inv * g[lane];
      x2 = x2 * inv * g[lane + HALF];
      const float2 cs = a.rope[(size_t)pos * HALF + lane];
      const float y1 = x1 * cs.x - x2 * cs.y;
      const float y2 = x2 * cs.x + x1 * cs.y;
      x1 = y1;
      x2 = y2;
    }
  }
  // Q8_0 blocks: dims d and d + HALF of lane d fall in blocks d / 32 and
  // (d + HALF) / 32, each spanning one aligned 32-lane half of the wave
  float d1 = 0.f, d2 = 0.f;
  if constexpr (Q8) {
    if (kind > 0) {
      d1 = half32_max(fabsf(x1)) / 127.0f;
      d2 = half32_max(fabsf(x2)) / 127.0f;
    }
  }
  if (!act) return;
  // q back in place; with a Q8_0 cache k too, since the attention of this
  // call reads its own rows unquantised from here (v is read as projected)
  if (kind == 0 || (Q8 && kind == 1)) {
    x[lane] = x1;
    x[lane + HALF] = x2;
  }
  if (kind > 0) {
    char* rowp = reinterpret_cast<char*>(kind == 1 ? a.kc : a.vc) +
                 ((size_t)(seq * nkv + kvh) * a.cap + pos) * KVIO<KVT>::row_bytes(HD);
    if constexpr (Q8) {
      const float i1 = d1 > 0.f ? 1.0f / d1 : 0.f, i2 = d2 > 0.f ? 1.0f / d2 : 0.f;
      rowp[lane] = (char)(int8_t)roundf(x1 * i1);
      rowp[lane + HALF] = (char)(int8_t)roundf(x2 * i2);
      f16_t* sc = reinterpret_cast<f16_t*>(rowp + HD);
      if ((lane & 31) == 0) {
        sc[lane >> 5] = (f16_t)d1;
        sc[(lane + HALF) >> 5] = (f16_t)d2;
      }
    } else {
      KVT* c = reinterpret_cast<KVT*>(rowp);
      c[lane] = (KVT)x1;
      c[lane + HALF] = (KVT)x2;
    }
  }
}

template <int HD>
static void launch_qk_hd(KvKind kv, const QkArgs& a, const dim3& grid, hipStream_t st) {
  if (kv == KV_F16) hipLaunchKernelGGL((k_qk_rope_append<HD, f16_t>), grid, dim3(256), 0, st, a);
  else if (kv == KV_Q8) hipLaunchKernelGGL((k_qk_rope_append<HD, q8_t>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_qk_rope_append<HD, float>), grid, dim3(256), 0, st, a);
}

// K/V append only (q left to the matrix-core attention), float16 cache,
// head_dim 128: 16 lanes per (row, head) unit, lane i holding dims 4i..4i+3
// and their NEOX partners 64+4i..; all loads of a lane (x, gains, rotations)
// go out before its two 8-byte stores.  Units: row t, head hh < n_kv (K,
// RMSNorm + RoPE) or the V head hh - n_kv (as is).
__global__ __launch_bounds__(256) void k_kv_append_f16_128(QkArgs a) {
  const int nkv = a.n_kv_heads, nh = 2 * nkv;
  const int unit = blockIdx.x * 16 + (threadIdx.x >> 4), i = threadIdx.x & 15;
  if (unit >= a.rows.n * nh) return;  // whole 16-lane groups: only row16 reductions below
  const int t = unit / nh, hh = unit % nh;
  const bool is_k = hh < nkv;
  const int kvh = is_k ? hh : hh - nkv;
  const float* x = a.qkv + (size_t)t * a.ldqkv + (size_t)(a.n_heads + hh) * 128;
  const int seq = row_seq(a.rows, t), pos = row_pos(a.rows, t);
  float4 x1 = *reinterpret_cast<const float4*>(x + 4 * i);
  float4 x2 = *reinterpret_cast<const float4*>(x + 64 + 4 * i);
  if (is_k) {
    const float4 g1 = *reinterpret_cast<const float4*>(a.g_k + 4 * i);
    const float4 g2 = *reinterpret_cast<const float4*>(a.g_k + 64 + 4 * i);
    const float4 c01 = *reinterpret_cast<const float4*>(a.rope + (size_t)pos * 64 + 4 * i);
    const float4 c23 = *reinterpret_cast<const float4*>(a.rope + (size_t)pos * 64 + 4 * i + 2);
    k_row_norm_rope(x1, x2, g1, g2, c01, c23, a.eps);
  }
  f16_t* row = reinterpret_cast<f16_t*>(is_k ? a.kc : a.vc) + ((size_t)(seq * nkv + kvh) * a.cap + pos) * 128;
  typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
  const f16x4_t o1 = {(f16_t)x1.x, (f16_t)x1.y, (f16_t)x1.z, (f16_t)x1.w};
  const f16x4_t o2 = {(f16_t)x2.x, (f16_t)x2.y, (f16_t)x2.z, (f16_t)x2.w};
  *reinterpret_cast<f16x4_t*>(row + 4 * i) = o1;
  *reinterpret_cast<f16x4_t*>(row + 64 + 4 * i) = o2;
}

void launch_qk_rope_append(KvKind kv, QkArgs a, hipStream_t st) {
  if (kv == KV_F16 && a.skip_q && a.head_dim == 128) {
    const int nh = 2 * a.n_kv_heads;
    hipLaunchKernelGGL(k_kv_append_f16_128, dim3((a.rows.n * nh + 15) / 16), dim3(256), 0, st, a);
    return;
  }
  const int nh = (a.skip_q ? 0 : a.n_heads) + 2 * a.n_kv_heads;
  const dim3 grid((a.rows.n * nh + 3) / 4);
  if (a.head_dim == 128) launch_qk_hd<128>(kv, a, grid, st);
  else launch_qk_hd<64>(kv, a, grid, st);
}

// ---------------------------------------------------------------------------
// Split-KV attention.  grid (n_splits, n_kv, rows), 256 threads (4 waves).
// Block (c, g, t) owns keys [c*kps, min((c+1)*kps, pos+1)) of KV head g for
// row t and serves all G query heads of the group from one read of K and V.
// Lane roles: a slot is one 16-lane row of a wave (16 slots per block), lane
// sub of a slot holds dims sub*DPL .. +DPL.  Slot s of wave w takes keys
// kb + 16u + 4w + s (u < U) of each 16U-key tile, so one wave instruction
// loads 4 consecutive key rows.  Every slot keeps its own online softmax (log2
// units: q carries scale * log2(e)), so the key loop has no cross-slot
// reduction and no barrier; the next tile's rows are loaded (clamped to the
// last key, always a written row) before the current tile's arithmetic.  The
// slots are combined once at the end: within a wave by lane swaps, across the
// 4 waves through LDS.  Partials (o unnormalised, m in log2 units, l) go to
// part_o / part_ml for k_attn_merge, or with one split straight to out.

template <typename KVT, int N>
struct KvRaw;
// get(f): the lane's N values, up to scale(): the factor that turns them
// into the cached values (1 for float rows; the block scale for Q8_0 codes,
// applied once to a dot product or a softmax weight instead of to every value)
template <int N>
struct KvRaw<f16_t, N> {
  typedef _Float16 vec __attribute__((ext_vector_type(N)));
  vec v;
  __device__ __forceinline__ void load(const char* row, int, int d) {
    v = *reinterpret_cast<const vec*>(reinterpret_cast<const f16_t*>(row) + d);
  }
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = (float)v[i];
  }
  __device__ __forceinline__ float scale() const { return 1.f; }
};
template <int N>
struct KvRaw<float, N> {
  typedef float vec __attribute__((ext_vector_type(N)));
  vec v;
  __device__ __forceinline__ void load(const char* row, int, int d) {
    v = *reinterpret_cast<const vec*>(reinterpret_cast<const float*>(row) + d);
  }
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = v[i];
  }
  __device__ __forceinline__ float scale() const { return 1.f; }
};
// signed byte k of w as a float in one instruction (SDWA byte select with
// sign extension)
template <int K>
__device__ __forceinline__ float i8_to_f32(uint32_t w);
template <>
__device__ __forceinline__ float i8_to_f32<0>(uint32_t w) {
  float r;
  asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
  return r;
}
template <>
__device__ __forceinline__ float i8_to_f32<1>(uint32_t w) {
  float r;
  asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  return r;
}
template <>
__device__ __forceinline__ float i8_to_f32<2>(uint32_t w) {
  float r;
  asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  return r;
}
template <>
__device__ __forceinline__ float i8_to_f32<3>(uint32_t w) {
  float r;
  asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}
template <int N>
struct KvRaw<q8_t, N> {  // N (4, 8 or 16) codes of one 32-value block and its scale
  // loads of at most 8 bytes: Q8_0 rows are 136 bytes, so 8-byte aligned
  static constexpr int W = N < 8 ? N : 8;
  typedef signed char vec __attribute__((ext_vector_type(W)));
  vec c[N / W];
  f16_t sc;
  __device__ __forceinline__ void load(const char* row, int hd, int d) {
#pragma unroll
    for (int i = 0; i < N / W; ++i) c[i] = *reinterpret_cast<const vec*>(row + d + W * i);
    sc = *reinterpret_cast<const f16_t*>(row + hd + (d >> 5) * 2);
  }
  // the codes as floats (the scale stays apart)
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int i = 0; i < N / W; ++i) {
#pragma unroll
      for (int j = 0; j < W / 4; ++j) {
        uint32_t w;
        __builtin_memcpy(&w, reinterpret_cast<const char*>(&c[i]) + 4 * j, 4);
        f[W * i + 4 * j] = i8_to_f32<0>(w);
        f[W * i + 4 * j + 1] = i8_to_f32<1>(w);
        f[W * i + 4 * j + 2] = i8_to_f32<2>(w);
        f[W * i + 4 * j + 3] = i8_to_f32<3>(w);
      }
    }
  }
  __device__ __forceinline__ float scale() const { return (float)sc; }
};
// sum over each aligned group of 8 lanes, in every lane of the group
// (lanes i and 7 - i, then quad swaps)
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  return v;
}

template <int HD, int G, typename KVT, int OUT>
__global__ __launch_bounds__(256) void k_attn_decode(AttnArgs a) {
  constexpr bool Q8 = std::is_same<KVT, q8_t>::value;
  // lanes per key row: 16 for float rows (8 values of 16 bytes per lane at
  // head_dim 128); 8 for Q8_0 rows, so that a lane takes 16 codes (two
  // 8-byte loads) and the one scale of their 32-value block (up to two query
  // heads per KV head: more would not fit the registers)
  constexpr int LPR = Q8 && G <= 2 ? 8 : 16;
  constexpr int SPW = 64 / LPR;     // slots per wave
  constexpr int DPL = HD / LPR;
  constexpr int U = LPR == 8 ? 1 : 16 / SPW;  // keys per slot and tile
  constexpr int TILE = 4 * SPW * U;           // keys per tile (64; 32 for Q8_0 rows)
  __shared__ __attribute__((aligned(16))) float s_acc[4][G][HD];
  __shared__ float s_m[4][G], s_l[4][G];

  const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane / LPR, sub = lane % LPR;
  const int nq = a.n_heads, nkv = a.n_kv_heads;
  const int seq = row_seq(a.rows, t), pos = row_pos(a.rows, t);
  const int k_begin = c * a.keys_per_split;
  const int k_end = min(pos + 1, k_begin + a.keys_per_split);

  if (k_begin >= k_end) {  // this split lies past the row's context
    if (OUT == ATT_PARTIAL && tid < G) {
      float* ml = a.part_ml + ((size_t)(t * nq + g * G + tid) * a.n_splits + c) * 2;
      ml[0] = -INFINITY;
      ml[1] = 0.f;
    }
    return;
  }

  constexpr size_t RB = KVIO<KVT>::row_bytes(HD);
  const size_t head_off = (size_t)(seq * nkv + g) * a.cap * RB;
  const char* Kp = reinterpret_cast<const char*>(a.kc) + head_off;
  const char* Vp = reinterpret_cast<const char*>(a.vc) + head_off;
  // Q8_0 cache: keys from `fresh` on are rows of this call, read unquantised
  // from the projection buffer (key j is row t - (pos - j): the call's rows
  // of one sequence are consecutive rows at consecutive positions)
  const int fresh = a.rows.uniform == 0 ? pos : a.rows.p0;
  const float* Kf = a.q + (size_t)(nq + g) * HD + sub * DPL;
  const float* Vf = a.q + (size_t)(nq + nkv + g) * HD + sub * DPL;

  float qr[G][DPL];
  const float qscale = a.scale * 1.4426950408889634f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qp = a.q + (size_t)t * a.ldq + (size_t)(g * G + h) * HD + sub * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) qr[h][e] = qp[e] * qscale;
  }
  // running maxima start at a finite floor far below any score, so no step
  // has to single out a slot, wave or split without keys: their weight
  // 2^(floor - max) is 0, and among themselves 2^0 = 1 times l = 0 and o = 0
  constexpr float FLOOR = -1e30f;
  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = FLOOR;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }

  const int kofs = SPW * wave + slot;
  KvRaw<KVT, DPL> kr[U], vr[U];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(kb + 4 * SPW * u + kofs, k_end - 1);
      kr[u].load(Kp + (size_t)j * RB, HD, sub * DPL);
      vr[u].load(Vp + (size_t)j * RB, HD, sub * DPL);
    }
  };
  load_tile(k_begin);
  for (int kb = k_begin; kb < k_end; kb += TILE) {
    float kf[U][DPL], vf[U][DPL], ks[U], vs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u].get(kf[u]);
      vr[u].get(vf[u]);
      ks[u] = kr[u].scale();
      vs[u] = vr[u].scale();
    }
    load_tile(kb + TILE < k_end ? kb + TILE : kb);  // next tile (the last one reloads itself)
    if (Q8 && kb + TILE > fresh) {  // rows of this call: as computed
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(kb + 4 * SPW * u + kofs, k_end - 1);
        if (j >= fresh) {
          const size_t r = (size_t)(t - pos + j) * a.ldq;
#pragma unroll
          for (int e = 0; e < DPL; ++e) {
            kf[u][e] = Kf[r + e];
            vf[u][e] = Vf[r + e];
          }
          ks[u] = vs[u] = 1.f;
        }
      }
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = kb + 4 * SPW * u + kofs < k_end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) d = fmaf(qr[h][e], kf[u][e], d);
        d *= ks[u];  // a lane's values share one Q8_0 block scale
        d = LPR == 16 ? row16_sum(d) : group8_sum(d);
        sc[u][h] = ok ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);
      float p[U], ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(sc[u][h] - mx);  // 0 for a masked key (-inf)
        ps += p[u];
      }
      l[h] = fmaf(l[h], alpha, ps);
      float pv[U];  // softmax weight times the value rows' scale
#pragma unroll
      for (int u = 0; u < U; ++u) pv[u] = p[u] * vs[u];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        float v = acc[h][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) v = fmaf(pv[u], vf[u][e], v);
        acc[h][e] = v;
      }
      m[h] = mx;
    }
  }

  // the 4 slots of a wave: scale each by 2^(m_slot - m_wave) and add them
  // (slots are the wave's 16-lane rows: swaps across 16 and 32 lanes)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // (Q8_0: 8 slots per wave, lanes l and l ^ 8 of each 16-lane row first)
    const float m8 = LPR == 16 ? m[h] : fmaxf(m[h], dpp_mov<0x128>(m[h]));
    const float mw4 = half_xor16_max(half_xor32_max(m8));
    const float scl = __builtin_amdgcn_exp2f(m[h] - mw4);
    auto slot_sum = [&](float v) { return xor_sum4(LPR == 16 ? v : v + dpp_mov<0x128>(v)); };
    const float lw = slot_sum(l[h] * scl);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = slot_sum(acc[h][e] * scl);
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) s_acc[wave][h][sub * DPL + e] = acc[h][e];
    }
    if (lane == 0) {
      s_m[wave][h] = mw4;
      s_l[wave][h] = lw;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int h = idx / HD, d = idx % HD;
    float M = FLOOR;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = __builtin_amdgcn_exp2f(s_m[w][h] - M);
      o = fmaf(wt, s_acc[w][h][d], o);
      L = fmaf(wt, s_l[w][h], L);
    }
    const int qh = g * G + h;
    if (OUT == ATT_PARTIAL) {
      const size_t base = (size_t)(t * nq + qh) * a.n_splits + c;
      a.part_o[base * HD + d] = o;
      if (d == 0) {
        a.part_ml[base * 2] = M;
        a.part_ml[base * 2 + 1] = L;
      }
    } else {
      const float v = o / L;
      const size_t oi = (size_t)t * a.ldo + (size_t)qh * HD + d;
      if (OUT == ATT_F32) reinterpret_cast<float*>(a.out)[oi] = v;
      else reinterpret_cast<bf16_t*>(a.out)[oi] = (bf16_t)f32_to_bf16(v);
    }
  }
}

// grid (n_heads, rows), head_dim threads: combine the splits' (o, m, l) of
// one (row, query head).  The splits' weights 2^(m_c - M) / L are formed
// once in LDS; each thread then sums its dim over the splits with the loads
// of 8 splits in flight.  Output float32, or bf16 (the A operand of the
// matrix-core o_proj).
template <bool BF16>
__global__ __launch_bounds__(128) void k_attn_merge(AttnArgs a) {
  __shared__ float s_w[MAX_SPLITS];
  const int h = blockIdx.x, t = blockIdx.y, d = threadIdx.x;
  const int ns = a.n_splits, HD = a.head_dim;
  const size_t base = (size_t)(t * a.n_heads + h) * ns;
  const float* ml = a.part_ml + base * 2;
  const float* po = a.part_o + base * HD + d;
  // the first PF splits' values are requested before the weights, so the
  // two reads overlap
  constexpr int PF = 16;
  float pv[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) pv[i] = i < ns ? po[(size_t)i * HD] : 0.f;
  if (d < 64) {  // one wave forms the weights
    float M = -INFINITY;
    for (int c = d; c < ns; c += 64) M = fmaxf(M, ml[2 * c]);
    M = wave_max(M);
    float L = 0.f;
    for (int c = d; c < ns; c += 64) {
      const float lc = ml[2 * c + 1];
      const float w = lc > 0.f ? __builtin_amdgcn_exp2f(ml[2 * c] - M) : 0.f;
      s_w[c] = w;
      L = fmaf(w, lc, L);
    }
    L = wave_sum(L);
    for (int c = d; c < ns; c += 64) s_w[c] /= L;
  }
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (i < ns) o = fmaf(s_w[i], pv[i], o);
  int c = PF;
  for (; c + 8 <= ns; c += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = po[(size_t)(c + i) * HD];
#pragma unroll
    for (int i = 0; i < 8; ++i) o = fmaf(s_w[c + i], v[i], o);
  }
  for (; c < ns; ++c) o = fmaf(s_w[c], po[(size_t)c * HD], o);
  const size_t oi = (size_t)t * a.ldo + (size_t)h * HD + d;
  if (BF16) reinterpret_cast<bf16_t*>(a.out)[oi] = (bf16_t)f32_to_bf16(o);
  else reinterpret_cast<float*>(a.out)[oi] = o;
}

template <int HD, typename KVT, int OUT>
static void launch_g(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.n_splits, a.n_kv_heads, a.rows.n);
  switch (a.n_heads / a.n_kv_heads) {
    case 1: hipLaunchKernelGGL((k_attn_decode<HD, 1, KVT, OUT>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_attn_decode<HD, 2, KVT, OUT>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_attn_decode<HD, 4, KVT, OUT>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_attn_decode<HD, 8, KVT, OUT>), grid, dim3(256), 0, st, a); break;
  }
}

template <int HD, typename KVT>
static void launch_o(AttnOut mode, const AttnArgs& a, hipStream_t st) {
  if (mode == ATT_PARTIAL) launch_g<HD, KVT, ATT_PARTIAL>(a, st);
  else if (mode == ATT_F32) launch_g<HD, KVT, ATT_F32>(a, st);
  else launch_g<HD, KVT, ATT_BF16>(a, st);
}

template <int HD>
static void launch_kv(KvKind kv, AttnOut mode, const AttnArgs& a, hipStream_t st) {
  if (kv == KV_F16) launch_o<HD, f16_t>(mode, a, st);
  else if (kv == KV_Q8) launch_o<HD, q8_t>(mode, a, st);
  else launch_o<HD, float>(mode, a, st);
}

void launch_attn_decode(KvKind kv, AttnOut mode, AttnArgs a, hipStream_t st) {
  if (a.head_dim == 128) launch_kv<128>(kv, mode, a, st);
  else launch_kv<64>(kv, mode, a, st);
}

void launch_attn_merge(AttnArgs a, bool bf16_out, hipStream_t st) {
  if (bf16_out) hipLaunchKernelGGL(k_attn_merge<true>, dim3(a.n_heads, a.rows.n), dim3(a.head_dim), 0, st, a);
  else hipLaunchKernelGGL(k_attn_merge<false>, dim3(a.n_heads, a.rows.n), dim3(a.head_dim), 0, st, a);
}

// ---------------------------------------------------------------------------
// small helpers

__global__ void k_rope_table(float2* tab, int cap, int half, int hd, double theta) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)cap * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)hd);
  const double ang = (double)pos * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

void launch_rope_table(float2* tab, int cap, int head_dim, double theta, hipStream_t st) {
  const int half = head_dim / 2;
  const size_t n = (size_t)cap * half;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab, cap,
                     half, head_dim, theta);
}

// grid (len, n_kv), hd / 4 threads: 4 values of one row each
template <typename KVT>
__global__ void k_kv_to_f32(const char* src, int cap, int len, int hd, float* dst) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x * 4;
  float f[4];
  kv_load<KVT, 4>(src + ((size_t)h * cap + t) * KVIO<KVT>::row_bytes(hd), hd, d, f);
  *reinterpret_cast<float4*>(dst + ((size_t)h * len + t) * hd + d) = make_float4(f[0], f[1], f[2], f[3]);
}

void launch_kv_to_f32(KvKind kv, const void* src, int n_kv, int cap, int len, int hd, float* dst,
                      hipStream_t st) {
  if (len <= 0) return;
  const dim3 grid(len, n_kv);
  const char* s = reinterpret_cast<const char*>(src);
  if (kv == KV_F16) hipLaunchKernelGGL(k_kv_to_f32<f16_t>, grid, dim3(hd / 4), 0, st, s, cap, len, hd, dst);
  else if (kv == KV_Q8) hipLaunchKernelGGL(k_kv_to_f32<q8_t>, grid, dim3(hd / 4), 0, st, s, cap, len, hd, dst);
  else hipLaunchKernelGGL(k_kv_to_f32<float>, grid, dim3(hd / 4), 0, st, s, cap, len, hd, dst);
}

// grid (len, n_kv, 2), hd / 4 threads: positions 0 .. len-1 of one
// sequence's K (z = 0) and V (z = 1) as float16 rows [n_kv][cap][hd], for the
// matrix-core prefill attention: positions below `fresh` dequantised from the
// Q8_0 cache, the call's own rows (position fresh + r is row r) from the
// projection buffer, K after its norm and RoPE
__global__ void k_kv_q8_to_f16(const char* kq, const char* vq, int cap, int hd, f16_t* k16,
                               f16_t* v16, int fresh, const float* qkv, int ldqkv, int nq,
                               int nkv) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x * 4;
  const char* src = blockIdx.z ? vq : kq;
  f16_t* dst = blockIdx.z ? v16 : k16;
  float f[4];
  if (t >= fresh) {
    const float4 v = *reinterpret_cast<const float4*>(
        qkv + (size_t)(t - fresh) * ldqkv + (size_t)(nq + blockIdx.z * nkv + h) * hd + d);
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  } else {
    kv_load<q8_t, 4>(src + ((size_t)h * cap + t) * KVIO<q8_t>::row_bytes(hd), hd, d, f);
  }
  typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 h4;
  h4 o;
  o[0] = (f16_t)f[0];
  o[1] = (f16_t)f[1];
  o[2] = (f16_t)f[2];
  o[3] = (f16_t)f[3];
  *reinterpret_cast<h4*>(dst + ((size_t)h * cap + t) * hd + d) = o;
}

void launch_kv_q8_to_f16(const void* kq, const void* vq, int n_kv, int cap, int len, int hd,
                         f16_t* k16, f16_t* v16, int fresh, const float* qkv, int ldqkv, int nq,
                         hipStream_t st) {
  if (len <= 0) return;
  hipLaunchKernelGGL(k_kv_q8_to_f16, dim3(len, n_kv, 2), dim3(hd / 4), 0, st,
                     reinterpret_cast<const char*>(kq), reinterpret_cast<const char*>(vq), cap, hd,
                     k16, v16, fresh, qkv, ldqkv, nq, n_kv);
}

size_t kv_row_bytes(KvKind kv, int hd) {
  return kv == KV_F16 ? KVIO<f16_t>::row_bytes(hd)
                      : (kv == KV_Q8 ? KVIO<q8_t>::row_bytes(hd) : KVIO<float>::row_bytes(hd));
}

}  // namespace qtalk
