// Causal GQA prefill attention on the matrix cores, reading the f16 KV cache.
//
// Semantics as the per-row attention ("qwentts.cpp src/talker-forward.h",
// talker_layer_forward: scores q.k / sqrt(head_dim) over the cache window,
// causal mask key <= position, softmax, weighted sum of V; "transcribe.cpp
// src/causal_lm/causal_lm.cpp", block_prefill: query head h reads KV head
// h / (n_heads / n_kv_heads)).  The rows' own K/V were appended to the cache
// before this kernel runs, so keys are read back in their cache precision.
//
// Work split: a block owns one KV head g and PB consecutive positions; its 4
// waves each own 32 positions of one query head of the group, so one staging
// of a 64-key K/V tile in LDS serves every query head that shares it.  Per
// wave and tile (flash-attention order, online softmax in float32):
//   S^T[key][row] = K . Q^T   v_mfma_f32_32x32x16_f16, A = K tile rows, B = q
//   P = exp2(S' - m)          S' carries 1/sqrt(hd) * log2(e) through q
//   O^T[hd][row] += V^T . P^T v_mfma_f32_32x32x16_f16, A = V^T (LDS), B = P
// Computing the transposed products makes the score accumulator of a lane
// hold one query row, which is exactly the lane role of the B operand of the
// value product, so P never leaves registers.  The key order inside a
// 32-key score tile is permuted (tau below) so that each lane's 8 value
// slots are 8 consecutive keys: one 16-byte LDS read of the transposed V.
#include "kernels.h"

namespace qtalk {
namespace pa {

constexpr int NWV = 4;        // waves per block
constexpr int NT = NWV * 64;  // threads per block
constexpr int KT = 64;        // keys per tile

// key (0..31) held by score-tile row m: m = a*8 + h*4 + b -> (a>>1)*16 + h*8 + (a&1)*4 + b
__device__ __forceinline__ int tau(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// Transposed V tile in LDS: hd row d holds the tile's 64 keys; the 8-key
// groups of a row are XOR-swizzled so that both the transposing dword stores
// (16 rows at once) and the 16-byte operand reads (32 rows at once) spread
// over the banks.
__device__ __forceinline__ int vt_index(int d, int key) {
  return d * KT + (key ^ ((((d >> 3) ^ d) & 7) << 3));
}

}  // namespace pa

template <int HD, int G>
__global__ __launch_bounds__(pa::NT, 2) void k_attn_prefill(PrefillAttnArgs a) {
  using namespace pa;
  constexpr int PB = 32 * NWV / G;  // positions per block
  constexpr int KSTR = HD + 8;      // K row stride in LDS (halfs)
  constexpr int NKS = HD / 16;      // k-steps of the score product
  constexpr int NMT = HD / 32;      // hd tiles of the value product
  constexpr int CPR = HD / 8;       // 16-byte chunks per key row
  constexpr int NLD = KT * CPR / NT;         // K chunks per thread per tile
  constexpr int NLDV = KT / 2 * CPR / NT;   // V chunk pairs per thread per tile
  static_assert(KT * CPR % NT == 0 && KT / 2 * CPR % NT == 0, "staging split");
  __shared__ __attribute__((aligned(16))) f16_t Ks[KT * KSTR];
  __shared__ __attribute__((aligned(16))) f16_t Vt[HD * KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nkv = a.n_kv_heads;
  const int g = blockIdx.x % nkv;
  const int nqb = (a.T + PB - 1) / PB;
  const int qb = nqb - 1 - (int)(blockIdx.x / nkv);  // longest blocks first
  const int P0 = a.p0 + qb * PB;
  const int P1 = min(P0 + PB, a.p0 + a.T);  // block positions [P0, P1)
  const int kend = P1;                      // keys [0, kend)
  const int nkt = (kend + KT - 1) / KT;

  const int hq = g * G + wave % G;
  const int Pw = P0 + (wave / G) * 32;  // wave positions [Pw, Pw + 32)
  const bool wave_live = Pw < P1;
  const int wave_last = min(Pw + 31, P1 - 1);
  const int n = lane & 31, h = lane >> 5;
  const int posn = Pw + n;

  const size_t head_off = (size_t)(a.seq * nkv + g) * a.cap * HD;
  const f16_t* Kg = a.kc + head_off;
  const f16_t* Vg = a.vc + head_off;

  // q (B operand of the score product): row posn, hd ks*16 + h*8 .. +8
  f16x8_t qf[NKS];
  {
    const int t = min(posn - a.p0, a.T - 1);
    const float* qp = a.q + (size_t)t * a.ldq + (size_t)hq * HD + h * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const float4 u = *reinterpret_cast<const float4*>(qp + ks * 16);
      const float4 v = *reinterpret_cast<const float4*>(qp + ks * 16 + 4);
      qf[ks] = f16x8_t{(f16_t)(u.x * a.qscale), (f16_t)(u.y * a.qscale), (f16_t)(u.z * a.qscale),
                       (f16_t)(u.w * a.qscale), (f16_t)(v.x * a.qscale), (f16_t)(v.y * a.qscale),
                       (f16_t)(v.z * a.qscale), (f16_t)(v.w * a.qscale)};
    }
  }

  // staging, per 64-key tile.  K: chunk i of this thread is key (tid + NT*i) / CPR,
  // column chunk (tid + NT*i) % CPR (16 lanes cover one 256-byte key row).  V:
  // the same chunk of two adjacent keys, so that the transposed store writes
  // whole dwords (keys 2kp, 2kp+1 of one hd row).
  uint4 rk[NLD], rv[NLDV][2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, key = kt * KT + idx / CPR, c = idx % CPR;
      rk[i] = key < kend ? *reinterpret_cast<const uint4*>(Kg + (size_t)key * HD + c * 8)
                         : make_uint4(0, 0, 0, 0);  // never-written slots read as 0
    }
#pragma unroll
    for (int i = 0; i < NLDV; ++i) {
      const int idx = tid + NT * i, key = kt * KT + 2 * (idx / CPR), c = idx % CPR;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        rv[i][u] = key + u < kend
                       ? *reinterpret_cast<const uint4*>(Vg + (size_t)(key + u) * HD + c * 8)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, key = idx / CPR, c = idx % CPR;
      *reinterpret_cast<uint4*>(&Ks[key * KSTR + c * 8]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < NLDV; ++i) {
      const int idx = tid + NT * i, key = 2 * (idx / CPR), c = idx % CPR;
      const uint32_t w0[4] = {rv[i][0].x, rv[i][0].y, rv[i][0].z, rv[i][0].w};
      const uint32_t w1[4] = {rv[i][1].x, rv[i][1].y, rv[i][1].z, rv[i][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = c * 8 + e;
        const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xFFFFu);
        const uint32_t hi = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xFFFFu);
        *reinterpret_cast<uint32_t*>(&Vt[vt_index(d, key)]) = lo | (hi << 16);
      }
    }
  };

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // A-operand row of the score product held by this lane: key tau(n) of each 32-key half
  const int krow = tau(n);

  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int kbase = kt * KT;
    if (wave_live && kbase <= wave_last) {
      // scores of two 32-key halves
      f32x16_t s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const f16x8_t kf =
              *reinterpret_cast<const f16x8_t*>(&Ks[(st * 32 + krow) * KSTR + ks * 16 + h * 8]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[st], 0, 0, 0);
        }
      }
      // causal mask (key <= position) on the tiles that reach the block's rows
      if (kbase + KT - 1 > Pw) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + st * 32 + (r >> 3) * 16 + h * 8 + ((r >> 2) & 1) * 4 + (r & 3);
            if (key > posn) s[st][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
      f16x8_t pf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[st][r] - m_new);  // masked: exp2(-inf) = 0
          psum += p;
          pf[st][r >> 3][r & 7] = (f16_t)p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
      // O^T += V^T P^T over the tile's 64 keys (4 k-steps of 16)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int sk = 0; sk < 2; ++sk)
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            const f16x8_t vf = *reinterpret_cast<const f16x8_t*>(
                &Vt[vt_index(mt * 32 + n, st * 32 + sk * 16 + h * 8)]);
            o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[st][sk], o[mt], 0, 0, 0);
          }
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      lstore();
      __syncthreads();
    }
  }

  if (!wave_live || posn >= P1) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  bf16_t* orow = a.out + (size_t)(posn - a.p0) * a.ldo + (size_t)hq * HD;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = mt * 32 + rg * 8 + h * 4;
      uint2 w;
      w.x = f32_to_bf16(o[mt][rg * 4] * inv) | (f32_to_bf16(o[mt][rg * 4 + 1] * inv) << 16);
      w.y = f32_to_bf16(o[mt][rg * 4 + 2] * inv) | (f32_to_bf16(o[mt][rg * 4 + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
}

bool attn_prefill_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4);
}

template <int HD, int G>
static void launch_hg(const PrefillAttnArgs& a, hipStream_t st) {
  constexpr int PB = 32 * pa::NWV / G;
  const int nqb = (a.T + PB - 1) / PB;
  hipLaunchKernelGGL((k_attn_prefill<HD, G>), dim3(nqb * a.n_kv_heads), dim3(pa::NT), 0, st, a);
}

void launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t st) {
  const int G = a.n_heads / a.n_kv_heads;
  if (a.head_dim == 128) {
    if (G == 1) launch_hg<128, 1>(a, st);
    else if (G == 2) launch_hg<128, 2>(a, st);
    else launch_hg<128, 4>(a, st);
  } else {
    if (G == 1) launch_hg<64, 1>(a, st);
    else if (G == 2) launch_hg<64, 2>(a, st);
    else launch_hg<64, 4>(a, st);
  }
}

}  // namespace qtalk
