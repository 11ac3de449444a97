// Causal GQA prefill attention on the matrix cores, reading the f16 KV cache.
//
// Semantics as the per-row attention ("qwentts.cpp src/talker-forward.h",
// talker_layer_forward: per-head RMSNorm of q with the shared q_norm gain,
// NEOX RoPE at the absolute position, scores q.k / sqrt(head_dim) over the
// cache window, causal mask key <= position, softmax, weighted sum of V;
// "transcribe.cpp src/causal_lm/causal_lm.cpp", block_prefill: query head h
// reads KV head h / (n_heads / n_kv_heads)).  The rows' own K/V were
// appended to the cache before this kernel runs, so keys are read back in
// their cache precision.  q arrives raw from the QKV projection; its QK-norm
// and RoPE are applied here, on the fragment each lane already holds.
//
// Work split (two query heads per KV head): a block owns one KV head g and
// 32 consecutive positions; its 4 waves are (query head of the group) x (key
// half), so one staging of a 64-key K/V tile in LDS serves both query heads,
// and each wave runs the MFMAs of one 32-key half of every tile with its own
// online softmax.  The two halves are merged (log-sum-exp) at the end.  Small
// blocks (480 of them at 2048 rows) spread the causal triangle over all CUs
// two blocks deep, longest first.
//
// Per wave and tile (flash-attention order, softmax state in float32):
//   S^T[key][row] = K . Q^T   v_mfma_f32_32x32x16_f16, A = K rows, B = q
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
constexpr int PB = 32;        // positions per block
constexpr int G = 2;          // query heads per KV head

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

// value of lane l ^ 32 combined with lane l's own: v_permlane32_swap exchanges
// the upper half of one operand with the lower half of the other, so the two
// results hold {v[l], v[l ^ 32]} in every lane
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HD>
__global__ __launch_bounds__(pa::NT, 2) void k_attn_prefill(PrefillAttnArgs a) {
  using namespace pa;
  constexpr int KSTR = HD + 8;              // K row stride in LDS (halfs)
  constexpr int NKS = HD / 16;              // k-steps of the score product
  constexpr int NMT = HD / 32;              // hd tiles of the value product
  constexpr int CPR = HD / 8;               // 16-byte chunks per key row
  constexpr int NLD = KT * CPR / NT;        // K chunks per thread per tile
  constexpr int NLDV = KT / 2 * CPR / NT;   // V chunk pairs per thread per tile
  static_assert(KT * CPR % NT == 0 && KT / 2 * CPR % NT == 0, "staging split");
  constexpr int LDS_HALFS = KT * KSTR + HD * KT;
  __shared__ __attribute__((aligned(16))) f16_t lds[LDS_HALFS];
  __shared__ __attribute__((aligned(16))) f16_t qlds[G * NKS * 64 * 8];  // q fragments
  f16_t* Ks = lds;
  f16_t* Vt = lds + KT * KSTR;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nkv = a.n_kv_heads;
  const int nqb = (a.T + PB - 1) / PB;
  // work item r (0 = longest: the last 32 positions) of this block.  Blocks b
  // and b + ncu are dispatched to the same CU when the whole grid fits two
  // deep, so the second one takes the item complementary to the first
  // (longest with shortest) and every CU gets about the same number of key
  // tiles; otherwise plain longest first.
  const int nb = nqb * nkv, b = blockIdx.x;
  const int r = (b < a.ncu || nb > 2 * a.ncu) ? b : nb - 1 - (b - a.ncu);
  const int g = r % nkv;
  const int qb = nqb - 1 - r / nkv;
  const int P0 = a.p0 + qb * PB;
  const int P1 = min(P0 + PB, a.p0 + a.T);  // block positions [P0, P1)
  const int kend = P1;                      // keys [0, kend)
  const int nkt = (kend + KT - 1) / KT;

  const int hh = wave >> 1, kh = wave & 1;  // query head of the group, key half
  const int hq = g * G + hh;
  const int last = P1 - 1;
  const int n = lane & 31, h = lane >> 5;
  const int posn = P0 + n;

  // batched prefill: this block's sequence and its rows of q and out
  const int bz = blockIdx.y;
  const int seq = a.nbatch > 1 ? a.seqs[bz] : a.seq;
  const float* qrows = a.q + (size_t)bz * a.T * a.ldq;
  bf16_t* orows = a.out + (size_t)bz * a.T * a.ldo;
  const size_t head_off = (size_t)(seq * nkv + g) * a.cap * HD;
  const f16_t* Kg = a.kc + head_off;
  const f16_t* Vg = a.vc + head_off;

  // q (B operand of the score product): row posn, hd ks*16 + h*8 + e.  The
  // lane pair (n, n + 32) holds the whole head, and the RoPE partner d + 64 of
  // hd d < 64 sits in the same lane at ks + NKS/2.  The key-half-0 wave of a
  // query head prepares the fragments and hands them to its partner through
  // LDS; both keep them in registers for the whole key loop.
  if (kh == 0) {
    const int t = min(posn - a.p0, a.T - 1);
    const int pr = min(posn, a.p0 + a.T - 1);
    const float* qp = qrows + (size_t)t * a.ldq + (size_t)hq * HD + h * 8;
    float qv[NKS][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const float4 u = *reinterpret_cast<const float4*>(qp + ks * 16);
      const float4 v = *reinterpret_cast<const float4*>(qp + ks * 16 + 4);
      qv[ks][0] = u.x; qv[ks][1] = u.y; qv[ks][2] = u.z; qv[ks][3] = u.w;
      qv[ks][4] = v.x; qv[ks][5] = v.y; qv[ks][6] = v.z; qv[ks][7] = v.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(qv[ks][e], qv[ks][e], ss);
    }
    ss += __shfl_xor(ss, 32);
    const float inv = rsqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[ks][e] *= inv * a.g_q[ks * 16 + h * 8 + e];
    const float2* cs = a.rope + (size_t)pr * (HD / 2) + h * 8;
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 c = cs[ks * 16 + e];
        const float x1 = qv[ks][e], x2 = qv[ks + NKS / 2][e];
        qv[ks][e] = (x1 * c.x - x2 * c.y) * a.qscale;
        qv[ks + NKS / 2][e] = (x2 * c.x + x1 * c.y) * a.qscale;
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f16x8_t f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (f16_t)qv[ks][e];
      *reinterpret_cast<f16x8_t*>(&qlds[((hh * NKS + ks) * 64 + lane) * 8]) = f;
    }
  }

  // staging, per 64-key tile, in two register stages (tile kt in stage kt & 1,
  // requested two tiles ahead of its use).  K: chunk i of this thread is key
  // (tid + NT*i) / CPR, column chunk (tid + NT*i) % CPR (16 lanes cover one
  // 256-byte key row).  V: the same chunk of two adjacent keys, so that the
  // transposed store writes whole dwords (keys 2kp, 2kp+1 of one hd row).
  // Offsets are fixed per thread; only the tile base moves.  Named registers:
  // an array here would be left in private memory.
  static_assert(NLD == 4 || NLD == 2, "K chunks per thread");
  static_assert(NLDV == 2 || NLDV == 1, "V pairs per thread");
  const int kkey0 = tid / CPR, kc0 = tid % CPR;  // chunk i: key kkey0 + i*(NT/CPR)
  constexpr int KSTEP = NT / CPR;
  const int vkey0 = 2 * (tid / CPR);             // pair i: keys vkey0 + i*2*KSTEP, +1
  uint4 s0k0, s0k1, s0k2, s0k3, s0v0, s0v1, s0v2, s0v3;  // stage 0
  uint4 s1k0, s1k1, s1k2, s1k3, s1v0, s1v1, s1v2, s1v3;  // stage 1
  // Loads read a clamped key row (always in bounds) and run unconditionally;
  // keys past the block's last position are zeroed when the stage is stored.
  // (A conditional load would make the compiler drain every outstanding load
  // at the join, the prefetch of the other stage included.)
#define QA_LD(BASE, KEY) \
  (*reinterpret_cast<const uint4*>((BASE) + (size_t)min((KEY), kend - 1) * HD + kc0 * 8))
#define QA_GLOAD(S, KT)                                          \
  do {                                                           \
    const int kb_ = (KT) * KT_;                                  \
    S##k0 = QA_LD(Kg, kb_ + kkey0);                              \
    S##k1 = QA_LD(Kg, kb_ + kkey0 + KSTEP);                      \
    if (NLD == 4) {                                              \
      S##k2 = QA_LD(Kg, kb_ + kkey0 + 2 * KSTEP);                \
      S##k3 = QA_LD(Kg, kb_ + kkey0 + 3 * KSTEP);                \
    }                                                            \
    S##v0 = QA_LD(Vg, kb_ + vkey0);                              \
    S##v1 = QA_LD(Vg, kb_ + vkey0 + 1);                          \
    if (NLDV == 2) {                                             \
      S##v2 = QA_LD(Vg, kb_ + vkey0 + 2 * KSTEP);                \
      S##v3 = QA_LD(Vg, kb_ + vkey0 + 2 * KSTEP + 1);            \
    }                                                            \
  } while (0)
#define QA_LSTORE_M(S, KT, MASK)                                           \
  do {                                                                     \
    const int kb_ = (KT) * KT_;                                            \
    store_k(0, kb_, S##k0, MASK);                                          \
    store_k(1, kb_, S##k1, MASK);                                          \
    if (NLD == 4) {                                                        \
      store_k(2, kb_, S##k2, MASK);                                        \
      store_k(3, kb_, S##k3, MASK);                                        \
    }                                                                      \
    store_v(0, kb_, S##v0, S##v1, MASK);                                   \
    if (NLDV == 2) store_v(1, kb_, S##v2, S##v3, MASK);                    \
  } while (0)
  // only the tile holding the block's last key needs its tail zeroed
#define QA_LSTORE(S, KT)                                                   \
  do {                                                                     \
    if (((KT) + 1) * KT_ <= kend) QA_LSTORE_M(S, KT, false);               \
    else QA_LSTORE_M(S, KT, true);                                         \
  } while (0)
  constexpr int KT_ = KT;
  f16_t* const kst = &Ks[kkey0 * KSTR + kc0 * 8];
  auto zero_past = [&](const uint4& r, int key, bool mask) {
    if (!mask) return r;
    const bool ok = key < kend;
    return make_uint4(ok ? r.x : 0u, ok ? r.y : 0u, ok ? r.z : 0u, ok ? r.w : 0u);
  };
  auto store_k = [&](int i, int kb, const uint4& r, bool mask) {
    *reinterpret_cast<uint4*>(kst + i * KSTEP * KSTR) = zero_past(r, kb + kkey0 + i * KSTEP, mask);
  };
  // transposed V: hd row d = kc0*8 + e; its swizzle (((d >> 3) ^ d) & 7) is
  // (kc0 ^ e) & 7, so the 8 row addresses of a pair differ only in e
  // (one byte permute per dword: halves e of key and key + 1)
  auto store_v = [&](int i, int kb, const uint4& q0, const uint4& q1, bool mask) {
    const int key = vkey0 + i * 2 * KSTEP;
    const uint4 r0 = zero_past(q0, kb + key, mask), r1 = zero_past(q1, kb + key + 1, mask);
    const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
    const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // bytes 0-3 select from w0[e/2], 4-7 from w1[e/2]: low half of each for
      // even e, high half for odd e
      const uint32_t dw = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1],
                                                (e & 1) ? 0x07060302u : 0x05040100u);
      const int d = kc0 * 8 + e;
      *reinterpret_cast<uint32_t*>(&Vt[d * KT + (key ^ (((kc0 ^ e) & 7) << 3))]) = dw;
    }
  };

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  // A-operand row of the score product held by this lane: key tau(n) of this
  // wave's 32-key half
  const int krow = kh * 32 + tau(n);
  f16x8_t qf[NKS];

  auto compute = [&](int kt) {
    const int kbase = kt * KT + kh * 32;  // this wave's first key
    if (kbase > last) return;
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f16x8_t kf = *reinterpret_cast<const f16x8_t*>(&Ks[krow * KSTR + ks * 16 + h * 8]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s, 0, 0, 0);
    }
    // causal mask (key <= position) where the half reaches the block's rows
    if (kbase + 31 > P0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + (r >> 3) * 16 + h * 8 + ((r >> 2) & 1) * 4 + (r & 3);
        if (key > posn) s[r] = -INFINITY;
      }
    }
    float t8[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) t8[r] = fmaxf(s[r], s[r + 8]);
#pragma unroll
    for (int r = 0; r < 4; ++r) t8[r] = fmaxf(t8[r], t8[r + 4]);
    float mx = fmaxf(fmaxf(t8[0], t8[2]), fmaxf(t8[1], t8[3]));
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) return;  // no key of this half is visible to any row yet
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    f16x8_t pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] - m_new);  // masked: exp2(-inf) = 0
      psum += p;
      pf[r >> 3][r & 7] = (f16_t)p;
    }
    l_run = l_run * alpha + psum;
    if (!__all(alpha == 1.0f)) {  // once the running max settles this is skipped
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
    }
    // O^T += V^T P^T over this half's 32 keys (2 k-steps of 16)
#pragma unroll
    for (int sk = 0; sk < 2; ++sk)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const f16x8_t vf = *reinterpret_cast<const f16x8_t*>(
            &Vt[vt_index(mt * 32 + n, kh * 32 + sk * 16 + h * 8)]);
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[sk], o[mt], 0, 0, 0);
      }
  };

  // loads run unconditionally (past the last tile they repeat it) so both
  // register stages stay in registers
  QA_GLOAD(s0, 0);
  QA_GLOAD(s1, min(1, nkt - 1));
  QA_LSTORE(s0, 0);
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = *reinterpret_cast<const f16x8_t*>(&qlds[((hh * NKS + ks) * 64 + lane) * 8]);
  for (int kt = 0; kt < nkt; kt += 2) {
    // tile kt in LDS, tile kt + 1 in flight in stage 1
    QA_GLOAD(s0, min(kt + 2, nkt - 1));
    compute(kt);
    __syncthreads();
    if (kt + 1 >= nkt) break;
    QA_LSTORE(s1, kt + 1);
    __syncthreads();
    // tile kt + 1 in LDS, tile kt + 2 in flight in stage 0
    QA_GLOAD(s1, min(kt + 3, nkt - 1));
    compute(kt + 1);
    __syncthreads();
    if (kt + 2 >= nkt) break;
    QA_LSTORE(s0, kt + 2);
    __syncthreads();
  }
#undef QA_LD
#undef QA_GLOAD
#undef QA_LSTORE

  // merge the two key halves of each query head through LDS (the tiles are
  // no longer needed): the key-half-1 wave hands over (m, l, O), the key-half-0
  // wave combines and writes
  float* xs = reinterpret_cast<float*>(lds);  // [G][64 lanes][NMT*16 + 2]
  constexpr int XS = NMT * 16 + 2;
  static_assert((size_t)G * 64 * XS * 4 <= sizeof(f16_t) * LDS_HALFS, "merge buffer");
  float* mine = xs + ((size_t)hh * 64 + lane) * XS;
  if (kh == 1) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[mt * 16 + r] = o[mt][r];
    mine[NMT * 16] = m_run;
    mine[NMT * 16 + 1] = l_run;
  }
  __syncthreads();
  if (kh == 1 || posn >= P1) return;
  const float m1 = mine[NMT * 16], l1 = mine[NMT * 16 + 1];
  const float M = fmaxf(m_run, m1);  // finite: key 0 is visible to every row
  const float a0 = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  const float a1 = m1 == -INFINITY ? 0.f : exp2f(m1 - M);
  const float l = l_run * a0 + l1 * a1;
  const float inv = 1.0f / xor32_sum(l);
  bf16_t* orow = orows + (size_t)(posn - a.p0) * a.ldo + (size_t)hq * HD;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = mt * 32 + rg * 8 + h * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (o[mt][rg * 4 + j] * a0 + mine[mt * 16 + rg * 4 + j] * a1) * inv;
      uint2 w;
      w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
}

bool attn_prefill_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && group == pa::G;
}

void launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t st) {
  const int nqb = (a.T + pa::PB - 1) / pa::PB;
  const dim3 grid(nqb * a.n_kv_heads, a.nbatch > 1 ? a.nbatch : 1);
  if (a.head_dim == 128) hipLaunchKernelGGL(k_attn_prefill<128>, grid, dim3(pa::NT), 0, st, a);
  else hipLaunchKernelGGL(k_attn_prefill<64>, grid, dim3(pa::NT), 0, st, a);
}

}  // namespace qtalk
