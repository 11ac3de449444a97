// Causal GQA prefill attention on the matrix cores, reading the f16 KV cache.
//
// Semantics as the per-row attention ("qwentts.cpp src/talker-forward.h",
// talker_layer_forward: per-head RMSNorm of q with the shared q_norm gain,
// NEOX RoPE at the absolute position, scores q.k / sqrt(head_dim) over the
// cache window, causal mask key <= position, softmax, weighted sum of V;
// "transcribe.cpp src/causal_lm/causal_lm.cpp", block_prefill: query head h
// reads KV head h / (n_heads / n_kv_heads)).  The rows' own K/V were
// appended to the cache before this kernel runs, so keys are read back in
// their cache precision.  q arrives either prepared by the QKV projection's
// epilogue (q16: normed, rotated, scaled, float16, read straight into the
// fragments) or raw in float32, and then its QK-norm and RoPE are applied
// here, on the fragment each lane already holds.
//
// Work split (two query heads per KV head): a block owns one KV head g and
// 32 or 64 consecutive positions; its waves are (query head of the group) x
// (32-row half of the positions) x (key half), so one staging of a 64-key
// K/V tile in LDS serves both query heads and all the block's rows, and each
// wave runs the MFMAs of one 32-key half of every tile with its own online
// softmax.  The two key halves are merged (log-sum-exp) at the end.  Blocks
// of 32 positions (4 waves, 480 blocks at 2048 rows) spread a causal
// triangle over all CUs two blocks deep, longest first; blocks of 64
// positions (8 waves, one block per CU) stage each K/V byte for twice the
// query rows, which pays where the blocks' key ranges are of similar length
// (a chunk far into the context).
//
// Per wave and tile (flash-attention order, softmax state in float32):
//   S^T[key][row] = K . Q^T   v_mfma_f32_32x32x16_f16, A = K rows, B = q
//   P = exp2(S' - m)          S' carries 1/sqrt(hd) * log2(e) through q
//   O^T[hd][row] += V^T . P^T v_mfma_f32_32x32x16_f16, A = V^T (LDS), B = P
// Computing the transposed products makes the score accumulator of a lane
// hold one query row, which is exactly the lane role of the B operand of the
// value product, so P never leaves registers.  The key order inside a
// 32-key score tile is permuted (tau below) so that each lane's 8 value
// slots are 8 consecutive keys, which two transposing LDS reads
// (ds_read_b64_tr_b16) fetch from the key-major V tile.
#include "kernels.h"
#include "lds_dma.h"

namespace qtalk {
namespace pa {

constexpr int PR = 32;        // positions per row half (one MFMA tile of query rows)
constexpr float LAZY = 8.f;   // online softmax: headroom of the running maximum (log2 units)
constexpr int G = 2;          // query heads per KV head

// key (0..31) held by score-tile row m: m = a*8 + h*4 + b -> (a>>1)*16 + h*8 + (a&1)*4 + b
__device__ __forceinline__ int tau(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
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

// NKQ key groups per block, NR row halves of 32 positions: waves (query
// head, row half, key group), 32 keys of every tile per wave, tiles of 32 NKQ
// keys.  NKQ = 2, NR = 1: 4 waves, two blocks per CU; NKQ = 2, NR = 2: 8
// waves, one block per CU.  Either way two waves share a SIMD.
template <int HD, int NKQ, int NR>
__global__ __launch_bounds__(64 * pa::G * NKQ * NR, NKQ * NR == 2 ? 2 : 1) void k_attn_prefill(PrefillAttnArgs a) {
  using namespace pa;
  constexpr int PB = PR * NR;               // positions per block
  constexpr int NWV = G * NR * NKQ;         // waves per block
  constexpr int KT = 32 * NKQ;              // keys per tile
  constexpr int NKS = HD / 16;              // k-steps of the score product
  constexpr int NMT = HD / 32;              // hd tiles of the value product
  constexpr int CPR = HD / 8;               // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;             // key rows per 1 KiB load instruction
  constexpr int NLI = KT / RPI / NWV;       // load instructions per wave, tile and operand
  static_assert((HD == 128 || HD == 64) && KT % (RPI * NWV) == 0, "staging split");
  // two tile buffers (tile kt in buffer kt & 1): the two K tiles, then the
  // two V tiles, so that a buffer is one immediate offset (KT * HD halfs)
  // away from the other; rows key-major, 16-byte chunk c of key row k stored
  // in slot c ^ swz(k).  At
  // head_dim 128 (256-byte rows, one row per pass over the 64 banks) swz
  // rotates the low four key bits, (k % 4) * 4 + (k / 4) % 4: the K reads
  // (16 lanes, 16 consecutive keys, one chunk) and the transposing V reads
  // (32 lanes, 4 consecutive keys, 4 aligned chunks) then both fall on 16
  // distinct 16-byte bank groups (k % 16 alone gave the V reads four-way
  // conflicts).  At head_dim 64 swz(k) = k % 8.  With one row half the q
  // fragments pass through the K tile of buffer 1 before the key loop; the
  // key-group merge at the end reuses the tiles' space
  constexpr int TILE = 2 * KT * HD;  // halfs per buffer
  constexpr int XS = HD / 32 * 16 + 2;                    // merge record: O, m, l of one lane
  constexpr int MERGE_HALFS = G * NR * (NKQ - 1) * 64 * XS * 2;
  constexpr int LDS_HALFS = 2 * TILE > MERGE_HALFS ? 2 * TILE : MERGE_HALFS;
  __shared__ __attribute__((aligned(1024))) f16_t lds[LDS_HALFS];
  f16_t* const qlds = lds + KT * HD;  // K tile of buffer 1
  static_assert(NR != 1 || G * NKS * 64 * 8 <= KT * HD, "q fragments fit one K tile");

  auto swz = [](int k) { return CPR == 16 ? ((k & 3) << 2) | ((k >> 2) & 3) : (k & (CPR - 1)); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int nkv = a.n_kv_heads;
  const int nqb = (a.T + PB - 1) / PB;
  // work item r (0 = longest: the last 32 positions) of this block.  Blocks b
  // and b + ncu are dispatched to the same CU when the whole grid fits two
  // deep, so the second one takes the item complementary to the first
  // (longest with shortest) and every CU gets about the same number of key
  // tiles; otherwise plain longest first.
  const int nb = nqb * nkv, b = blockIdx.x;
  const int r = (NKQ * NR != 2 || b < a.ncu || nb > 2 * a.ncu) ? b : nb - 1 - (b - a.ncu);
  const int g = r % nkv;
  const int qb = nqb - 1 - r / nkv;
  const int P0 = a.p0 + qb * PB;
  const int P1 = min(P0 + PB, a.p0 + a.T);  // block positions [P0, P1)
  const int kend = P1;                      // keys [0, kend)
  const int nkt = (kend + KT - 1) / KT;

  // query head of the group, row half, key group
  const int hh = wave / (NKQ * NR), rh = (wave / NKQ) % NR, kh = wave % NKQ;
  const int hq = g * G + hh;
  const int R0 = P0 + rh * PR;              // this wave's first position
  const int last = min(R0 + PR, P1) - 1;    // its last key (below R0 when the half is past the end)
  const int n = lane & 31, h = lane >> 5;
  const int posn = R0 + n;

  // batched prefill: this block's sequence and its rows of q and out
  const int bz = blockIdx.y;
  const int seq = a.nbatch > 1 ? a.seqs[bz] : a.seq;
  const float* qrows = a.q + (size_t)bz * a.T * a.ldq;
  bf16_t* orows = a.out + (size_t)bz * a.T * a.ldo;
  const size_t head_off = (size_t)(seq * nkv + g) * a.cap * HD;
  const f16_t* Kg = a.kc + head_off;
  const f16_t* Vg = a.vc + head_off;
  // buffer resources over this KV head's rows (whole tiles are read through
  // them: a scalar tile offset and a constant lane offset per instruction)
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(Kg, a.cap * HD * 2);
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(Vg, a.cap * HD * 2);

  // q (B operand of the score product): row posn, hd ks*16 + h*8 + e.  The
  // lane pair (n, n + 32) holds the whole head, and the RoPE partner d + 64 of
  // hd d < 64 sits in the same lane at ks + NKS/2.  The key-half-0 wave of a
  // query head prepares the fragments and hands them to its partner through
  // LDS (with two row halves, every wave prepares its own); all keep them in
  // registers for the whole key loop.
  f16x8_t qf[NKS];
  if ((NR == 2 || kh == 0) && !a.q16) {
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
      if (NR == 2) qf[ks] = f;
      else *reinterpret_cast<f16x8_t*>(&qlds[((hh * NKS + ks) * 64 + lane) * 8]) = f;
    }
  }

  // staging: tiles go from the cache straight into LDS (global_load_lds_dwordx4,
  // no registers, no LDS store instructions).  Load instruction i of wave w
  // covers key rows RPI (w * NLI + i) .. +RPI-1 of the tile; lane l takes row
  // l / CPR and global chunk (l % CPR) ^ (row % CPR), so the rows land
  // swizzled.  Rows are clamped to the block's last key (always in bounds;
  // keys past it are masked in the scores, and their P is 0 against finite V).
  const int srow = lane / CPR, sslot = lane % CPR;
  // byte offset of this lane's 16 bytes in load instruction i, from the
  // tile's first row (a tile wholly before the block's last key is read
  // from a uniform base plus these; a tile that reaches past it clamps rows)
  uint32_t goff[NLI];
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int key_ = RPI * (wave * NLI + i) + srow;
    goff[i] = (uint32_t)(key_ * HD + (sslot ^ swz(key_)) * 8) * 2;
  }
#define QA_ISSUE(KT_, BUF)                                                                \
  do {                                                                                    \
    if (((KT_) + 1) * KT <= kend) {                                                       \
      const uint32_t soff_ = (uint32_t)(KT_) * KT * HD * 2;                               \
      _Pragma("unroll") for (int i = 0; i < NLI; ++i) {                                   \
        f16_t* const l_ = lds + (BUF) * KT * HD + RPI * (wave * NLI + i) * HD;            \
        lds_load16_buf(krs, goff[i], soff_, l_);                                          \
        lds_load16_buf(vrs, goff[i], soff_, l_ + 2 * KT * HD);                            \
      }                                                                                   \
    } else {                                                                              \
      _Pragma("unroll") for (int i = 0; i < NLI; ++i) {                                   \
        const int r0_ = RPI * (wave * NLI + i), key_ = r0_ + srow;                        \
        const size_t g_ = (size_t)min((KT_) * KT + key_, kend - 1) * HD + (sslot ^ swz(key_)) * 8; \
        f16_t* const l_ = lds + (BUF) * KT * HD + r0_ * HD;                               \
        lds_load16(Kg + g_, l_);                                                          \
        lds_load16(Vg + g_, l_ + 2 * KT * HD);                                            \
      }                                                                                   \
    }                                                                                     \
  } while (0)

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  float mref = 0.f;            // the scores' reference: m_run once finite
  float thr = -INFINITY;       // a row maximum (relative to mref) past this moves the reference
  f32x16_t cin = f32x16_t{};   // -mref in every register: the score accumulator's start

  // A-operand row of the score product held by this lane: key tau(n) of this
  // wave's 32-key half
  const int krow = kh * 32 + tau(n);
  // operand reads are inline asm with explicit waits: the compiler would wait
  // for every outstanding direct-to-LDS load (the next tile's) before a read.
  // K fragment of step ks: row krow, chunk 2 ks + h (swizzled).  V^T fragment
  // (hd rows mt*32 + n, keys kk .. kk+7, kk = kh*32 + sk*16 + h*8) from the
  // key-major V rows by two ds_read_b64_tr_b16: in each 16-lane group lane
  // 4e + q of the group supplies 4 consecutive dims (4q ..) of key e, and lane
  // j receives dim j of keys 0..3 (then 4..7 from the second read).
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int gq = lane >> 4, rq = lane & 15;
  // this lane's V source: key (gq >> 1) * 8 + (rq >> 2) of the 16-key step,
  // dims (gq & 1) * 16 + (rq & 3) * 4 of the 32-dim tile
  const int vkey = (gq >> 1) * 8 + (rq >> 2), vdim = (gq & 1) * 16 + (rq & 3) * 4;
  // this lane's operand addresses in buffer 0, formed once (buffer 1 is the
  // immediate offset KT * HD * 2 bytes further)
  uint32_t koff[NKS], voff[2][NMT][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    koff[ks] = lds_base + (uint32_t)(krow * HD + (((2 * ks + h) ^ swz(krow)) * 8)) * 2;
#pragma unroll
  for (int sk = 0; sk < 2; ++sk)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = kh * 32 + sk * 16 + vkey + hf * 4, dim = mt * 32 + vdim;
        voff[sk][mt][hf] = lds_base + (uint32_t)(2 * KT * HD + key * HD + (((dim >> 3) ^ swz(key)) << 3) + (dim & 7)) * 2;
      }

  auto compute = [&](int kt, auto bufc) {
    constexpr uint32_t BOFF = decltype(bufc)::value * KT * HD * 2;  // buffer byte offset
    const int kbase = kt * KT + kh * 32;  // this wave's first key
    if (kbase > last) return;
    f16x8_t kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[ks]) : "v"(koff[ks]), "n"(BOFF));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(kf[ks]));
    // the row's current reference enters as the accumulator's start (cin,
    // kept in registers and rebuilt only when the reference moves), so s
    // holds the scores minus mref (log2 units; mref 0 while the row has none)
    f32x16_t s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[0], qf[0], cin, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qf[ks], s, 0, 0, 0);
    // causal mask (key <= position) where the half reaches the block's rows
    if (kbase + 31 > R0) {
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
    if (__all(mx == -INFINITY)) return;  // no key of this group is visible to any row
    // V^T fragments of both 16-key steps, all 4 hd tiles
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    s16x4_t vr[2][NMT][2];
#pragma unroll
    for (int sk = 0; sk < 2; ++sk)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(vr[sk][mt][hf]) : "v"(voff[sk][mt][hf]), "n"(BOFF));
    // lazy rescaling: the reference m_run moves only when a row's maximum
    // passes it by more than LAZY (log2 units), so P <= 2^LAZY (exact in
    // float16 up to its rounding) and the O/l rescale, once the maxima have
    // settled, almost never runs; the final 1/l and the merge of the key
    // groups use the same reference, so the result is the softmax itself
    // (mx is relative to mref; thr is -inf while the row has no reference,
    // so any visible key sets one, then LAZY)
    if (__any(mx > thr)) {
      const float m_new = fmaxf(m_run, mx + mref);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      // scores relative to the new reference (a row with no visible key
      // yet keeps reference 0: its P is 0 either way); O and l rescaled
      const float mref_new = m_new == -INFINITY ? 0.f : m_new;
      const float shift = mref_new - mref;
      mref = mref_new;
      thr = m_new == -INFINITY ? -INFINITY : LAZY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] -= shift;
        cin[r] = -mref;
      }
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
    }
    f16x8_t pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (f16_t)__builtin_amdgcn_exp2f(s[r]);  // masked: exp2(-inf) = 0
    // l sums the float16 weights the value product uses, two per dot2
    // instruction (float32 accumulation), in two chains
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ps0 = __builtin_amdgcn_fdot2(h2_t{pf[0][2 * q], pf[0][2 * q + 1]}, one2, ps0, false);
      ps1 = __builtin_amdgcn_fdot2(h2_t{pf[1][2 * q], pf[1][2 * q + 1]}, one2, ps1, false);
    }
    l_run += ps0 + ps1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int sk = 0; sk < 2; ++sk)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) asm volatile("" : "+v"(vr[sk][mt][hf]));
    // O^T += V^T P^T over this half's 32 keys (2 k-steps of 16)
#pragma unroll
    for (int sk = 0; sk < 2; ++sk)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const s16x4_t lo = vr[sk][mt][0], hi = vr[sk][mt][1];
        const s16x4_t v8a = lo, v8b = hi;
        f16x8_t vf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[e] = __builtin_bit_cast(f16_t, (short)v8a[e]);
          vf[e + 4] = __builtin_bit_cast(f16_t, (short)v8b[e]);
        }
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[sk], o[mt], 0, 0, 0);
      }
  };

  // key loop: one tile in flight.  Each iteration waits for its own loads of
  // tile kt, then the raw barrier (not __syncthreads, which would also wait
  // for loads just issued) makes every wave's part of tile kt visible and
  // frees the other buffer, whose next tile is requested before the products.
  QA_ISSUE(0, 0);
  if (a.q16) {  // prepared by the projection: each wave loads its own fragments
    const int t = min(posn - a.p0, a.T - 1);
    const f16_t* qp = reinterpret_cast<const f16_t*>(qrows) + (size_t)t * 2 * a.ldq + (size_t)hq * HD + h * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const f16x8_t*>(qp + ks * 16);
  }
  if constexpr (NR == 1) {
    __syncthreads();  // q fragments (K tile of buffer 1) written
    if (!a.q16) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = *reinterpret_cast<const f16x8_t*>(&qlds[((hh * NKS + ks) * 64 + lane) * 8]);
    }
  }
  // two tiles per iteration, so that each names its buffer as a constant
  for (int kt = 0; kt < nkt; kt += 2) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nkt) QA_ISSUE(kt + 1, 1);
    compute(kt, std::integral_constant<int, 0>{});
    if (kt + 1 >= nkt) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < nkt) QA_ISSUE(kt + 2, 0);
    compute(kt + 1, std::integral_constant<int, 1>{});
  }
#undef QA_ISSUE
  __syncthreads();

  // merge the key groups of each query head through LDS (the tiles are no
  // longer needed): the other groups hand over (m, l, O), the group-0 wave
  // combines and writes
  float* xs = reinterpret_cast<float*>(lds);  // [G][NR][NKQ-1][64 lanes][NMT*16 + 2]
  static_assert(XS == NMT * 16 + 2 && (size_t)G * NR * (NKQ - 1) * 64 * XS * 4 <= sizeof(f16_t) * LDS_HALFS,
                "merge buffer");
  if (kh != 0) {
    float* mine = xs + ((size_t)((hh * NR + rh) * (NKQ - 1) + kh - 1) * 64 + lane) * XS;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[mt * 16 + r] = o[mt][r];
    mine[NMT * 16] = m_run;
    mine[NMT * 16 + 1] = l_run;
  }
  __syncthreads();
  if (kh != 0 || posn >= P1) return;
  const float* part[NKQ - 1];
  float M = m_run;  // finite: key 0 is visible to every row
#pragma unroll
  for (int j = 0; j < NKQ - 1; ++j) {
    part[j] = xs + ((size_t)((hh * NR + rh) * (NKQ - 1) + j) * 64 + lane) * XS;
    M = fmaxf(M, part[j][NMT * 16]);
  }
  const float a0 = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  float aj[NKQ - 1];
  float l = l_run * a0;
#pragma unroll
  for (int j = 0; j < NKQ - 1; ++j) {
    const float mj = part[j][NMT * 16];
    aj[j] = mj == -INFINITY ? 0.f : exp2f(mj - M);
    l += part[j][NMT * 16 + 1] * aj[j];
  }
  const float inv = 1.0f / xor32_sum(l);
  bf16_t* orow = orows + (size_t)(posn - a.p0) * a.ldo + (size_t)hq * HD;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = mt * 32 + rg * 8 + h * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float acc = o[mt][rg * 4 + j] * a0;
#pragma unroll
        for (int p = 0; p < NKQ - 1; ++p) acc += part[p][mt * 16 + rg * 4 + j] * aj[p];
        v[j] = acc * inv;
      }
      uint2 w;
      w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
}

bool attn_prefill_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && group == pa::G;
}

int attn_prefill_rows_per_block(const PrefillAttnArgs& a) {
  if (a.head_dim != 128 || a.rows_per_block == 32) return 32;
  if (a.rows_per_block == 64) return 64;
  // 64 positions per block halve the K/V staging per flop but give every CU
  // one block, so the longest block sets the time: taken where the chunk
  // starts at least its own length into the context (the key ranges of its
  // blocks then differ by at most a factor of two) and the grid fills the
  // chip
  const int nb = (a.T + 63) / 64 * a.n_kv_heads * (a.nbatch > 1 ? a.nbatch : 1);
  return (a.p0 >= a.T && nb >= a.ncu) ? 64 : 32;
}

void launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t st) {
  const int pb = attn_prefill_rows_per_block(a);
  const int nqb = (a.T + pb - 1) / pb;
  const dim3 grid(nqb * a.n_kv_heads, a.nbatch > 1 ? a.nbatch : 1);
  // two key groups per block (four key groups on one item, one block per
  // CU, finished a causal triangle from position 0 sooner while q was
  // prepared here; with q from the projection's epilogue two groups are
  // faster there too)
  if (a.head_dim == 128 && pb == 64)
    hipLaunchKernelGGL((k_attn_prefill<128, 2, 2>), grid, dim3(64 * pa::G * 2 * 2), 0, st, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((k_attn_prefill<128, 2, 1>), grid, dim3(64 * pa::G * 2), 0, st, a);
  else
    hipLaunchKernelGGL((k_attn_prefill<64, 2, 1>), grid, dim3(64 * pa::G * 2), 0, st, a);
}

}  // namespace qtalk
