// Batch-1 decode of the whole Talker stack in ONE persistent launch.
//
// Why: a decode token at the Talker's shapes is ~170 dependent steps of at
// most a few MiB each; as separate launches every step pays launch and ramp
// latency.  Here 256 blocks (one per CU, all resident together) walk the
// layers together.  Between steps they exchange activations as
// 8-byte words (float value, 32-bit epoch) written with device-coherent
// stores: a reader polls the words themselves until every epoch matches the
// current launch, so data and synchronisation travel together and no grid
// barrier is needed.  Each block issues the weight loads of its next step
// before it waits, so the HBM stream overlaps the exchange latency.
//
// Steps per layer (math as in "qwentts.cpp src/talker-forward.h",
// talker_layer_forward), block (g, c) = (group, chunk):
//   QKV : x -> RMSNorm(g_in) -> 16 rows of head group g's [q|k|v]     -> E1
//   ATT : q/k norm + NEOX RoPE, new K/V appended (f16), split-KV causal GQA
//         over 32 key chunks per KV head, one online softmax per slot;
//         slots combined in-wave (permlane swaps), then across waves   -> P
//   MRG : dims 8(c%16)..+7 of q head 2g+c/16 merged over the 32 chunks
//         (log-sum-exp)                                                  -> OG
//   OP  : o_proj split by group: rows 32c..32c+31 of Wo[:, 256g..256g+255]
//         times head group g's output                                   -> OP
//   XM  : x + sum of the 8 groups' partials for rows 32c..32c+31        -> XM
//   GU  : RMSNorm(g_post), gate|up pairs 384g+12c..+11, silu(g)*u       -> A
//   DP  : down split by group: rows 32c..32c+31 of Wd[:, 384g..384g+383] -> DP
//   XD  : x + sum of the 8 groups' down partials, rows 32c..32c+31      -> XD
// then final RMSNorm + codec_head rows hr*b..hr*b+hr-1 (hr = vocab / 256)
// -> logits.  Only OP and DP
// are read across groups, 256 words per block; every other exchange stays
// inside a group.  The RMSNorms
// are folded into the exchange: the received vector is stored times its gain
// while the sum of squares accumulates, and the norm scale multiplies the dot
// products, so a norm costs no extra block barrier.
//
// Two kinds of exchange.  Words that blocks on other XCDs read are stored and
// polled at device scope; that traffic meets at the memory side (~0.6 us one
// way).  Blocks are dealt to the 8 XCDs in turn, so block b runs on XCD
// (b + r) % 8 for some rotation r.  KV head g is given to the 32 blocks on
// XCD g, which share one L2, and the QKV -> attention and attention -> merge
// exchanges stay inside that L2 when head group g's q/k/v rows are also
// produced there: plain stores (the vector L1 writes through to L2) and
// non-temporal loads (which are not served from a stale L1 line) make a hop
// of ~0.3 us.  The placement is checked when the library is set up; the
// device-scope variant is the fallback.
//
// Specialised to the Talker geometry (hidden 1024, 16/8 heads of 128,
// intermediate 3072, vocab 3072, bf16 weights, f16 cache); other shapes use
// the per-step kernels.
#include <climits>

#include "kernels.h"

namespace qtalk {
namespace pd {

constexpr int NB = 256;
constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int H = 1024, QD = 2048, KVD = 1024, QKV = QD + 2 * KVD, I = 3072;
constexpr int HD = 128, NQ = 16, NKV = 8, G = 2;
constexpr int NCH = NB / NKV;  // key chunks per KV head
// exchange regions of one layer (words); "group" = the 32 blocks of one KV
// head, which share an XCD when the exchanges are XCD-local
constexpr int OFF_E1 = 0;                   // QKV rows [4096], by group
constexpr int OFF_OG = OFF_E1 + QKV;        // merged attention output [8 groups][32 blocks][16]
                                            // (8 used: dims 8(c%16).. of q head 2g + c/16), by group
constexpr int OFF_OP = OFF_OG + NKV * 512;  // o_proj partials [8 groups][1024], all blocks
constexpr int OFF_XM = OFF_OP + NKV * H;    // x after attention [8 groups][1024], one copy per group
constexpr int OFF_A = OFF_XM + NKV * H;     // SwiGLU output [8 groups][32 blocks][16] (12 used)
constexpr int OFF_DP = OFF_A + NKV * 512;   // down partials [8 groups][1024], all blocks
constexpr int OFF_XD = OFF_DP + NKV * H;    // layer output [8 groups][1024], one copy per group
constexpr int WORDS_PER_LAYER = OFF_XD + NKV * H;
// after the two layer regions: each block's candidate of the greedy pick
// (value word, index word)
constexpr int PICK_WORDS = 2 * NB;
constexpr int ISEG = I / NKV, OSEG = QD / NKV;  // down / o_proj input columns per group
// chunk partial (o[HD], m, l) padded to 144 words: each block writes whole
// 128-byte lines, so no line holds words of two writers
constexpr int PST = 144;
constexpr int PART_WORDS = NKV * NCH * G * PST;  // per layer

static_assert(QKV % NB == 0 && H % NB == 0 && I % NB == 0, "row split");

}  // namespace pd



namespace pd {

__device__ __forceinline__ uint64_t ld_ll(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ll(uint64_t* p, float v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// XCD-local exchange words: written with plain stores into the shared L2 and
// read with non-temporal loads, which are not served from a (possibly stale)
// vector L1 line
__device__ __forceinline__ uint64_t ld_loc(const uint64_t* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void st_loc(uint64_t* p, float v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_WAVEFRONT);
}
template <bool LOCAL>
__device__ __forceinline__ uint64_t ld_x(const uint64_t* p) {
  if constexpr (LOCAL) return ld_loc(p);
  else return ld_ll(p);
}
template <bool LOCAL>
__device__ __forceinline__ void st_x(uint64_t* p, float v, uint32_t ep) {
  if constexpr (LOCAL) st_loc(p, v, ep);
  else st_ll(p, v, ep);
}
// v[l] + v[l ^ 32]: v_permlane32_swap exchanges the upper half of one operand
// with the lower half of the other, so its two results hold both values in
// every lane
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// v[l] + v[l ^ 16], by v_permlane16_swap, which exchanges the odd rows (16
// lanes) of one operand with the even rows of the other
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Reduce-scatter steps over the 4 rows of a wave: swap16_add(a, b) holds
// a[l] + a[l ^ 16] in even rows and b[l] + b[l ^ 16] in odd rows;
// swap32_add(a, b) holds a[l] + a[l ^ 32] in lanes 0-31, b[l] + b[l ^ 32] in
// lanes 32-63.
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool err_set(const int* err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}
__device__ __forceinline__ void raise_err(int* err, int code) {
  __hip_atomic_store(err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// where a wait reports that it gave up, and after how many re-polls
struct Bail {
  int* err;
  long limit;
};

// Exchange-word wait split in two: issue() sends the first poll, so the
// caller can queue the next step's weight loads behind it (loads complete in
// issue order); finish() re-polls stale words until every epoch equals `ep`
// and stores the values to dst (LDS).  finish() is false if the wait gave up.
template <int MAXW, bool LOCAL = false>
struct LLWait {
  uint64_t v[MAXW];
  const uint64_t* src;
  int n;
  __device__ __forceinline__ void issue(const uint64_t* s, int count) {
    src = s;
    n = count;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if (k * NT + tid < n) v[k] = ld_x<LOCAL>(src + k * NT + tid);
  }
  template <typename Store>
  __device__ __forceinline__ bool finish(uint32_t ep, const Bail& bl, Store store) {
    const int tid = threadIdx.x;
    long spins = 0;
    while (true) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < MAXW; ++k)
        if (k * NT + tid < n && (uint32_t)(v[k] >> 32) != ep) ok = false;
      if (ok) break;
      ++spins;
      if ((spins & 255) == 0 && err_set(bl.err)) return false;
      if (spins > bl.limit) {
        raise_err(bl.err, 1);
        return false;
      }
      // re-poll at once: a poll round trip is the detection granularity,
      // which measured more expensive than the poll traffic
      asm volatile("" ::: "memory");  // the words change under us: reload them
#pragma unroll
      for (int k = 0; k < MAXW; ++k)
        if (k * NT + tid < n && (uint32_t)(v[k] >> 32) != ep) v[k] = ld_x<LOCAL>(src + k * NT + tid);
    }
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if (k * NT + tid < n) store(k * NT + tid, __uint_as_float((uint32_t)v[k]));
    return true;
  }
  __device__ __forceinline__ bool finish_to(uint32_t ep, const Bail& bl, float* dst) {
    return finish(ep, bl, [&](int i, float x) { dst[i] = x; });
  }
};

// A block's share of one matrix-vector step: `units` (<= MAXU) (row, K-part)
// units over the block's waves; each unit reads KSEG contiguous bf16 of its
// row.
template <int MAXU, int S, int KSEG>
struct Gp {
  static constexpr int NU = (MAXU + NW - 1) / NW;
  static constexpr int NL = KSEG / 512;
  static_assert(KSEG % 512 == 0, "k segment");
  uint4 w[NU][NL];
  int units;

  // rowp(r): pointer to the weight row of the block's r-th output row
  template <typename RowP>
  __device__ __forceinline__ void load(RowP rowp, int wave, int lane, int n_units = MAXU) {
    units = n_units;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (u < units) {
        const bf16_t* p = rowp(u / S) + (u % S) * KSEG + lane * 8;
#pragma unroll
        for (int l = 0; l < NL; ++l) w[i][l] = ld_stream16(p + l * 512);
      }
    }
  }
  // out[i] = dot(unit wave + NW*i's weights, xs segment), in every lane
  __device__ __forceinline__ void dot_all(const float* xs, float (&out)[NU], int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      out[i] = 0.f;
      if (u < units) {
        const float* xb = xs + (u % S) * KSEG + lane * 8;
        float acc = 0.f;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          float f[8];
          unpack8_bf16(w[i][l], f);
          const float4 a = *reinterpret_cast<const float4*>(xb + l * 512);
          const float4 b = *reinterpret_cast<const float4*>(xb + l * 512 + 4);
          acc = fmaf(f[0], a.x, acc);
          acc = fmaf(f[1], a.y, acc);
          acc = fmaf(f[2], a.z, acc);
          acc = fmaf(f[3], a.w, acc);
          acc = fmaf(f[4], b.x, acc);
          acc = fmaf(f[5], b.y, acc);
          acc = fmaf(f[6], b.z, acc);
          acc = fmaf(f[7], b.w, acc);
        }
        out[i] = wave_sum(acc);
      }
    }
  }
  // red[u] = dot(unit u's weights, xs segment)
  __device__ __forceinline__ void dot(const float* xs, float* red, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (u < units) {
        const float* xb = xs + (u % S) * KSEG + lane * 8;
        float acc = 0.f;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          float f[8];
          unpack8_bf16(w[i][l], f);
          const float4 a = *reinterpret_cast<const float4*>(xb + l * 512);
          const float4 b = *reinterpret_cast<const float4*>(xb + l * 512 + 4);
          acc = fmaf(f[0], a.x, acc);
          acc = fmaf(f[1], a.y, acc);
          acc = fmaf(f[2], a.z, acc);
          acc = fmaf(f[3], a.w, acc);
          acc = fmaf(f[4], b.x, acc);
          acc = fmaf(f[5], b.y, acc);
          acc = fmaf(f[6], b.z, acc);
          acc = fmaf(f[7], b.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) red[u] = acc;
      }
    }
  }
};

// The gain of the norm over H = 2 * NT: thread t holds g[t] and g[t + NT],
// loaded early so no global load sits on the critical path.
struct Gain2 {
  float g0, g1;
  __device__ __forceinline__ void load(const float* g) {
    g0 = g[threadIdx.x];
    g1 = g[threadIdx.x + NT];
  }
};
static_assert(H == 2 * NT, "two hidden channels per thread");

// Receive an H-vector: x[k] to `x` (LDS), x[k] * g[k] to `xg` (LDS), and this
// thread's share of sum(x^2) to *ss.  RMSNorm is then applied as one scale
// on the dot products: W (x * rsqrt(mean(x^2) + eps) * g) = rsqrt(.) * W (x g).
template <bool LOCAL>
__device__ __forceinline__ bool recv_norm(LLWait<2, LOCAL>& w, uint32_t ep, const Bail& bl, float* x,
                                          float* xg, const Gain2& g, float* ss) {
  float s = 0.f;
  const bool ok = w.finish(ep, bl, [&](int i, float v) {
    x[i] = v;
    xg[i] = v * (i < NT ? g.g0 : g.g1);
    s = fmaf(v, v, s);
  });
  *ss = s;
  return ok;
}

// A block's 32 rows of a column slice of SEG bf16 weights per row: wave w
// takes rows 4w .. 4w+3, 16 lanes per row, SEG / 128 chunks of 8 per lane.
template <int SEG>
struct Slab {
  static constexpr int NC = SEG / 128;
  static_assert(SEG % 128 == 0, "slab width");
  uint4 w[NC];
  // rowp(r): pointer to the first weight of the block's row r (0..31)
  template <typename RowP>
  __device__ __forceinline__ void load(RowP rowp, int wave, int lane) {
    const bf16_t* p = rowp(4 * wave + (lane >> 4)) + (lane & 15) * 8;
#pragma unroll
    for (int j = 0; j < NC; ++j) w[j] = ld_stream16(p + j * 128);
  }
  // dot of the lane's row with xs[0 .. SEG), in all 16 lanes of the row
  __device__ __forceinline__ float dot(const float* xs, int lane) const {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float f[8];
      unpack8_bf16(w[j], f);
      const float* xb = xs + (lane & 15) * 8 + j * 128;
      const float4 a = *reinterpret_cast<const float4*>(xb);
      const float4 b = *reinterpret_cast<const float4*>(xb + 4);
      acc = fmaf(f[0], a.x, acc);
      acc = fmaf(f[1], a.y, acc);
      acc = fmaf(f[2], a.z, acc);
      acc = fmaf(f[3], a.w, acc);
      acc = fmaf(f[4], b.x, acc);
      acc = fmaf(f[5], b.y, acc);
      acc = fmaf(f[6], b.z, acc);
      acc = fmaf(f[7], b.w, acc);
    }
    return row16_sum(acc);
  }
};

// 1 / sqrt(mean(x^2) + eps) from per-wave partial sums in redw[0..NW)
__device__ __forceinline__ float inv_rms(const float* redw, float eps) {
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += redw[i];
  return rsqrtf(t / (float)H + eps);
}

// max over each aligned 32-lane half of the wave
__device__ __forceinline__ float half32_max(float v) { return xor16_max(row16_max(v)); }

// greedy-pick candidate order: the larger value, then the lower index; an
// empty candidate (index INT_MAX) loses to any other.  Candidates hold
// distinct indices, so the order is total and any reduction tree gives the
// same pick.
__device__ __forceinline__ bool pick_better(float v, int i, float bv, int bi) {
  if (bi == INT_MAX) return i != INT_MAX;
  if (i == INT_MAX) return false;
  return v > bv || (v == bv && i < bi);
}

}  // namespace pd

// LOCAL: group exchanges inside the XCD; Q8: Q8_0 cache rows (HD codes, then
// HD / 32 float16 scales) instead of float16 rows; PICK: the greedy pick of
// the logits after the head step
template <bool LOCAL, bool Q8, bool PICK, bool SINGLE>
__global__ __launch_bounds__(pd::NT, 1) void k_decode_fused(FusedDecodeArgs a) {
  using namespace pd;
  constexpr size_t RB = Q8 ? HD + HD / 16 : HD * 2;  // bytes per cache row
  __shared__ __attribute__((aligned(16))) float xres[H];  // residual stream
  __shared__ __attribute__((aligned(16))) float xin[I];   // input of the current product
  __shared__ float araw[QKV / NKV];                        // this head group's q0 | q1 | k | v
  __shared__ float red[32];
  __shared__ float redw[NW];
  __shared__ float qs[G][HD];                              // normed, roped, scaled q
  __shared__ float knew[HD], vnew[HD];                     // the new position's K, V as attended
  __shared__ signed char kcode[HD], vcode[HD];             // Q8_0: its codes
  __shared__ f16_t kscl[HD / 32], vscl[HD / 32];           // Q8_0: its block scales
  __shared__ __attribute__((aligned(16))) float ow[NW][G * HD];  // per-wave attention sums
  __shared__ __attribute__((aligned(16))) float mws[G][NW];      // per-wave softmax max
  __shared__ __attribute__((aligned(16))) float lws[G][NW];      // per-wave softmax sum
  __shared__ float mg[NCH * 10];  // merge input: 8 o values, m, l of each chunk
  __shared__ __attribute__((aligned(16))) float cwt[NCH];  // merge weights of the chunks

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Bail bl{a.err, a.spin_limit};
  // block-wide "some thread gave up": sticky (a block that gives up leaves
  // the kernel), so one barrier per step suffices; a wave that reads a later
  // step's flag early only leaves earlier, which the barrier tolerates
  // (ended waves no longer take part in it)
  __shared__ int s_bail;
  if (tid == 0) s_bail = 0;
  __syncthreads();
  auto sync_bail = [&](bool bail) -> bool {
    if (bail) s_bail = 1;
    __syncthreads();
    return s_bail != 0;
  };
  // exchange words carry epoch (launch epoch * 64 + layer); layers of equal
  // parity share one buffer region (see the layer loop)
  const uint32_t ep0 = a.epoch * 64u;
  const int pos = a.pos;
  const int n_ctx = pos + 1;
  // attention role of this block: KV head g, key chunk c.  With
  // XCD-local exchanges g is the XCD the block runs on: the dispatcher deals
  // blocks to the 8 XCDs in turn (starting where the previous dispatch left
  // off), so blocks 8c .. 8c+7 cover every XCD once and (g, c) is a bijection.
  const int g = LOCAL ? (int)xcc_id() : b % NKV, c = b / NKV;
  // SINGLE (up to 64 keys: the code predictor's contexts, a Talker's first
  // steps): chunk 0 of each KV head takes them all and publishes the
  // normalised output itself, so the merge step and its exchange drop out
  constexpr bool single = SINGLE;
  const int kpb = single ? 64 : (n_ctx + NCH - 1) / NCH;
  const int k0 = c * kpb, k1 = min(k0 + kpb, n_ctx);
  const float scale = 1.4426950408889634f * rsqrtf((float)HD);  // log2(e) / sqrt(HD)
  const int slot = tid >> 4, sub = tid & 15;

  // QKV rows of this block (16 of the packed [q | k | v]).  XCD-local: the
  // rows of head group g (q heads 2g, 2g+1, then k and v of head g) come from
  // the 32 blocks of XCD g, chunk c taking rows 16c .. 16c+15 of that group.
  // Otherwise rows 16b .. 16b+15.
  const int qkv_row0 = !LOCAL ? b * 16
                              : (c < 16 ? g * 2 * HD + c * 16
                                        : (c < 24 ? QD + g * HD + (c - 16) * 16
                                                  : QD + KVD + g * HD + (c - 24) * 16));
  if (LOCAL && g >= NKV) {  // more XCDs than KV heads: not the expected device
    if (tid == 0) raise_err(a.err, 3);
    return;
  }

  // Bulk loads (weight slices, cached K/V rows, norm gains) are issued right
  // after a step's exchange wait has succeeded, for use one step later.  The
  // polls of a wave complete in issue order behind its outstanding loads, so a
  // bulk load requested while a poll is still repeating would hold that poll
  // back by a full HBM round trip; requested after the wait, it has the
  // step's arithmetic plus the next exchange to land.
  Gp<16, 1, H> gq;   // Wqkv rows qkv_row0 .. +15 (two per wave); after the
                     // last layer, codec_head rows 12b .. 12b+11
  Slab<OSEG> go;     // Wo rows 32c .. +31, columns 256g .. +255
  Gp<24, 1, H> gg;   // gate|up row pairs of SwiGLU outputs gu_row0 .. +11
  Slab<ISEG> gd;     // Wd rows 32c .. +31, columns 384g .. +383
  const int gu_row0 = g * ISEG + c * 12;
  auto wqkv_row = [&](int l) {
    const bf16_t* W = a.w + (size_t)l * a.layer_stride;
    return [=](int r) { return W + (size_t)(qkv_row0 + r) * H; };
  };
  // cached K/V rows of keys kb + slot and kb + 32 + slot, dims sub*8 .. +8.
  // The loads are unconditional, their key clamped to the last position
  // (n_ctx - 1 = pos < cap, always in bounds); keys at or past the chunk end
  // are masked by selects in the attention step.  (A conditional load would
  // make the compiler wait for every outstanding load where the branches
  // join, including the weight slices in flight for the next step.)
  // f16 rows: 8 values per lane; Q8_0 rows: 8 codes and the scale of their
  // 32-value block (codes then scales in each row)
  f16x8_t kr[2], vr[2];
  uint2 kq[2], vq[2];
  f16_t ksc[2], vsc[2];
  auto load_rows = [&](const char* K, const char* V, int kb) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int j = min(kb + p * 32 + slot, n_ctx - 1);
      const char* kp = K + (size_t)j * RB;
      const char* vp = V + (size_t)j * RB;
      if constexpr (Q8) {
        kq[p] = *reinterpret_cast<const uint2*>(kp + sub * 8);
        vq[p] = *reinterpret_cast<const uint2*>(vp + sub * 8);
        ksc[p] = *reinterpret_cast<const f16_t*>(kp + HD + (sub >> 2) * 2);
        vsc[p] = *reinterpret_cast<const f16_t*>(vp + HD + (sub >> 2) * 2);
      } else {
        kr[p] = *reinterpret_cast<const f16x8_t*>(kp + sub * 16);
        vr[p] = *reinterpret_cast<const f16x8_t*>(vp + sub * 16);
      }
    }
  };
  // the first 64 keys of this block's chunk in layer l (the new position is
  // replaced in the attention step)
  auto load_kv = [&](int l) {
    const size_t hoff = (size_t)l * a.layer_kv_bytes + ((size_t)(a.seq * NKV + g) * a.cap) * RB;
    load_rows(a.kc + hoff, a.vc + hoff, k0);
  };
  // Rows 32c .. 32c+31 of x + (sum of the 8 groups' partials in PP): thread t
  // polls partial t & 15 (duplicated for t & 15 >= 8, weighted 0) of row
  // 32c + t / 16 (device scope); a fixed-order 16-lane sum adds them onto the
  // residual and lane 0 of the row publishes it to this group's copy XOUT.
  auto reduce_rows = [&](const uint64_t* PP, uint32_t epw, uint64_t* XOUT) -> bool {
    const int jr = tid >> 4, gp = tid & 15;
    const uint64_t* word = PP + (gp & 7) * H + 32 * c + jr;
    LLWait<1> wr;
    wr.issue(word - tid, NT);
    float v = 0.f;
    const bool ok = wr.finish(epw, bl, [&](int, float x) { v = x; });
    const float s = row16_sum(gp < NKV ? v : 0.f);
    if (gp == 0) st_x<LOCAL>(XOUT + g * H + 32 * c + jr, xres[32 * c + jr] + s, epw);
    return ok;
  };
  Gain2 gin;  // input-norm gain of the next layer
  // layer-0 input: emb, or one table row looked up here (the code
  // predictor's previous code; a sum of several tables is formed by a gather
  // kernel before the launch).  Its loads go out first, the bulk loads
  // behind them, and the values reach LDS once they have landed.
  float e0, e1;
  bool e_bad = false;
  if (a.n_gather) {
    const int id = a.gids[0];
    e_bad = id < 0 || id >= a.grows[0];
    const float* row = a.gtab[0] + (size_t)min(max(id, 0), a.grows[0] - 1) * H;
    e0 = row[tid];
    e1 = row[tid + NT];
    if (a.goverlay) {
      e0 += a.goverlay[tid];
      e1 += a.goverlay[tid + NT];
    }
  } else {
    e0 = a.emb[tid];
    e1 = a.emb[tid + NT];
  }
  gq.load(wqkv_row(0), wave, lane);
  load_kv(0);
  gin.load(a.norms);
  if (e_bad) {  // an id outside the table: a NaN row, reported at sync
    e0 = e1 = __int_as_float(0x7fc00000);
    if (b == 0 && tid == 0) *a.gstatus = 5;
  }
  xres[tid] = e0;
  xres[tid + NT] = e1;

  for (int l = 0; l < a.n_layers; ++l) {
    const bf16_t* Wl = a.w + (size_t)l * a.layer_stride;
    const bf16_t* Wo = Wl + (size_t)QKV * H;
    const bf16_t* Wgu = Wo + (size_t)H * QD;
    const bf16_t* Wd = Wgu + (size_t)2 * I * H;
    const float* nl = a.norms + (size_t)l * a.norm_stride;
    const float *g_post = nl + H, *g_q = nl + 2 * H, *g_k = nl + 2 * H + HD;
    // Layers l and l + 2 share the exchange and partial regions (parity
    // double buffering keeps them cache-resident).  Reuse is safe: a block
    // writes layer l + 2's words only after it has received words of layer
    // l + 1 that, through the chain of waits, every block produced after it
    // finished reading layer l's words.  The epoch tells the two layers apart.
    const uint32_t ep = ep0 + (uint32_t)l;
    uint64_t* E = a.ll + (size_t)(l & 1) * WORDS_PER_LAYER;
    uint64_t* Eprev = a.ll + (size_t)((l + 1) & 1) * WORDS_PER_LAYER;
    uint64_t* P = a.part + (size_t)(l & 1) * PART_WORDS;  // this layer's chunk partials
    const size_t hoff = (size_t)l * a.layer_kv_bytes + ((size_t)(a.seq * NKV + g) * a.cap) * RB;
    char* Kp = a.kc + hoff;
    char* Vp = a.vc + hoff;

    // ---------------- XD (previous layer's output) + QKV ----------------
    float gn, gnp;  // QK-norm gains of this thread's attention channel and of its RoPE partner
    float2 cs;      // RoPE (cos, sin) of this thread's pair
    {
      float ss;
      bool bail = false;
      if (l > 0) {
        // layer l - 1's down partials -> its output rows -> this group's copy
        bail = !reduce_rows(Eprev + OFF_DP, ep - 1, Eprev + OFF_XD);
        LLWait<2, LOCAL> wx;
        wx.issue(Eprev + OFF_XD + g * H, H);
        bail = bail || !recv_norm(wx, ep - 1, bl, xres, xin, gin, &ss);
      } else {
        // the layer-0 input row, loaded before the loop into xres (this
        // thread's own two elements: no barrier)
        const float x0 = xres[tid], x1 = xres[tid + NT];
        xin[tid] = x0 * gin.g0;
        xin[tid + NT] = x1 * gin.g1;
        ss = x0 * x0 + x1 * x1;
      }
      // next step's bulk loads
      const float* gsel = tid < 256 ? g_q : g_k;
      gn = gsel[tid & 127];
      gnp = gsel[(tid & 127) ^ 64];
      cs = a.rope[(size_t)pos * (HD / 2) + (tid & 63)];
      go.load([&](int r) { return Wo + (size_t)(32 * c + r) * QD + g * OSEG; }, wave, lane);
      ss = wave_sum(ss);
      if (lane == 0) redw[wave] = ss;
      if (sync_bail(bail)) return;
      const float inv = inv_rms(redw, a.eps);
      float v[2];  // rows wave and wave + 8 of this block's 16
      gq.dot_all(xin, v, wave, lane);
      if (lane < 2) st_x<LOCAL>(E + OFF_E1 + qkv_row0 + wave + NW * lane, (lane ? v[1] : v[0]) * inv, ep);
    }

    // ---------------- attention ----------------
    {
      {
        // q0 | q1 | k | v of head group g, one word per thread
        LLWait<1, LOCAL> w1;
        const int src = tid < 256 ? OFF_E1 + g * 256 + tid
                                  : (tid < 384 ? OFF_E1 + QD + g * HD + (tid - 256)
                                               : OFF_E1 + QD + KVD + g * HD + (tid - 384));
        w1.issue(E + src - tid, tid + 1);  // word tid of (E + src - tid)
        float v = 0.f;
        const bool bail = !w1.finish(ep, bl, [&](int, float x) { v = x; });
        araw[tid] = v;
        const float sq = wave_sum(v * v);  // waves 0-1 q0, 2-3 q1, 4-5 k, 6-7 v
        if (lane == 0) redw[wave] = sq;
        if (sync_bail(bail)) return;
      }
      // next step's bulk loads (the o_proj input comes from the merge, a
      // further exchange away)
      gg.load([&](int r) {
        // unit r: logical row 12b + r/2, gate (r even) or up (r odd); rows are
        // interleaved in blocks of 16 (gate rows, up rows)
        const int lr = gu_row0 + (r >> 1);
        return Wgu + ((size_t)(lr >> 4) * 32 + (lr & 15) + (r & 1) * 16) * H;
      }, wave, lane);
      // per-head RMSNorm, NEOX RoPE on (i, i + 64).  f16 cache: the new k and
      // v are attended as the cache stores them (read after write).  Q8_0
      // cache: they are attended unquantised, as computed, while the codes
      // and scales go to the cache (the 32-value block of a k or v dim is one
      // half of its wave)
      {
        float y;
        if (tid < 384) {
          const int hh = tid >> 7, j = tid & 127;
          const float inv = rsqrtf((redw[2 * hh] + redw[2 * hh + 1]) / (float)HD + a.eps);
          const float xj = araw[tid] * inv * gn;
          const float xp = araw[tid ^ 64] * inv * gnp;
          y = j < 64 ? xj * cs.x - xp * cs.y : xj * cs.x + xp * cs.y;
          if (hh < 2) qs[hh][j] = y * scale;
        } else {
          y = araw[tid];
        }
        if (tid >= 256) {  // k (waves 4-5) or v (waves 6-7) dim tid & 127
          const int j = tid & 127;
          float c;
          if constexpr (Q8) {
            const float d = half32_max(fabsf(y)) / 127.0f;
            const float code = roundf(y * (d > 0.f ? 1.0f / d : 0.f));
            (tid < 384 ? kcode : vcode)[j] = (signed char)code;
            if ((lane & 31) == 0) (tid < 384 ? kscl : vscl)[j >> 5] = (f16_t)d;
            c = y;
          } else {
            c = (float)(f16_t)y;
          }
          (tid < 384 ? knew : vnew)[j] = c;
        }
      }
      __syncthreads();
      if (k0 <= pos && pos < k1 && tid < HD) {  // this block owns the new position
        char* kp = Kp + (size_t)pos * RB;
        char* vp = Vp + (size_t)pos * RB;
        if constexpr (Q8) {
          kp[tid] = kcode[tid];
          vp[tid] = vcode[tid];
          if (tid < HD / 32) {
            reinterpret_cast<f16_t*>(kp + HD)[tid] = kscl[tid];
            reinterpret_cast<f16_t*>(vp + HD)[tid] = vscl[tid];
          }
        } else {
          reinterpret_cast<f16_t*>(kp)[tid] = (f16_t)knew[tid];
          reinterpret_cast<f16_t*>(vp)[tid] = (f16_t)vnew[tid];
        }
      }
      // keys [k0, k1), 64 per pass: thread (slot, sub) takes keys kb + slot and
      // kb + 32 + slot, dims sub*8 .. +8.  Each slot (16 lanes) keeps its own
      // online softmax, scores in log2 units (q carries log2(e)), so the loop
      // needs no reduction across slots; the 32 slots are combined once after.
      float qr[G][8], kn[8], vn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kn[e] = knew[sub * 8 + e];
        vn[e] = vnew[sub * 8 + e];
#pragma unroll
        for (int h = 0; h < G; ++h) qr[h][e] = qs[h][sub * 8 + e];
      }
      float acc[G][8];
      float m_run[G], l_run[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
      }
      // one pass over keys kb + slot, kb + 32 + slot held in kr, vr
      auto pass = [&](int kb, bool first) {
        const int j0 = kb + slot, j1 = kb + 32 + slot;
        float kf[2][8], vf[2][8];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if constexpr (Q8) {
            const float ks = (float)ksc[p], vs = (float)vsc[p];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              kf[p][e] = (float)(signed char)(kq[p].x >> (8 * e)) * ks;
              kf[p][e + 4] = (float)(signed char)(kq[p].y >> (8 * e)) * ks;
              vf[p][e] = (float)(signed char)(vq[p].x >> (8 * e)) * vs;
              vf[p][e + 4] = (float)(signed char)(vq[p].y >> (8 * e)) * vs;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kf[p][e] = (float)kr[p][e];
              vf[p][e] = (float)vr[p][e];
            }
          }
        }
        if (j1 >= pos) {  // rare: the new position (fresh K/V) or keys past the chunk
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int j = p ? j1 : j0;
            const bool fresh = j == pos, dead = j >= k1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              kf[p][e] = fresh ? kn[e] : kf[p][e];
              vf[p][e] = dead ? 0.f : (fresh ? vn[e] : vf[p][e]);  // stale rows out
            }
          }
        }
        float s[2][G];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qr[h][e], kf[p][e], d);
            s[p][h] = group_sum<16>(d);
          }
        if (j1 >= k1) {  // rare: keys past the chunk end
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (j0 >= k1) s[0][h] = -INFINITY;
            s[1][h] = -INFINITY;
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float m_new = fmaxf(m_run[h], fmaxf(s[0][h], s[1][h]));
          const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // slot with no key yet
          const float p0 = __builtin_amdgcn_exp2f(s[0][h] - m_ref);
          const float p1 = __builtin_amdgcn_exp2f(s[1][h] - m_ref);
          if (first) {
            l_run[h] = p0 + p1;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p1, vf[1][e], p0 * vf[0][e]);
          } else {
            const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_ref);
            l_run[h] = fmaf(l_run[h], alpha, p0 + p1);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc[h][e] = fmaf(p1, vf[1][e], fmaf(p0, vf[0][e], acc[h][e] * alpha));
          }
          m_run[h] = m_new;
        }
      };
      if (k0 < k1) pass(k0, true);                    // rows loaded a step ahead
      for (int kb = k0 + 64; kb < k1; kb += 64) {     // contexts above 32 x 64 keys
        load_rows(Kp, Vp, kb);
        pass(kb, false);
      }
      // combine the 32 slots.  Inside a wave (its 4 rows = 4 slots): scale
      // each slot by 2^(m_slot - m_wave) and add the rows by permlane swaps,
      // reduce-scattered so that row r ends with head r % 2, dims sub * 8 +
      // 4 (r / 2) .. +3.  Then across the 8 waves through LDS.
      {
        const int row = lane >> 4;
        float mwv[G], scv[G], lwv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          mwv[h] = xor32_max(xor16_max(m_run[h]));
          scv[h] = m_run[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - mwv[h]);
          lwv[h] = xor32_sum(xor16_sum(l_run[h] * scv[h]));
        }
        float r1[8];  // rows 0, 2: head 0; rows 1, 3: head 1 (sums of row pairs)
#pragma unroll
        for (int e = 0; e < 8; ++e) r1[e] = swap16_add(acc[0][e] * scv[0], acc[1][e] * scv[1]);
        float r2[4];  // rows 0, 1: dims 0..3; rows 2, 3: dims 4..7 (sums of all rows)
#pragma unroll
        for (int e = 0; e < 4; ++e) r2[e] = swap32_add(r1[e], r1[e + 4]);
        *reinterpret_cast<float4*>(&ow[wave][(row & 1) * HD + sub * 8 + (row >> 1) * 4]) =
            make_float4(r2[0], r2[1], r2[2], r2[3]);
        if (lane < G) {
          mws[lane][wave] = lane ? mwv[1] : mwv[0];
          lws[lane][wave] = lane ? lwv[1] : lwv[0];
        }
      }
      __syncthreads();
      // partial words of (head g, query head h, chunk c) at
      // P + ((g * G + h) * NCH + c) * PST: o[128] (unnormalised), m (log2
      // units), l.  o value (h, i) = output wave * 32 + lane % 32 is summed
      // over waves 4 (lane / 32) .. +3 in each half-wave and the halves added
      // across lanes l and l ^ 32.
      {
        const int out = wave * 32 + (lane & 31), h = out >> 7, i = out & (HD - 1), half = lane >> 5;
        const float4 ma = *reinterpret_cast<const float4*>(&mws[h][0]);
        const float4 mb = *reinterpret_cast<const float4*>(&mws[h][4]);
        const float M = fmaxf(fmaxf(fmaxf(ma.x, ma.y), fmaxf(ma.z, ma.w)), fmaxf(fmaxf(mb.x, mb.y), fmaxf(mb.z, mb.w)));
        // a wave with no key (-inf) weighs 0; so does a chunk past the context
        auto wt = [&](float m) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M); };
        const float4 mm = half ? mb : ma;
        const int w0 = 4 * half;
        float o = wt(mm.x) * ow[w0][out];
        o = fmaf(wt(mm.y), ow[w0 + 1][out], o);
        o = fmaf(wt(mm.z), ow[w0 + 2][out], o);
        o = fmaf(wt(mm.w), ow[w0 + 3][out], o);
        o = xor32_sum(o);
        uint64_t* pw = P + ((size_t)(g * G + h) * NCH + c) * PST;
        if (single) {  // chunk 0 holds every key: o / l into the merged-output words
          if (c == 0 && half == 0) {
            const float4 la = *reinterpret_cast<const float4*>(&lws[h][0]);
            const float4 lb = *reinterpret_cast<const float4*>(&lws[h][4]);
            const float L = wt(ma.x) * la.x + wt(ma.y) * la.y + wt(ma.z) * la.z + wt(ma.w) * la.w +
                            (wt(mb.x) * lb.x + wt(mb.y) * lb.y + wt(mb.z) * lb.z + wt(mb.w) * lb.w);
            st_x<LOCAL>(E + OFF_OG + g * 512 + 16 * (h * 16 + (i >> 3)) + (i & 7), o / L, ep);
          }
        } else if (half == 0) {
          st_x<LOCAL>(pw + i, o, ep);
        }
        if (!single && half == 1 && i < PST - HD) {  // m, l of head h (-inf, 0 past the context), padding
          float v = i == 0 ? M : 0.f;
          if (i == 1) {
            const float4 la = *reinterpret_cast<const float4*>(&lws[h][0]);
            const float4 lb = *reinterpret_cast<const float4*>(&lws[h][4]);
            v = wt(ma.x) * la.x + wt(ma.y) * la.y + wt(ma.z) * la.z + wt(ma.w) * la.w +
                (wt(mb.x) * lb.x + wt(mb.y) * lb.y + wt(mb.z) * lb.z + wt(mb.w) * lb.w);
          }
          st_x<LOCAL>(pw + HD + i, v, ep);
        }
      }
      static_assert(NW * 32 == G * HD && NW == 8 && G == 2, "combine split");
    }
    // ---------------- merge: 8 output dims per block ----------------
    // block (g, c) merges dims d0 .. d0+7 (d0 = 8 (c % 16)) of query head
    // 2g + c / 16 over the group's 32 chunk partials (log-sum-exp): thread
    // t < 320 polls chunk t / 10's word t % 10 (8 o values, then m and l)
    if (!single) {
      const int h = c >> 4, d0 = (c & 15) * 8;
      const uint64_t* pbase = P + (size_t)(g * G + h) * NCH * PST;
      const int tm = min(tid, NCH * 10 - 1), cc = tm / 10, k = tm % 10;
      LLWait<1, LOCAL> wm;
      wm.issue(pbase + cc * PST + (k < 8 ? d0 + k : HD + k - 8) - tid, NCH * 10);
      const bool bail = !wm.finish(ep, bl, [&](int, float x) { mg[tm] = x; });
      if (sync_bail(bail)) return;
      if (wave == 0) {  // lane cc < NCH: chunk cc's weight 2^(m_c - M) / L
        const float mc = lane < NCH ? mg[lane * 10 + 8] : -INFINITY;
        const float lc = lane < NCH ? mg[lane * 10 + 9] : 0.f;
        const float M = wave_max(mc);
        const float wgt = lc > 0.f ? __builtin_amdgcn_exp2f(mc - M) : 0.f;
        const float L = wave_sum(wgt * lc);
        if (lane < NCH) cwt[lane] = wgt / L;
        // one wave: its LDS writes are seen by its later reads.  Lane
        // (q, k) = (lane / 8, lane % 8) sums chunks 4q .. 4q+3 of dim k, then
        // the 8 lanes of each dim are added (lanes k + 8q)
        const int k = lane & 7, q = lane >> 3;
        const float4 w4 = *reinterpret_cast<const float4*>(&cwt[4 * q]);
        float o = w4.x * mg[(4 * q) * 10 + k];
        o = fmaf(w4.y, mg[(4 * q + 1) * 10 + k], o);
        o = fmaf(w4.z, mg[(4 * q + 2) * 10 + k], o);
        o = fmaf(w4.w, mg[(4 * q + 3) * 10 + k], o);
        o += dpp_mov<0x128>(o);  // row_ror:8 -> lane k + 8 of the row
        o = xor32_sum(xor16_sum(o));
        if (lane < 8) st_x<LOCAL>(E + OFF_OG + g * 512 + 16 * c + lane, o, ep);
      }
    }

    // ---------------- o_proj partial of this group ----------------
    Gain2 gpost;
    {
      LLWait<1, LOCAL> wo;  // head group g's merged output, 8 words from each block
      const int to = min(tid, OSEG - 1);
      wo.issue(E + OFF_OG + g * 512 + 16 * (to >> 3) + (to & 7) - tid, OSEG);
      const bool bail = !wo.finish_to(ep, bl, xin);
      // bulk loads: the next step's gain, the next layer's cached keys
      gpost.load(g_post);
      if (l + 1 < a.n_layers) load_kv(l + 1);
      if (sync_bail(bail)) return;
      const float s = go.dot(xin, lane);
      if ((lane & 15) == 0) st_ll(E + OFF_OP + g * H + 32 * c + 4 * wave + (lane >> 4), s, ep);
    }

    // ---------------- XM + gate|up + SwiGLU ----------------
    {
      bool bail = !reduce_rows(E + OFF_OP, ep, E + OFF_XM);
      LLWait<2, LOCAL> wx;
      wx.issue(E + OFF_XM + g * H, H);
      float ss;
      bail = bail || !recv_norm(wx, ep, bl, xres, xin, gpost, &ss);
      // bulk loads: the next layer's input-norm gain and the down step's
      // weight slice (the next layer's QKV slice follows after the down
      // publish)
      if (l + 1 < a.n_layers) {
        gin.load(a.norms + (size_t)(l + 1) * a.norm_stride);
      } else {
        gin.load(a.g_final);
      }
      gd.load([&](int r) { return Wd + (size_t)(32 * c + r) * I + g * ISEG; }, wave, lane);
      ss = wave_sum(ss);
      if (lane == 0) redw[wave] = ss;
      if (sync_bail(bail)) return;
      const float inv = inv_rms(redw, a.eps);
      gg.dot(xin, red, wave, lane);
      __syncthreads();
      if (tid < 12)
        st_x<LOCAL>(E + OFF_A + g * 512 + 16 * c + tid,
                    silu_f(red[2 * tid] * inv) * (red[2 * tid + 1] * inv), ep);
    }

    // ---------------- down partial of this group ----------------
    {
      // SwiGLU outputs 384g .. 384g+383: thread t < 384 reads block t / 12's
      // word t % 12
      LLWait<1, LOCAL> wa;
      const int ta = min(tid, ISEG - 1);
      wa.issue(E + OFF_A + g * 512 + 16 * (ta / 12) + ta % 12 - tid, ISEG);
      const bool bail = !wa.finish_to(ep, bl, xin);
      if (sync_bail(bail)) return;
      const float s = gd.dot(xin, lane);
      if ((lane & 15) == 0) st_ll(E + OFF_DP + g * H + 32 * c + 4 * wave + (lane >> 4), s, ep);
      // after the publish: the next layer's QKV slice, or after the last layer
      // the block's head_rows head rows (unconditional loads; units past them
      // re-read the last one and are not used)
      const bool last = l + 1 == a.n_layers;
      const int hr = a.head_rows;
      const bf16_t* Wn = a.w + (size_t)(last ? l : l + 1) * a.layer_stride;
      gq.load([&](int r) {
        return last ? a.head + (size_t)(b * hr + min(r, hr - 1)) * H : Wn + (size_t)(qkv_row0 + r) * H;
      }, wave, lane);
      gq.units = last ? hr : 16;
    }
  }

  // ---------------- final output rows, norm + codec head ----------------
  {
    const uint32_t epl = ep0 + (uint32_t)(a.n_layers - 1);
    uint64_t* El = a.ll + (size_t)((a.n_layers - 1) & 1) * WORDS_PER_LAYER;
    bool bail = !reduce_rows(El + OFF_DP, epl, El + OFF_XD);
    LLWait<2, LOCAL> wx;
    wx.issue(El + OFF_XD + g * H, H);
    float ss;
    bail = bail || !recv_norm(wx, epl, bl, xres, xin, gin, &ss);  // gin = final gain
    ss = wave_sum(ss);
    if (lane == 0) redw[wave] = ss;
    if (sync_bail(bail)) return;
    const float inv = inv_rms(redw, a.eps);
    if (b == 0 && a.hidden_out)
      for (int k = tid; k < H; k += NT) a.hidden_out[k] = xin[k] * inv;
    gq.dot(xin, red, wave, lane);
    __syncthreads();
    if (tid < a.head_rows) a.logits[b * a.head_rows + tid] = red[tid] * inv;
    if (!PICK) return;
    // greedy pick: wave 0 forms the block's candidate over its head rows and
    // publishes (value, index); block 0 polls the 256 candidates and keeps,
    // in block order, the larger value (the lower index among equals)
    uint64_t* PK = a.ll + (size_t)2 * WORDS_PER_LAYER;
    if (wave == 0) {
      float v = -INFINITY;
      int i = INT_MAX;
      const int id = b * a.head_rows + lane;
      if (lane < a.head_rows && !(id >= a.pick_suppress && id != a.pick_keep)) {
        v = red[lane] * inv;
        v = v != v ? -INFINITY : v;
        i = id;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(i, off);
        if (pick_better(ov, oi, v, i)) {
          v = ov;
          i = oi;
        }
      }
      if (lane == 0) {
        st_ll(PK + 2 * b, v, ep0);
        st_ll(PK + 2 * b + 1, __int_as_float(i), ep0);
      }
    }
    if (b != 0) return;
    // the candidates land in the attention step's per-wave sums (free now)
    float* cv = &ow[0][0];
    int* ci = reinterpret_cast<int*>(&ow[1][0]);
    static_assert(G * HD >= NB, "candidate arrays");
    {
      LLWait<1> wp;
      wp.issue(PK, PICK_WORDS);
      const bool bail = !wp.finish(ep0, bl, [&](int k, float x) {
        if (k & 1) ci[k >> 1] = __float_as_int(x);
        else cv[k >> 1] = x;
      });
      if (sync_bail(bail)) return;
    }
    if (wave == 0) {  // lane l takes blocks l, l + 64, ...: block order kept by the tie rule
      float v = cv[lane];
      int i = ci[lane];
      for (int k = lane + 64; k < NB; k += 64)
        if (pick_better(cv[k], ci[k], v, i)) {
          v = cv[k];
          i = ci[k];
        }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(i, off);
        if (pick_better(ov, oi, v, i)) {
          v = ov;
          i = oi;
        }
      }
      if (lane == 0) *a.pick_out = i == INT_MAX ? -1 : i;
    }
  }
}

bool fused_decode_supported(int hidden, int q_dim, int kv_dim, int inter, int vocab, int n_heads,
                            int n_kv_heads, int head_dim) {
  return hidden == pd::H && q_dim == pd::QD && kv_dim == pd::KVD && inter == pd::I &&
         vocab % pd::NB == 0 && vocab / pd::NB >= 1 && vocab / pd::NB <= 16 && n_heads == pd::NQ &&
         n_kv_heads == pd::NKV && head_dim == pd::HD;
}

size_t fused_decode_ll_words(int) { return (size_t)2 * pd::WORDS_PER_LAYER + pd::PICK_WORDS; }
size_t fused_decode_part_words(int) { return (size_t)2 * pd::PART_WORDS; }
int fused_decode_blocks() { return pd::NB; }

// The NB blocks must be resident together.  An ordinary launch gets that
// from fused_decode_fits() (one block per compute unit, NB <= compute units)
// and from the caller running no other persistent decode on the device at
// the same time; work that merely occupies compute units for a while only
// delays the late blocks, and a wait that outlasts the spin limit becomes
// error 1.  `cooperative == true` has the runtime guarantee it (or fail the
// launch), at ~18 us more per launch.
hipError_t launch_decode_fused(const FusedDecodeArgs& args, hipStream_t st, bool cooperative) {
  FusedDecodeArgs a = args;
  // the greedy pick and the short-context attention are separate
  // instantiations: their code in the common kernel measured 2-3% slower per
  // token even where not taken
  const void* fns[2][2][2][2] = {
      {{{(const void*)k_decode_fused<false, false, false, false>, (const void*)k_decode_fused<false, false, false, true>},
        {(const void*)k_decode_fused<false, false, true, false>, (const void*)k_decode_fused<false, false, true, true>}},
       {{(const void*)k_decode_fused<false, true, false, false>, (const void*)k_decode_fused<false, true, false, true>},
        {(const void*)k_decode_fused<false, true, true, false>, (const void*)k_decode_fused<false, true, true, true>}}},
      {{{(const void*)k_decode_fused<true, false, false, false>, (const void*)k_decode_fused<true, false, false, true>},
        {(const void*)k_decode_fused<true, false, true, false>, (const void*)k_decode_fused<true, false, true, true>}},
       {{(const void*)k_decode_fused<true, true, false, false>, (const void*)k_decode_fused<true, true, false, true>},
        {(const void*)k_decode_fused<true, true, true, false>, (const void*)k_decode_fused<true, true, true, true>}}}};
  const void* fn = fns[a.xcd_local ? 1 : 0][a.kv_q8 ? 1 : 0][a.pick_out ? 1 : 0][a.pos + 1 <= 64 ? 1 : 0];
  void* params[] = {&a};
  if (!cooperative) return hipLaunchKernel(fn, dim3(pd::NB), dim3(pd::NT), params, 0, st);
  return hipLaunchCooperativeKernel(fn, dim3(pd::NB), dim3(pd::NT), params, 0, st);
}

__global__ void k_fill_zero(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

void launch_fill_zero(uint64_t* p, size_t n, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_zero, dim3(256), dim3(256), 0, st, p, n);
}

__global__ void k_xcc_ids(int* ids) {
  if (threadIdx.x == 0) ids[blockIdx.x] = (int)pd::xcc_id();
}

// Whether a co-resident grid of NB blocks places blocks 8c .. 8c+7 on 8
// different XCDs for every c (the dispatcher's round-robin), which the
// XCD-local exchanges rely on.
bool fused_decode_xcd_layout_ok(hipStream_t st, bool cooperative) {
  int* d = nullptr;
  if (hipMalloc(&d, pd::NB * sizeof(int)) != hipSuccess) return false;
  void* params[] = {&d};
  int h[pd::NB];
  hipError_t e;
  if (cooperative) {
    e = hipLaunchCooperativeKernel((const void*)k_xcc_ids, dim3(pd::NB), dim3(64), params, 0, st);
  } else {
    hipLaunchKernelGGL(k_xcc_ids, dim3(pd::NB), dim3(64), 0, st, d);
    e = hipGetLastError();
  }
  bool ok = e == hipSuccess &&
            hipMemcpyAsync(h, d, sizeof(h), hipMemcpyDeviceToHost, st) == hipSuccess &&
            hipStreamSynchronize(st) == hipSuccess;
  for (int c = 0; ok && c < pd::NB / pd::NKV; ++c) {
    unsigned seen = 0;
    for (int i = 0; i < pd::NKV; ++i) {
      const int x = h[c * pd::NKV + i];
      ok = ok && x >= 0 && x < pd::NKV && !(seen >> x & 1u);
      seen |= ok ? 1u << x : 0u;
    }
  }
  (void)hipFree(d);
  return ok;
}

bool fused_decode_fits() {
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)k_decode_fused<true, false, true, false>, pd::NT, 0) !=
      hipSuccess)
    return false;
  return (long)per * ncu >= pd::NB;
}

}  // namespace qtalk
