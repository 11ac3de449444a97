// Batch-1 decode of the whole Talker stack in ONE persistent launch.
//
// Why: a decode token at the Talker's shapes is ~170 dependent steps of at
// most a few MiB each; as separate launches every step pays launch and ramp
// latency.  Here 256 blocks (one per CU, co-resident by cooperative launch)
// walk the layers together.  Between steps they exchange activations as
// 8-byte words (float value, 32-bit epoch) written with device-coherent
// stores: a reader polls the words themselves until every epoch matches the
// current launch, so data and synchronisation travel together and no grid
// barrier is needed.  Each block issues the weight loads of its next step
// before it waits, so the HBM stream overlaps the exchange latency.
//
// Steps per layer (math as in "qwentts.cpp src/talker-forward.h",
// talker_layer_forward):
//   QKV : x -> RMSNorm(g_in) -> [q|k|v] rows 16b..16b+15      -> E1
//   ATT : q/k norm + NEOX RoPE, new K/V appended (f16), split-KV causal GQA
//         over 32 key chunks per KV head; the last chunk block of a head
//         merges the chunks (log-sum-exp)                    -> E2
//   O   : x + o @ Wo^T, rows 4b..4b+3                         -> E3
//   GU  : RMSNorm(g_post), 12 gate|up row pairs, silu(g)*u    -> E4
//   D   : x + a @ Wd^T, rows 4b..4b+3                         -> E5
// then final RMSNorm + codec_head rows 12b..12b+11 -> logits.
//
// Specialised to the Talker geometry (hidden 1024, 16/8 heads of 128,
// intermediate 3072, vocab 3072, bf16 weights, f16 cache); other shapes use
// the per-step kernels.
#include "kernels.h"

namespace qtalk {
namespace pd {

constexpr int NB = 256;
constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int H = 1024, QD = 2048, KVD = 1024, QKV = QD + 2 * KVD, I = 3072, V = 3072;
constexpr int HD = 128, NQ = 16, NKV = 8, G = 2;
constexpr int NCH = NB / NKV;  // key chunks per KV head
constexpr int OFF_E1 = 0, OFF_E2 = OFF_E1 + QKV, OFF_E3 = OFF_E2 + QD, OFF_E4 = OFF_E3 + H,
              OFF_E5 = OFF_E4 + I, WORDS_PER_LAYER = OFF_E5 + H;
constexpr int PART_WORDS = NKV * NCH * G * (HD + 2);  // per layer
constexpr long SPIN_LIMIT = 1L << 21;

static_assert(QKV % NB == 0 && H % NB == 0 && I % NB == 0 && V % NB == 0, "row split");

}  // namespace pd



namespace pd {

__device__ __forceinline__ uint64_t ld_ll(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ll(uint64_t* p, float v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
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

// Exchange-word wait split in two: issue() sends the first poll, so the
// caller can queue the next step's weight loads behind it (loads complete in
// issue order); finish() re-polls stale words until every epoch equals `ep`
// and stores the values to dst (LDS).  finish() is false if the wait gave up.
template <int MAXW>
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
      if (k * NT + tid < n) v[k] = ld_ll(src + k * NT + tid);
  }
  template <typename Store>
  __device__ __forceinline__ bool finish(uint32_t ep, int* err, Store store) {
    const int tid = threadIdx.x;
    long spins = 0;
    while (true) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < MAXW; ++k)
        if (k * NT + tid < n && (uint32_t)(v[k] >> 32) != ep) ok = false;
      if (ok) break;
      ++spins;
      if ((spins & 255) == 0 && err_set(err)) return false;
      if (spins > SPIN_LIMIT) {
        raise_err(err, 1);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < MAXW; ++k)
        if (k * NT + tid < n && (uint32_t)(v[k] >> 32) != ep) v[k] = ld_ll(src + k * NT + tid);
    }
#pragma unroll
    for (int k = 0; k < MAXW; ++k)
      if (k * NT + tid < n) store(k * NT + tid, __uint_as_float((uint32_t)v[k]));
    return true;
  }
  __device__ __forceinline__ bool finish_to(uint32_t ep, int* err, float* dst) {
    return finish(ep, err, [&](int i, float x) { dst[i] = x; });
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

// xn[k] = x[k] * rsqrt(mean(x^2) + eps) * g[k] over K = H
__device__ __forceinline__ void rms_to(const float* x, const Gain2& g, float eps, float* xn,
                                       float* redw) {
  const int tid = threadIdx.x;
  const float x0 = x[tid], x1 = x[tid + NT];
  const float ss = block_sum<NT>(x0 * x0 + x1 * x1, redw);
  const float inv = rsqrtf(ss / (float)H + eps);
  xn[tid] = x0 * inv * g.g0;
  xn[tid + NT] = x1 * inv * g.g1;
  __syncthreads();
}

}  // namespace pd

__global__ __launch_bounds__(pd::NT, 1) void k_decode_fused(FusedDecodeArgs a) {
  using namespace pd;
  __shared__ __attribute__((aligned(16))) float xres[H];  // residual stream
  __shared__ __attribute__((aligned(16))) float xin[I];   // input of the current step
  __shared__ float red[32];
  __shared__ float redw[NW];
  __shared__ float qs[G][HD];                              // roped, scaled q
  __shared__ float knew[HD], vnew[HD];
  __shared__ float sp[G][64];
  __shared__ float s_m[G], s_l[G], s_alpha[G];
  __shared__ __attribute__((aligned(16))) float ored[NCH][G * HD];  // slot sums; chunk o's
  __shared__ float mlbuf[NCH][G][2];

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ep = a.epoch;
  const int pos = a.pos;
  const int n_ctx = pos + 1;
  // attention role of this block: KV head g (= the XCD it runs on), key chunk
  // c; the c == 0 block of each head also merges the head's chunks
  const int g = b % NKV, c = b / NKV;
  const int kpb = (n_ctx + NCH - 1) / NCH;
  const int k0 = c * kpb, k1 = min(k0 + kpb, n_ctx);
  const float scale = rsqrtf((float)HD);
  const int slot = tid >> 4, sub = tid & 15;

  // Every step's weight slice is requested one step ahead of its use, right
  // behind that step's first exchange poll, so the HBM stream of step k+1
  // overlaps step k's exchange wait and arithmetic.
  Gp<16, 1, H> gq;        // Wqkv rows 16b .. 16b+15; after the last layer,
                          // codec_head rows 12b .. 12b+11
  Gp<8, 2, QD / 2> go;    // Wo rows 4b .. 4b+3, two K halves
  Gp<24, 1, H> gg;        // 12 gate|up row pairs
  Gp<8, 2, I / 2> gd;     // Wd rows 4b .. 4b+3, two K halves
  auto wqkv_row = [&](int l) {
    const bf16_t* W = a.w + (size_t)l * a.layer_stride;
    return [=](int r) { return W + (size_t)(b * 16 + r) * H; };
  };
  gq.load(wqkv_row(0), wave, lane);

  for (int k = tid; k < H; k += NT) xres[k] = a.emb[k];
  __syncthreads();

  for (int l = 0; l < a.n_layers; ++l) {
    const bf16_t* Wl = a.w + (size_t)l * a.layer_stride;
    const bf16_t* Wo = Wl + (size_t)QKV * H;
    const bf16_t* Wgu = Wo + (size_t)H * QD;
    const bf16_t* Wd = Wgu + (size_t)2 * I * H;
    const float* nl = a.norms + (size_t)l * a.norm_stride;
    const float *g_in = nl, *g_post = nl + H, *g_q = nl + 2 * H, *g_k = nl + 2 * H + HD;
    uint64_t* E = a.ll + (size_t)l * WORDS_PER_LAYER;
    const uint64_t* Eprev = a.ll + (size_t)(l == 0 ? a.n_layers : l - 1) * WORDS_PER_LAYER;
    uint64_t* P = a.part + (size_t)l * PART_WORDS;  // this layer's chunk partials
    const size_t hoff = (size_t)l * a.layer_kv_elems + ((size_t)(a.seq * NKV + g) * a.cap) * HD;
    f16_t* Kp = a.kc + hoff;
    f16_t* Vp = a.vc + hoff;

    // ---------------- QKV ----------------
    {
      LLWait<2> w5;
      if (l > 0) w5.issue(Eprev + OFF_E5, H);
      Gain2 gin;
      gin.load(g_in);
      // the first 64 keys of this block's chunk, for the attention step (in
      // bounds: keys < n_ctx <= cap; the new position is replaced later)
      f16x8_t kr[2], vr[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int j = k0 + p * 32 + slot;
        kr[p] = f16x8_t{};
        vr[p] = f16x8_t{};
        if (j < k1) {
          kr[p] = *reinterpret_cast<const f16x8_t*>(Kp + (size_t)j * HD + sub * 8);
          vr[p] = *reinterpret_cast<const f16x8_t*>(Vp + (size_t)j * HD + sub * 8);
        }
      }
      __asm__ volatile("" ::: "memory");  // keep the prefetch here, ahead of the wait
      if (l > 0) {
        const bool bail = !w5.finish_to(ep, a.err, xres);
        if (__syncthreads_or(bail)) return;
      }
      rms_to(xres, gin, a.eps, xin, redw);
      gq.dot(xin, red, wave, lane);
      __syncthreads();
      if (tid < 16) st_ll(E + OFF_E1 + b * 16 + tid, red[tid], ep);

      // ---------------- attention ----------------
      // this head group's q (2 heads), k, v: one word per thread
      float* raw = xin;  // [0,256) q, [256,384) k, [384,512) v
      float gn;          // QK-norm gain of this thread's channel
      float2 cs;         // RoPE (cos, sin) of this thread's pair
      {
        LLWait<1> w1;
        const int src = tid < 256 ? OFF_E1 + g * 256 + tid
                                  : (tid < 384 ? OFF_E1 + QD + g * HD + (tid - 256)
                                               : OFF_E1 + QD + KVD + g * HD + (tid - 384));
        w1.issue(E + src - tid, tid + 1);  // word tid of (E + src - tid)
        go.load([&](int r) { return Wo + (size_t)(b * 4 + r) * QD; }, wave, lane);
        gn = tid < 256 ? g_q[tid & 127] : g_k[tid & 127];
        if (tid < 192) cs = a.rope[(size_t)pos * (HD / 2) + (tid & 63)];
        const bool bail = !w1.finish(ep, a.err, [&](int, float x) { raw[tid] = x; });
        if (__syncthreads_or(bail)) return;
      }
      // per-head RMSNorm over 128 dims: waves 0-1 q head 0, 2-3 q head 1, 4-5 k
      {
        const float xv = raw[tid];
        const float ss = wave_sum(tid < 384 ? xv * xv : 0.f);
        if (lane == 0) redw[wave] = ss;
        __syncthreads();
        if (tid < 384) {
          const int hh = tid >> 7;  // 0, 1: q heads; 2: k
          const float inv = rsqrtf((redw[2 * hh] + redw[2 * hh + 1]) / (float)HD + a.eps);
          xin[512 + tid] = xv * inv * gn;
        }
        __syncthreads();
      }
      // NEOX RoPE on (i, i + 64); k and v round through the cache type
      if (tid < 192) {
        const int hh = tid >> 6, i = tid & 63;
        const float x1 = xin[512 + hh * 128 + i], x2 = xin[512 + hh * 128 + i + 64];
        const float y1 = x1 * cs.x - x2 * cs.y, y2 = x2 * cs.x + x1 * cs.y;
        if (hh < 2) {
          qs[hh][i] = y1 * scale;
          qs[hh][i + 64] = y2 * scale;
        } else {
          knew[i] = (float)(f16_t)y1;
          knew[i + 64] = (float)(f16_t)y2;
        }
      } else if (tid >= 384) {
        vnew[tid - 384] = (float)(f16_t)raw[tid];
      }
      if (tid < G) {
        s_m[tid] = -INFINITY;
        s_l[tid] = 0.f;
      }
      __syncthreads();
      if (k0 <= pos && pos < k1 && tid < HD) {  // this block owns the new position
        Kp[(size_t)pos * HD + tid] = (f16_t)knew[tid];
        Vp[(size_t)pos * HD + tid] = (f16_t)vnew[tid];
      }
      float acc[G][8];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
      // q of this thread's 8 dims, both heads of the group
      float qr[G][8];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[h][e] = qs[h][sub * 8 + e];
      // one sub-chunk of 64 keys [kb, kb + 64) from registers kk / vv
      auto sub_chunk = [&](int kb, f16x8_t (&kk)[2], f16x8_t (&vv)[2]) {
        if (kb <= pos && pos < kb + 64) {  // the new position: take the fresh K/V
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (kb + p * 32 + slot == pos) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                kk[p][e] = (f16_t)knew[sub * 8 + e];
                vv[p][e] = (f16_t)vnew[sub * 8 + e];
              }
            }
          }
        }
        // scores: 16 lanes per key, 8 dims per lane
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int jl = p * 32 + slot, j = kb + jl;
          float kf[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) kf[e] = (float)kk[p][e];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qr[h][e], kf[e], d);
            d = group_sum<16>(d);
            if (sub == 0) sp[h][jl] = j < k1 ? d : -INFINITY;
          }
        }
        __syncthreads();
        if (wave < G) {  // online softmax, one wave per query head
          const int h = wave;
          const float s = sp[h][lane];
          const float mold = s_m[h];
          const float mnew = fmaxf(mold, wave_max(s));
          const float pv = (s == -INFINITY) ? 0.f : __expf(s - mnew);
          sp[h][lane] = pv;
          const float ps = wave_sum(pv);
          if (lane == 0) {
            const float alpha = (mold == -INFINITY) ? 0.f : __expf(mold - mnew);
            s_alpha[h] = alpha;
            s_l[h] = s_l[h] * alpha + ps;
            s_m[h] = mnew;
          }
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float al = s_alpha[h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int jl = p * 32 + slot;
          float vf[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = (float)vv[p][e];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            // keys past the chunk have probability 0; their (unloaded)
            // registers are zeroed first so no stale value can reach acc
            const float pv = sp[h][jl];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
          }
        }
        __syncthreads();
      };
      if (k0 < k1) sub_chunk(k0, kr, vr);
      for (int kb = k0 + 64; kb < k1; kb += 64) {  // contexts above 32 x 64 keys
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int j = kb + p * 32 + slot;
          kr[p] = f16x8_t{};
          vr[p] = f16x8_t{};
          if (j < k1) {
            kr[p] = *reinterpret_cast<const f16x8_t*>(Kp + (size_t)j * HD + sub * 8);
            vr[p] = *reinterpret_cast<const f16x8_t*>(Vp + (size_t)j * HD + sub * 8);
          }
        }
        sub_chunk(kb, kr, vr);
      }
      // reduce the 32 key slots; publish this chunk's (o, m, l) as words
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) ored[slot][h * HD + sub * 8 + e] = acc[h][e];
      __syncthreads();
      // partial words of (head g, query head h, chunk c) at
      // P + ((g * G + h) * NCH + c) * (HD + 2): o[128], m, l
      if (tid < G * HD) {
        float o = 0.f;
#pragma unroll 8
        for (int s = 0; s < 32; ++s) o += ored[s][tid];
        st_ll(P + ((size_t)(g * G + (tid >> 7)) * NCH + c) * (HD + 2) + (tid & 127), o, ep);
      } else if (tid < G * HD + G) {
        const int h = tid - G * HD;
        const bool empty = k0 >= k1;
        uint64_t* pw = P + ((size_t)(g * G + h) * NCH + c) * (HD + 2);
        st_ll(pw + HD, empty ? -INFINITY : s_m[h], ep);
        st_ll(pw + HD + 1, empty ? 0.f : s_l[h], ep);
      }
      __syncthreads();
    }
    if (c < G) {  // chunk blocks 0 and 1 merge query heads 2g and 2g+1 (log-sum-exp)
      const int h = c;
      constexpr int NWD = NCH * (HD + 2);
      LLWait<(NWD + NT - 1) / NT> wp;
      wp.issue(P + (size_t)(g * G + h) * NWD, NWD);
      const bool bail = !wp.finish(ep, a.err, [&](int i, float x) {
        const int cc = i / (HD + 2), k = i % (HD + 2);
        if (k < HD) ored[cc][k] = x;
        else mlbuf[cc][0][k - HD] = x;
      });
      if (__syncthreads_or(bail)) return;
      if (tid < HD) {
        float M = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) M = fmaxf(M, mlbuf[cc][0][0]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          const float lc = mlbuf[cc][0][1];
          const float wgt = lc > 0.f ? __expf(mlbuf[cc][0][0] - M) : 0.f;
          L = fmaf(wgt, lc, L);
          o = fmaf(wgt, ored[cc][tid], o);
        }
        st_ll(E + OFF_E2 + (g * G + h) * HD + tid, o / L, ep);
      }
    }

    // ---------------- o_proj + residual ----------------
    {
      LLWait<4> w2;
      w2.issue(E + OFF_E2, QD);
      // unit r of the gate|up step: logical row 12b + r/2, gate (r even) or
      // up (r odd); rows are interleaved in blocks of 16 (gate rows, up rows)
      gg.load([&](int r) {
        const int lr = b * 12 + (r >> 1);
        return Wgu + ((size_t)(lr >> 4) * 32 + (lr & 15) + (r & 1) * 16) * H;
      }, wave, lane);
      const bool bail = !w2.finish_to(ep, a.err, xin);
      if (__syncthreads_or(bail)) return;
      go.dot(xin, red, wave, lane);
      __syncthreads();
      if (tid < 4)
        st_ll(E + OFF_E3 + b * 4 + tid, xres[b * 4 + tid] + red[2 * tid] + red[2 * tid + 1], ep);
    }

    // ---------------- gate|up + SwiGLU ----------------
    {
      LLWait<2> w3;
      w3.issue(E + OFF_E3, H);
      Gain2 gpost;
      gpost.load(g_post);
      gd.load([&](int r) { return Wd + (size_t)(b * 4 + r) * I; }, wave, lane);
      const bool bail = !w3.finish_to(ep, a.err, xres);
      if (__syncthreads_or(bail)) return;
      rms_to(xres, gpost, a.eps, xin, redw);
      gg.dot(xin, red, wave, lane);
      __syncthreads();
      if (tid < 12) st_ll(E + OFF_E4 + b * 12 + tid, silu_f(red[2 * tid]) * red[2 * tid + 1], ep);
    }

    // ---------------- down + residual ----------------
    {
      LLWait<6> w4;
      w4.issue(E + OFF_E4, I);
      if (l + 1 < a.n_layers) gq.load(wqkv_row(l + 1), wave, lane);
      else gq.load([&](int r) { return a.head + (size_t)(b * 12 + r) * H; }, wave, lane, 12);
      const bool bail = !w4.finish_to(ep, a.err, xin);
      if (__syncthreads_or(bail)) return;
      gd.dot(xin, red, wave, lane);
      __syncthreads();
      if (tid < 4)
        st_ll(E + OFF_E5 + b * 4 + tid, xres[b * 4 + tid] + red[2 * tid] + red[2 * tid + 1], ep);
    }
  }

  // ---------------- final norm + codec head ----------------
  Gain2 gfin;
  {
    LLWait<2> w5;
    w5.issue(a.ll + (size_t)(a.n_layers - 1) * WORDS_PER_LAYER + OFF_E5, H);
    gfin.load(a.g_final);
    const bool bail = !w5.finish_to(ep, a.err, xres);
    if (__syncthreads_or(bail)) return;
  }
  rms_to(xres, gfin, a.eps, xin, redw);
  if (b == 0 && a.hidden_out)
    for (int k = tid; k < H; k += NT) a.hidden_out[k] = xin[k];
  gq.dot(xin, red, wave, lane);
  __syncthreads();
  if (tid < 12) a.logits[b * 12 + tid] = red[tid];
}

bool fused_decode_supported(int hidden, int q_dim, int kv_dim, int inter, int vocab, int n_heads,
                            int n_kv_heads, int head_dim) {
  return hidden == pd::H && q_dim == pd::QD && kv_dim == pd::KVD && inter == pd::I &&
         vocab == pd::V && n_heads == pd::NQ && n_kv_heads == pd::NKV && head_dim == pd::HD;
}

size_t fused_decode_ll_words(int n_layers) { return (size_t)(n_layers + 1) * pd::WORDS_PER_LAYER; }
size_t fused_decode_part_words(int n_layers) { return (size_t)n_layers * pd::PART_WORDS; }
int fused_decode_blocks() { return pd::NB; }
int fused_decode_threads() { return pd::NT; }

// Cooperative launch guarantees that all NB blocks are resident together (or
// fails).  `cooperative == false` issues an ordinary launch of the same grid,
// for tracing tools that cannot follow cooperative launches; residency then
// rests on fused_decode_fits() and on this stream running nothing else at the
// same time, which holds for the library's single in-order stream.
hipError_t launch_decode_fused(const FusedDecodeArgs& args, hipStream_t st, bool cooperative) {
  FusedDecodeArgs a = args;
  if (!cooperative) {
    hipLaunchKernelGGL(k_decode_fused, dim3(pd::NB), dim3(pd::NT), 0, st, a);
    return hipGetLastError();
  }
  void* params[] = {&a};
  return hipLaunchCooperativeKernel((const void*)k_decode_fused, dim3(pd::NB), dim3(pd::NT), params,
                                    0, st);
}

bool fused_decode_fits() {
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)k_decode_fused, pd::NT, 0) !=
      hipSuccess)
    return false;
  return (long)per * ncu >= pd::NB;
}

}  // namespace qtalk
