// Matrix-vector products for decode (and short prefill): bf16 or f32 weights,
// float32 activations, float32 accumulation.
//
// The pages' projections are bias-free mul_mat(W, x) with W stored [out][in]
// ("qwentts.cpp src/talker-forward.h", talker_layer_forward) and must
// accumulate in float32 ("transcribe.cpp src/causal_lm/causal_lm.cpp",
// mul_mat_f32acc).  Each wave streams whole weight rows with 16-byte loads
// (1 KiB per wave per step, fully coalesced); activations sit in LDS, already
// RMS-normalised when the call fuses the pre-norm.  Up to 8 activation rows
// share every weight load (4 where 8 rows of float32 would pass 64 KiB of LDS).
#include "kernels.h"

namespace qtalk {

template <typename WT>
struct WTraits;
template <>
struct WTraits<float> {
  static constexpr int E = 4;  // elements per 16-byte load
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};
template <>
struct WTraits<bf16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    unpack8_bf16(v, f);
  }
};

constexpr int GEMV_NT = 256;
constexpr int GEMV_WAVES = GEMV_NT / 64;

template <typename WT, int NR, int EPI>
__global__ __launch_bounds__(GEMV_NT) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];  // [NR][K]
  __shared__ float red[GEMV_WAVES];
  __shared__ float inv_s[NR];
  constexpr int E = WTraits<WT>::E;
  const int K = a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nr = a.nrows;

  // stage the activation rows; optional fused RMSNorm
  for (int r = 0; r < NR; ++r) {
    float ss = 0.f;
    if (r < nr) {
      const float* xr = a.X + (size_t)r * a.ldx;
      for (int k = tid * 4; k < K; k += GEMV_NT * 4) {
        float4 v = *reinterpret_cast<const float4*>(xr + k);
        *reinterpret_cast<float4*>(xs + r * K + k) = v;
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    } else {
      for (int k = tid * 4; k < K; k += GEMV_NT * 4)
        *reinterpret_cast<float4*>(xs + r * K + k) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (a.gain) {
      ss = block_sum<GEMV_NT>(ss, red);
      if (tid == 0) inv_s[r] = rsqrtf(ss / (float)K + a.eps);
    }
  }
  __syncthreads();
  if (a.gain) {
    for (int r = 0; r < nr; ++r) {
      const float inv = inv_s[r];
      for (int k = tid; k < K; k += GEMV_NT) xs[r * K + k] = xs[r * K + k] * inv * a.gain[k];
    }
    __syncthreads();
    if (a.norm_out && blockIdx.x == 0) {
      for (int r = 0; r < nr; ++r)
        for (int k = tid; k < K; k += GEMV_NT) a.norm_out[(size_t)r * a.ld_norm + k] = xs[r * K + k];
    }
  }

  constexpr int RW = (EPI == EPI_SWIGLU) ? 2 : 1;  // weight rows per wave
  const int lrow = blockIdx.x * GEMV_WAVES + wave;  // logical output row
  if (lrow >= a.O) return;
  const WT* W = reinterpret_cast<const WT*>(a.W);
  size_t wrow[RW];
  if (EPI == EPI_SWIGLU) {
    const size_t pg = (size_t)(lrow >> 4) * 32 + (lrow & 15);
    wrow[0] = pg;
    if (RW > 1) wrow[RW - 1] = pg + 16;
  } else {
    wrow[0] = (size_t)lrow;
  }

  float acc[NR][RW];
#pragma unroll
  for (int n = 0; n < NR; ++n)
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[n][j] = 0.f;

  const int nsteps = (K + 64 * E - 1) / (64 * E);
#pragma unroll 4
  for (int s = 0; s < nsteps; ++s) {
    const int k0 = (s * 64 + lane) * E;
    if (k0 < K) {
      float wf[RW][E];
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const uint4 wv = ld_stream16(W + wrow[j] * (size_t)K + k0);
        WTraits<WT>::unpack(wv, wf[j]);
      }
#pragma unroll
      for (int n = 0; n < NR; ++n) {
        float xv[E];
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(xs + n * K + k0 + e);
          xv[e] = v.x;
          xv[e + 1] = v.y;
          xv[e + 2] = v.z;
          xv[e + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < RW; ++j)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[n][j] = fmaf(wf[j][e], xv[e], acc[n][j]);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NR; ++n)
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[n][j] = wave_sum(acc[n][j]);

  if (lane == 0) {
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      if (n < nr) {
        float* y = a.Y + (size_t)n * a.ldy + lrow;
        if (EPI == EPI_STORE) *y = acc[n][0];
        else if (EPI == EPI_ADD) *y += acc[n][0];
        else *y = silu_f(acc[n][0]) * acc[n][RW - 1];
      }
    }
  }
}

template <typename WT, int NR>
static void launch_nr(Epilogue epi, const GemvArgs& a, hipStream_t st) {
  const dim3 grid((a.O + GEMV_WAVES - 1) / GEMV_WAVES);
  const size_t lds = (size_t)NR * a.K * sizeof(float);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((k_gemv<WT, NR, EPI_STORE>), grid, dim3(GEMV_NT), lds, st, a); break;
    case EPI_ADD: hipLaunchKernelGGL((k_gemv<WT, NR, EPI_ADD>), grid, dim3(GEMV_NT), lds, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemv<WT, NR, EPI_SWIGLU>), grid, dim3(GEMV_NT), lds, st, a); break;
  }
}

// Each pass streams the whole weight matrix once for up to 8 rows (4 when
// 8 rows of x would not fit 64 KiB of LDS), so a batch of n rows reads the
// weights ceil(n / rows per pass) times.
template <typename WT>
static void launch_t(Epilogue epi, GemvArgs a, hipStream_t st) {
  const int n = a.nrows;
  const int per = (size_t)8 * a.K * sizeof(float) <= 65536 ? 8 : 4;
  for (int r0 = 0; r0 < n; r0 += per) {
    GemvArgs g = a;
    g.X = a.X + (size_t)r0 * a.ldx;
    g.Y = a.Y + (size_t)r0 * a.ldy;
    g.norm_out = a.norm_out ? a.norm_out + (size_t)r0 * a.ld_norm : nullptr;
    g.nrows = n - r0 < per ? n - r0 : per;
    if (g.nrows == 1) launch_nr<WT, 1>(epi, g, st);
    else if (g.nrows == 2) launch_nr<WT, 2>(epi, g, st);
    else if (g.nrows <= 4) launch_nr<WT, 4>(epi, g, st);
    else launch_nr<WT, 8>(epi, g, st);
  }
}

void launch_gemv(bool w_bf16, Epilogue epi, GemvArgs a, hipStream_t st) {
  if (w_bf16) launch_t<bf16_t>(epi, a, st);
  else launch_t<float>(epi, a, st);
}

}  // namespace qtalk
