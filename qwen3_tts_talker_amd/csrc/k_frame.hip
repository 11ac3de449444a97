// Frame-step glue around the Talker, on the device so that a frame of codes
// never returns to the host:
//  * k_embed_sum: the step embedding of each slot, the codec table's row of
//    the codebook-0 id plus each acoustic table's row of its codebook's id
//    plus the slot's overlay row ("qwentts.cpp src/talker-forward.h", the
//    batched step graph's input_embed; "rightkit-qts 0.2.3
//    src/pipeline/tts_transformer.rs", build_talker_step_embedding);
//  * k_argmax: the greedy pick of each logits row with ids from
//    suppress_begin up excluded except keep_id (the codebook-0 suppression
//    before select_token in the same file), lowest index among equal maxima;
//    optionally also the table row of the pick, the code predictor's next
//    input (forward_code_pred_step_cached in the same file embeds the
//    previous code).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "kernels.h"

namespace qtalk {

namespace {

// One block per slot, hidden / 4 threads (<= 1024), one float4 each.  The
// tables are summed in order (0, 1, ..., G-1, overlay) in float32.  An id
// outside its table writes NaN for the slot and status 5.
__global__ void k_embed_sum(EmbedSumArgs a) {
  const int s = blockIdx.x, c = threadIdx.x * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  bool bad = false;
  for (int g = 0; g < a.n_groups; ++g) {
    const int id = a.ids[(size_t)g * a.n + s];
    if (id < 0 || id >= a.rows[g]) {
      bad = true;
      continue;
    }
    const float4 r = *reinterpret_cast<const float4*>(a.tables[g] + (size_t)id * a.hidden + c);
    if (g == 0) {
      acc = r;
    } else {
      acc.x += r.x;
      acc.y += r.y;
      acc.z += r.z;
      acc.w += r.w;
    }
  }
  if (a.overlay) {
    const float4 o = *reinterpret_cast<const float4*>(a.overlay + (size_t)s * a.hidden + c);
    acc.x += o.x;
    acc.y += o.y;
    acc.z += o.z;
    acc.w += o.w;
  }
  if (bad) {
    acc = make_float4(__int_as_float(0x7fc00000), __int_as_float(0x7fc00000),
                      __int_as_float(0x7fc00000), __int_as_float(0x7fc00000));
    if (threadIdx.x == 0) *a.status = 5;
  }
  *reinterpret_cast<float4*>(a.out + (size_t)s * a.hidden + c) = acc;
}

// (value, index) candidate order: larger value first, then lower index; an
// empty candidate (index INT_MAX) loses to any other
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  if (bi == INT_MAX) return i != INT_MAX;
  if (i == INT_MAX) return false;
  return v > bv || (v == bv && i < bi);
}

// One block of 256 threads per row.  NaN counts as -inf.
__global__ __launch_bounds__(256) void k_argmax(ArgmaxArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lg = a.logits + (size_t)row * a.vocab;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int t = tid; t < a.vocab; t += 256) {
    if (t >= a.suppress_begin && t != a.keep_id) continue;
    float v = lg[t];
    if (v != v) v = -INFINITY;
    if (better(v, t, bv, bi)) {
      bv = v;
      bi = t;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    // no candidate at all (suppress_begin <= 0 and keep_id outside the row)
    bi = bi == INT_MAX ? -1 : bi;
    a.out[row] = bi;
    si[0] = bi;
  }
  if (!a.table) return;
  // the next step's input: row `pick` of the table (NaN and status 5 when
  // there is none)
  __syncthreads();
  const int pick = si[0];
  const bool bad = pick < 0 || pick >= a.table_rows;
  if (bad && tid == 0) *a.status = 5;
  const float nan = __int_as_float(0x7fc00000);
  for (int c = tid * 4; c < a.hidden; c += 1024) {
    const float4 r = bad ? make_float4(nan, nan, nan, nan)
                         : *reinterpret_cast<const float4*>(a.table + (size_t)pick * a.hidden + c);
    *reinterpret_cast<float4*>(a.rows_out + (size_t)row * a.hidden + c) = r;
  }
}

}  // namespace

void launch_embed_sum(const EmbedSumArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_embed_sum, dim3(a.n), dim3(a.hidden / 4), 0, st, a);
}

void launch_argmax(const ArgmaxArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(a.n), dim3(256), 0, st, a);
}

}  // namespace qtalk
