// Host-side launchers of the Talker kernels (internal to the library).
#pragma once

#include "common.h"

namespace qtalk {

enum Epilogue { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

// largest K of the matrix-vector kernel: 4 rows of float32 activations in LDS
constexpr int MAX_GEMV_K = 8192;

// y[n][o] (=|+=) sum_k W[o][k] * xn[n][k], xn = RMSNorm(x[n]) * gain when
// `gain` is set (else xn = x).  EPI_SWIGLU reads W as gate|up rows
// interleaved in blocks of 16 (see pack order in the runtime) and writes
// silu(gate) * up for O logical rows.  norm_out (nullable) receives xn.
struct GemvArgs {
  const void* W;
  int O;
  int K;
  const float* X;
  int ldx;
  int nrows;
  const float* gain;
  float eps;
  float* Y;
  int ldy;
  float* norm_out;
  int ld_norm;
};
void launch_gemv(bool w_bf16, Epilogue epi, GemvArgs a, hipStream_t st);

// QK RMSNorm + NEOX RoPE on q (in place) and k, then K/V append into the
// cache; with a Q8_0 cache the normed and roped k also goes back in place.
struct QkArgs {
  float* qkv;
  int ldqkv;
  int n_heads, n_kv_heads, head_dim;
  const float* g_q;
  const float* g_k;
  float eps;
  const float2* rope;  // [cap][head_dim/2] (cos, sin)
  void* kc;
  void* vc;  // cache base of this layer: [S][n_kv][cap][hd]
  int cap;
  int skip_q;  // 1: leave q as is (the matrix-core attention norms and ropes it)
  RowMeta rows;
};
// KV cache storage: float32, float16, or Q8_0 rows (head_dim int8 codes then
// head_dim / 32 float16 scales)
enum KvKind { KV_F32 = 0, KV_F16 = 1, KV_Q8 = 2 };
size_t kv_row_bytes(KvKind kv, int head_dim);
// positions 0 .. len-1 of one sequence (K and V, [n_kv][cap] rows each) as
// float16 [n_kv][cap][hd] copies: below `fresh` dequantised from the Q8_0
// cache, from `fresh` on the call's own rows (row r = position fresh + r) of
// the projection buffer qkv [rows][ldqkv] (K normed and roped in place)
void launch_kv_q8_to_f16(const void* kq, const void* vq, int n_kv, int cap, int len, int hd,
                         f16_t* k16, f16_t* v16, int fresh, const float* qkv, int ldqkv, int nq,
                         hipStream_t st);
void launch_qk_rope_append(KvKind kv, QkArgs a, hipStream_t st);

// Causal GQA attention of the listed rows over the cache (split over keys).
enum AttnOut { ATT_PARTIAL = 0, ATT_F32 = 1, ATT_BF16 = 2 };
struct AttnArgs {
  const float* q;  // q of row t, head h at q + t*ldq + h*hd
  int ldq;
  const void* kc;
  const void* vc;  // [S][n_kv][cap][hd] of this layer
  int n_heads, n_kv_heads, head_dim, cap;
  float scale;
  int keys_per_split;
  int n_splits;
  float* part_o;   // [rows][n_heads][n_splits][hd]
  float* part_ml;  // [rows][n_heads][n_splits][2]: m (log2 units), l
  void* out;       // final output row t at out + t*ldo (f32 or bf16)
  int ldo;
  RowMeta rows;
};
constexpr int MAX_SPLITS = 128;  // key splits per row of the split-KV attention
void launch_attn_decode(KvKind kv, AttnOut mode, AttnArgs a, hipStream_t st);
// combine the ATT_PARTIAL splits into out (float32, or bf16 with bf16_out)
void launch_attn_merge(AttnArgs a, bool bf16_out, hipStream_t st);

// Causal GQA attention of T uniform rows (positions p0 .. p0+T-1 of one
// sequence) over the f16 cache on the matrix cores; output bf16 rows.
struct PrefillAttnArgs {
  const float* q;  // raw q of row t, head h at q + t*ldq + h*head_dim
  int ldq;
  const float* g_q;     // [head_dim] QK-norm gain of q
  float eps;
  const float2* rope;   // [cap][head_dim/2] (cos, sin)
  const f16_t* kc;
  const f16_t* vc;  // [S][n_kv][cap][hd] of this layer
  int n_heads, n_kv_heads, head_dim, cap;
  int seq, p0, T;
  float qscale;  // log2(e) / sqrt(head_dim)
  // 1: q arrives normed, rotated and scaled, float16 (row t's head h at halfs
  // t * 2 * ldq + h * head_dim); 0: raw float32 as above
  int q16;
  // positions per block: 32, 64 (head_dim 128 only), or 0 to let the
  // launcher pick from the chunk's offset and the grid size
  int rows_per_block;
  bf16_t* out;   // row t at out + t*ldo
  int ldo;
  int ncu;  // compute units (block placement only)
  // batched prefill: nbatch > 1 sequences seqs[z] of T rows each, stacked
  // (q and out rows z*T .. z*T+T-1); nbatch <= 1: the single sequence `seq`
  int nbatch;
  int seqs[MAX_ROWS];
};
bool attn_prefill_supported(int head_dim, int group);
void launch_attn_prefill(const PrefillAttnArgs& a, hipStream_t st);
int attn_prefill_rows_per_block(const PrefillAttnArgs& a);

// C = A[M][K] (bf16) * B[N][K]^T (bf16) on MFMA, float32 accumulation.
struct GemmArgs {
  const bf16_t* A;
  int lda;
  const bf16_t* B;
  int M, N, K;
  void* C;  // f32 [M][ldc] for STORE/ADD; bf16 [M][ldc] for SWIGLU
  int ldc;
  float* work;  // split-K partials [ksplit][M][N]
  size_t work_elems;
  // EPI_STORE, the Q|K|V projection (head_dim 128): columns 0 .. kcol-1
  // are q rows, which get the per-head RMSNorm (gain g_q), NEOX RoPE and the
  // score scale qscale and go as float16 into C in place (row r's head h at
  // halfs h * 128 of the row: the first kcol halfs of its ldc floats);
  // columns kcol .. vcol-1 are K rows, which get the per-head RMSNorm (gain g_k),
  // NEOX RoPE at the row's position (table rope [cap][64]) and go as
  // float16 to kcache; columns from vcol on are V rows, which go as float16
  // to vcache.  Row r belongs to sequence kv_seqs[r / kv_per] at position
  // vpos0 + r % kv_per (kv_per = 0: sequence kv_seqs[0], position vpos0 +
  // r); its cache row for head (col - kcol or vcol) / 128 is element
  // seq * kv_seq_stride + (head * vcap + position) * 128 of the layer's
  // cache; K and V do not go to C.  All of this applies when
  // gemm_writes_kv(a) holds; otherwise C receives every column in float32.
  f16_t* kcache = nullptr;
  f16_t* vcache = nullptr;
  int kcol = 0, vcol = 0, vcap = 0, vpos0 = 0;
  size_t kv_seq_stride = 0;
  int kv_per = 0;
  int kv_seqs[MAX_ROWS] = {};
  const float* g_k = nullptr;
  const float* g_q = nullptr;
  const float2* rope = nullptr;
  float eps = 0.f, qscale = 0.f;
};
void launch_gemm(Epilogue epi, GemmArgs a, hipStream_t st);
// whether launch_gemm(EPI_STORE, a) forms q, K and V in its epilogue (q as
// float16 into C, K and V into the cache): the 256-row matrix-core product
// with whole 128-column tiles and no K split; otherwise C holds the raw
// float32 product and the caller appends K and V itself
bool gemm_writes_kv(const GemmArgs& a);
// C += A * B^T (C = the f32 residual stream [M][N]), then hn = bf16(RMSNorm(C) * g)
// row by row; split-K partials are reduced in the same pass as the norm.
void launch_gemm_add_norm(GemmArgs a, const float* g, float eps, bf16_t* hn, int ldh,
                          hipStream_t st);
bool gemm_shape_ok(int M, int N, int K);
// shapes the skinny (<= 128-row) product takes: N % 32 == 0, K % 128 == 0
bool skinny_shape_ok(int N, int K);

// out[t][k] = bf16(RMSNorm(x[t]) * g); also the float32 values to out32 when set
void launch_rmsnorm_bf16(const float* x, int ldx, int T, int K, const float* g,
                         float eps, bf16_t* out, int ldo, hipStream_t st, float* out32 = nullptr,
                         int ld32 = 0);

// cos/sin table [cap][half], angle pos * theta^(-2i/hd), float64 math
void launch_rope_table(float2* tab, int cap, int head_dim, double theta,
                       hipStream_t st);

// dst[h][t][d] = float(cache[h][t][d]) for t < len
void launch_kv_to_f32(KvKind kv, const void* src, int n_kv, int cap, int len,
                      int hd, float* dst, hipStream_t st);

// Batch-1 decode of the whole stack in one persistent launch (Talker
// geometry, bf16 weights, f16 cache).  See k_decode_fused.hip.
struct FusedDecodeArgs {
  const bf16_t* w;  // layer l at w + l * layer_stride: [Wqkv | Wo | Wgu | Wd]
  size_t layer_stride;
  const float* norms;  // layer l at norms + l * norm_stride: g_in, g_post, g_q, g_k
  size_t norm_stride;
  const bf16_t* head;
  const float* g_final;
  char* kc;
  char* vc;  // [L][S][NKV][cap] rows of HD values (f16, or Q8_0: codes then scales)
  size_t layer_kv_bytes;
  int kv_q8;  // 1: Q8_0 rows
  int cap, seq, pos, n_layers;
  float eps;
  const float2* rope;
  const float* emb;
  float* logits;
  float* hidden_out;
  uint64_t* ll;    // [2][words per layer] exchange words (layer parity)
  uint64_t* part;  // [2][NKV][G][NCH][144] chunk partials (o, m, l, padding), as words
  int* err;        // 0; 1 a wait gave up; 3 a block ran on an unexpected XCD
  long spin_limit; // re-polls after which a wait gives up (error 1)
  uint32_t epoch;  // >= 1 and < 2^26; words carry epoch * 64 + layer
  int xcd_local;   // QKV -> attention -> merge exchanges inside each XCD's L2
  int head_rows;   // vocab / 256: codec head rows per block (1..16)
  // layer-0 input looked up on the device when n_gather == 1 (emb unused):
  // x = gtab[0][gids[0]] (+ goverlay); an id outside the table gives a NaN
  // row and *gstatus = 5 (the decode status word: rolled back at sync)
  int n_gather;
  const float* gtab[1];
  int grows[1];
  const int32_t* gids;
  const float* goverlay;
  int* gstatus;
  // when set: the greedy pick of the logits (ids >= pick_suppress excluded
  // except pick_keep; NaN as -inf; the lowest id among equal maxima; -1 if
  // nothing is left) written to *pick_out
  int32_t* pick_out;
  int pick_suppress, pick_keep;
};
// default bounded-wait limit of the persistent decode (~1-2 s of polling)
constexpr long FUSED_SPIN_LIMIT = 1L << 21;
bool fused_decode_supported(int hidden, int q_dim, int kv_dim, int inter, int vocab, int n_heads,
                            int n_kv_heads, int head_dim);
bool fused_decode_fits();
bool fused_decode_xcd_layout_ok(hipStream_t st, bool cooperative);
int fused_decode_blocks();
size_t fused_decode_ll_words(int n_layers);
size_t fused_decode_part_words(int n_layers);
hipError_t launch_decode_fused(const FusedDecodeArgs& a, hipStream_t st, bool cooperative);
// zero n 8-byte words (a kernel, not a memset node)
void launch_fill_zero(uint64_t* p, size_t n, hipStream_t st);

// frame-step glue (k_frame.hip)
constexpr int MAX_EMBED_GROUPS = 32;
struct EmbedSumArgs {
  const float* tables[MAX_EMBED_GROUPS];  // [rows[g]][hidden] float32 each
  int rows[MAX_EMBED_GROUPS];
  int n_groups, n, hidden;  // hidden % 4 == 0, hidden <= 4096
  const int32_t* ids;       // [n_groups][n] (group-major)
  const float* overlay;     // [n][hidden] or null
  float* out;               // [n][hidden]
  int* status;              // set to 5 when an id is outside its table
};
void launch_embed_sum(const EmbedSumArgs& a, hipStream_t st);
struct ArgmaxArgs {
  const float* logits;  // [n][vocab]
  int n, vocab, suppress_begin, keep_id;
  int32_t* out;         // [n]
  // optional, the pick's row lookup: rows_out[i] = table[out[i]]
  const float* table;   // [table_rows][hidden] or null
  int table_rows, hidden;  // hidden % 4 == 0
  float* rows_out;      // [n][hidden]
  int* status;          // set to 5 when a pick has no table row
};
void launch_argmax(const ArgmaxArgs& a, hipStream_t st);

}  // namespace qtalk
