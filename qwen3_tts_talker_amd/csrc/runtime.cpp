// Host runtime of the C ABI in include/qtalk.h: weight repack, KV cache and
// scratch ownership, argument validation and the per-layer launch sequence.
//
// Forward order per layer ("qwentts.cpp src/talker-forward.h",
// talker_layer_forward): input RMSNorm -> QKV projection -> QK-norm + RoPE +
// K/V append -> causal GQA attention over the cache -> o_proj + residual ->
// post-attention RMSNorm -> gate|up projection + SwiGLU -> down + residual.
// After the stack: final RMSNorm + codec_head on the last row
// (talker_forward_core), or on every row of a batched decode
// (talker_forward_decode).
//
// Two launch paths compute the same thing:
//  - matrix-vector path (decode, short or float32 prefill): activations stay
//    float32, weights are upcast in the kernels;
//  - matrix-core path (bf16 prefill longer than 16 rows): activations are
//    rounded to bf16 as the A operand of MFMA GEMMs, accumulation is float32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qtalk.h"
#include "kernels.h"

using namespace qtalk;

namespace {

constexpr int GEMV_ROWS = MAX_ROWS;  // rows per matrix-vector pass
constexpr int MFMA_MIN_ROWS = 17;    // prefill rows that switch to the matrix cores
constexpr int BATCH_MFMA_MIN = 8;    // batched-decode rows that switch to the matrix cores
constexpr int MAX_CHUNK = 2048;      // rows per matrix-core pass
// prefill / extend of at most this many rows runs as consecutive persistent
// single-row launches when the persistent decode is available (one launch
// costs less than the matrix-vector path's per-layer launches up to here)
constexpr int FUSED_MAX_ROWS = 2;
constexpr size_t WORK_ELEMS = (size_t)8 << 20;  // split-K workspace (floats)

struct LayerDev {
  void* wqkv;  // [q_dim + 2 kv_dim][H]: q rows, then k rows, then v rows
  void* wo;    // [H][q_dim]
  void* wgu;   // [2 I][H]: 16 gate rows, 16 up rows, repeated
  void* wd;    // [H][I]
  float *g_in, *g_post, *g_q, *g_k;
};

}  // namespace

struct qtalk_ctx {
  qtalk_config cfg{};
  hipStream_t stream = nullptr;
  bool w_bf16 = true, kv_f16 = true;
  KvKind kv = KV_F16;  // cache storage
  f16_t* kv16 = nullptr;  // Q8 cache: float16 copy of one sequence's K then V for the matrix-core prefill attention
  size_t kv_rb = 0;    // bytes per cache row (one position of one KV head)
  size_t welem = 2;
  int q_dim = 0, kv_dim = 0, qkv_dim = 0;
  std::vector<LayerDev> layers;
  void* wblob = nullptr;
  float* nblob = nullptr;
  void* head = nullptr;  // [n_out_heads][vocab][hidden]
  int n_out_heads = 1;
  int head_sel = 0;  // head of the logits of the following calls (qtalk_select_head)
  float* g_final = nullptr;
  void *kc = nullptr, *vc = nullptr;
  size_t layer_kv_elems = 0;  // values of one layer's cache (all sequences)
  size_t layer_kv_rows() const { return layer_kv_elems / (size_t)cfg.head_dim; }
  float2* rope = nullptr;
  std::vector<int32_t> cur_len;
  int tc = 0;  // rows per matrix-core pass
  float *x = nullptr, *qkv = nullptr, *att = nullptr, *act = nullptr;
  bf16_t* hn = nullptr;
  float *part_o = nullptr, *part_ml = nullptr;
  float* work = nullptr;
  // persistent batch-1 decode (Talker geometry only)
  bool fused = false;
  // launch of the persistent decode: an ordinary launch of the 256-block
  // grid (one block per compute unit, checked at create; persistent decodes
  // of all contexts in the process serialised per device, see DecodeChain),
  // or with QTALK_COOPERATIVE=1 a cooperative launch, which the runtime
  // guarantees co-resident but which costs ~18 us more per token
  bool coop = false;
  int dev = 0;
  hipEvent_t chain_ev = nullptr;  // marks another context's stream (DecodeChain)
  int ncu = 256;  // compute units of the device (placement heuristics only)
  int attn_rows = 0;  // prefill attention positions per block (0: the launcher picks)
  // QKV -> attention -> merge exchanges of the persistent decode inside each
  // XCD (needs the dispatcher's block b -> XCD b % 8 placement, checked at
  // create and by every launch); QTALK_XCD_LOCAL=0 turns it off
  bool xcd_local = false;
  uint64_t* ll = nullptr;
  uint64_t* fpart = nullptr;
  int* ferr = nullptr;
  long spin_limit = FUSED_SPIN_LIMIT;  // persistent decode: re-polls before a wait gives up
  // per sequence, the first position written by a persistent launch since
  // the last qtalk_sync (-1: none); a launch that gave up rolls it back
  std::vector<int32_t> fused_first;
  int* aux_err = nullptr;  // frame-step kernels: 5 when an id was outside its table
  float* step_in = nullptr;  // [hidden]: a gathered step input (qtalk_decode_step without the persistent decode)
  uint32_t epoch = 0;
  size_t per_layer = 0, norms_per_layer = 0;
  std::string err;
};

namespace {

// Persistent decodes run one at a time per device across every context of
// the process.  Without a cooperative launch nothing stops two persistent
// grids from sharing the compute units, and each would then wait for blocks
// that the other one occupies (until the spin limit turns it into an error).
// Launches on one stream are ordered by the stream; a launch on another
// stream first waits for everything enqueued so far on the stream of the
// previous persistent decode.
struct DecodeChain {
  std::mutex mu;
  hipStream_t stream = nullptr;  // stream of the latest persistent decode on the device
};
constexpr int MAX_DEVICES = 64;
DecodeChain g_chain[MAX_DEVICES];

// Exchange words and chunk partials of the persistent decode for
// qtalk_decode_noalloc, in a static device array instead of the context's
// buffers: each device holds its own copy until the process ends.  Host code
// uses only the address resolved per device at qtalk_create (the array's name
// in host code is a stand-in, not a device address).  Every persistent launch
// through it takes a fresh epoch from the device's counter, so words left by
// an earlier launch (of any context) never match; the launches are
// serialised per device (DecodeChain), whose mutex guards these entries.
constexpr size_t SCRATCH_BYTES = (size_t)2 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
struct StaticScratch {
  void* ptr = nullptr;  // this device's copy of `scratch`
  bool resolved = false;
  uint32_t epoch = 0;   // last epoch used in it
};
StaticScratch g_scratch[MAX_DEVICES];

// resolve `scratch` on the current device (once per device)
void resolve_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_chain[dev].mu);
  StaticScratch& z = g_scratch[dev];
  if (z.resolved) return;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) z.ptr = p;
  else (void)hipGetLastError();
  z.resolved = true;
}

// where a persistent launch exchanges its words: the context's buffers or
// the device's static array, each with its own epoch counter
struct Exchange {
  uint64_t* ll;
  uint64_t* part;
  uint32_t* epoch;
};

qtalk_status fail(qtalk_ctx* c, qtalk_status s, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return s;
}

bool dev_alloc(void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  return hipMalloc(p, bytes) == hipSuccess;
}

void free_all(qtalk_ctx* c) {
  void* ptrs[] = {c->wblob, c->nblob, c->head, c->kc,     c->vc,    c->rope,   c->x,
                  c->qkv,   c->att,   c->act,  c->hn,     c->part_o, c->part_ml, c->work,
                  c->ll,    c->fpart, c->ferr, c->aux_err, c->kv16, c->step_in};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
}

const char* check_config(const qtalk_config* g) {
  if (g->n_layers < 1 || g->hidden < 1 || g->n_heads < 1 || g->n_kv_heads < 1 ||
      g->intermediate < 1 || g->vocab < 1 || g->max_seq_len < 1 || g->max_seqs < 1)
    return "every size must be >= 1";
  if (g->head_dim != 64 && g->head_dim != 128) return "head_dim must be 64 or 128";
  if (g->n_heads % g->n_kv_heads) return "n_heads must be a multiple of n_kv_heads";
  const int G = g->n_heads / g->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return "n_heads / n_kv_heads must be 1, 2, 4 or 8";
  if (g->hidden % 64 || g->intermediate % 64 || (g->n_heads * g->head_dim) % 64)
    return "hidden, intermediate and n_heads*head_dim must be multiples of 64";
  if (!(g->rms_eps >= 0.f) || !(g->rope_theta > 0.f)) return "bad rms_eps or rope_theta";
  if (g->weight_dtype != QTALK_F32 && g->weight_dtype != QTALK_BF16)
    return "weight_dtype must be F32 or BF16";
  if (g->kv_dtype != QTALK_F32 && g->kv_dtype != QTALK_F16 && g->kv_dtype != QTALK_Q8)
    return "kv_dtype must be F32, F16 or Q8";
  if (g->n_output_heads < 0 || g->n_output_heads > 64) return "n_output_heads must be 0..64";
  // the matrix-vector kernel keeps up to 4 activation rows of float32 in LDS
  if (g->hidden > MAX_GEMV_K || g->intermediate > MAX_GEMV_K || g->n_heads * g->head_dim > MAX_GEMV_K)
    return "hidden, intermediate and n_heads*head_dim must be <= 8192";
  return nullptr;
}

// ---------------------------------------------------------------------------

struct Fwd {
  qtalk_ctx* c;
  hipStream_t st;
  const qtalk_config& g;
  explicit Fwd(qtalk_ctx* cc) : c(cc), st(cc->stream), g(cc->cfg) {}

  char* kv_layer(void* base, int l) const {
    return reinterpret_cast<char*>(base) + (size_t)l * c->layer_kv_rows() * c->kv_rb;
  }

  void qk_append(int l, const RowMeta& rows, bool skip_q = false) {
    QkArgs q{};
    q.qkv = c->qkv;
    q.ldqkv = c->qkv_dim;
    q.n_heads = g.n_heads;
    q.n_kv_heads = g.n_kv_heads;
    q.head_dim = g.head_dim;
    q.g_q = c->layers[l].g_q;
    q.g_k = c->layers[l].g_k;
    q.eps = g.rms_eps;
    q.rope = c->rope;
    q.kc = kv_layer(c->kc, l);
    q.vc = kv_layer(c->vc, l);
    q.cap = g.max_seq_len;
    q.skip_q = skip_q ? 1 : 0;
    q.rows = rows;
    launch_qk_rope_append(c->kv, q, st);
  }

  AttnArgs attn_args(int l, const RowMeta& rows) const {
    AttnArgs a{};
    a.q = c->qkv;
    a.ldq = c->qkv_dim;
    a.kc = kv_layer(c->kc, l);
    a.vc = kv_layer(c->vc, l);
    a.n_heads = g.n_heads;
    a.n_kv_heads = g.n_kv_heads;
    a.head_dim = g.head_dim;
    a.cap = g.max_seq_len;
    a.scale = 1.0f / sqrtf((float)g.head_dim);
    a.part_o = c->part_o;
    a.part_ml = c->part_ml;
    a.out = c->att;
    a.ldo = c->q_dim;
    a.rows = rows;
    return a;
  }

  static int max_ctx(const RowMeta& r) {
    if (r.uniform == 1) return r.p0 + r.n;
    if (r.uniform == 2) return r.p0 + r.per;
    int m = 0;
    for (int i = 0; i < r.n; ++i) m = std::max(m, r.pos[i] + 1);
    return m;
  }

  // Key splits of the split-KV attention: about 1024 blocks over all rows
  // and KV heads (multiples of 64 keys), at most MAX_SPLITS per row.
  void set_splits(AttnArgs& a, const RowMeta& r) const {
    long total = 0;
    for (int t = 0; t < r.n; ++t)
      total += 1 + (r.uniform == 1 ? r.p0 + t : (r.uniform == 2 ? r.p0 + t % r.per : r.pos[t]));
    total *= g.n_kv_heads;
    const int mx = max_ctx(r);
    int kps = 64 * (int)((total + 1024L * 64 - 1) / (1024L * 64));
    kps = std::max(kps, 64 * ((mx + 64 * MAX_SPLITS - 1) / (64 * MAX_SPLITS)));
    a.keys_per_split = kps;
    a.n_splits = (mx + kps - 1) / kps;
  }

  void gemv(const void* W, int O, int K, const float* X, int ldx, int n, const float* gain,
            float* Y, int ldy, Epilogue epi, float* norm_out = nullptr, int ld_norm = 0) {
    GemvArgs a{W, O, K, X, ldx, n, gain, g.rms_eps, Y, ldy, norm_out, ld_norm};
    launch_gemv(c->w_bf16, epi, a, st);
  }

  // matrix-vector layer on rows.n <= GEMV_ROWS rows held in c->x
  void layer_gemv(int l, const RowMeta& rows) {
    const LayerDev& L = c->layers[l];
    const int n = rows.n, H = g.hidden;
    gemv(L.wqkv, c->qkv_dim, H, c->x, H, n, L.g_in, c->qkv, c->qkv_dim, EPI_STORE);
    qk_append(l, rows);
    AttnArgs a = attn_args(l, rows);
    set_splits(a, rows);
    launch_attn_decode(c->kv, ATT_PARTIAL, a, st);
    launch_attn_merge(a, false, st);
    gemv(L.wo, H, c->q_dim, c->att, c->q_dim, n, nullptr, c->x, H, EPI_ADD);
    gemv(L.wgu, g.intermediate, H, c->x, H, n, L.g_post, c->act, g.intermediate, EPI_SWIGLU);
    gemv(L.wd, H, g.intermediate, c->act, g.intermediate, n, nullptr, c->x, H, EPI_ADD);
  }

  void gemm(const bf16_t* A, int lda, const void* B, int M, int N, int K, void* C, int ldc,
            Epilogue epi) {
    GemmArgs a{A, lda, reinterpret_cast<const bf16_t*>(B), M, N, K, C, ldc, c->work, WORK_ELEMS};
    launch_gemm(epi, a, st);
  }

  // matrix-core layer on rows.n <= c->tc uniform rows held in c->x.  On entry
  // c->hn holds RMSNorm(x) * g_in when `normed` (the previous layer's down
  // projection produced it); on return it holds the next layer's input norm
  // unless this is the last layer.
  // q's score scale: log2(e) / sqrt(head_dim) (softmax in exp2 units)
  float attn_qscale() const { return 1.4426950408889634f / sqrtf((float)g.head_dim); }

  void layer_mfma(int l, const RowMeta& rows, bool normed) {
    const LayerDev& L = c->layers[l];
    const int T = rows.n, H = g.hidden, I = g.intermediate;
    bf16_t* att_b = reinterpret_cast<bf16_t*>(c->att);
    bf16_t* act_b = reinterpret_cast<bf16_t*>(c->act);
    if (!normed) launch_rmsnorm_bf16(c->x, H, T, H, L.g_in, g.rms_eps, c->hn, H, st);
    const bool sup = attn_prefill_supported(g.head_dim, g.n_heads / g.n_kv_heads);
    // a Q8 cache reaches the matrix cores through a float16 copy of the
    // sequence's positions 0 .. p0+T-1 (one sequence at a time): earlier
    // positions dequantised, this chunk's rows as computed
    const bool q8_mfma = c->kv == KV_Q8 && c->kv16 && sup && rows.uniform == 1;
    const bool mfma_attn = (c->kv == KV_F16 && sup) || q8_mfma;
    // one sequence or stacked sequences, float16 cache, head_dim 128: the
    // projection forms K (norm, RoPE) and V in its epilogue and writes them
    // straight into the cache where its tiling allows; otherwise the append
    // kernel does
    GemmArgs qa{c->hn, H, reinterpret_cast<const bf16_t*>(L.wqkv), T, c->qkv_dim, H, c->qkv, c->qkv_dim,
                c->work, WORK_ELEMS};
    if (c->kv == KV_F16 && mfma_attn && g.head_dim == 128 && (rows.uniform == 1 || rows.uniform == 2)) {
      qa.kcache = reinterpret_cast<f16_t*>(kv_layer(c->kc, l));
      qa.vcache = reinterpret_cast<f16_t*>(kv_layer(c->vc, l));
      qa.kv_seq_stride = (size_t)g.n_kv_heads * g.max_seq_len * g.head_dim;
      if (rows.uniform == 2) {
        qa.kv_per = rows.per;
        for (int z = 0; z < T / rows.per; ++z) qa.kv_seqs[z] = rows.seq[z];
      } else {
        qa.kv_seqs[0] = rows.seq0;
      }
      qa.kcol = c->q_dim;
      qa.vcol = c->q_dim + c->kv_dim;
      qa.vcap = g.max_seq_len;
      qa.vpos0 = rows.p0;
      qa.g_k = L.g_k;
      qa.g_q = L.g_q;
      qa.rope = c->rope;
      qa.eps = g.rms_eps;
      qa.qscale = attn_qscale();
    }
    const bool kv_done = gemm_writes_kv(qa);
    if (!kv_done) qa.kcache = qa.vcache = nullptr;
    launch_gemm(EPI_STORE, qa, st);
    if (!kv_done) qk_append(l, rows, mfma_attn);
    if (mfma_attn) {
      PrefillAttnArgs p{};
      p.q = c->qkv;
      p.ldq = c->qkv_dim;
      p.g_q = L.g_q;
      p.eps = g.rms_eps;
      p.rope = c->rope;
      p.kc = reinterpret_cast<const f16_t*>(kv_layer(c->kc, l));
      p.vc = reinterpret_cast<const f16_t*>(kv_layer(c->vc, l));
      if (q8_mfma) {
        const size_t seq_rows = (size_t)rows.seq0 * g.n_kv_heads * g.max_seq_len;
        f16_t* k16 = c->kv16;
        f16_t* v16 = c->kv16 + (size_t)g.n_kv_heads * g.max_seq_len * g.head_dim;
        launch_kv_q8_to_f16(kv_layer(c->kc, l) + seq_rows * c->kv_rb, kv_layer(c->vc, l) + seq_rows * c->kv_rb,
                            g.n_kv_heads, g.max_seq_len, rows.p0 + T, g.head_dim, k16, v16, rows.p0,
                            c->qkv, c->qkv_dim, g.n_heads, st);
        p.kc = k16;
        p.vc = v16;
      }
      p.n_heads = g.n_heads;
      p.n_kv_heads = g.n_kv_heads;
      p.head_dim = g.head_dim;
      p.cap = g.max_seq_len;
      p.seq = rows.seq0;
      p.p0 = rows.p0;
      p.T = T;
      if (rows.uniform == 2) {  // T / per stacked sequences of per rows each
        p.T = rows.per;
        p.nbatch = T / rows.per;
        for (int z = 0; z < p.nbatch; ++z) p.seqs[z] = rows.seq[z];
        p.seq = rows.seq[0];
      }
      if (q8_mfma) p.seq = 0;  // the float16 copy holds this sequence only
      p.qscale = attn_qscale();
      p.q16 = kv_done ? 1 : 0;
      p.out = att_b;
      p.ldo = c->q_dim;
      p.ncu = c->ncu;
      p.rows_per_block = c->attn_rows;
      launch_attn_prefill(p, st);
    } else {
      AttnArgs a = attn_args(l, rows);
      a.keys_per_split = max_ctx(rows);
      a.n_splits = 1;
      launch_attn_decode(c->kv, ATT_BF16, a, st);
    }
    gemm_add_norm(att_b, c->q_dim, L.wo, T, H, c->q_dim, L.g_post);
    gemm(c->hn, H, L.wgu, T, 2 * I, H, act_b, I, EPI_SWIGLU);
    if (l + 1 < g.n_layers) gemm_add_norm(act_b, I, L.wd, T, H, I, c->layers[l + 1].g_in);
    else gemm(act_b, I, L.wd, T, H, I, c->x, H, EPI_ADD);
  }

  // Matrix-core layer for decode rows held in c->x (one row per sequence,
  // any positions: the batched decode).  The projections read bf16
  // activations, as in the matrix-core prefill; the attention is the split-KV
  // kernel, merged straight into bf16 for o_proj.  `normed` as in layer_mfma.
  void layer_rows_mfma(int l, const RowMeta& rows, bool normed) {
    const LayerDev& L = c->layers[l];
    const int n = rows.n, H = g.hidden, I = g.intermediate;
    bf16_t* att_b = reinterpret_cast<bf16_t*>(c->att);
    bf16_t* act_b = reinterpret_cast<bf16_t*>(c->act);
    if (!normed) launch_rmsnorm_bf16(c->x, H, n, H, L.g_in, g.rms_eps, c->hn, H, st);
    gemm(c->hn, H, L.wqkv, n, c->qkv_dim, H, c->qkv, c->qkv_dim, EPI_STORE);
    qk_append(l, rows);
    AttnArgs a = attn_args(l, rows);
    set_splits(a, rows);
    launch_attn_decode(c->kv, ATT_PARTIAL, a, st);
    launch_attn_merge(a, true, st);
    gemm_add_norm(att_b, c->q_dim, L.wo, n, H, c->q_dim, L.g_post);
    gemm(c->hn, H, L.wgu, n, 2 * I, H, act_b, I, EPI_SWIGLU);
    if (l + 1 < g.n_layers) gemm_add_norm(act_b, I, L.wd, n, H, I, c->layers[l + 1].g_in);
    else gemm(act_b, I, L.wd, n, H, I, c->x, H, EPI_ADD);
  }

  bool rows_mfma_ok() const {
    return c->w_bf16 && skinny_shape_ok(c->qkv_dim, g.hidden) && skinny_shape_ok(g.hidden, c->q_dim) &&
           skinny_shape_ok(2 * g.intermediate, g.hidden) && skinny_shape_ok(g.hidden, g.intermediate) &&
           g.intermediate % 16 == 0;
  }

  // x += A * B^T, then hn = bf16(RMSNorm(x) * gain)
  void gemm_add_norm(const bf16_t* A, int lda, const void* B, int M, int N, int K, const float* gain) {
    GemmArgs a{A, lda, reinterpret_cast<const bf16_t*>(B), M, N, K, c->x, N, c->work, WORK_ELEMS};
    launch_gemm_add_norm(a, gain, g.rms_eps, c->hn, N, st);
  }

  const void* head_w() const {
    return reinterpret_cast<const char*>(c->head) + (size_t)c->head_sel * g.vocab * g.hidden * c->welem;
  }

  void head(const float* X, int n, float* logits, float* hidden_out) {
    gemv(head_w(), g.vocab, g.hidden, X, g.hidden, n, c->g_final, logits, g.vocab, EPI_STORE,
         hidden_out, g.hidden);
  }

  // rows of one sequence at positions p0 .. p0+T-1 (prefill / extend)
  qtalk_status run_sequence(int seq, int p0, const float* emb, int T, float* logits, float* hidden_out) {
    const bool mfma = c->w_bf16 && T >= MFMA_MIN_ROWS &&
                      gemm_shape_ok(1, c->qkv_dim, g.hidden) && gemm_shape_ok(1, g.hidden, c->q_dim) &&
                      gemm_shape_ok(1, 2 * g.intermediate, g.hidden) &&
                      gemm_shape_ok(1, g.hidden, g.intermediate) && g.intermediate % 16 == 0;
    const int chunk = mfma ? c->tc : GEMV_ROWS;
    int done = 0;
    while (done < T) {
      const int n = std::min(chunk, T - done);
      RowMeta rows{};
      rows.n = n;
      rows.uniform = 1;
      rows.seq0 = seq;
      rows.p0 = p0 + done;
      if (hipMemcpyAsync(c->x, emb + (size_t)done * g.hidden, (size_t)n * g.hidden * 4,
                         hipMemcpyDeviceToDevice, st) != hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot copy the input rows");
      for (int l = 0; l < g.n_layers; ++l) {
        if (mfma && n >= MFMA_MIN_ROWS) layer_mfma(l, rows, l > 0);
        else layer_gemv(l, rows);
      }
      done += n;
      if (done == T) head(c->x + (size_t)(n - 1) * g.hidden, 1, logits, hidden_out);
    }
    return QTALK_OK;
  }

  // batched prefill: n sequences of T rows each from position 0, stacked in
  // groups that fit one matrix-core pass; each group's logits from its
  // sequences' last rows
  qtalk_status run_batch_prefill(const int32_t* seqs, int n, const float* emb, int T, float* logits,
                                 float* hidden_out) {
    const int H = g.hidden;
    const bool mfma = c->w_bf16 && gemm_shape_ok(1, c->qkv_dim, H) && gemm_shape_ok(1, H, c->q_dim) &&
                      gemm_shape_ok(1, 2 * g.intermediate, H) && gemm_shape_ok(1, H, g.intermediate) &&
                      g.intermediate % 16 == 0;
    const int cap_rows = mfma ? std::max(c->tc, GEMV_ROWS) : GEMV_ROWS;
    if (T > cap_rows) {  // a sequence's rows exceed one pass: one prefill per sequence
      for (int b = 0; b < n; ++b) {
        const qtalk_status s = run_sequence(seqs[b], 0, emb + (size_t)b * T * H, T,
                                            logits + (size_t)b * g.vocab,
                                            hidden_out ? hidden_out + (size_t)b * H : nullptr);
        if (s != QTALK_OK) return s;
      }
      return QTALK_OK;
    }
    const int per_group = std::min(MAX_ROWS, cap_rows / T);
    for (int b0 = 0; b0 < n; b0 += per_group) {
      const int nb = std::min(per_group, n - b0), M = nb * T;
      RowMeta rows{};
      rows.n = M;
      rows.p0 = 0;
      if (M <= GEMV_ROWS && !(mfma && M >= MFMA_MIN_ROWS)) {
        rows.uniform = 0;
        for (int t = 0; t < M; ++t) {
          rows.seq[t] = seqs[b0 + t / T];
          rows.pos[t] = t % T;
        }
      } else {
        rows.uniform = 2;
        rows.per = T;
        rows.seq0 = seqs[b0];
        for (int z = 0; z < nb; ++z) rows.seq[z] = seqs[b0 + z];
      }
      if (hipMemcpyAsync(c->x, emb + (size_t)b0 * T * H, (size_t)M * H * 4, hipMemcpyDeviceToDevice, st) !=
          hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot copy the input rows");
      for (int l = 0; l < g.n_layers; ++l) {
        if (mfma && M >= MFMA_MIN_ROWS) layer_mfma(l, rows, l > 0);
        else layer_gemv(l, rows);
      }
      // last row of each sequence: rows T-1, 2T-1, ... (stride T rows)
      gemv(head_w(), g.vocab, H, c->x + (size_t)(T - 1) * H, T * H, nb, c->g_final,
           logits + (size_t)b0 * g.vocab, g.vocab, EPI_STORE,
           hidden_out ? hidden_out + (size_t)b0 * H : nullptr, H);
    }
    return QTALK_OK;
  }

  // one row of sequence `seq` at position `pos` as one persistent launch,
  // exchanging through the context's buffers or (static_words) the device's
  // static array; the input row is emb, or gathered on the device (gather);
  // with pick set, the greedy pick of the logits goes to pick->out
  struct Pick {
    int32_t* out;
    int suppress, keep;
  };
  qtalk_status run_fused(int seq, int pos, const float* emb, float* logits, float* hidden_out,
                         bool static_words = false, const qtalk_gather* gather = nullptr,
                         const Pick* pick = nullptr) {
    FusedDecodeArgs a{};
    if (gather) {  // one table (several are summed by a gather kernel first)
      a.n_gather = 1;
      a.gtab[0] = gather->tables[0];
      a.grows[0] = gather->table_rows[0];
      a.gids = gather->ids;
      a.goverlay = gather->overlay;
      a.gstatus = c->ferr;
    }
    if (pick) {
      a.pick_out = pick->out;
      a.pick_suppress = pick->suppress;
      a.pick_keep = pick->keep;
    }
    a.w = reinterpret_cast<const bf16_t*>(c->wblob);
    a.layer_stride = c->per_layer;
    a.norms = c->nblob;
    a.norm_stride = c->norms_per_layer;
    a.head = reinterpret_cast<const bf16_t*>(head_w());
    a.head_rows = g.vocab / fused_decode_blocks();
    a.g_final = c->g_final;
    a.kc = reinterpret_cast<char*>(c->kc);
    a.vc = reinterpret_cast<char*>(c->vc);
    a.layer_kv_bytes = c->layer_kv_rows() * c->kv_rb;
    a.kv_q8 = c->kv == KV_Q8;
    a.cap = g.max_seq_len;
    a.seq = seq;
    a.pos = pos;
    a.n_layers = g.n_layers;
    a.eps = g.rms_eps;
    a.rope = c->rope;
    a.emb = emb;
    a.logits = logits;
    a.hidden_out = hidden_out;
    a.err = c->ferr;
    a.spin_limit = c->spin_limit;
    a.xcd_local = c->xcd_local;
    DecodeChain& ch = g_chain[c->dev];
    std::lock_guard<std::mutex> lock(ch.mu);
    Exchange x{c->ll, c->fpart, &c->epoch};
    if (static_words) {
      char* base = reinterpret_cast<char*>(g_scratch[c->dev].ptr);
      x = Exchange{reinterpret_cast<uint64_t*>(base),
                   reinterpret_cast<uint64_t*>(base + fused_decode_ll_words(g.n_layers) * 8),
                   &g_scratch[c->dev].epoch};
    }
    a.ll = x.ll;
    a.part = x.part;
    if (*x.epoch + 1 >= (1u << 26)) {  // epochs would wrap: clear the words and restart
      launch_fill_zero(x.ll, fused_decode_ll_words(g.n_layers), st);
      launch_fill_zero(x.part, fused_decode_part_words(g.n_layers), st);
      *x.epoch = 0;
    }
    a.epoch = *x.epoch + 1;
    if (ch.stream && ch.stream != st) {
      if (hipEventRecord(c->chain_ev, ch.stream) != hipSuccess ||
          hipStreamWaitEvent(st, c->chain_ev, 0) != hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot order the persistent decode after another context's");
    }
    const hipError_t e = launch_decode_fused(a, st, c->coop);
    if (e != hipSuccess)
      return fail(c, QTALK_E_DEVICE, "persistent decode launch failed: %s", hipGetErrorString(e));
    ch.stream = st;
    *x.epoch += 1;
    int32_t& first = c->fused_first[seq];
    first = first < 0 ? pos : std::min(first, pos);
    return QTALK_OK;
  }

  // one row per listed sequence (batched decode): 8 or more rows on the
  // matrix cores (each weight matrix read once per pass), fewer on the
  // matrix-vector kernel
  qtalk_status run_batch(const int32_t* seqs, int n, const float* emb, float* logits, float* hidden_out) {
    const bool mfma = rows_mfma_ok();
    for (int b0 = 0; b0 < n; b0 += GEMV_ROWS) {
      const int nb = std::min(GEMV_ROWS, n - b0);
      RowMeta rows{};
      rows.n = nb;
      rows.uniform = 0;
      for (int i = 0; i < nb; ++i) {
        rows.seq[i] = seqs[b0 + i];
        rows.pos[i] = c->cur_len[seqs[b0 + i]];
      }
      if (hipMemcpyAsync(c->x, emb + (size_t)b0 * g.hidden, (size_t)nb * g.hidden * 4,
                         hipMemcpyDeviceToDevice, st) != hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot copy the input rows");
      for (int l = 0; l < g.n_layers; ++l) {
        if (mfma && nb >= BATCH_MFMA_MIN) layer_rows_mfma(l, rows, l > 0);
        else layer_gemv(l, rows);
      }
      float* hid = hidden_out ? hidden_out + (size_t)b0 * g.hidden : nullptr;
      if (mfma && nb >= BATCH_MFMA_MIN && skinny_shape_ok(g.vocab, g.hidden)) {
        // the head on the matrix cores too (bf16 normed rows, as the layers'
        // projections): the weights are read once for all rows
        launch_rmsnorm_bf16(c->x, g.hidden, nb, g.hidden, c->g_final, g.rms_eps, c->hn, g.hidden, st, hid,
                            g.hidden);
        gemm(c->hn, g.hidden, head_w(), nb, g.vocab, g.hidden, logits + (size_t)b0 * g.vocab, g.vocab,
             EPI_STORE);
      } else {
        head(c->x, nb, logits + (size_t)b0 * g.vocab, hid);
      }
    }
    return QTALK_OK;
  }
};

qtalk_status launch_status(qtalk_ctx* c) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(c, QTALK_E_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return QTALK_OK;
}

qtalk_status copy_in(void* dst, const void* src, size_t bytes) {
  return hipMemcpy(dst, src, bytes, hipMemcpyDefault) == hipSuccess ? QTALK_OK : QTALK_E_DEVICE;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

qtalk_status qtalk_create(const qtalk_config* config, const qtalk_weights* w, void* hip_stream,
                          qtalk_ctx** out) {
  if (!out) return QTALK_E_INVAL;
  *out = nullptr;
  if (!config || !w || !w->layers || !w->final_norm || !w->codec_head) return QTALK_E_INVAL;
  if (check_config(config)) return QTALK_E_INVAL;
  const qtalk_config& g = *config;
  for (int l = 0; l < g.n_layers; ++l) {
    const qtalk_layer_weights& lw = w->layers[l];
    if (!lw.q_proj || !lw.k_proj || !lw.v_proj || !lw.o_proj || !lw.gate_proj || !lw.up_proj ||
        !lw.down_proj || !lw.input_norm || !lw.post_attn_norm || !lw.q_norm || !lw.k_norm)
      return QTALK_E_INVAL;
  }

  qtalk_ctx* c = new qtalk_ctx();
  c->cfg = g;
  c->stream = reinterpret_cast<hipStream_t>(hip_stream);
  c->w_bf16 = g.weight_dtype == QTALK_BF16;
  c->kv_f16 = g.kv_dtype == QTALK_F16;
  c->kv = g.kv_dtype == QTALK_F16 ? KV_F16 : (g.kv_dtype == QTALK_Q8 ? KV_Q8 : KV_F32);
  c->kv_rb = kv_row_bytes(c->kv, g.head_dim);
  c->welem = c->w_bf16 ? 2 : 4;
  c->n_out_heads = std::max(1, (int)g.n_output_heads);
  c->q_dim = g.n_heads * g.head_dim;
  c->kv_dim = g.n_kv_heads * g.head_dim;
  c->qkv_dim = c->q_dim + 2 * c->kv_dim;
  const size_t H = g.hidden, I = g.intermediate, we = c->welem;
  const size_t n_qkv = (size_t)c->qkv_dim * H, n_o = H * c->q_dim, n_gu = 2 * I * H, n_d = H * I;
  const size_t per_layer = n_qkv + n_o + n_gu + n_d;
  const size_t norms_per_layer = 2 * H + 2 * (size_t)g.head_dim;
  c->layer_kv_elems = (size_t)g.max_seqs * g.n_kv_heads * g.max_seq_len * g.head_dim;
  // rows per matrix-core pass: a prefill chunk of one sequence, or the
  // stacked rows of a batched prefill over several
  c->tc = (int)std::min<long long>((long long)g.max_seq_len * g.max_seqs, MAX_CHUNK);
  const int part_rows = GEMV_ROWS;
  const int rows = std::max(c->tc, GEMV_ROWS);


  bool ok = dev_alloc(&c->wblob, per_layer * g.n_layers * we) &&
            dev_alloc((void**)&c->nblob, (norms_per_layer * g.n_layers + H) * 4) &&
            dev_alloc(&c->head, (size_t)c->n_out_heads * g.vocab * H * we) &&
            dev_alloc(&c->kc, c->layer_kv_rows() * c->kv_rb * g.n_layers) &&
            dev_alloc(&c->vc, c->layer_kv_rows() * c->kv_rb * g.n_layers) &&
            dev_alloc((void**)&c->rope, (size_t)g.max_seq_len * (g.head_dim / 2) * sizeof(float2)) &&
            dev_alloc((void**)&c->x, (size_t)rows * H * 4) &&
            dev_alloc((void**)&c->aux_err, 4) &&
            dev_alloc((void**)&c->step_in, H * 4) &&
            dev_alloc((void**)&c->ferr, 4) &&
            (c->kv != KV_Q8 || !c->w_bf16 ||
             !attn_prefill_supported(g.head_dim, g.n_heads / g.n_kv_heads) ||
             dev_alloc((void**)&c->kv16, (size_t)2 * g.n_kv_heads * g.max_seq_len * g.head_dim * 2)) &&
            dev_alloc((void**)&c->qkv, (size_t)rows * c->qkv_dim * 4) &&
            dev_alloc((void**)&c->att, (size_t)rows * c->q_dim * 4) &&
            dev_alloc((void**)&c->act, (size_t)rows * I * 4) &&
            dev_alloc((void**)&c->hn, (size_t)rows * H * 2) &&
            dev_alloc((void**)&c->part_o, (size_t)part_rows * g.n_heads * MAX_SPLITS * g.head_dim * 4) &&
            dev_alloc((void**)&c->part_ml, (size_t)part_rows * g.n_heads * MAX_SPLITS * 2 * 4) &&
            dev_alloc((void**)&c->work, WORK_ELEMS * 4);
  c->per_layer = per_layer;
  c->norms_per_layer = norms_per_layer;
  const char* env = getenv("QTALK_FUSED_DECODE");
  const char* env_coop = getenv("QTALK_COOPERATIVE");
  c->coop = env_coop && env_coop[0] == '1';
  if (const char* env_rows = getenv("QTALK_ATTN_ROWS")) c->attn_rows = atoi(env_rows) == 64 ? 64 : atoi(env_rows) == 32 ? 32 : 0;
  {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      c->ncu = ncu;
    c->dev = dev;
  }
  c->fused = ok && c->w_bf16 && (c->kv == KV_F16 || c->kv == KV_Q8) && !(env && env[0] == '0') &&
             c->dev < MAX_DEVICES &&
             g.n_layers <= 64 &&
             fused_decode_supported(g.hidden, c->q_dim, c->kv_dim, g.intermediate, g.vocab,
                                    g.n_heads, g.n_kv_heads, g.head_dim) &&
             fused_decode_fits();
  if (c->fused) {
    resolve_scratch(c->dev);
    if (hipEventCreateWithFlags(&c->chain_ev, hipEventDisableTiming) != hipSuccess) ok = false;
    const char* env_loc = getenv("QTALK_XCD_LOCAL");
    c->xcd_local = !(env_loc && env_loc[0] == '0') && fused_decode_xcd_layout_ok(c->stream, c->coop);
    ok = dev_alloc((void**)&c->ll, fused_decode_ll_words(g.n_layers) * 8) &&
         dev_alloc((void**)&c->fpart, fused_decode_part_words(g.n_layers) * 8);
  }
  if (!ok) {
    (void)hipGetLastError();
    free_all(c);
    delete c;
    return QTALK_E_NOMEM;
  }

  qtalk_status s = QTALK_OK;
  char* wb = reinterpret_cast<char*>(c->wblob);
  c->layers.resize(g.n_layers);
  for (int l = 0; l < g.n_layers && s == QTALK_OK; ++l) {
    const qtalk_layer_weights& lw = w->layers[l];
    LayerDev& L = c->layers[l];
    char* base = wb + (size_t)l * per_layer * we;
    L.wqkv = base;
    L.wo = base + n_qkv * we;
    L.wgu = base + (n_qkv + n_o) * we;
    L.wd = base + (n_qkv + n_o + n_gu) * we;
    float* nb = c->nblob + (size_t)l * norms_per_layer;
    L.g_in = nb;
    L.g_post = nb + H;
    L.g_q = nb + 2 * H;
    L.g_k = nb + 2 * H + g.head_dim;
    char* qkv = reinterpret_cast<char*>(L.wqkv);
    if (copy_in(qkv, lw.q_proj, (size_t)c->q_dim * H * we) ||
        copy_in(qkv + (size_t)c->q_dim * H * we, lw.k_proj, (size_t)c->kv_dim * H * we) ||
        copy_in(qkv + (size_t)(c->q_dim + c->kv_dim) * H * we, lw.v_proj, (size_t)c->kv_dim * H * we) ||
        copy_in(L.wo, lw.o_proj, n_o * we) || copy_in(L.wd, lw.down_proj, n_d * we) ||
        copy_in(L.g_in, lw.input_norm, H * 4) || copy_in(L.g_post, lw.post_attn_norm, H * 4) ||
        copy_in(L.g_q, lw.q_norm, g.head_dim * 4) || copy_in(L.g_k, lw.k_norm, g.head_dim * 4))
      s = QTALK_E_DEVICE;
    // gate|up interleaved in blocks of 16 rows: [g0..g15, u0..u15, g16.., u16..]
    const size_t blk = 16 * H * we;
    if (s == QTALK_OK &&
        (hipMemcpy2D(L.wgu, 2 * blk, lw.gate_proj, blk, blk, I / 16, hipMemcpyDefault) != hipSuccess ||
         hipMemcpy2D(reinterpret_cast<char*>(L.wgu) + blk, 2 * blk, lw.up_proj, blk, blk, I / 16,
                     hipMemcpyDefault) != hipSuccess))
      s = QTALK_E_DEVICE;
  }
  c->g_final = c->nblob + (size_t)g.n_layers * norms_per_layer;
  if (s == QTALK_OK && (copy_in(c->g_final, w->final_norm, H * 4) ||
                        copy_in(c->head, w->codec_head, (size_t)c->n_out_heads * g.vocab * H * we)))
    s = QTALK_E_DEVICE;
  if (s == QTALK_OK) {
    const size_t kv_bytes = c->layer_kv_rows() * c->kv_rb * g.n_layers;
    if (hipMemsetAsync(c->kc, 0, kv_bytes, c->stream) != hipSuccess ||
        hipMemsetAsync(c->vc, 0, kv_bytes, c->stream) != hipSuccess ||
        hipMemsetAsync(c->aux_err, 0, 4, c->stream) != hipSuccess)
      s = QTALK_E_DEVICE;
    if (hipMemsetAsync(c->ferr, 0, 4, c->stream) != hipSuccess ||
        (c->fused &&
         (hipMemsetAsync(c->ll, 0, fused_decode_ll_words(g.n_layers) * 8, c->stream) != hipSuccess ||
          hipMemsetAsync(c->fpart, 0, fused_decode_part_words(g.n_layers) * 8, c->stream) != hipSuccess)))
      s = QTALK_E_DEVICE;
    launch_rope_table(c->rope, g.max_seq_len, g.head_dim, (double)g.rope_theta, c->stream);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(c->stream) != hipSuccess)
      s = QTALK_E_DEVICE;
  }
  if (s != QTALK_OK) {
    free_all(c);
    delete c;
    return s;
  }
  c->cur_len.assign(g.max_seqs, 0);
  c->fused_first.assign(g.max_seqs, -1);
  *out = c;
  return QTALK_OK;
}

void qtalk_destroy(qtalk_ctx* c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->stream);
  if (c->fused) {
    DecodeChain& ch = g_chain[c->dev];
    std::lock_guard<std::mutex> lock(ch.mu);
    if (ch.stream == c->stream) ch.stream = nullptr;
  }
  if (c->chain_ev) (void)hipEventDestroy(c->chain_ev);
  free_all(c);
  delete c;
}

static qtalk_status seq_call(qtalk_ctx* c, int32_t seq, const float* emb, int32_t T, float* logits,
                             float* hidden_out, bool rewind) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", seq);
  if (T < 1) return fail(c, QTALK_E_INVAL, "T must be >= 1 (got %d)", T);
  if (!emb || !logits) return fail(c, QTALK_E_INVAL, "emb and logits must not be null");
  const int p0 = rewind ? 0 : c->cur_len[seq];
  if ((long long)p0 + T > c->cfg.max_seq_len)
    return fail(c, QTALK_E_OVERFLOW, "cache overflow: %d + %d > %d", p0, T, c->cfg.max_seq_len);
  Fwd f(c);
  qtalk_status s = QTALK_OK;
  if (c->fused && (T == 1 || (T <= FUSED_MAX_ROWS && c->kv != KV_Q8))) {
    // a row or two (the code predictor's prefill) as consecutive persistent
    // launches: row t attends to positions 0 .. p0 + t, as in the prefill.
    // Not for two rows over a Q8 cache: there the second row attends to the
    // first unquantised, and a launch per row would read it back quantised.
    for (int t = 0; t < T && s == QTALK_OK; ++t)
      s = f.run_fused(seq, p0 + t, emb + (size_t)t * c->cfg.hidden, logits,
                      t + 1 == T ? hidden_out : nullptr);
  } else {
    s = f.run_sequence(seq, p0, emb, T, logits, hidden_out);
    if (s == QTALK_OK) s = launch_status(c);
  }
  if (s == QTALK_OK) c->cur_len[seq] = p0 + T;
  return s;
}

qtalk_status qtalk_prefill(qtalk_ctx* c, int32_t seq, const float* emb, int32_t T, float* logits,
                           float* hidden_out) {
  return seq_call(c, seq, emb, T, logits, hidden_out, true);
}

qtalk_status qtalk_extend(qtalk_ctx* c, int32_t seq, const float* emb, int32_t T, float* logits,
                          float* hidden_out) {
  return seq_call(c, seq, emb, T, logits, hidden_out, false);
}

qtalk_status qtalk_prefill_batch(qtalk_ctx* c, int32_t n, const int32_t* seqs, const float* emb,
                                 int32_t T, float* logits, float* hidden_out) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (n < 1 || !seqs) return fail(c, QTALK_E_INVAL, "n must be >= 1 and seqs non-null");
  if (T < 1) return fail(c, QTALK_E_INVAL, "T must be >= 1 (got %d)", T);
  if (!emb || !logits) return fail(c, QTALK_E_INVAL, "emb and logits must not be null");
  std::vector<char> seen(c->cfg.max_seqs, 0);
  for (int b = 0; b < n; ++b) {
    if (seqs[b] < 0 || seqs[b] >= c->cfg.max_seqs)
      return fail(c, QTALK_E_INVAL, "bad sequence id %d", seqs[b]);
    if (seen[seqs[b]]) return fail(c, QTALK_E_INVAL, "sequence %d listed twice", seqs[b]);
    seen[seqs[b]] = 1;
  }
  if (T > c->cfg.max_seq_len)
    return fail(c, QTALK_E_OVERFLOW, "cache overflow: %d > %d", T, c->cfg.max_seq_len);
  Fwd f(c);
  qtalk_status s = f.run_batch_prefill(seqs, n, emb, T, logits, hidden_out);
  if (s == QTALK_OK) s = launch_status(c);
  if (s == QTALK_OK)
    for (int b = 0; b < n; ++b) c->cur_len[seqs[b]] = T;
  return s;
}

qtalk_status qtalk_decode(qtalk_ctx* c, int32_t seq, const float* emb, float* logits,
                          float* hidden_out) {
  if (!c || !c->fused) return seq_call(c, seq, emb, 1, logits, hidden_out, false);
  c->err.clear();
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", seq);
  if (!emb || !logits) return fail(c, QTALK_E_INVAL, "emb and logits must not be null");
  if (c->cur_len[seq] + 1 > c->cfg.max_seq_len)
    return fail(c, QTALK_E_OVERFLOW, "cache overflow: %d + 1 > %d", c->cur_len[seq],
                c->cfg.max_seq_len);
  Fwd f(c);
  const qtalk_status s = f.run_fused(seq, c->cur_len[seq], emb, logits, hidden_out);
  if (s == QTALK_OK) c->cur_len[seq] += 1;
  return s;
}

qtalk_status qtalk_decode_step(qtalk_ctx* c, int32_t seq, const float* emb, const qtalk_gather* gather,
                              float* logits, float* hidden_out, int32_t suppress_begin, int32_t keep_id,
                              int32_t* out_id) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", seq);
  if (!logits) return fail(c, QTALK_E_INVAL, "logits must not be null");
  if (!emb == !gather) return fail(c, QTALK_E_INVAL, "give exactly one of emb and gather");
  if (gather) {
    if (gather->n_tables < 1 || gather->n_tables > QTALK_MAX_GATHER || !gather->ids)
      return fail(c, QTALK_E_INVAL, "gather: n_tables must be 1..%d and ids non-null", QTALK_MAX_GATHER);
    for (int q = 0; q < gather->n_tables; ++q)
      if (!gather->tables[q] || gather->table_rows[q] < 1)
        return fail(c, QTALK_E_INVAL, "gather: table %d is null or empty", q);
    if (c->cfg.hidden % 4 || c->cfg.hidden > 4096)
      return fail(c, QTALK_E_INVAL, "gather: hidden must be a multiple of 4 and <= 4096");
  }
  if (c->cur_len[seq] + 1 > c->cfg.max_seq_len)
    return fail(c, QTALK_E_OVERFLOW, "cache overflow: %d + 1 > %d", c->cur_len[seq], c->cfg.max_seq_len);
  Fwd f(c);
  qtalk_status s = QTALK_OK;
  if (c->fused && (!gather || gather->n_tables == 1)) {
    // one launch: a one-table lookup and the pick inside the persistent decode
    const Fwd::Pick pk{out_id, suppress_begin, keep_id};
    s = f.run_fused(seq, c->cur_len[seq], emb, logits, hidden_out, false, gather, out_id ? &pk : nullptr);
  } else if (c->fused) {
    // a sum of several tables: the gather kernel, then one launch with the pick
    EmbedSumArgs e{};
    for (int q = 0; q < gather->n_tables; ++q) {
      e.tables[q] = gather->tables[q];
      e.rows[q] = gather->table_rows[q];
    }
    e.n_groups = gather->n_tables;
    e.n = 1;
    e.hidden = c->cfg.hidden;
    e.ids = gather->ids;
    e.overlay = gather->overlay;
    e.out = c->step_in;
    e.status = c->ferr;  // the decode status word: the position is rolled back at sync
    launch_embed_sum(e, c->stream);
    const Fwd::Pick pk{out_id, suppress_begin, keep_id};
    s = f.run_fused(seq, c->cur_len[seq], c->step_in, logits, hidden_out, false, nullptr,
                    out_id ? &pk : nullptr);
  } else {
    // the same steps as separate launches: gather, decode, pick
    if (gather) {
      EmbedSumArgs e{};
      for (int q = 0; q < gather->n_tables; ++q) {
        e.tables[q] = gather->tables[q];
        e.rows[q] = gather->table_rows[q];
      }
      e.n_groups = gather->n_tables;
      e.n = 1;
      e.hidden = c->cfg.hidden;
      e.ids = gather->ids;
      e.overlay = gather->overlay;
      e.out = c->step_in;
      e.status = c->ferr;  // like the persistent decode's: the position is rolled back at sync
      launch_embed_sum(e, c->stream);
      emb = c->step_in;
      int32_t& first = c->fused_first[seq];
      first = first < 0 ? c->cur_len[seq] : std::min(first, c->cur_len[seq]);
    }
    s = f.run_sequence(seq, c->cur_len[seq], emb, 1, logits, hidden_out);
    if (s == QTALK_OK && out_id) {
      ArgmaxArgs am{logits, 1, c->cfg.vocab, suppress_begin, keep_id, out_id, nullptr, 0, 0, nullptr, nullptr};
      launch_argmax(am, c->stream);
    }
    if (s == QTALK_OK) s = launch_status(c);
  }
  if (s == QTALK_OK) c->cur_len[seq] += 1;
  return s;
}

qtalk_status qtalk_decode_noalloc(qtalk_ctx* c, int32_t seq, const float* emb, float* logits,
                                  float* hidden_out) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (!c->fused)
    return fail(c, QTALK_E_INVAL, "qtalk_decode_noalloc needs the persistent decode (Talker geometry, bf16 weights)");
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", seq);
  if (!emb || !logits) return fail(c, QTALK_E_INVAL, "emb and logits must not be null");
  const size_t need = (fused_decode_ll_words(c->cfg.n_layers) + fused_decode_part_words(c->cfg.n_layers)) * 8;
  if (need > SCRATCH_BYTES)
    return fail(c, QTALK_E_INVAL, "qtalk_decode_noalloc needs %zu bytes of static scratch, it holds %zu", need,
                SCRATCH_BYTES);
  if (!g_scratch[c->dev].ptr)
    return fail(c, QTALK_E_DEVICE, "the static scratch array has no address on device %d", c->dev);
  if (c->cur_len[seq] + 1 > c->cfg.max_seq_len)
    return fail(c, QTALK_E_OVERFLOW, "cache overflow: %d + 1 > %d", c->cur_len[seq], c->cfg.max_seq_len);
  Fwd f(c);
  const qtalk_status s = f.run_fused(seq, c->cur_len[seq], emb, logits, hidden_out, true);
  if (s == QTALK_OK) c->cur_len[seq] += 1;
  return s;
}

qtalk_status qtalk_decode_batch(qtalk_ctx* c, int32_t n, const int32_t* seqs, const float* emb,
                                float* logits, float* hidden_out) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (n < 1 || n > c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "n must be in [1, max_seqs]");
  if (!seqs || !emb || !logits) return fail(c, QTALK_E_INVAL, "seqs, emb and logits must not be null");
  std::vector<char> seen(c->cfg.max_seqs, 0);
  for (int i = 0; i < n; ++i) {
    const int s = seqs[i];
    if (s < 0 || s >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", s);
    if (seen[s]) return fail(c, QTALK_E_INVAL, "sequence %d listed twice", s);
    seen[s] = 1;
    if (c->cur_len[s] + 1 > c->cfg.max_seq_len)
      return fail(c, QTALK_E_OVERFLOW, "cache overflow on sequence %d", s);
  }
  Fwd f(c);
  qtalk_status st = f.run_batch(seqs, n, emb, logits, hidden_out);
  if (st == QTALK_OK) st = launch_status(c);
  if (st == QTALK_OK)
    for (int i = 0; i < n; ++i) c->cur_len[seqs[i]] += 1;
  return st;
}

qtalk_status qtalk_kv_rewind(qtalk_ctx* c, int32_t seq, int32_t n_keep) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(c, QTALK_E_INVAL, "bad sequence id %d", seq);
  if (n_keep < 0 || n_keep > c->cur_len[seq])
    return fail(c, QTALK_E_INVAL, "n_keep %d outside [0, %d]", n_keep, c->cur_len[seq]);
  c->cur_len[seq] = n_keep;
  return QTALK_OK;
}

int32_t qtalk_kv_len(const qtalk_ctx* c, int32_t seq) {
  if (!c || seq < 0 || seq >= c->cfg.max_seqs) return -1;
  return c->cur_len[seq];
}

qtalk_status qtalk_kv_read(qtalk_ctx* c, int32_t seq, int32_t layer, int32_t kv, float* dst) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (seq < 0 || seq >= c->cfg.max_seqs || layer < 0 || layer >= c->cfg.n_layers ||
      (kv != 0 && kv != 1) || !dst)
    return fail(c, QTALK_E_INVAL, "bad kv_read arguments");
  const qtalk_config& g = c->cfg;
  const char* base = reinterpret_cast<const char*>(kv ? c->vc : c->kc) +
                     ((size_t)layer * c->layer_kv_rows() + (size_t)seq * g.n_kv_heads * g.max_seq_len) *
                         c->kv_rb;
  launch_kv_to_f32(c->kv, base, g.n_kv_heads, g.max_seq_len, c->cur_len[seq], g.head_dim, dst,
                   c->stream);
  return launch_status(c);
}

qtalk_status qtalk_embed_sum(qtalk_ctx* c, int32_t n_groups, const float* const* tables,
                             const int32_t* table_rows, const int32_t* ids, int32_t n,
                             const float* overlay, float* out) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (n_groups < 1 || n_groups > MAX_EMBED_GROUPS)
    return fail(c, QTALK_E_INVAL, "n_groups must be 1..%d", MAX_EMBED_GROUPS);
  if (n < 1) return fail(c, QTALK_E_INVAL, "n must be >= 1");
  if (!tables || !table_rows || !ids || !out)
    return fail(c, QTALK_E_INVAL, "tables, table_rows, ids and out must not be null");
  if (c->cfg.hidden % 4 || c->cfg.hidden > 4096)
    return fail(c, QTALK_E_INVAL, "hidden must be a multiple of 4 and <= 4096");
  EmbedSumArgs a{};
  for (int g = 0; g < n_groups; ++g) {
    if (!tables[g] || table_rows[g] < 1) return fail(c, QTALK_E_INVAL, "table %d is null or empty", g);
    a.tables[g] = tables[g];
    a.rows[g] = table_rows[g];
  }
  a.n_groups = n_groups;
  a.n = n;
  a.hidden = c->cfg.hidden;
  a.ids = ids;
  a.overlay = overlay;
  a.out = out;
  a.status = c->aux_err;
  launch_embed_sum(a, c->stream);
  return launch_status(c);
}

qtalk_status qtalk_argmax(qtalk_ctx* c, const float* logits, int32_t n, int32_t vocab,
                          int32_t suppress_begin, int32_t keep_id, int32_t* out_ids) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (!logits || !out_ids) return fail(c, QTALK_E_INVAL, "logits and out_ids must not be null");
  if (n < 1 || vocab < 1) return fail(c, QTALK_E_INVAL, "n and vocab must be >= 1");
  ArgmaxArgs a{logits, n, vocab, suppress_begin, keep_id, out_ids, nullptr, 0, 0, nullptr, nullptr};
  launch_argmax(a, c->stream);
  return launch_status(c);
}

qtalk_status qtalk_argmax_embed(qtalk_ctx* c, const float* logits, int32_t n, int32_t vocab,
                                int32_t suppress_begin, int32_t keep_id, const float* table,
                                int32_t table_rows, int32_t* out_ids, float* out_rows) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (!logits || !out_ids || !table || !out_rows)
    return fail(c, QTALK_E_INVAL, "logits, table, out_ids and out_rows must not be null");
  if (n < 1 || vocab < 1 || table_rows < 1) return fail(c, QTALK_E_INVAL, "n, vocab and table_rows must be >= 1");
  ArgmaxArgs a{logits, n, vocab, suppress_begin, keep_id, out_ids,
               table, table_rows, c->cfg.hidden, out_rows, c->aux_err};
  launch_argmax(a, c->stream);
  return launch_status(c);
}

qtalk_status qtalk_select_head(qtalk_ctx* c, int32_t head) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (head < 0 || head >= c->n_out_heads)
    return fail(c, QTALK_E_INVAL, "head %d out of range 0..%d", head, c->n_out_heads - 1);
  c->head_sel = head;
  return QTALK_OK;
}

qtalk_status qtalk_sync(qtalk_ctx* c) {
  if (!c) return QTALK_E_INVAL;
  const hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return fail(c, QTALK_E_DEVICE, "stream failed: %s", hipGetErrorString(e));
  std::string msg;
  {
    int code = 0;
    if (hipMemcpy(&code, c->ferr, 4, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(c, QTALK_E_DEVICE, "cannot read the decode status word");
    if (code) {
      // a persistent launch gave up (1) or ran on unexpected XCDs (3), or a
      // step input's id was outside its table (5): the positions written by
      // such launches since the last sync, and everything after them, are
      // dropped; later launches start clean
      if (hipMemset(c->ferr, 0, 4) != hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot clear the decode status word");
      if (code == 3) c->xcd_local = false;  // later steps use device-scope exchanges
      char buf[160];
      snprintf(buf, sizeof buf, "%s (code %d); rolled back:",
               code == 3   ? "persistent decode: blocks did not run on the expected XCDs"
               : code == 5 ? "decode step: an id of the gathered input was outside its table"
                           : "persistent decode gave up waiting",
               code);
      msg = buf;
      for (int s = 0; s < c->cfg.max_seqs; ++s) {
        const int32_t f = c->fused_first[s];
        if (f >= 0 && f < c->cur_len[s]) {
          snprintf(buf, sizeof buf, " seq %d to %d;", s, f);
          msg += buf;
          c->cur_len[s] = f;
        }
      }
    }
    std::fill(c->fused_first.begin(), c->fused_first.end(), -1);
  }
  {
    int code = 0;
    if (hipMemcpy(&code, c->aux_err, 4, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(c, QTALK_E_DEVICE, "cannot read the frame-step status word");
    if (code) {
      if (hipMemset(c->aux_err, 0, 4) != hipSuccess)
        return fail(c, QTALK_E_DEVICE, "cannot clear the frame-step status word");
      msg += msg.empty() ? "" : " ";
      msg += "frame step: an id was outside its table (those rows hold NaN)";
    }
  }
  if (!msg.empty()) return fail(c, QTALK_E_DEVICE, "%s", msg.c_str());
  return QTALK_OK;
}

qtalk_status qtalk_set_wait_limit(qtalk_ctx* c, int64_t polls) {
  if (!c) return QTALK_E_INVAL;
  c->err.clear();
  if (polls < 0) return fail(c, QTALK_E_INVAL, "polls must be >= 0");
  c->spin_limit = polls ? (long)polls : FUSED_SPIN_LIMIT;
  return QTALK_OK;
}

const char* qtalk_last_error(const qtalk_ctx* c) { return c ? c->err.c_str() : "null context"; }

}  // extern "C"
#pragma GCC visibility pop
