// Prefill projections on the matrix cores: C[M][N] = A[M][K] * B[N][K]^T with
// A the (normalised) activations in bf16 and B a weight matrix stored
// [out][in] in bf16, float32 accumulation ("transcribe.cpp
// src/causal_lm/causal_lm.cpp", mul_mat_f32acc).  Both operands are
// K-contiguous, so every lane feeds v_mfma_f32_16x16x32_bf16 with one 16-byte
// LDS read per operand.
//
// Tiles: BM x 128 per 256-thread block (4 waves as 2 x 2, each BM/2 x 64),
// BK = 64, rows padded to 72 elements in LDS.  Global loads for the next K
// tile are issued before the MFMAs of the current one.  Small-M shapes split
// K over blockIdx.z into a float32 workspace that a second kernel sums in a
// fixed order (deterministic), applying the epilogue there.
#include "kernels.h"
#include "kv_row.h"
#include "lds_dma.h"

namespace qtalk {

constexpr int GB_N = 128;
constexpr int GB_K = 64;
constexpr int G_STRIDE = GB_K + 8;  // bf16 elements per LDS row

template <int BM, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs a, int k_per_split) {
  constexpr int BN = GB_N;
  constexpr int TM = BM / 32;  // 16-row MFMA tiles per wave (M)
  constexpr int TN = BN / 32;  // 16-col MFMA tiles per wave (N)
  constexpr int AR = BM / 32;  // 16-byte A chunks per thread per K tile
  constexpr int BR = BN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * G_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * G_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int kbeg = blockIdx.z * k_per_split;
  const int nkt = k_per_split / GB_K;
  const int M = a.M, K = a.K;

  // global -> register staging roles
  const int lrow = tid >> 3, lchunk = (tid & 7) * 8;
  const bf16_t* Ag[AR];
  const bf16_t* Bg[BR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    int r = m0 + lrow + 32 * i;
    r = r < M ? r : M - 1;
    Ag[i] = a.A + (size_t)r * a.lda + kbeg + lchunk;
  }
#pragma unroll
  for (int i = 0; i < BR; ++i) Bg[i] = a.B + (size_t)(n0 + lrow + 32 * i) * K + kbeg + lchunk;

  // staging registers as named scalars (AR is 2 or 4, BR is 4): an array
  // here is left in private memory by the compiler
  static_assert((AR == 2 || AR == 4) && BR == 4, "staging layout");
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define QG_LDA(I, KT) (*reinterpret_cast<const uint4*>(Ag[I] + (KT) * GB_K))
#define QG_GLOAD(KT)                                                    \
  do {                                                                  \
    const int kt_ = (KT);                                               \
    ra0 = QG_LDA(0, kt_);                                               \
    ra1 = QG_LDA(1, kt_);                                               \
    if (AR == 4) {                                                      \
      ra2 = QG_LDA(AR == 4 ? 2 : 0, kt_);                               \
      ra3 = QG_LDA(AR == 4 ? 3 : 0, kt_);                               \
    }                                                                   \
    rb0 = ld_stream16(Bg[0] + kt_ * GB_K);                              \
    rb1 = ld_stream16(Bg[1] + kt_ * GB_K);                              \
    rb2 = ld_stream16(Bg[2] + kt_ * GB_K);                              \
    rb3 = ld_stream16(Bg[3] + kt_ * GB_K);                              \
  } while (0)
#define QG_ST(BUF, ROW, V) *reinterpret_cast<uint4*>(&BUF[(lrow + (ROW)) * G_STRIDE + lchunk]) = (V)
#define QG_LSTORE()                  \
  do {                               \
    QG_ST(As, 0, ra0);               \
    QG_ST(As, 32, ra1);              \
    if (AR == 4) {                   \
      QG_ST(As, 64, ra2);            \
      QG_ST(As, 96, ra3);            \
    }                                \
    QG_ST(Bs, 0, rb0);               \
    QG_ST(Bs, 32, rb1);              \
    QG_ST(Bs, 64, rb2);              \
    QG_ST(Bs, 96, rb3);              \
  } while (0)

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  QG_GLOAD(0);
  QG_LSTORE();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    QG_GLOAD(min(kt + 1, nkt - 1));  // unconditional (repeats the last tile) so ra/rb stay in registers
#pragma unroll
    for (int ks = 0; ks < GB_K; ks += 32) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            &As[(wm * (BM / 2) + i * 16 + fr) * G_STRIDE + ks + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            &Bs[(wn * (BN / 2) + j * 16 + fr) * G_STRIDE + ks + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      QG_LSTORE();
      __syncthreads();
    }
  }
#undef QG_LDA
#undef QG_GLOAD
#undef QG_ST
#undef QG_LSTORE

  // epilogue: lane holds C[rbase + r][cbase + (lane & 15)], r = 0..3
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int rbase = m0 + wm * (BM / 2) + i * 16 + rq;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rbase + r;
        if (row >= M) continue;
        const float v = acc[i][j][r];
        if (SPLIT) {
          a.work[((size_t)blockIdx.z * M + row) * a.N + col] = v;
        } else if (EPI == EPI_STORE) {
          reinterpret_cast<float*>(a.C)[(size_t)row * a.ldc + col] = v;
        } else if (EPI == EPI_ADD) {
          reinterpret_cast<float*>(a.C)[(size_t)row * a.ldc + col] += v;
        } else if ((j & 1) == 0) {  // SwiGLU: tile j = gate block, j+1 = up block
          const float u = acc[i][j + 1 < TN ? j + 1 : j][r];
          const int oc = (n0 + wn * (BN / 2) + j * 16) / 2 + fr;
          reinterpret_cast<bf16_t*>(a.C)[(size_t)row * a.ldc + oc] =
              (bf16_t)f32_to_bf16(silu_f(v) * u);
        }
      }
    }
  }
}

// Large-M variant with direct-to-LDS loads: 256 x BN block tile over 8 waves
// (4 x 2, a 64 x BN/2 tile each, 32x32x16 MFMA), K tiles of BK.  Global
// tiles go straight into LDS with global_load_lds_dwordx4 (no register
// staging, no LDS store instructions) into NS stages, NS - 1 tiles in flight
// while one is read.  LDS rows (BK bf16) are unpadded; 16-byte chunk c of
// row r sits in slot c ^ ((r / RB) % CPR), RB rows per 256 bytes, CPR chunks
// per row.  The LDS serves a 16-byte read of 16 lanes per clock from its 64
// banks, and an operand read gives 16 lanes 16 consecutive rows of one
// chunk, which this layout spreads over all 64 banks.  The loads produce it
// by giving lane l of the instruction that starts at row R (a multiple of
// RPI = 64 / CPR rows) row R + l / CPR and chunk (l % CPR) ^ (((R + l / CPR)
// / RB) % CPR).  BN = 192 gives the 6144-wide gate|up projection exactly 256
// tiles at M = 2048.  (32-deep tiles with five or six stages measured 4-8%
// slower at 1920 rows: the copy is bound by L2 bandwidth, not by the bytes
// in flight.)

template <int BN>
struct DmaCfg {
  static constexpr int BK = 64;
  static constexpr int NS = BN == 128 ? 3 : 2;  // LDS stages: 144 or 112 KiB
};

template <int BN, int EPI, bool SPLIT>
__global__ __launch_bounds__(512) void k_gemm_dma(GemmArgs a, int k_per_split) {
  constexpr int BM = 256, BK = DmaCfg<BN>::BK, NS = DmaCfg<BN>::NS;
  constexpr int CPR = BK / 8, RPI = 64 / CPR, RB = 128 / BK;
  constexpr int KS = BK / 16;                 // MFMA k-steps per tile
  constexpr int JA = BM / RPI / 8;            // A load instructions per wave and tile
  constexpr int NB = BN / RPI;                // B load instructions per tile
  constexpr int JB = (NB + 7) / 8;            // ... per wave, at most
  constexpr int WTM = BM / 4, WTN = BN / 2;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(KS % 2 == 0 && (BM / RPI) % 8 == 0, "tile split");
  __shared__ __attribute__((aligned(1024))) bf16_t As[NS][BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t Bs[NS][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // Blocks are dealt round-robin over the 8 XCDs (block i to XCD i % 8).
  // Split-K grids take logical tile i / 8 + (i % 8) * (grid / 8), so each
  // XCD runs a run of consecutive logical tiles (column tiles fastest): the
  // column tiles of a few row tiles in one K range, which share their A
  // tiles in that XCD's L2 (the hardware order would give an XCD one column
  // tile and every row tile and K range, and no A tile twice).
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (SPLIT) {
    const int nx = gridDim.x, nxy = nx * gridDim.y, total = nxy * gridDim.z;
    if (total % 8 == 0) {
      const int lin = blockIdx.x + nx * (blockIdx.y + gridDim.y * blockIdx.z);
      const int lg = (lin & 7) * (total >> 3) + (lin >> 3);
      bz = lg / nxy;
      by = (lg - bz * nxy) / nx;
      bx = lg - bz * nxy - by * nx;
    }
  }
  const int n0 = bx * BN, m0 = by * BM;
  const int kbeg = bz * k_per_split;
  const int nkt = k_per_split / BK;
  const int M = a.M, K = a.K;

  // this wave's load instructions: A rows (wave + 8 j) * RPI for j < JA, then
  // B rows (wave + 8 j) * RPI; the last B slot only for waves below NB % 8
  // (A rows past M re-read row M - 1; never stored)
  const bool bx_last = (NB % 8 == 0) || wave < NB % 8;
  const bf16_t* ag[JA];
  const bf16_t* bg[JB];
  auto src_chunk = [&](int R) { return ((lane % CPR) ^ (((R + lane / CPR) / RB) % CPR)) * 8; };
#pragma unroll
  for (int j = 0; j < JA; ++j) {
    const int R = (wave + 8 * j) * RPI;
    ag[j] = a.A + (size_t)min(m0 + R + lane / CPR, M - 1) * a.lda + kbeg + src_chunk(R);
  }
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int R = (j == JB - 1 && !bx_last ? 0 : wave + 8 * j) * RPI;  // unused slot: any valid row
    bg[j] = a.B + (size_t)(n0 + R + lane / CPR) * K + kbeg + src_chunk(R);
  }
  const int lpt = JA + (NB / 8) + (NB % 8 != 0 && bx_last ? 1 : 0);  // loads per wave and tile

#define QD_ISSUE(KT, S)                                                                           \
  do {                                                                                            \
    const int kt_ = (KT), s_ = (S);                                                               \
    _Pragma("unroll") for (int j = 0; j < JA; ++j)                                                \
        lds_load16(ag[j] + kt_ * BK, &As[s_][(wave + 8 * j) * RPI * BK]);                         \
    _Pragma("unroll") for (int j = 0; j < JB; ++j) if (j < JB - 1 || bx_last)                      \
        lds_load16(bg[j] + kt_ * BK, &Bs[s_][(wave + 8 * j) * RPI * BK]);                         \
  } while (0)
  // wait until this wave has at most T tiles of loads outstanding (loads retire in order)
#define QD_WAIT_TILES(T)                                                                          \
  do {                                                                                            \
    if (lpt == JA + NB / 8) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((T) * (JA + NB / 8)) : "memory"); \
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((T) * (JA + NB / 8 + 1)) : "memory");           \
  } while (0)

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  // operand reads: row (l % 32) of each 32-row fragment, chunk 2 s + l / 32
  // (fragments start at multiples of 32 rows, so the slot is a function of l).
  // They are inline asm: the compiler would otherwise wait for every
  // outstanding direct-to-LDS load (tiles in flight included) before the
  // first read.  The statements after the wait name the fragments it guards,
  // so no MFMA is scheduled above it.  The reads of the next k-step go out
  // while the MFMAs of this one run; a register they refill was last read by
  // an MFMA already issued (MFMAs take their A/B operands at issue).
  const int fr = lane & 31, fh = lane >> 5, fx = (fr / RB) % CPR;
  const uint32_t a_off = (uint32_t)(uintptr_t)(As[0] + (wm * WTM + fr) * BK);
  const uint32_t b_off = (uint32_t)(uintptr_t)(Bs[0] + (wn * WTN + fr) * BK);
  constexpr int NF = TM + TN;  // fragments per k-step: A 0..TM-1, then B
#define QD_READ(X, S, KS_)                                                                    \
  do {                                                                                        \
    const uint32_t ab_ = a_off + (S) * (BM * BK * 2), bb_ = b_off + (S) * (BN * BK * 2);      \
    const uint32_t slot_ = (((2 * (KS_) + fh) ^ fx) * 16);                                    \
    _Pragma("unroll") for (int q = 0; q < NF; ++q) {                                          \
      const uint32_t addr_ = (q < TM ? ab_ + q * 32 * BK * 2 : bb_ + (q - TM) * 32 * BK * 2) + slot_; \
      asm volatile("ds_read_b128 %0, %1" : "=v"(X[q]) : "v"(addr_));                         \
    }                                                                                         \
  } while (0)

  // Pipeline.  The prologue requests tiles 0 .. NS-1 (one per stage).
  // Operand reads run two k-steps ahead, one fragment set per k-step of the
  // tile (KS = 4 sets).  At k-step 2 of tile kt every read of tile kt has
  // been issued; the wave waits for all of them and for its loads of tile
  // kt + 1, and the raw barrier (not __syncthreads, which would also wait
  // for the loads in flight) makes every wave's part of tile kt + 1 visible
  // and tells that tile kt's stage has been read by all waves: tile kt + NS
  // goes there, and the reads of tile kt + 1's k-steps 0 and 1 are issued
  // under tile kt's last two steps of MFMAs.
  static_assert(KS == 4, "four k-steps per tile");
  bf16x8_t fb[KS][NF];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nkt) QD_ISSUE(s, s);
  if (nkt >= NS) QD_WAIT_TILES(NS - 1);
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  QD_READ(fb[0], 0, 0);
  QD_READ(fb[1], 0, 1);
#define QD_MFMA(X)                                                                            \
  do {                                                                                        \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                            \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) acc[i][j] =                            \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(X[i], X[TM + j], acc[i][j], 0, 0, 0);     \
  } while (0)
#define QD_FENCE(X) _Pragma("unroll") for (int q = 0; q < NF; ++q) asm volatile("" : "+v"(X[q]))
  int st = 0;  // stage of tile kt
  for (int kt = 0; kt < nkt; ++kt) {
    const int nst = st + 1 == NS ? 0 : st + 1;
    // k-step 0: its reads done, those of step 1 may be outstanding (LDS
    // reads retire in order)
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NF) : "memory");
    QD_FENCE(fb[0]);
    QD_READ(fb[2], st, 2);
    QD_MFMA(fb[0]);
    // k-step 1
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(NF) : "memory");
    QD_FENCE(fb[1]);
    QD_READ(fb[3], st, 3);
    QD_MFMA(fb[1]);
    // k-step 2: every read of tile kt done
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    QD_FENCE(fb[2]);
    QD_FENCE(fb[3]);
    if (kt + 1 < nkt) {
      if (kt + NS - 1 < nkt) QD_WAIT_TILES(NS - 2);
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + NS < nkt) QD_ISSUE(kt + NS, st);
      QD_READ(fb[0], nst, 0);
    }
    QD_MFMA(fb[2]);
    // k-step 3
    if (kt + 1 < nkt) QD_READ(fb[1], nst, 1);
    QD_MFMA(fb[3]);
    st = nst;
  }
#undef QD_MFMA
#undef QD_FENCE

#undef QD_ISSUE
#undef QD_WAIT_TILES
#undef QD_READ

  // epilogue: register r of lane l is C[row (r/4)*8 + (l/32)*4 + r%4][col l%32]
  if constexpr (EPI == EPI_SWIGLU && !SPLIT) {
    // SwiGLU: columns 0..15 of each 32-column fragment are gate rows of the
    // weight, 16..31 the matching up rows.  v_permlane16_swap of registers
    // 2p and 2p + 1 (rows r and r + 1) swaps the odd 16-lane rows of the
    // first with the even rows of the second, which leaves every lane the
    // gate and the up value of one output: lanes 16..31 of each half take
    // row r + 1.  The bf16 tile is staged in the A stages (free once every
    // wave has read the last one) and leaves in 16-byte row chunks.
    constexpr int OC = BN / 2, OLD = OC + 8;  // output columns, LDS row stride
    static_assert(BM * OLD <= NS * BM * BK && OC % 8 == 0, "output tile staging");
    bf16_t* const os = &As[0][0];
    __syncthreads();
    const int odd = (lane >> 4) & 1, c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int rb = wm * WTM + i * 32 + (lane >> 5) * 4 + odd;
        const int oc = (wn * WTN + j * 32) / 2 + c16;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][2 * p]),
                                                           __float_as_uint(acc[i][j][2 * p + 1]), false, false);
          const int row = rb + (p >> 1) * 8 + (p & 1) * 2;
          os[row * OLD + oc] = (bf16_t)f32_to_bf16(silu_f(__uint_as_float(sw[0])) * __uint_as_float(sw[1]));
        }
      }
    __syncthreads();
    constexpr int CH = OC / 8;  // 16-byte chunks per output row
    bf16_t* const cb = reinterpret_cast<bf16_t*>(a.C) + n0 / 2;
    for (int q = tid; q < BM * CH; q += 512) {
      const int row = q / CH, ch = q % CH;
      if (m0 + row < M)
        *reinterpret_cast<uint4*>(cb + (size_t)(m0 + row) * a.ldc + ch * 8) =
            *reinterpret_cast<const uint4*>(os + row * OLD + ch * 8);
    }
    return;
  }
  if constexpr (EPI == EPI_STORE && !SPLIT && BN == 128) {
    // Row r's position, and the element offset (head 0) of its cache row:
    // one sequence, base0 + r * 128; stacked sequences, formed for the 8
    // rows i * 32 + tid / 16 this thread stores before any store (a load
    // issued after a store waits for it), with the sequence index (r + 1/2)
    // / kv_per taken in float32 (exact for the row counts a product holds)
    // instead of an integer division
    const int per = a.kv_per;
    const float inv_per = per > 0 ? 1.0f / (float)per : 0.f;
    auto kv_seq = [&](int r) { return per > 0 ? (int)(((float)r + 0.5f) * inv_per) : 0; };
    auto kv_pos = [&](int r) { return a.vpos0 + r - kv_seq(r) * per; };
    const size_t base0 = (size_t)a.kv_seqs[0] * a.kv_seq_stride + (size_t)(a.vpos0 + m0) * 128;
    size_t roff[8];
    if (per > 0 && a.kcache != nullptr && n0 >= a.kcol) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = min(m0 + i * 32 + (tid >> 4), M - 1);
        const int z = kv_seq(r);
        roff[i] = (size_t)a.kv_seqs[z] * a.kv_seq_stride + (size_t)(a.vpos0 + r - z * per) * 128;
      }
    }
    if (a.kcache != nullptr && n0 < a.vcol) {
      // a q or K head (128 columns): float32 rows staged in the free A
      // stages, 128 rows at a time; 16 lanes per row, lane i holding dims
      // 4i .. 4i+3 and their RoPE partners 64 + 4i .. (the arithmetic of the
      // append kernel: per-head RMSNorm, NEOX rotation; q then times the
      // score scale), float16 to the cache (K) or in place into C (q)
      const bool is_q = n0 < a.kcol;
      const float* const gain = is_q ? a.g_q : a.g_k;
      const float scale = is_q ? a.qscale : 1.0f;
      constexpr int FLD = 128 + 4;  // LDS row stride (floats)
      static_assert(128 * FLD * 4 <= NS * BM * BK * 2, "q/K tile staging");
      float* const fs = reinterpret_cast<float*>(&As[0][0]);
      const int i4 = (tid & 15) * 4;
      const float4 g1 = *reinterpret_cast<const float4*>(gain + i4);
      const float4 g2 = *reinterpret_cast<const float4*>(gain + 64 + i4);
      // rotations of every row this thread forms (8 passes of 32 rows),
      // requested before the staging so that they have landed by then
      float4 cr[8][2];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int pos = kv_pos(min(m0 + p * 32 + (tid >> 4), M - 1));
        cr[p][0] = *reinterpret_cast<const float4*>(a.rope + (size_t)pos * 64 + i4);
        cr[p][1] = *reinterpret_cast<const float4*>(a.rope + (size_t)pos * 64 + i4 + 2);
      }
      f16_t* const khead = a.kcache + (size_t)((is_q ? 0 : n0 - a.kcol) / 128) * a.vcap * 128;
      f16_t* const qhead = reinterpret_cast<f16_t*>(reinterpret_cast<float*>(a.C) + (size_t)m0 * a.ldc) + n0;
      typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        __syncthreads();  // LDS free: the last K stage read, or the previous half formed
        if ((wm >> 1) == half) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = (wm & 1) * WTM + i * 32 + (lane >> 5) * 4 + (r >> 2) * 8 + (r & 3);
                fs[row * FLD + wn * WTN + j * 32 + fr] = acc[i][j][r];
              }
        }
        __syncthreads();
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int rr = pp * 32 + (tid >> 4);  // row within this half
          const int row = half * 128 + rr;
          float4 x1 = *reinterpret_cast<const float4*>(fs + rr * FLD + i4);
          float4 x2 = *reinterpret_cast<const float4*>(fs + rr * FLD + 64 + i4);
          k_row_norm_rope(x1, x2, g1, g2, cr[half * 4 + pp][0], cr[half * 4 + pp][1], a.eps);
          if (is_q) {  // q: the score scale
            x1.x *= scale; x1.y *= scale; x1.z *= scale; x1.w *= scale;
            x2.x *= scale; x2.y *= scale; x2.z *= scale; x2.w *= scale;
          }
          if (m0 + row < M) {
            f16_t* const kdst = is_q ? qhead + (size_t)row * a.ldc * 2
                                     : khead + (per > 0 ? roff[half * 4 + pp] : base0 + (size_t)row * 128);
            const f16x4_t o1 = {(f16_t)x1.x, (f16_t)x1.y, (f16_t)x1.z, (f16_t)x1.w};
            const f16x4_t o2 = {(f16_t)x2.x, (f16_t)x2.y, (f16_t)x2.z, (f16_t)x2.w};
            *reinterpret_cast<f16x4_t*>(kdst + i4) = o1;
            *reinterpret_cast<f16x4_t*>(kdst + 64 + i4) = o2;
          }
        }
      }
      return;
    }
    if (a.vcache != nullptr && n0 >= a.vcol) {
      // a V head (128 columns): float16 rows staged in the free A stages,
      // then 16-byte chunks of the 256-byte cache rows (the same round to
      // nearest as the append kernel)
      constexpr int OLD = 128 + 8;  // LDS row stride (halfs)
      static_assert(BM * OLD * 2 <= NS * BM * BK * 2, "V tile staging");
      f16_t* const os = reinterpret_cast<f16_t*>(&As[0][0]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * WTM + i * 32 + (lane >> 5) * 4 + (r >> 2) * 8 + (r & 3);
            os[row * OLD + wn * WTN + j * 32 + fr] = (f16_t)acc[i][j][r];
          }
      __syncthreads();
      f16_t* const vhead = a.vcache + (size_t)((n0 - a.vcol) / 128) * a.vcap * 128;
      static_assert(BM * 16 == 8 * 512, "8 rows per thread");
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = i * 32 + (tid >> 4), ch = tid & 15;
        if (m0 + row < M)
          *reinterpret_cast<uint4*>(vhead + (per > 0 ? roff[i] : base0 + (size_t)row * 128) + ch * 8) =
              *reinterpret_cast<const uint4*>(os + row * OLD + ch * 8);
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int rbase = m0 + wm * WTM + i * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cbase = n0 + wn * WTN + j * 32;
      const int col = cbase + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + (r >> 2) * 8 + (r & 3);
        const float v = acc[i][j][r];
        if (row >= M) continue;
        if (SPLIT) a.work[((size_t)bz * M + row) * a.N + col] = v;
        else if (EPI == EPI_STORE) reinterpret_cast<float*>(a.C)[(size_t)row * a.ldc + col] = v;
        else reinterpret_cast<float*>(a.C)[(size_t)row * a.ldc + col] += v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny products, M <= 128 rows (short prefills): latency-bound, so every
// wave keeps a whole chunk in flight and the loads are coalesced.  Block =
// one 32 x 32 output tile; its nw waves (<= 8) take the chunks of 128 K
// values round robin.  A chunk (32 activation rows and 32 weight rows, 256
// bytes each) is read with 16-byte loads of 16 lanes per row (8 cache lines
// per instruction), written to the wave's own LDS region (rows padded by 16
// bytes), then read back in the v_mfma_f32_32x32x16_bf16 operand layout for
// 8 MFMAs while the next chunk's loads fly.  The waves' tiles are added
// through LDS in wave order (deterministic) before the epilogue: no split-K
// workspace, no second kernel.  (Measured slower at these sizes: splitting K
// over more blocks with the last block of a tile adding the splits, whose
// store / arrival / reload chain costs more than the wider grid gains; and
// two chunks in flight per wave.)
constexpr int SK_KC = 128;             // K values per chunk
constexpr int SK_LD = SK_KC + 8;       // bf16 per LDS row
constexpr int SK_WAVE = 2 * 32 * SK_LD;  // bf16 per wave region (A rows, then B rows)

// SPLIT: block z of the grid's third dimension takes the z-th of gridDim.z
// equal K ranges and writes its partial tile to work[z] (EPI_ADD only; the
// fused reduce adds the splits, the residual and the next RMSNorm)
template <int EPI, bool SPLIT = false>
__global__ __launch_bounds__(512) void k_gemm_skinny(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];  // nw * SK_WAVE; also the wave tiles at the end
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int M = a.M;
  const int nch = a.K / SK_KC / gridDim.z;  // chunks of this block's K range
  const int kofs = blockIdx.z * nch * SK_KC;
  bf16_t* W = lds + wave * SK_WAVE;
  // staging: instruction i covers rows 4i .. 4i+3, lane l row 4i + l/16,
  // columns 8 (l % 16) .. +7 of the chunk
  const int sr = lane >> 4, sc = (lane & 15) * 8;  // sc: column inside the chunk (LDS and global)
  const bf16_t* Ag = a.A + kofs + sc;
  const bf16_t* Bg = a.B + (size_t)(n0 + sr) * a.K + kofs + sc;
  const size_t bstep = (size_t)4 * a.K;
  const int arow_max = M - 1 - m0;  // last valid row of the tile (rows past it: not stored)
  bf16x8_t ra[8], rb[8];  // vector types: the arrays stay in registers
  int ch = wave;
  if (ch < nch) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = min(4 * i + sr, arow_max);
      ra[i] = *reinterpret_cast<const bf16x8_t*>(Ag + (size_t)(m0 + r) * a.lda + ch * SK_KC);
      rb[i] = *reinterpret_cast<const bf16x8_t*>(Bg + i * bstep + ch * SK_KC);
    }
  }
  f32x16_t acc = f32x16_t{};
  for (; ch < nch; ch += nw) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<bf16x8_t*>(W + (4 * i + sr) * SK_LD + sc) = ra[i];
      *reinterpret_cast<bf16x8_t*>(W + (32 + 4 * i + sr) * SK_LD + sc) = rb[i];
    }
    const int nx = ch + nw;
    if (nx < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = min(4 * i + sr, arow_max);
        ra[i] = *reinterpret_cast<const bf16x8_t*>(Ag + (size_t)(m0 + r) * a.lda + nx * SK_KC);
        rb[i] = *reinterpret_cast<const bf16x8_t*>(Bg + i * bstep + nx * SK_KC);
      }
    }
    // operand layout: lane l, step s: row l % 32, K 8 (l / 32) + 16 s .. +7
    const bf16_t* ar = W + (lane & 31) * SK_LD + (lane >> 5) * 8;
    const bf16_t* br = W + (32 + (lane & 31)) * SK_LD + (lane >> 5) * 8;
#pragma unroll
    for (int s2 = 0; s2 < SK_KC / 16; ++s2) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(ar + s2 * 16);
      const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(br + s2 * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with its staging region
  float* part = reinterpret_cast<float*>(lds);  // [wave][lane * 16 + register]
#pragma unroll
  for (int q = 0; q < 16; q += 4)
    *reinterpret_cast<float4*>(&part[wave * 1024 + lane * 16 + q]) = make_float4(acc[q], acc[q + 1], acc[q + 2], acc[q + 3]);
  __syncthreads();
  // thread t < 1024 of the tile: lane t / 16, register t % 16; register q of
  // lane l is row (q/4)*8 + (l/32)*4 + q%4, column l%32 of the tile
  for (int t = threadIdx.x; t < 1024; t += blockDim.x) {
    const int l = t >> 4, q = t & 15;
    const int row = m0 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3), col = l & 31;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += part[w * 1024 + t];
    if (EPI == EPI_SWIGLU) {
      // columns 0..15 of the tile are gate rows, 16..31 the matching up rows:
      // lane l + 16 holds the up value of lane l's gate value
      if (col >= 16 || row >= M) continue;
      float u = 0.f;
      for (int w = 0; w < nw; ++w) u += part[w * 1024 + t + 16 * 16];
      reinterpret_cast<bf16_t*>(a.C)[(size_t)row * a.ldc + n0 / 2 + col] = (bf16_t)f32_to_bf16(silu_f(v) * u);
      continue;
    }
    if (row >= M) continue;
    if (SPLIT) {
      a.work[((size_t)blockIdx.z * M + row) * a.N + n0 + col] = v;
      continue;
    }
    float* c = reinterpret_cast<float*>(a.C) + (size_t)row * a.ldc + n0 + col;
    if (EPI == EPI_STORE) *c = v;
    else *c += v;
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs a, int ks) {
  const size_t MN = (size_t)a.M * a.N;
  const size_t n_out = (EPI == EPI_SWIGLU) ? MN / 2 : MN;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_out;
       idx += (size_t)gridDim.x * blockDim.x) {
    if (EPI == EPI_SWIGLU) {
      const int half = a.N / 2;
      const int row = (int)(idx / half), r = (int)(idx % half);
      const size_t p = (size_t)row * a.N + (size_t)(r >> 4) * 32 + (r & 15);
      float gsum = 0.f, usum = 0.f;
      for (int z = 0; z < ks; ++z) {
        gsum += a.work[z * MN + p];
        usum += a.work[z * MN + p + 16];
      }
      reinterpret_cast<bf16_t*>(a.C)[(size_t)row * a.ldc + r] =
          (bf16_t)f32_to_bf16(silu_f(gsum) * usum);
    } else {
      const int row = (int)(idx / a.N), col = (int)(idx % a.N);
      float s = 0.f;
      for (int z = 0; z < ks; ++z) s += a.work[z * MN + idx];
      float* c = reinterpret_cast<float*>(a.C) + (size_t)row * a.ldc + col;
      if (EPI == EPI_ADD) *c += s;
      else *c = s;
    }
  }
}

bool gemm_shape_ok(int M, int N, int K) {
  return M >= 1 && N % GB_N == 0 && K % GB_K == 0;
}
// (N % 128 == 0 also covers the 256 x 128 tiles of the large-M kernel)

// ---------------------------------------------------------------------------
// Split-K reduce fused with the residual add and the next pre-norm: row t of
// C (= the residual stream x) becomes x + sum_z work[z][t], and
// hn[t] = bf16(RMSNorm(x[t]) * g).  One block per row (N <= 1024).

constexpr int SPLITK_MAX = 8;  // splits the fused reduce takes

__global__ __launch_bounds__(256) void k_splitk_reduce_add_norm(GemmArgs a, int ks, const float* g,
                                                                float eps, bf16_t* hn, int ldh) {
  // N <= 1024: one float4 of the row per thread.  Every load (x, the splits,
  // the gains) is issued before the first store, and the sums stay in
  // registers for the norm pass: a load issued after a store waits for it
  // (loads and stores retire through one in-order counter).  The splits are
  // added in split order (deterministic).
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, k = tid * 4;
  const size_t MN = (size_t)a.M * a.N;
  float* xr = reinterpret_cast<float*>(a.C) + (size_t)t * a.ldc;
  const bool act = k < a.N;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f), gg = x;
  float q[SPLITK_MAX][4];
  if (act) {
    x = *reinterpret_cast<const float4*>(xr + k);
    gg = *reinterpret_cast<const float4*>(g + k);
#pragma unroll
    for (int z = 0; z < SPLITK_MAX; ++z) {
      if (z >= ks) break;
      const float4 p = *reinterpret_cast<const float4*>(a.work + z * MN + (size_t)t * a.N + k);
      q[z][0] = p.x;
      q[z][1] = p.y;
      q[z][2] = p.z;
      q[z][3] = p.w;
    }
#pragma unroll
    for (int z = 0; z < SPLITK_MAX; ++z) {
      if (z >= ks) break;
      x.x += q[z][0];
      x.y += q[z][1];
      x.z += q[z][2];
      x.w += q[z][3];
    }
    *reinterpret_cast<float4*>(xr + k) = x;
  }
  const float ss = block_sum<256>(x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w, red);
  const float inv = rsqrtf(ss / (float)a.N + eps);
  if (act) {
    uint2 o;
    o.x = f32_to_bf16(x.x * inv * gg.x) | (f32_to_bf16(x.y * inv * gg.y) << 16);
    o.y = f32_to_bf16(x.z * inv * gg.z) | (f32_to_bf16(x.w * inv * gg.w) << 16);
    *reinterpret_cast<uint2*>(hn + (size_t)t * ldh + k) = o;
  }
}

bool skinny_shape_ok(int N, int K) { return N % 32 == 0 && K % SK_KC == 0; }

static bool skinny_ok(const GemmArgs& a) {
  return a.M >= 1 && a.M <= 128 && skinny_shape_ok(a.N, a.K);
}

// waves per block: the largest divisor of the chunk count up to 8 (every
// wave takes the same number of chunks)
template <int EPI>
static void launch_skinny(GemmArgs a, hipStream_t st) {
  const int nch = a.K / SK_KC;
  int nw = 8;
  while (nch % nw) --nw;
  hipLaunchKernelGGL((k_gemm_skinny<EPI>), dim3(a.N / 32, (a.M + 31) / 32), dim3(64 * nw),
                     nw * SK_WAVE * sizeof(bf16_t), st, a);
}

template <int BM, int EPI>
static void launch_bm(GemmArgs a, int ks, hipStream_t st) {
  const dim3 grid(a.N / GB_N, (a.M + BM - 1) / BM, ks);
  const int kps = a.K / ks;
  if (ks == 1) {
    hipLaunchKernelGGL((k_gemm_bf16<BM, EPI, false>), grid, dim3(256), 0, st, a, kps);
  } else {
    hipLaunchKernelGGL((k_gemm_bf16<BM, EPI, true>), grid, dim3(256), 0, st, a, kps);
    const size_t n_out = (size_t)a.M * a.N / (EPI == EPI_SWIGLU ? 2 : 1);
    const unsigned blocks = (unsigned)((n_out + 255) / 256 < 4096 ? (n_out + 255) / 256 : 4096);
    hipLaunchKernelGGL((k_splitk_reduce<EPI>), dim3(blocks), dim3(256), 0, st, a, ks);
  }
}

template <int BN, int EPI>
static void launch_dma(GemmArgs a, int ks, hipStream_t st) {
  const dim3 grid(a.N / BN, (a.M + 255) / 256, ks);
  const int kps = a.K / ks;
  if (ks == 1) {
    hipLaunchKernelGGL((k_gemm_dma<BN, EPI, false>), grid, dim3(512), 0, st, a, kps);
  } else if constexpr (BN == 128) {  // the 192-wide tile is never split
    hipLaunchKernelGGL((k_gemm_dma<BN, EPI, true>), grid, dim3(512), 0, st, a, kps);
    const size_t n_out = (size_t)a.M * a.N / (EPI == EPI_SWIGLU ? 2 : 1);
    const unsigned blocks = (unsigned)((n_out + 255) / 256 < 4096 ? (n_out + 255) / 256 : 4096);
    hipLaunchKernelGGL((k_splitk_reduce<EPI>), dim3(blocks), dim3(256), 0, st, a, ks);
  }
}

static void launch_dma_epi(Epilogue epi, GemmArgs a, int ks, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: launch_dma<128, EPI_STORE>(a, ks, st); break;
    case EPI_ADD: launch_dma<128, EPI_ADD>(a, ks, st); break;
    case EPI_SWIGLU: launch_dma<128, EPI_SWIGLU>(a, ks, st); break;
  }
}

static int dma_splits(const GemmArgs& a) {
  const int nkt = a.K / GB_K;
  const int tiles = ((a.M + 255) / 256) * (a.N / 128);
  int ks = 1;
  while (tiles * ks * 2 <= 256 && nkt % (ks * 2) == 0 && nkt / (ks * 2) >= 4 &&
         (size_t)(ks * 2) * a.M * a.N <= a.work_elems)
    ks *= 2;
  return ks;
}

void launch_gemm_add_norm(GemmArgs a, const float* g, float eps, bf16_t* hn, int ldh,
                          hipStream_t st) {
  if (skinny_ok(a) && a.N % 4 == 0 && a.N <= 1024) {
    // few rows: a narrow output (o_proj, down: N / 32 = 32 tiles) would
    // leave most CUs idle, so K is split over up to 8 blocks per tile and
    // the splits meet in the fused reduce, which also adds the residual and
    // forms the next RMSNorm's bf16 rows
    const int nch = a.K / SK_KC, tiles = (a.N / 32) * ((a.M + 31) / 32);
    int ks = 1;
    while (ks * 2 <= SPLITK_MAX && tiles * ks * 2 <= 256 && nch % (ks * 2) == 0 && nch / (ks * 2) >= 2 &&
           (size_t)(ks * 2) * a.M * a.N <= a.work_elems)
      ks *= 2;
    if (ks > 1) {
      int nw = 8;
      while ((nch / ks) % nw) --nw;
      hipLaunchKernelGGL((k_gemm_skinny<EPI_ADD, true>), dim3(a.N / 32, (a.M + 31) / 32, ks), dim3(64 * nw),
                         nw * SK_WAVE * sizeof(bf16_t), st, a);
      hipLaunchKernelGGL(k_splitk_reduce_add_norm, dim3(a.M), dim3(256), 0, st, a, ks, g, eps, hn, ldh);
      return;
    }
  }
  if (a.M >= 512 && a.N % 4 == 0 && a.N <= 1024) {
    const int ks = dma_splits(a);
    if (ks > 1 && ks <= SPLITK_MAX) {
      const dim3 grid(a.N / 128, (a.M + 255) / 256, ks);
      hipLaunchKernelGGL((k_gemm_dma<128, EPI_ADD, true>), grid, dim3(512), 0, st, a, a.K / ks);
      hipLaunchKernelGGL(k_splitk_reduce_add_norm, dim3(a.M), dim3(256), 0, st, a, ks, g, eps, hn,
                         ldh);
      return;
    }
  }
  launch_gemm(EPI_ADD, a, st);
  launch_rmsnorm_bf16(reinterpret_cast<const float*>(a.C), a.ldc, a.M, a.N, g, eps, hn, ldh, st);
}

bool gemm_writes_kv(const GemmArgs& a) {
  // the path launch_gemm takes for EPI_STORE at M >= 512: 128-column DMA
  // tiles, split over K only when the grid is short of 256 blocks
  // (stacked sequences: whole sequences, at most MAX_ROWS of them, and few
  // enough rows for the float32 sequence index to be exact)
  const bool rows_ok = a.kv_per == 0 || (a.M % a.kv_per == 0 && a.M / a.kv_per <= MAX_ROWS && a.M < (1 << 22));
  return a.kcache != nullptr && a.vcache != nullptr && a.M >= 512 && a.N % 128 == 0 && a.kcol % 128 == 0 &&
         a.vcol % 128 == 0 && a.kcol < a.vcol && a.vcol < a.N && rows_ok && dma_splits(a) == 1;
}

void launch_gemm(Epilogue epi, GemmArgs a, hipStream_t st) {
  const int nkt = a.K / GB_K;
  if (skinny_ok(a)) {
    switch (epi) {
      case EPI_STORE: launch_skinny<EPI_STORE>(a, st); break;
      case EPI_ADD: launch_skinny<EPI_ADD>(a, st); break;
      case EPI_SWIGLU: launch_skinny<EPI_SWIGLU>(a, st); break;
    }
    return;
  }
  // the 256-row tiles' SwiGLU epilogue writes 16-byte chunks of output rows
  const bool vec_out = epi != EPI_SWIGLU || (a.ldc % 8 == 0 && ((uintptr_t)a.C & 15) == 0);
  if (a.M >= 512 && vec_out) {
    // 256-row tiles.  The gate|up projection takes 192-column blocks when
    // that gives the grid whole rounds of 256 CUs (6144 wide at M = 2048);
    // otherwise 128 columns, splitting K while the doubled grid still fits
    // one round of 256 blocks (the split-K reduce costs a full pass over C,
    // so a full grid is never split).
    const int mt = (a.M + 255) / 256;
    if (epi == EPI_SWIGLU && a.N % 192 == 0 && (mt * (a.N / 192)) % 256 == 0) {
      launch_dma<192, EPI_SWIGLU>(a, 1, st);
      return;
    }
    launch_dma_epi(epi, a, dma_splits(a), st);
    return;
  }
  const int BM = a.M > 64 ? 128 : 64;
  const int tiles = (a.N / GB_N) * ((a.M + BM - 1) / BM);
  int ks = 1;
  // split K while the grid is short of the 256 CUs and each split keeps >= 4
  // K tiles; ks divides the K tile count
  while (tiles * ks < 256 && nkt % (ks * 2) == 0 && nkt / (ks * 2) >= 4 &&
         (size_t)(ks * 2) * a.M * a.N <= a.work_elems)
    ks *= 2;
  if (BM == 128) {
    switch (epi) {
      case EPI_STORE: launch_bm<128, EPI_STORE>(a, ks, st); break;
      case EPI_ADD: launch_bm<128, EPI_ADD>(a, ks, st); break;
      case EPI_SWIGLU: launch_bm<128, EPI_SWIGLU>(a, ks, st); break;
    }
  } else {
    switch (epi) {
      case EPI_STORE: launch_bm<64, EPI_STORE>(a, ks, st); break;
      case EPI_ADD: launch_bm<64, EPI_ADD>(a, ks, st); break;
      case EPI_SWIGLU: launch_bm<64, EPI_SWIGLU>(a, ks, st); break;
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm to bf16 rows (the A operand of the next projection)

__global__ __launch_bounds__(256) void k_rmsnorm_bf16(const float* x, int ldx, int K,
                                                      const float* g, float eps, bf16_t* out,
                                                      int ldo, float* out32, int ld32) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)t * ldx;
  float ss = 0.f;
  for (int k = tid * 4; k < K; k += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + k);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum<256>(ss, red);
  const float inv = rsqrtf(ss / (float)K + eps);
  for (int k = tid * 4; k < K; k += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + k);
    const float4 gg = *reinterpret_cast<const float4*>(g + k);
    const float4 y = make_float4(v.x * inv * gg.x, v.y * inv * gg.y, v.z * inv * gg.z, v.w * inv * gg.w);
    uint2 o;
    o.x = f32_to_bf16(y.x) | (f32_to_bf16(y.y) << 16);
    o.y = f32_to_bf16(y.z) | (f32_to_bf16(y.w) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)t * ldo + k) = o;
    if (out32) *reinterpret_cast<float4*>(out32 + (size_t)t * ld32 + k) = y;
  }
}

void launch_rmsnorm_bf16(const float* x, int ldx, int T, int K, const float* g, float eps,
                         bf16_t* out, int ldo, hipStream_t st, float* out32, int ld32) {
  hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(T), dim3(256), 0, st, x, ldx, K, g, eps, out, ldo, out32, ld32);
}

}  // namespace qtalk
