// bf16 MFMA GEMM for gfx950: C[M,N] = A[M,K] . B[N,K]^T with fp32 accumulate.
//
// Every projection of the MLA forward is an nn.Linear product y = x W^T with
// W stored [out, in] (the module layout shown on the "Kimi K2 · Key-value
// compression" page).  Both operands are therefore K-contiguous, which is
// exactly the per-lane operand shape of v_mfma_f32_32x32x16_bf16 (each lane
// holds 8 consecutive K values of one row), so tiles go global -> registers
// -> LDS (XOR-swizzled 16-byte chunks, conflict-free ds_read_b128) -> MFMA
// with no transposition anywhere.
//
// Tile: BM x BN x 64, WM x WN waves, each wave (BM/WM) x (BN/WN) built from
// 32x32 MFMA blocks.  Two LDS stages and two MFMA-fragment register sets form
// a software pipeline (see the main loop).  Split-K writes fp32 partials
// whose consumer sums them in a fixed order (deterministic).
//
// Epilogues (bf16 outputs are staged through LDS and written with 16-byte
// coalesced stores):
//   EPI_F32    fp32 store (split-K partial or fp32 result)
//   EPI_BF16   bf16 store
//   EPI_RESID  bf16 store of R + acc (residual add of the dense block)
//   EPI_SWIGLU dual-B product: 32-column blocks alternate W1 / W3 rows, so a
//              lane holds g and u of the same output column and writes
//              silu(g) * u (the SwiGLU steps of the dense block)
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

#define MLA_SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
// Direct-to-LDS pipeline shape: k per stage and ring depth.  Measured on the
// prefill shapes: 64-k stages (whole 128-byte lines per tile row) in a
// 2-deep ring beat 32-k stages in a 3- or 4-deep ring (o_proj 187 vs 205 us):
// half-line requests cost more than the shorter prefetch distance, and a
// deeper ring would cost the 128x128 tile its second workgroup per CU.
#ifndef GEMM_DMA_SK
#define GEMM_DMA_SK(bm) 64
#endif
#ifndef GEMM_DMA_NSTG
#define GEMM_DMA_NSTG(bm) 2
#endif
enum { SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200 };

// LDS swizzle of the 16-byte chunk of a 128-byte tile row.  gfx950 serves a
// ds_read_b128 16 lanes at a time from 64 banks (256 bytes), so the 16 rows a
// half-wave reads must land on 16 distinct 16-byte bank groups: even and odd
// rows share a 256-byte line, and (row >> 1) spreads eight line pairs.
MLA_DEV int gemm_swz(int r) { return (r >> 1) & 7; }

// Wave-wide direct-to-LDS load of 16 bytes per lane (global rsrc.base + voff
// -> LDS byte m0 + 16 lane); issued from asm so the compiler's wait counting
// (which cannot tell ring stages apart) stays out: the kernel waits with
// explicit vmcnt values.
MLA_DEV void gemm_dma16(unsigned m0, int voff, u32x4 rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
MLA_DEV u32x4 gemm_rsrc(const void* base) {
  const unsigned long a = (unsigned long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = 0x7fffffffu;  // rows are clamped in range; offsets stay below 2^31
  r[3] = 0x00020000u;
  return r;
}

// One launch may carry two independent products (same tile shape and
// epilogue, no batch or K split): workgroups [0, tiles0) of the logical order
// compute product 0, the rest product 1.
struct GemmGroup {
  GemmParams p[2];
  int n;               // 1 or 2 products
  int tiles0, tiles1;  // tiles of each product
};

// Logical (product, tile) of workgroup b.  The dispatcher hands workgroup b
// to XCD b % 8, in order; each XCD gets a contiguous range of each product's
// tiles, product 0's first, so every XCD runs the same mix and the longer
// product (placed first by the caller) starts first.
MLA_DEV void gemm_tile_of(const GemmGroup& g, int b, int& prob, int& lt) {
  if (g.n == 1) {
    prob = 0;
    lt = xcd_remap(b, g.tiles0);
    return;
  }
  const int total = g.tiles0 + g.tiles1;
  const int x = b % 8, slot = b / 8;
  const int before = x * (total / 8) + min(x, total % 8);  // workgroups on XCDs < x
  const int s0 = x * (g.tiles0 / 8) + min(x, g.tiles0 % 8);
  const int n0 = g.tiles0 / 8 + (x < g.tiles0 % 8 ? 1 : 0);
  if (slot < n0) {
    prob = 0;
    lt = s0 + slot;
  } else {
    prob = 1;
    lt = (before - s0) + (slot - n0);
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool DMA>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(GemmGroup gg) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int ROWS_PER_PASS = NT / 8;               // 8 threads x 16 B cover one 64-wide K row
  constexpr int A_CH = BM / ROWS_PER_PASS;
  constexpr int B_CH = BN / ROWS_PER_PASS;
  constexpr int NLD = A_CH + B_CH;                    // 16-byte loads per thread per K tile
  constexpr int NMF = FM * FN;                        // MFMAs per wave per 16-wide K step
  constexpr int NRD = FM + FN;                        // fragment reads per K step
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for the block");
  static_assert(EPI != EPI_SWIGLU || (WTN % 64) == 0, "SwiGLU pairs 32-column blocks inside a wave");
  // Accumulator orientation: every epilogue takes D = B.A^T per 32x32 block,
  // so that a lane holds one output row and four consecutive output columns
  // (8 g + 4 (lane >> 5) + 0..3).  The staged bf16 epilogues write them to LDS
  // as one 8-byte chunk; the fp32 partial epilogue stores them straight to
  // memory as 16-byte vectors (four times fewer stores than one column per
  // lane: the joint down-projection 73.2 -> 70.4 us).

  // LDS: the two-stage register-staged layout, or the direct-to-LDS ring
  constexpr int LDS_U4_REG = 2 * (BM + BN) * 8;
  constexpr int LDS_U4_DMA = DMA ? GEMM_DMA_NSTG(BM) * (BM + BN) * GEMM_DMA_SK(BM) * 2 / 16 : 0;
  constexpr int LDS_U4 = LDS_U4_REG > LDS_U4_DMA ? LDS_U4_REG : LDS_U4_DMA;
  __shared__ u32x4 lds_raw[LDS_U4];
  u32x4 (*lds)[(BM + BN) * 8] = reinterpret_cast<u32x4 (*)[(BM + BN) * 8]>(lds_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // ---- product and tile coordinates (XCD-aware, grouped along M) ----
  int prob, lin;
  gemm_tile_of(gg, blockIdx.x, prob, lin);
  const GemmParams& p = gg.p[prob];
  const int GM = p.group_m;
  const int group = lin / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gm = min(p.tiles_m - first_m, GM);
  const int within = lin - group * GM * p.tiles_n;
  const int tm = first_m + within % gm;
  const int tn = within / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int bidx = blockIdx.y / p.ksplit;
  const int split = blockIdx.y % p.ksplit;
  const bf16_t* __restrict__ A = p.A + (long)bidx * p.sA;
  const bf16_t* __restrict__ B = p.B + (long)bidx * p.sB;
  const bf16_t* __restrict__ B2 = p.B2;
  const int k_begin = split * p.kchunk;
  const int k_end = min(p.K, k_begin + p.kchunk);
  const int nk = (k_end - k_begin) / 64;

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int lr = lane & 31, lg = lane >> 5;

  if constexpr (DMA) {
    // Direct-to-LDS pipeline.  K advances in stages of SK (tile rows of SK*2
    // bytes, CH chunks of 16 B; chunk c of row r at position c ^ swz(r), with
    // swz spreading the rows that share a 256-byte bank window).  An NSTG
    // ring: the loads of stage t + NSTG are issued in iteration t, after the
    // barrier that frees stage t's buffer.  Within a stage, k-step s + 1's
    // fragments are read under k-step s's MFMAs; the barrier sits before the
    // last k-step, whose MFMAs cover the next stage's first fragment reads.
    constexpr int SK = GEMM_DMA_SK(BM);
    constexpr int NSTG = GEMM_DMA_NSTG(BM);
    constexpr int KSTEPS = SK / 16, CH = SK / 8, ROWB = SK * 2;
    constexpr int RPW = 256 / ROWB;  // rows per 256-byte bank window
    constexpr int NW = WM * WN;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE_B = A_BYTES + B_BYTES;
    constexpr int A_DMA = A_BYTES / 1024 / NW, B_DMA = B_BYTES / 1024 / NW;  // per wave per stage
    constexpr int DPW = A_DMA + B_DMA;
    constexpr int RPD = 1024 / ROWB;  // rows per DMA
    static_assert(KSTEPS % 2 == 0, "k-steps per stage");
    static_assert(A_DMA >= 1 && B_DMA >= 1 && A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0,
                  "DMA split");
    static_assert(NSTG * STAGE_B <= LDS_U4 * 16, "ring does not fit the LDS");
    auto swz = [](int r) { return (r / RPW) & (CH - 1); };
    const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)&lds[0][0];
    const int wv = __builtin_amdgcn_readfirstlane(wid);
    // DMA d of this wave fills tile rows RPD g .. RPD g + RPD - 1 (g = wv *
    // X_DMA + d): lane l -> row RPD g + l / CH, chunk position l % CH
    int a_vo[A_DMA], b_vo[B_DMA];
    unsigned b_src2 = 0;  // bit d: DMA d reads from B2
#pragma unroll
    for (int d = 0; d < A_DMA; ++d) {
      const int r = RPD * (wv * A_DMA + d) + lane / CH;
      const int c = (lane % CH) ^ swz(r);
      a_vo[d] = (min(m0 + r, p.M - 1) * (int)p.lda + k_begin + 8 * c) * 2;
    }
#pragma unroll
    for (int d = 0; d < B_DMA; ++d) {
      const int r = RPD * (wv * B_DMA + d) + lane / CH;
      const int c = (lane % CH) ^ swz(r);
      int src;
      if (EPI == EPI_SWIGLU) {
        const int rb = r >> 5;
        src = min(n0 / 2 + (rb >> 1) * 32 + (r & 31), p.N / 2 - 1);
        if (rb & 1) b_src2 |= 1u << d;
      } else {
        src = min(n0 + r, p.N - 1);
        if (p.b_split > 0 && n0 + RPD * (wv * B_DMA + d) >= p.b_split) {
          src -= p.b_split;
          b_src2 |= 1u << d;
        }
      }
      b_vo[d] = (src * (int)p.ldb + k_begin + 8 * c) * 2;
    }
    const u32x4 ra = gemm_rsrc(A), rb1 = gemm_rsrc(B), rb2 = gemm_rsrc(B2 ? B2 : B);
    const int nst = (k_end - k_begin) / SK;
#define GD_ISSUE(u_)                                                                         \
  do {                                                                                       \
    const unsigned sb_ = lds_base + ((u_) % NSTG) * STAGE_B;                                 \
    const int ko_ = ROWB * (u_);                                                             \
    _Pragma("unroll") for (int d = 0; d < A_DMA; ++d)                                        \
      gemm_dma16(sb_ + 1024 * (wv * A_DMA + d), a_vo[d] + ko_, ra);                          \
    _Pragma("unroll") for (int d = 0; d < B_DMA; ++d)                                        \
      gemm_dma16(sb_ + A_BYTES + 1024 * (wv * B_DMA + d), b_vo[d] + ko_,                     \
                 ((b_src2 >> d) & 1) ? rb2 : rb1);                                           \
  } while (0)
#define GD_WAIT(n_after)                                                                     \
  do {                                                                                       \
    if ((n_after) >= 2 && NSTG >= 4) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * DPW) : "memory"); \
    else if ((n_after) >= 1 && NSTG >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(DPW) : "memory"); \
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                    \
  } while (0)
    // fragment rows are lr (mod 32), so swz(row) = swz(lr) for every fragment
    const int sw = swz(lr);
    const int a_rd = (wm * WTM + lr) * ROWB, b_rd = A_BYTES + (wn * WTN + lr) * ROWB;
    const char* ldsc = (const char*)&lds[0][0];
#define GD_FREAD(u_, s_, slot)                                                               \
  do {                                                                                       \
    const char* sb_ = ldsc + ((u_) % NSTG) * STAGE_B;                                        \
    const int co_ = 16 * ((2 * (s_) + lg) ^ sw);                                             \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                           \
      fa[slot][i] = *(const bf16x8*)(sb_ + a_rd + i * 32 * ROWB + co_);                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
      fb[slot][j] = *(const bf16x8*)(sb_ + b_rd + j * 32 * ROWB + co_);                      \
  } while (0)
#define GD_MFMAS(slot)                                                                       \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    const int i = q / FN, j = q % FN;                                                        \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);  \
  }
#define GD_SCHED()                                                                           \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    MLA_SGB(SG_MFMA, 1);                                                                     \
    if (q < NRD) MLA_SGB(SG_DS_RD, 1);                                                       \
  }
    bf16x8 fa[2][FM], fb[2][FN];
    for (int u = 0; u < NSTG - 1 && u < nst; ++u) GD_ISSUE(u);
    if (nst > 0) {
      GD_WAIT(min(NSTG - 2, nst - 1));
      __syncthreads();
      if (nst > NSTG - 1) GD_ISSUE(NSTG - 1);
      GD_FREAD(0, 0, 0);
    }
    for (int t = 0; t < nst; ++t) {
#pragma unroll
      for (int s = 0; s + 1 < KSTEPS; ++s) {
        GD_FREAD(t, s + 1, (s + 1) & 1);
        GD_MFMAS(s & 1)
        GD_SCHED()
      }
      // Straight-line on purpose (the last iteration re-reads its own
      // stage): a branch around these reads would make the compiler wait
      // for them before the MFMAs below, at the join.
      GD_WAIT(min(NSTG - 2, nst - 2 - t));
      __syncthreads();
      if (t + NSTG < nst) GD_ISSUE(t + NSTG);  // into stage t's buffer, free now
      GD_FREAD(min(t + 1, nst - 1), 0, 0);
      GD_MFMAS(1)
      GD_SCHED()
    }
#undef GD_ISSUE
#undef GD_WAIT
#undef GD_FREAD
#undef GD_MFMAS
#undef GD_SCHED
  } else {
  // ---- per-thread global source rows as 32-bit element offsets (rows past
    //      the edge are clamped: loaded from a valid row and never stored) ----
    const int ch = tid & 7;
    int a_off[A_CH], b_off[B_CH];
  #pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int r = tid / 8 + i * ROWS_PER_PASS;
      int gr = min(m0 + r, p.M - 1);
      a_off[i] = gr * (int)p.lda + ch * 8 + k_begin;
    }
    unsigned b2mask = 0;  // bit i: chunk row i comes from B2
  #pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int r = tid / 8 + i * ROWS_PER_PASS;
      int src;
      if (EPI == EPI_SWIGLU) {
        int rb = r >> 5;
        src = min(n0 / 2 + (rb >> 1) * 32 + (r & 31), p.N / 2 - 1);
        if (rb & 1) b2mask |= 1u << i;
      } else {
        src = min(n0 + r, p.N - 1);
        if (p.b_split > 0 && src >= p.b_split) {
          src -= p.b_split;
          b2mask |= 1u << i;
        }
      }
      b_off[i] = src * (int)p.ldb + ch * 8 + k_begin;
    }
    // LDS slots this thread stores into (u32x4 units)
    int st_idx[NLD];
  #pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = tid / 8 + i * ROWS_PER_PASS;
      st_idx[i] = r * 8 + (ch ^ gemm_swz(r));
    }
  #pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = tid / 8 + i * ROWS_PER_PASS;
      st_idx[A_CH + i] = (BM + r) * 8 + (ch ^ gemm_swz(r));
    }
  
    // Software pipeline: the K tile in LDS buffer `cur` is multiplied in four
    // 16-wide steps while (step 0) the next tile's global loads are issued,
    // (steps 0-2) the next step's MFMA fragments are read from LDS into the
    // other fragment register set, and (step 3) the next tile is stored to the
    // other LDS buffer, one barrier is passed and its first fragments are read.
    // sched_group_barrier interleaves those memory instructions with the MFMAs
    // so the matrix pipe is never left waiting on a load issued just before.
    u32x4 stg[NLD];
    bf16x8 fa[2][FM], fb[2][FN];
  
  #define GEMM_GLOAD(kt_)                                                                   \
    do {                                                                                    \
      const int ko_ = (kt_) * 64;                                                           \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                      \
          stg[i] = *(const u32x4*)(A + a_off[i] + ko_);                                      \
      _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                    \
        const bf16_t* src_ = ((b2mask >> i) & 1) ? B2 : B;                                   \
        stg[A_CH + i] = *(const u32x4*)(src_ + b_off[i] + ko_);                              \
      }                                                                                     \
    } while (0)
  #define GEMM_SSTORE(buf)                                                                  \
    do {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < NLD; ++i) lds[buf][st_idx[i]] = stg[i];         \
    } while (0)
  #define GEMM_FREAD(buf, s, slot)                                                          \
    do {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                      \
        const int r = wm * WTM + i * 32 + lr;                                               \
        fa[slot][i] = __builtin_bit_cast(bf16x8, lds[buf][r * 8 + ((2 * (s) + lg) ^ gemm_swz(r))]); \
      }                                                                                     \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                      \
        const int r = wn * WTN + j * 32 + lr;                                               \
        fb[slot][j] = __builtin_bit_cast(bf16x8, lds[buf][(BM + r) * 8 + ((2 * (s) + lg) ^ gemm_swz(r))]); \
      }                                                                                     \
    } while (0)
  #define GEMM_MFMAS(slot, lo, hi)                                                          \
    do {                                                                                    \
      _Pragma("unroll") for (int q = (lo); q < (hi); ++q) {                                 \
        const int i = q / FN, j = q % FN;                                                   \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);  \
      }                                                                                     \
    } while (0)
  
    if (nk > 0) {
      GEMM_GLOAD(0);
      GEMM_SSTORE(0);
    }
    __syncthreads();
    if (nk > 0) GEMM_FREAD(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1, nxt = cur ^ 1;
      const int kn = min(kt + 1, nk - 1);  // the last iteration reloads a valid tile
      // step 0
      GEMM_GLOAD(kn);
      GEMM_FREAD(cur, 1, 1);
      GEMM_MFMAS(0, 0, NMF);
  #pragma unroll
      for (int q = 0; q < NMF; ++q) {
        MLA_SGB(SG_MFMA, 1);
        if (q < NLD) MLA_SGB(SG_VMEM_RD, (NLD + NMF - 1) / NMF);
        if (q < NRD) MLA_SGB(SG_DS_RD, (NRD + NMF - 1) / NMF);
      }
      // step 1
      GEMM_FREAD(cur, 2, 0);
      GEMM_MFMAS(1, 0, NMF);
  #pragma unroll
      for (int q = 0; q < NMF; ++q) {
        MLA_SGB(SG_MFMA, 1);
        MLA_SGB(SG_DS_RD, (NRD + NMF - 1) / NMF);
      }
      // step 2
      GEMM_FREAD(cur, 3, 1);
      GEMM_MFMAS(0, 0, NMF);
  #pragma unroll
      for (int q = 0; q < NMF; ++q) {
        MLA_SGB(SG_MFMA, 1);
        MLA_SGB(SG_DS_RD, (NRD + NMF - 1) / NMF);
      }
      // step 3: store the next tile under half the MFMAs, barrier, read its
      // first fragments under the other half
      GEMM_SSTORE(nxt);
      GEMM_MFMAS(1, 0, NMF / 2);
  #pragma unroll
      for (int q = 0; q < NMF / 2; ++q) {
        MLA_SGB(SG_MFMA, 1);
        MLA_SGB(SG_DS_WR, (2 * NLD + NMF - 1) / NMF);
      }
      __syncthreads();
      GEMM_FREAD(nxt, 0, 0);
      GEMM_MFMAS(1, NMF / 2, NMF);
  #pragma unroll
      for (int q = 0; q < NMF / 2; ++q) {
        MLA_SGB(SG_MFMA, 1);
        MLA_SGB(SG_DS_RD, (2 * NRD + NMF - 1) / NMF);
      }
    }
  
  #undef GEMM_FREAD
  #undef GEMM_MFMAS
  #undef GEMM_GLOAD
  #undef GEMM_SSTORE
  }

  // ---- epilogue.  A lane holds column (lane & 31) of each 32x32 block and
  //      rows 8*i + 4*(lane >> 5) + j in acc[...][4*i + j]. ----
  const int lr_ = lane & 31;
  if (EPI == EPI_F32) {
    // B.A^T orientation: a lane holds row m0 + wm WTM + 32 i + lr of C and the
    // four consecutive columns 32 j + 8 g + 4 lg + 0..3 of its wave's block
    float* C = (float*)p.C + (long)bidx * p.sC + (long)split * p.split_stride;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = m0 + wm * WTM + i * 32 + lr_;
      if (row >= p.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * WTN + j * 32 + 8 * g + 4 * lg;
          const floatx4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          float* dst = C + (long)row * p.ldc + col;
          if (col + 4 <= p.N && (p.ldc & 3) == 0) {
            *(floatx4*)dst = v;
          } else {
            for (int q = 0; q < 4; ++q)
              if (col + q < p.N) dst[q] = v[q];
          }
        }
    }
    return;
  }
  constexpr int OUTN = (EPI == EPI_SWIGLU) ? BN / 2 : BN;   // output columns of the tile
  static_assert(OUTN % 64 == 0, "output tile width");
  const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  const int on0 = (EPI == EPI_SWIGLU) ? n0 / 2 : n0;
  bf16_t* C = (bf16_t*)p.C + (long)bidx * p.sC;
  // kernel arguments the store loops need, read once
  const int rows_M = p.M;
  const long ldc = p.ldc, ldr = p.ldr;
  const bf16_t* __restrict__ Rres = p.R;
  const bf16_t* __restrict__ bias = (EPI != EPI_SWIGLU) ? p.bias : nullptr;
  constexpr int CH8 = OUTN / 8;  // 8-output (16-byte bf16) chunks per output row
  // output column (in the tile) of acc[i][j][4 g + q], q = 0..3
  auto tcol = [&](int j, int g) {
    if (EPI == EPI_SWIGLU) return ((wn * WTN) / 32 + j) / 2 * 32 + 8 * g + 4 * lg;
    return wn * WTN + j * 32 + 8 * g + 4 * lg;
  };
  if constexpr (EPI != EPI_RESID) {
    // bf16 outputs (plain, bias, SwiGLU): the rounded tile is staged whole
    // in the (now free) LDS, 16-byte chunk s of row r at s ^ (r % NSL), then
    // every thread writes 8 consecutive outputs with one 16-byte store.
    constexpr int ROWB = OUTN * 2;
    constexpr int NSL = CH8 < 16 ? CH8 : 16;
    static_assert(BM * ROWB <= (int)sizeof(lds_raw), "epilogue staging does not fit the LDS");
    char* cst = (char*)&lds[0][0];
    // bias of this lane's output columns (the same for all its rows), loaded
    // once; columns past the output read as zero
    float bcol[EPI == EPI_SWIGLU ? 1 : FN][4][4];
    if (EPI != EPI_SWIGLU && bias) {
#pragma unroll
      for (int j = 0; j < (EPI == EPI_SWIGLU ? 1 : FN); ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cc = on0 + tcol(j, g) + q;
            bcol[j][g][q] = cc < out_cols ? bf2f(bias[cc]) : 0.f;
          }
    }
    __syncthreads();  // last K tile read
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + lr_;
#pragma unroll
      for (int j = 0; j < FN; j += (EPI == EPI_SWIGLU ? 2 : 1))
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = tcol(j, g);
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (EPI == EPI_SWIGLU) {
              const float gg = acc[i][j][4 * g + q], uu = acc[i][j + 1][4 * g + q];
              v[q] = gg / (1.f + __expf(-gg)) * uu;
            } else {
              v[q] = acc[i][j][4 * g + q];
            }
          }
          if (EPI != EPI_SWIGLU && bias) {
            // o_proj of the attention_bias variant: y = x W^T + b
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] += bcol[EPI == EPI_SWIGLU ? 0 : j][g][q];
          }
          *(u32x2*)(cst + r * ROWB + 16 * ((c >> 3) ^ (r % NSL)) + 8 * ((c >> 2) & 1)) =
              u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
        }
    }
    __syncthreads();
    constexpr int NIT = BM * CH8 / NT;
    static_assert((BM * CH8) % NT == 0, "epilogue store loop");
    u32x4 sv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * NT, rl = idx / CH8, c8 = idx % CH8;
      sv[it] = *(const u32x4*)(cst + rl * ROWB + 16 * (c8 ^ (rl % NSL)));
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * NT, rl = idx / CH8, c8 = idx % CH8;
      const int row = m0 + rl, col = on0 + 8 * c8;
      if (row >= rows_M || col >= out_cols) continue;
      if (col + 8 <= out_cols) {
        *(u32x4*)(C + (long)row * ldc + col) = sv[it];
      } else {
        for (int q = 0; q < out_cols - col; ++q)
          C[(long)row * ldc + col + q] = (bf16_t)((q & 1) ? (sv[it][q >> 1] >> 16) : (sv[it][q >> 1] & 0xffffu));
      }
    }
  } else {
    // residual add: the fp32 tile is staged in passes of RP rows, 16-byte
    // chunk s of row r at s ^ 2 (r % 8) (pairs of chunks stay together), and
    // the store loop adds R in fp32 before the one rounding.
    constexpr int LDS_F = (int)sizeof(lds_raw) / 4;           // floats available
    constexpr int RP0 = LDS_F / OUTN;
    constexpr int RP = RP0 >= BM ? BM : (RP0 >= WTM ? (RP0 / WTM) * WTM : WTM);
    static_assert(RP * OUTN <= LDS_F, "epilogue staging does not fit the LDS");
    float* cst = (float*)&lds[0][0];
    auto cidx = [](int r, int c) { return r * OUTN + ((c >> 2) ^ (2 * (r & 7))) * 4 + (c & 3); };
    constexpr int NIT = RP * CH8 / NT;
    static_assert((RP * CH8) % NT == 0, "epilogue store loop");
#pragma unroll
    for (int pass = 0; pass < BM / RP; ++pass) {
      __syncthreads();  // LDS free: last K tile read (pass 0) or previous pass stored
      const int rlo = pass * RP;
      if (wm * WTM + WTM > rlo && wm * WTM < rlo + RP) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int rl = wm * WTM + i * 32 + lr_ - rlo;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *(floatx4*)&cst[cidx(rl, tcol(j, g))] =
                  floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
      }
      __syncthreads();
      floatx4 sv[NIT][2];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * NT, rl = idx / CH8, c8 = idx % CH8;
        sv[it][0] = *(const floatx4*)&cst[cidx(rl, 8 * c8)];
        sv[it][1] = *(const floatx4*)&cst[cidx(rl, 8 * c8 + 4)];
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * NT, rl = idx / CH8, c8 = idx % CH8;
        const int row = m0 + rlo + rl, col = on0 + 8 * c8;
        if (row >= rows_M || col >= out_cols) continue;
        float v[8] = {sv[it][0][0], sv[it][0][1], sv[it][0][2], sv[it][0][3],
                      sv[it][1][0], sv[it][1][1], sv[it][1][2], sv[it][1][3]};
        if (col + 8 <= out_cols) {
          const u32x4 r = *(const u32x4*)(Rres + (long)row * ldr + col);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] += lo_bf(r[q]);
            v[2 * q + 1] += hi_bf(r[q]);
          }
        } else {
          for (int q = 0; q < out_cols - col; ++q) v[q] += bf2f(Rres[(long)row * ldr + col + q]);
        }
        if (bias) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (col + q < out_cols) v[q] += bf2f(bias[col + q]);
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack2bf(v[2 * q], v[2 * q + 1]);
        if (col + 8 <= out_cols) {
          *(u32x4*)(C + (long)row * ldc + col) = o;
        } else {
          for (int q = 0; q < out_cols - col; ++q)
            C[(long)row * ldc + col + q] = (bf16_t)((q & 1) ? (o[q >> 1] >> 16) : (o[q >> 1] & 0xffffu));
        }
      }
    }
  }
}

// direct-to-LDS pipeline: whole k stages, byte offsets within 2^31, B2 rows
// starting on a 16-row boundary
template <int BM, int EPI>
static bool dma_ok(const GemmParams& p) {
  const long rowsA = p.M, rowsB = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  return BM >= 128 && p.kchunk % GEMM_DMA_SK(BM) == 0 && p.K % GEMM_DMA_SK(BM) == 0 &&
         rowsA * p.lda * 2 < 0x7fffffffL && rowsB * p.ldb * 2 < 0x7fffffffL &&
         (p.b_split <= 0 || p.b_split % 16 == 0);
}

// M tiles per group of the tile order.  Each XCD runs a contiguous range of
// the order; the workgroups it holds at once read, through its L2, the A row
// blocks of `rows` M tiles and the B column blocks of about resident / rows N
// tiles, so the group height r that minimises r BM + (resident / r) BN
// minimises the fetches from beyond L2.  Groups of 8 unless another height
// (a divisor of the M tile count, so that every group is alike) saves at
// least a fifth: the joint down-projection at T = 2048 (9 tiles x 3 K
// slices per XCD) takes 4 (7 blocks per XCD instead of 10), which measured
// 2-3% faster.
template <int BM, int BN>
static int pick_group_m(int tiles_m, int tiles_n, int ksplit) {
  const long per_xcd = ((long)tiles_m * tiles_n + 7) / 8;
  const int per_cu = BM >= 256 ? 1 : 2;  // workgroups of this tile one CU holds
  const long resident = std::min<long>(per_xcd, std::max(1, 32 * per_cu / std::max(1, ksplit)));
  auto cost = [&](int r) { return (long)r * BM + (resident + r - 1) / r * BN; };
  const int r0 = std::min(tiles_m, 8);
  int best = r0;
  for (int r = std::min(tiles_m, 32); r >= 1; --r)
    if (tiles_m % r == 0 && cost(r) < cost(best)) best = r;
  return cost(best) * 5 <= cost(r0) * 4 ? best : 8;
}

// ---------------------------------------------------------------------------
// 256 x 224 tiles for products 7168 columns wide (o_proj, the dense block's
// W2).  7168 = 28 x 256, so 256 x 256 tiles come in multiples of 28 per 256
// rows: 224 tiles for 2048 rows leave 32 of the 256 CUs idle, 448 for 4096
// rows run as 1.75 waves.  Cutting every 256-column tile into seven 32-column
// strips for a "main" tile plus one strip left over gives 8 x 28 / 7 = 32
// tiles of seven strips per 256 rows: the 28 main tiles (strips 0..6 of
// 256-column tile t) and 4 gathered tiles (strip 7 of tiles 7 u .. 7 u + 6).
// Every tile is a whole-K 256 x 224 product, so the launch fills whole waves
// (256 tiles for 2048 rows, 512 for 4096) and all workgroups of an XCD still
// move through K in step, sharing A and B stages in its L2.
//
// Eight waves: wave w owns rows 64 (w % 4) .. + 63 (two 32-row MFMA blocks)
// and strips 0..3 (w < 4) or 4..6 (w >= 4).  The eight waves of a workgroup
// land on the four SIMDs in a pattern of period four (read back from the
// HW_ID register), so the two waves of a SIMD, w and w + 4, issue
// 8 + 6 = 14 v_mfma_f32_32x32x16_bf16 per 16-wide k step, every SIMD the same.  Operands arrive by direct-to-LDS loads in a
// two-stage ring of 64-k stages (A 32 KB + B 28 KB), as in the generic tile.
// ---------------------------------------------------------------------------
namespace {
constexpr int V_BM = 256, V_NS = 7, V_BN = 32 * V_NS, V_SK = 64, V_ROWB = 128, V_NSTG = 2;
constexpr int V_A_BYTES = V_BM * V_ROWB, V_B_BYTES = V_BN * V_ROWB, V_STAGE = V_A_BYTES + V_B_BYTES;
constexpr int V_LDS = V_NSTG * V_STAGE;  // 120 KB, reused by the epilogue staging
}  // namespace

// first output column of strip j (0..6) of column tile tv; nt = N / 256
MLA_DEV int v224_col(int tv, int j, int nt) {
  return tv < nt ? 256 * tv + 32 * j : 256 * (7 * (tv - nt) + j) + 224;
}

// K loop of one wave: FN strips (4 or 3) starting at strip s0, rows 64 rg ...
template <int FN>
MLA_DEV void v224_loop(floatx16 (&acc)[2][4], const char* ldsc, unsigned lds_base, int nst, int wv,
                       const int (&a_vo)[4], const int (&b_vo)[4], int b_dma0, u32x4 ra, u32x4 rb,
                       int a_rd, int b_rd, int sw, int lg) {
  constexpr int NMF = 2 * FN, NRD = 2 + FN, KSTEPS = V_SK / 16;
#define V_ISSUE(u_)                                                                          \
  do {                                                                                       \
    const unsigned sb_ = lds_base + ((u_) % V_NSTG) * V_STAGE;                               \
    const int ko_ = V_ROWB * (u_);                                                           \
    _Pragma("unroll") for (int d = 0; d < 4; ++d)                                            \
      gemm_dma16(sb_ + 1024 * (4 * wv + d), a_vo[d] + ko_, ra);                              \
    _Pragma("unroll") for (int d = 0; d < FN; ++d)                                           \
      gemm_dma16(sb_ + V_A_BYTES + 1024 * (b_dma0 + d), b_vo[d] + ko_, rb);                  \
  } while (0)
#define V_FREAD(u_, s_, slot)                                                                \
  do {                                                                                       \
    const char* sb_ = ldsc + ((u_) % V_NSTG) * V_STAGE;                                      \
    const int co_ = 16 * ((2 * (s_) + lg) ^ sw);                                             \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                            \
      fa[slot][i] = *(const bf16x8*)(sb_ + a_rd + i * 32 * V_ROWB + co_);                    \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
      fb[slot][j] = *(const bf16x8*)(sb_ + b_rd + j * 32 * V_ROWB + co_);                    \
  } while (0)
#define V_MFMAS(slot)                                                                        \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    const int i = q / FN, j = q % FN;                                                        \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0); \
  }
#define V_SCHED()                                                                            \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    MLA_SGB(SG_MFMA, 1);                                                                     \
    if (q < NRD) MLA_SGB(SG_DS_RD, 1);                                                       \
  }
  bf16x8 fa[2][2], fb[2][FN];
  if (nst <= 0) return;
  V_ISSUE(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nst > 1) V_ISSUE(1);
  V_FREAD(0, 0, 0);
  for (int t = 0; t < nst; ++t) {
#pragma unroll
    for (int s = 0; s + 1 < KSTEPS; ++s) {
      V_FREAD(t, s + 1, (s + 1) & 1);
      V_MFMAS(s & 1)
      V_SCHED()
    }
    // stage t + 1 landed (this wave's loads; the barrier covers the others')
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + V_NSTG < nst) V_ISSUE(t + V_NSTG);  // into stage t's buffer, read by now
    V_FREAD(min(t + 1, nst - 1), 0, 0);
    V_MFMAS(1)
    V_SCHED()
  }
#undef V_ISSUE
#undef V_FREAD
#undef V_MFMAS
#undef V_SCHED
}

// bf16 epilogue of one wave: bias (when given) added in fp32, the rounded
// tile staged in LDS (row pitch 448 B; 16-byte chunk c of row r at
// c ^ ((r >> 2) & 3), which stays inside c's aligned group of four)
template <int FN>
MLA_DEV void v224_stage_bf16(const floatx16 (&acc)[2][4], char* cst, int rg, int s0, int lr, int lg,
                             const bf16_t* __restrict__ bias, int tv, int nt) {
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int colg = v224_col(tv, s0 + j, nt);  // output column of this strip's column 0
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * (s0 + j) + 8 * g + 4 * lg;  // column in the tile
      float bq[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
#pragma unroll
        for (int q = 0; q < 4; ++q) bq[q] = bf2f(bias[colg + 8 * g + 4 * lg + q]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * rg + 32 * i + lr;
        const floatx16& a = acc[i][j];
        *(u32x2*)(cst + r * (V_BN * 2) + 16 * ((c >> 3) ^ ((r >> 2) & 3)) + 8 * ((c >> 2) & 1)) =
            u32x2{pack2bf(a[4 * g] + bq[0], a[4 * g + 1] + bq[1]), pack2bf(a[4 * g + 2] + bq[2], a[4 * g + 3] + bq[3])};
      }
    }
  }
}

// fp32 staging of rows [rlo, rlo + 128) for the residual epilogue: 4-float
// chunk c4 of row r at c4 ^ (r & 7), inside c4's aligned group of eight
MLA_DEV int v224_fidx(int r, int c) { return r * V_BN + (((c >> 2) ^ (r & 7)) << 2) + (c & 3); }
template <int FN>
MLA_DEV void v224_stage_f32(const floatx16 (&acc)[2][4], float* cst, int rg, int s0, int lr, int lg, int rlo) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rl = 64 * rg + 32 * i + lr - rlo;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * (s0 + j) + 8 * g + 4 * lg;
        *(floatx4*)&cst[v224_fidx(rl, c)] =
            floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
  }
}

template <int EPI>
__global__ __launch_bounds__(512) void gemm_v224_kernel(GemmParams p) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_RESID || EPI == EPI_F32, "bf16, residual and fp32-partial epilogues");
  __shared__ __attribute__((aligned(16))) char lds[V_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wv & 3, cg = wv >> 2;
  const int s0 = cg ? 4 : 0;  // first strip of this wave
  const int lr = lane & 31, lg = lane >> 5;
  const int nt = p.N / 256;

  // tile coordinates: XCD-aware, grouped along M (as the generic tile)
  const int lin = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  const int GM = p.group_m;
  const int group = lin / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gm = min(p.tiles_m - first_m, GM);
  const int within = lin - group * GM * p.tiles_n;
  const int tm = first_m + within % gm, tv = within / gm;
  const int m0 = tm * V_BM;
  // K slice of this workgroup (grid.y: fp32-partial launches cut K into ksplit slices)
  const int split = blockIdx.y;
  const int k_begin = split * p.kchunk, k_end = min(p.K, k_begin + p.kchunk);

  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  {
    // DMA d of a wave fills 8 rows of 128 B: lane l -> row 8 g + l / 8
    // (g = the DMA's index in its tile), chunk position l % 8 holding
    // logical chunk (l % 8) ^ swz(row), swz(r) = (r >> 1) & 7.  A: DMAs
    // 4 w .. 4 w + 3.  B: strip wv (DMAs 4 wv ..) for w < 4, DMAs
    // 16 + 3 (w - 4) .. for w >= 4; DMA g covers rows 8 (g % 4) .. of strip g / 4.
    int a_vo[4], b_vo[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r = 8 * (4 * wv + d) + lane / 8;
      const int c = (lane % 8) ^ gemm_swz(r);
      a_vo[d] = (min(m0 + r, p.M - 1) * (int)p.lda + k_begin + 8 * c) * 2;
    }
    const int b_dma0 = cg ? 16 + 3 * (wv - 4) : 4 * wv;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int g = b_dma0 + d;
      const int r = 8 * g + lane / 8;  // row of the B tile
      const int c = (lane % 8) ^ gemm_swz(r);
      const int src = min(v224_col(tv, min(g, 27) / 4, nt) + 8 * (g % 4) + lane / 8, p.N - 1);
      b_vo[d] = (src * (int)p.ldb + k_begin + 8 * c) * 2;
    }
    const u32x4 ra = gemm_rsrc(p.A), rb = gemm_rsrc(p.B);
    const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds;
    const int sw = gemm_swz(lr);  // fragment rows are lr (mod 32)
    const int a_rd = (64 * rg + lr) * V_ROWB, b_rd = V_A_BYTES + (32 * s0 + lr) * V_ROWB;
    const int nst = (k_end - k_begin) / V_SK;
    if (cg == 0)
      v224_loop<4>(acc, lds, lds_base, nst, wv, a_vo, b_vo, b_dma0, ra, rb, a_rd, b_rd, sw, lg);
    else
      v224_loop<3>(acc, lds, lds_base, nst, wv, a_vo, b_vo, b_dma0, ra, rb, a_rd, b_rd, sw, lg);
  }

  const int rows_M = p.M;
  const long ldc = p.ldc;
  bf16_t* C = (bf16_t*)p.C;
  const bf16_t* __restrict__ bias = p.bias;
  constexpr int CH8 = V_BN / 8;  // 28 16-byte output chunks per tile row
  if constexpr (EPI == EPI_BF16) {
    char* cst = lds;
    __syncthreads();  // last K stage read
    if (cg == 0) v224_stage_bf16<4>(acc, cst, rg, s0, lr, lg, bias, tv, nt);
    else v224_stage_bf16<3>(acc, cst, rg, s0, lr, lg, bias, tv, nt);
    __syncthreads();
    constexpr int NIT = V_BM * CH8 / 512;  // 14
    u32x4 sv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * 512, rl = idx / CH8, c8 = idx % CH8;
      sv[it] = *(const u32x4*)(cst + rl * (V_BN * 2) + 16 * (c8 ^ ((rl >> 2) & 3)));
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * 512, rl = idx / CH8, c8 = idx % CH8;
      const int row = m0 + rl;
      if (row >= rows_M) continue;
      *(u32x4*)(C + (long)row * ldc + v224_col(tv, c8 >> 2, nt) + 8 * (c8 & 3)) = sv[it];
    }
  } else if constexpr (EPI == EPI_F32) {
    // fp32 partial of this K slice, staged as the residual epilogue stages it
    // (two passes of 128 rows), 8 columns per thread as two 16-byte stores
    float* cst = (float*)lds;
    float* Cf = (float*)p.C + (long)split * p.split_stride;
    constexpr int NIT = 128 * CH8 / 512;  // 7
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      __syncthreads();  // LDS free: last K stage read (pass 0) or previous pass stored
      const int rlo = 128 * pass;
      if ((rg >> 1) == pass) {
        if (cg == 0) v224_stage_f32<4>(acc, cst, rg, s0, lr, lg, rlo);
        else v224_stage_f32<3>(acc, cst, rg, s0, lr, lg, rlo);
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * 512, rl = idx / CH8, c8 = idx % CH8;
        const int row = m0 + rlo + rl;
        const floatx4 a = *(const floatx4*)&cst[v224_fidx(rl, 8 * c8)];
        const floatx4 b = *(const floatx4*)&cst[v224_fidx(rl, 8 * c8 + 4)];
        if (row >= rows_M) continue;
        float* dst = Cf + (long)row * ldc + v224_col(tv, c8 >> 2, nt) + 8 * (c8 & 3);
        *(floatx4*)dst = a;
        *(floatx4*)(dst + 4) = b;
      }
    }
  } else {
    // residual add in two passes of 128 rows (waves with rg < 2, then rg >= 2)
    float* cst = (float*)lds;
    const bf16_t* __restrict__ Rres = p.R;
    const long ldr = p.ldr;
    constexpr int NIT = 128 * CH8 / 512;  // 7
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      __syncthreads();  // LDS free: last K stage read (pass 0) or previous pass stored
      const int rlo = 128 * pass;
      if ((rg >> 1) == pass) {
        if (cg == 0) v224_stage_f32<4>(acc, cst, rg, s0, lr, lg, rlo);
        else v224_stage_f32<3>(acc, cst, rg, s0, lr, lg, rlo);
      }
      __syncthreads();
      floatx4 sv[NIT][2];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * 512, rl = idx / CH8, c8 = idx % CH8;
        sv[it][0] = *(const floatx4*)&cst[v224_fidx(rl, 8 * c8)];
        sv[it][1] = *(const floatx4*)&cst[v224_fidx(rl, 8 * c8 + 4)];
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * 512, rl = idx / CH8, c8 = idx % CH8;
        const int row = m0 + rlo + rl;
        if (row >= rows_M) continue;
        const int col = v224_col(tv, c8 >> 2, nt) + 8 * (c8 & 3);
        float v[8] = {sv[it][0][0], sv[it][0][1], sv[it][0][2], sv[it][0][3],
                      sv[it][1][0], sv[it][1][1], sv[it][1][2], sv[it][1][3]};
        const u32x4 r = *(const u32x4*)(Rres + (long)row * ldr + col);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += lo_bf(r[q]);
          v[2 * q + 1] += hi_bf(r[q]);
        }
        if (bias) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += bf2f(bias[col + q]);
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack2bf(v[2 * q], v[2 * q + 1]);
        *(u32x4*)(C + (long)row * ldc + col) = o;
      }
    }
  }
}

// The 256 x 224 tiling applies to single products whose width is a multiple
// of 1792 (seven 256-column tiles) with no batch or second weight: bf16 and
// residual outputs over the whole K (chosen automatically when its whole
// waves beat the 256 x 256 tile's), or fp32 partials of K slices (chosen by
// the small-product plan).
static bool v224_shape_ok(const GemmParams& p, int epi) {
  if (epi != EPI_BF16 && epi != EPI_RESID && epi != EPI_F32) return false;
  if (p.N % 1792 != 0 || p.batch != 1 || p.b_split > 0 || p.B2 || p.K % V_SK != 0 || p.M <= 0) return false;
  if (epi != EPI_F32 && (p.ksplit != 1 || p.kchunk != p.K)) return false;
  if (p.kchunk % V_SK != 0 || p.kchunk <= 0 || (long)p.ksplit * p.kchunk < p.K) return false;
  if (epi == EPI_F32 && (p.bias || (p.ldc % 4) != 0)) return false;
  if ((long)p.M * p.lda * 2 >= 0x7fffffffL || (long)p.N * p.ldb * 2 >= 0x7fffffffL) return false;
  if ((p.ldc % 8) != 0 && epi != EPI_F32) return false;
  return epi != EPI_RESID || (p.ldr % 8) == 0;
}
static bool v224_ok(const GemmParams& p, int epi) {
  if (epi == EPI_F32 || !v224_shape_ok(p, epi)) return false;
  const long tm = (p.M + 255) / 256;
  const long w256 = (tm * (p.N / 256) + 255) / 256, w224 = (tm * (p.N / 224) + 255) / 256;
  return w224 * 7 < w256 * 8;
}

template <int EPI>
static hipError_t launch_v224(GemmParams p, hipStream_t s) {
  p.tiles_m = (p.M + 255) / 256;
  p.tiles_n = p.N / 224;
  p.group_m = pick_group_m<256, 224>(p.tiles_m, p.tiles_n, p.ksplit);
  hipLaunchKernelGGL(gemm_v224_kernel<EPI>, dim3(p.tiles_m * p.tiles_n, p.ksplit), dim3(512), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Persistent 256 x 256 tile loop for launches of more than one round of tiles
// with a bf16 or SwiGLU output.  With one workgroup per tile, every tile pays
// its own first-stage wait and an epilogue staged through the whole LDS with
// two workgroup barriers per pass (~5.5 us per tile on the paired
// up-projections, against 1.4 us per 64-k stage).  Here one workgroup per CU
// runs a list of tiles, and between two tiles:
//   - the next tile's first stage is issued into ring buffer 0 as soon as
//     every wave has read the last stage;
//   - each wave writes its own 128 x 64 part of the finished tile through a
//     private 4 KB LDS slot (the 32 KB beyond the 128 KB ring), 32 rows at a
//     time, and stores whole 128-byte row segments: no workgroup barrier,
//     since a wave's LDS operations complete in issue order;
//   - the second stage is issued after the stores, so that waiting until at
//     most one stage of loads is in flight (loads complete in order) proves
//     the first stage landed without waiting for the stores.
// The first k-step of every tile starts its MFMA chains from a zero C
// operand instead of zeroing 128 accumulators.
//
// Schedule (static, per XCD): the logical order is the one-workgroup-per-tile
// launch's (workgroup b on XCD b % 8, XCD-contiguous tile ranges, product 0
// first), and the W workgroups of an XCD split its slots longest first:
// product 0's slots round robin (slot w + k W to workgroup w), then
// product 1's slots in runs whose lengths the launcher computes by greedy
// least-loaded assignment with per-tile costs of (K / 64 + 2) stages.  The
// workgroups with one more product-0 slot (w < n0 % W) and the others each
// start equally loaded, and ties go to the lower index, so in each of the two
// groups the first e workgroups get a + 1 runs of product 1 and the rest a:
// four numbers per XCD describe the schedule (a kernel argument block of a
// kilobyte of per-workgroup tables launched measurably slower).
// Products with a bias keep the per-tile kernel.
// ---------------------------------------------------------------------------
struct PersSched {
  int W;                        // workgroups per XCD (grid 8 W)
  int aH[8], eH[8], aL[8], eL[8];  // pairs: product-1 run lengths per XCD (see above)
};

template <int EPI>
__global__ __launch_bounds__(512) void gemm_pers_kernel(GemmGroup gg, PersSched ps) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_SWIGLU, "bf16-output epilogues only");
  constexpr int BM = 256, BN = 256, WN = 4;
  constexpr int WTM = 128, WTN = 64, FM = WTM / 32, FN = WTN / 32, NMF = FM * FN, NRD = FM + FN;
  constexpr int KSTEPS = 4, CH = 8, ROWB = 128;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE_B = A_BYTES + B_BYTES;  // 64 KB
  constexpr int A_DMA = A_BYTES / 1024 / 8, B_DMA = B_BYTES / 1024 / 8;                 // 4 + 4
  static_assert(A_DMA + B_DMA == 8, "the stage wait below counts 8 loads per wave");
  constexpr int RPD = 1024 / ROWB;  // rows per DMA
  constexpr int WST = 4096;         // per-wave epilogue staging
  __shared__ u32x4 lds_raw[(2 * STAGE_B + 8 * WST) / 16];  // 160 KB
  char* ldsc = (char*)lds_raw;
  const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = tid >> 6, wv = __builtin_amdgcn_readfirstlane(wid);
  const int wm = wid / WN, wn = wid % WN;
  const int lr = lane & 31, lg = lane >> 5;

  // ---- this workgroup's slots ----
  const int x = blockIdx.x & 7, w = blockIdx.x >> 3, W = ps.W;
  const int total = gg.tiles0 + (gg.n == 2 ? gg.tiles1 : 0);
  const int slots = total / 8 + (x < total % 8 ? 1 : 0);
  const int n0 = gg.n == 2 ? gg.tiles0 / 8 + (x < gg.tiles0 % 8 ? 1 : 0) : slots;
  const int nl = w < n0 ? (n0 - w + W - 1) / W : 0;
  int ns = 0, sbase = n0;
  if (gg.n == 2) {
    const int r0 = n0 % W, aH = ps.aH[x], eH = ps.eH[x], aL = ps.aL[x], eL = ps.eL[x];
    if (w < r0) {
      ns = aH + (w < eH ? 1 : 0);
      sbase += w * aH + min(w, eH);
    } else {
      const int u = w - r0;
      ns = aL + (u < eL ? 1 : 0);
      sbase += r0 * aH + eH + u * aL + min(u, eL);
    }
  }
  const int nitems = nl + ns;
  if (nitems == 0) return;

  // ---- per-tile state: source offsets of this wave's DMAs, tile origin ----
  int a_vo[A_DMA], b_vo[B_DMA];
  unsigned b_src2 = 0;
  u32x4 ra, rb1, rb2;
  int nst = 0, prob = 0, m0 = 0, n0c = 0;
  auto setup = [&](int k) {
    const int slot = k < nl ? w + k * W : sbase + (k - nl);
    int lin;
    gemm_tile_of(gg, 8 * slot + x, prob, lin);
    const GemmParams& p = gg.p[prob];
    const int GM = p.group_m;
    const int group = lin / (GM * p.tiles_n);
    const int first_m = group * GM;
    const int gm = min(p.tiles_m - first_m, GM);
    const int within = lin - group * GM * p.tiles_n;
    m0 = (first_m + within % gm) * BM;
    n0c = (within / gm) * BN;
    nst = p.K / 64;
#pragma unroll
    for (int d = 0; d < A_DMA; ++d) {
      const int r = RPD * (wv * A_DMA + d) + lane / CH;
      const int c = (lane % CH) ^ gemm_swz(r);
      a_vo[d] = (min(m0 + r, p.M - 1) * (int)p.lda + 8 * c) * 2;
    }
    b_src2 = 0;
#pragma unroll
    for (int d = 0; d < B_DMA; ++d) {
      const int r = RPD * (wv * B_DMA + d) + lane / CH;
      const int c = (lane % CH) ^ gemm_swz(r);
      int src;
      if (EPI == EPI_SWIGLU) {
        const int rb = r >> 5;
        src = min(n0c / 2 + (rb >> 1) * 32 + (r & 31), p.N / 2 - 1);
        if (rb & 1) b_src2 |= 1u << d;
      } else {
        src = min(n0c + r, p.N - 1);
        if (p.b_split > 0 && n0c + RPD * (wv * B_DMA + d) >= p.b_split) {
          src -= p.b_split;
          b_src2 |= 1u << d;
        }
      }
      b_vo[d] = (src * (int)p.ldb + 8 * c) * 2;
    }
    ra = gemm_rsrc(p.A);
    rb1 = gemm_rsrc(p.B);
    rb2 = gemm_rsrc(p.B2 ? p.B2 : p.B);
  };

#define PS_ISSUE(u_)                                                                         \
  do {                                                                                       \
    const unsigned sb_ = lds_base + ((u_) & 1) * STAGE_B;                                    \
    const int ko_ = ROWB * (u_);                                                             \
    _Pragma("unroll") for (int d = 0; d < A_DMA; ++d)                                        \
      gemm_dma16(sb_ + 1024 * (wv * A_DMA + d), a_vo[d] + ko_, ra);                          \
    _Pragma("unroll") for (int d = 0; d < B_DMA; ++d)                                        \
      gemm_dma16(sb_ + A_BYTES + 1024 * (wv * B_DMA + d), b_vo[d] + ko_,                     \
                 ((b_src2 >> d) & 1) ? rb2 : rb1);                                           \
  } while (0)
  const int sw = gemm_swz(lr);  // fragment rows are lr (mod 32)
  const int a_rd = (wm * WTM + lr) * ROWB, b_rd = A_BYTES + (wn * WTN + lr) * ROWB;
#define PS_FREAD(u_, s_, slot)                                                               \
  do {                                                                                       \
    const char* sb_ = ldsc + ((u_) & 1) * STAGE_B;                                           \
    const int co_ = 16 * ((2 * (s_) + lg) ^ sw);                                             \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                           \
      fa[slot][i] = *(const bf16x8*)(sb_ + a_rd + i * 32 * ROWB + co_);                      \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
      fb[slot][j] = *(const bf16x8*)(sb_ + b_rd + j * 32 * ROWB + co_);                      \
  } while (0)
#define PS_MFMAS(slot, zero_)                                                                \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    const int i = q / FN, j = q % FN;                                                        \
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i],            \
                                                        (zero_) ? floatx16{} : acc[i][j], 0, 0, 0); \
  }
#define PS_SCHED()                                                                           \
  _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                          \
    MLA_SGB(SG_MFMA, 1);                                                                     \
    if (q < NRD) MLA_SGB(SG_DS_RD, 1);                                                       \
  }

  bf16x8 fa[2][FM], fb[2][FN];
  floatx16 acc[FM][FN];
  // one 64-k stage: k-step s + 1's fragments read under k-step s's MFMAs; the
  // barrier before the last k-step, whose MFMAs cover the next stage's first
  // fragment reads (FIRST: the stage that starts the accumulators)
  auto stage = [&](int t, auto first_) {
    constexpr bool FIRST = decltype(first_)::value;
#pragma unroll
    for (int s = 0; s + 1 < KSTEPS; ++s) {
      PS_FREAD(t, s + 1, (s + 1) & 1);
      PS_MFMAS(s & 1, FIRST && s == 0)
      PS_SCHED()
    }
    // stage t + 1 landed (this wave's loads; the barrier covers the others')
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < nst) PS_ISSUE(t + 2);  // into stage t's buffer, read by now
    PS_FREAD(min(t + 1, nst - 1), 0, 0);
    PS_MFMAS(1, false)
    PS_SCHED()
  };

  setup(0);
  PS_ISSUE(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nst > 1) PS_ISSUE(1);
  PS_FREAD(0, 0, 0);

  for (int k = 0; k < nitems; ++k) {
    stage(0, std::true_type{});
    for (int t = 1; t < nst; ++t) stage(t, std::false_type{});

    // ---- epilogue of this tile; the next tile's first stage loads meanwhile ----
    const int eprob = prob, em0 = m0, en0 = n0c;
    __syncthreads();  // every wave's last fragment reads done: both ring buffers free
    const bool more = k + 1 < nitems;
    if (more) {
      setup(k + 1);
      PS_ISSUE(0);
    }
    {
      const GemmParams& p = gg.p[eprob];
      // this wave's output part: rows wm WTM + 32 i + (0..31), OCW columns
      constexpr int OCW = (EPI == EPI_SWIGLU) ? WTN / 2 : WTN;
      constexpr int RB = OCW * 2, NCH = RB / 16;  // staged row bytes, 16-byte chunks per row
      constexpr int RPI = 64 / NCH;               // rows per 16-byte-per-lane read
      const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
      const int ocol0 = (EPI == EPI_SWIGLU) ? en0 / 2 + wn * OCW : en0 + wn * OCW;
      bf16_t* C = (bf16_t*)p.C;
      const int rows_M = p.M;
      const long ldc = p.ldc;
      char* wst = ldsc + 2 * STAGE_B + wid * WST;
      // chunk swizzle: the 32 rows one write instruction covers spread over all
      // 64 banks, and the rows one 16-lane read phase covers are disjoint
      auto swz = [](int r) { return (EPI == EPI_SWIGLU) ? ((r >> 2) & 3) : ((r >> 1) & 7); };
      const int rrow = lane / NCH, rch = lane % NCH;  // read-out: row within the group, chunk
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        asm volatile("" ::: "memory");  // the previous rows' reads stay before these writes
#pragma unroll
        for (int j = 0; j < FN; j += (EPI == EPI_SWIGLU ? 2 : 1))
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (EPI == EPI_SWIGLU) {
                const float gg_ = acc[i][j][4 * g + q], uu = acc[i][j + 1][4 * g + q];
                v[q] = gg_ / (1.f + __expf(-gg_)) * uu;
              } else {
                v[q] = acc[i][j][4 * g + q];
              }
            }
            const int c = (EPI == EPI_SWIGLU) ? g : 4 * j + g;  // 16-byte chunk of the row
            *(u32x2*)(wst + lr * RB + 16 * (c ^ swz(lr)) + 8 * lg) = u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
          }
        asm volatile("" ::: "memory");  // a wave's LDS operations complete in order
        u32x4 sv[32 / RPI];
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int r = it * RPI + rrow;
          sv[it] = *(const u32x4*)(wst + r * RB + 16 * (rch ^ swz(r)));
        }
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int row = em0 + wm * WTM + 32 * i + it * RPI + rrow, col = ocol0 + 8 * rch;
          if (row >= rows_M || col >= out_cols) continue;
          bf16_t* dst = C + (long)row * ldc + col;
          if (col + 8 <= out_cols) {
            *(u32x4*)dst = sv[it];
          } else {
            for (int q = 0; q < out_cols - col; ++q)
              dst[q] = (bf16_t)((q & 1) ? (sv[it][q >> 1] >> 16) : (sv[it][q >> 1] & 0xffffu));
          }
        }
      }
    }
    if (more) {
      // stage 1 goes after the stores: at most its 8 loads still in flight
      // means stage 0 has landed, whatever the stores are doing
      if (nst > 1) {
        PS_ISSUE(1);
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      PS_FREAD(0, 0, 0);
    }
  }
#undef PS_ISSUE
#undef PS_FREAD
#undef PS_MFMAS
#undef PS_SCHED
}

// Persistent launch of a 256 x 256 bf16 / SwiGLU product (or pair) without
// bias: one workgroup per CU when the tiles take more than one round.  Pairs
// need product 0 to be the longer one (it is scheduled first).
static bool pers_ok(const GemmGroup& g) {
  const long total = g.tiles0 + (g.n == 2 ? g.tiles1 : 0);
  if (total <= 256) return false;
  for (int i = 0; i < g.n; ++i)
    if (g.p[i].batch != 1 || g.p[i].ksplit != 1 || g.p[i].kchunk != g.p[i].K || g.p[i].K % 64 != 0 ||
        g.p[i].bias)
      return false;
  return g.n == 1 || g.p[0].K >= g.p[1].K;
}

// Greedy least-loaded split of each XCD's product-1 slots (ties to the lower
// workgroup index), in the compact form the kernel reads.  Within each of the
// two groups the loads differ by at most one product-1 tile and the
// least-loaded member is the first one holding the group's smallest count, so
// the greedy choice only compares the two groups' candidates: O(1) per slot.
static bool pers_plan(const GemmGroup& g, PersSched& ps) {
  constexpr int W = 32;  // workgroups per XCD: one per CU of the 256
  ps = PersSched{};
  ps.W = W;
  if (g.n != 2) return true;
  const long c0 = g.p[0].K / 64 + 2, c1 = g.p[1].K / 64 + 2;
  const int total = g.tiles0 + g.tiles1;
  for (int x = 0; x < 8; ++x) {
    const int slots = total / 8 + (x < total % 8 ? 1 : 0);
    const int n0 = g.tiles0 / 8 + (x < g.tiles0 % 8 ? 1 : 0);
    const int r0 = n0 % W, sz[2] = {r0, W - r0};
    const long base[2] = {(n0 / W + 1) * c0, (n0 / W) * c0};
    long cnt[2] = {0, 0};  // product-1 slots given to group H (w < r0) and L
    for (int j = n0; j < slots; ++j) {
      // the group's least-loaded member holds cnt / size slots
      long best = -1;
      int bg = 0;
      for (int gi = 0; gi < 2; ++gi) {
        if (sz[gi] == 0) continue;
        const long ld = base[gi] + (cnt[gi] / sz[gi]) * c1;
        if (best < 0 || ld < best) {  // equal loads: group H holds the lower index
          best = ld;
          bg = gi;
        }
      }
      ++cnt[bg];
    }
    ps.aH[x] = r0 ? (int)(cnt[0] / r0) : 0;
    ps.eH[x] = r0 ? (int)(cnt[0] % r0) : 0;
    ps.aL[x] = (int)(cnt[1] / (W - r0));
    ps.eL[x] = (int)(cnt[1] % (W - r0));
  }
  return true;
}

template <int BM, int BN, int WM, int WN, int EPI>
static hipError_t launch_cfg(const GemmParams* ps, int n, hipStream_t s) {
  GemmGroup g;
  g.n = n;
  bool dma = true;
  for (int i = 0; i < n; ++i) {
    g.p[i] = ps[i];
    g.p[i].tiles_m = (ps[i].M + BM - 1) / BM;
    g.p[i].tiles_n = (ps[i].N + BN - 1) / BN;  // SwiGLU: N counts both W1 and W3 columns
    g.p[i].group_m = pick_group_m<BM, BN>(g.p[i].tiles_m, g.p[i].tiles_n, ps[i].ksplit);
    dma = dma && dma_ok<BM, EPI>(ps[i]);
  }
  if (n == 1) g.p[1] = g.p[0];
  g.tiles0 = g.p[0].tiles_m * g.p[0].tiles_n;
  g.tiles1 = n == 2 ? g.p[1].tiles_m * g.p[1].tiles_n : 0;
  dim3 grid(g.tiles0 + g.tiles1, ps[0].batch * ps[0].ksplit);
  if constexpr (BM == 256 && BN == 256 && (EPI == EPI_BF16 || EPI == EPI_SWIGLU)) {
    PersSched sch;
    if (dma && pers_ok(g) && pers_plan(g, sch)) {
      hipLaunchKernelGGL(gemm_pers_kernel<EPI>, dim3(8 * sch.W), dim3(512), 0, s, g, sch);
      return hipGetLastError();
    }
  }
  if constexpr (BM >= 128) {
    if (dma) {
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI, true>), grid, dim3(WM * WN * 64), 0, s, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI, false>), grid, dim3(WM * WN * 64), 0, s, g);
  return hipGetLastError();
}
template <int BM, int BN, int WM, int WN, int EPI>
static hipError_t launch_cfg(GemmParams p, hipStream_t s) {
  return launch_cfg<BM, BN, WM, WN, EPI>(&p, 1, s);
}

template <int EPI>
static hipError_t launch_epi(const GemmParams* ps, int n, int cfg, hipStream_t s) {
  switch (cfg) {
    case GEMM_CFG_256x256: return launch_cfg<256, 256, 2, 4, EPI>(ps, n, s);
    case GEMM_CFG_128x128: return launch_cfg<128, 128, 2, 2, EPI>(ps, n, s);
    case GEMM_CFG_64x128: return launch_cfg<64, 128, 1, 2, EPI>(ps, n, s);
    default: return hipErrorInvalidValue;
  }
}
template <int EPI>
static hipError_t launch_epi(GemmParams p, int cfg, hipStream_t s) {
  return launch_epi<EPI>(&p, 1, cfg, s);
}

// Tile config and split-K count by a wave-quantisation cost model: a launch
// of T work units runs in ceil(T / 256) waves on the 256 CUs, each wave as
// long as one unit (a tile over K / S), and a 256x256 tile computes about
// 1.35x faster per CU than four 128x128 tiles (fewer LDS bytes per MFMA;
// measured 1.3-1.4 on the prefill shapes).
// Measured on the prefill shapes (M = 2048): it picks 256x256 with three
// K splits for the 2112 x 7168 down-projection, 128x128 for the q
// up-projection and 256x256 for kv and o_proj.
GemmPlan gemm_plan(int M, int N, int K, int batch, int max_split) {
  GemmPlan best{GEMM_CFG_64x128, 1, K};
  if (M <= 64) return best;
  double best_t = 1e30;
  const int kb = (K + 63) / 64;
  for (int cfg : {GEMM_CFG_256x256, GEMM_CFG_128x128}) {
    const int b = cfg == GEMM_CFG_256x256 ? 256 : 128;
    const double rate = cfg == GEMM_CFG_256x256 ? 1.35 : 1.0;
    const long tiles = (long)((M + b - 1) / b) * ((N + b - 1) / b) * batch;
    for (int S = 1; S <= max_split; ++S) {
      const int per = (kb + S - 1) / S;
      if (S > 1 && per < 8) break;  // keep >= 512 of K per split
      const int Sr = (kb + per - 1) / per;
      const long waves = (tiles * Sr + 255) / 256;
      const double t = (double)waves * b * b * per / rate;
      if (t < best_t * 0.999) {
        best_t = t;
        best = GemmPlan{cfg, Sr, per * 64};
      }
    }
  }
  return best;
}

int gemm_pick_cfg(int M, int N, int K, int batch) { return gemm_plan(M, N, K, batch, 1).cfg; }

// Plan for a product of a few hundred rows (64 < M <= 1024), where the tile
// grid alone leaves most CUs idle and splitting K pays even with the fp32
// partial traffic.  A time model in seconds, from rates measured on the
// prefill and chunked-prefill shapes: a CU running one 256x256 tile
// sustains 5.6 TFLOP/s; a 128x128 tile alone on its CU 2.46 TFLOP/s, two
// sharing a CU 4.2 TFLOP/s together; 5 us / 3 us of prologue and epilogue
// per tile; partials move at 5 TB/s.  With fp32_out the product's consumer
// reads fp32 partials anyway (only the extra splits cost); otherwise the
// partials are summed into bf16 by reduce_splits (one more launch).
GemmPlan gemm_plan_small(int M, int N, int K, bool fp32_out, int max_split) {
  GemmPlan best{GEMM_CFG_128x128, 1, K};
  double best_t = 1e30;
  const int kb = (K + 63) / 64;
  for (int cfg : {GEMM_CFG_256x256, GEMM_CFG_256x224, GEMM_CFG_128x128}) {
    // 256 x 224 tiles (products 1792k wide) run at the 256 x 256 tile's per-CU rate
    if (cfg == GEMM_CFG_256x224 && N % 1792 != 0) continue;
    const int b = cfg == GEMM_CFG_128x128 ? 128 : 256, bn = cfg == GEMM_CFG_256x224 ? 224 : b;
    const long tiles = (long)((M + b - 1) / b) * ((N + bn - 1) / bn);
    for (int S = 1; S <= max_split; ++S) {
      const int per = (kb + S - 1) / S;
      if (S > 1 && per < 8) break;  // keep >= 512 of K per split
      const int Sr = (kb + per - 1) / per;
      const long W = tiles * Sr;
      const double fl = 2.0 * b * bn * 64.0 * per;  // FLOPs of one tile
      double t;
      if (b == 256) t = (double)((W + 255) / 256) * (fl / 5.6e12 + 5e-6);
      else if (W <= 256) t = fl / 2.46e12 + 3e-6;
      else t = (double)((W + 511) / 512) * (2.0 * fl / 4.2e12 + 3e-6);
      const double mn = (double)M * N;
      if (fp32_out) t += (Sr - 1) * mn * 8.0 / 5e12;
      else if (Sr > 1) t += (Sr * mn * 8.0 + mn * 2.0) / 5e12 + 3e-6;
      if (t < best_t * 0.999) {
        best_t = t;
        best = GemmPlan{cfg, Sr, per * 64};
      }
    }
  }
  return best;
}

hipError_t gemm_bf16_pair(GemmParams a, GemmParams b, int epi, int cfg, hipStream_t s) {
  GemmParams ps[2] = {a, b};
  for (auto& p : ps) {
    if (p.batch > 1 || p.ksplit > 1) return hipErrorInvalidValue;
    p.batch = p.ksplit = 1;
    if (p.kchunk <= 0) p.kchunk = p.K;
  }
  const int bm = cfg == GEMM_CFG_256x256 ? 256 : cfg == GEMM_CFG_128x128 ? 128 : 64;
  const int bn = cfg == GEMM_CFG_256x256 ? 256 : 128;
  // the per-XCD split of the two tile ranges needs at least 8 tiles of each
  const long t0 = (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
  const long t1 = (long)((b.M + bm - 1) / bm) * ((b.N + bn - 1) / bn);
  if (t0 < 8 || t1 < 8) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_F32: return launch_epi<EPI_F32>(ps, 2, cfg, s);
    case EPI_BF16: return launch_epi<EPI_BF16>(ps, 2, cfg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_bf16(GemmParams p, int epi, int cfg, hipStream_t s) {
  if (p.batch <= 0) p.batch = 1;
  if (p.ksplit <= 0) p.ksplit = 1;
  if (p.kchunk <= 0) p.kchunk = p.K;
  if (cfg < 0 && v224_ok(p, epi))
    return epi == EPI_BF16 ? launch_v224<EPI_BF16>(p, s) : launch_v224<EPI_RESID>(p, s);
  if (cfg == GEMM_CFG_256x224) {
    // the plan's 256 x 224 choice; a product outside its shape takes the 256 x 256 tile
    if (v224_shape_ok(p, epi)) {
      if (epi == EPI_F32) return launch_v224<EPI_F32>(p, s);
      if (epi == EPI_BF16 || epi == EPI_RESID)
        return epi == EPI_BF16 ? launch_v224<EPI_BF16>(p, s) : launch_v224<EPI_RESID>(p, s);
    }
    cfg = GEMM_CFG_256x256;
  }
  if (cfg < 0) cfg = gemm_pick_cfg(p.M, p.N, p.kchunk, p.batch * p.ksplit);
  switch (epi) {
    case EPI_F32: return launch_epi<EPI_F32>(p, cfg, s);
    case EPI_BF16: return launch_epi<EPI_BF16>(p, cfg, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(p, cfg, s);
    case EPI_SWIGLU:
      if (cfg == GEMM_CFG_64x128) return launch_cfg<64, 128, 1, 2, EPI_SWIGLU>(p, s);
      if (cfg == GEMM_CFG_128x128) return launch_cfg<128, 128, 2, 2, EPI_SWIGLU>(p, s);
      return launch_cfg<256, 256, 2, 4, EPI_SWIGLU>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
