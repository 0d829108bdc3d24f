// Device bodies of the balanced weight-streaming GEMM and of its
// fixed-order split sum, shared by their own kernels (gemm_stream.hip) and by
// the persistent latent-decode kernel.
//
// Weight-streaming bf16 GEMM for decode-sized products (M <= 64 rows),
// balanced over the whole chip: C[M,N] = A[M,K] . B[N,K]^T.
//
// In a decode step every projection multiplies a handful of token rows by a
// full weight matrix, so the time is the weight stream from HBM.  The work is
// cut into units of (128 weight rows) x (128 k); the units, in n-block-major
// order, are dealt out as equal contiguous runs to a persistent grid of G
// workgroups (one per CU), so every CU streams the same number of bytes
// whatever the shape (split-K where a run crosses k, n-block changes where it
// crosses n).  A run never spans more than two n-blocks, so a workgroup keeps
// two accumulator sets and writes at most two fp32 partial blocks after its
// loop.  A fixed-order reduction (stream_sum4) adds the partials of each
// n-block in workgroup order: deterministic.
//
// Each unit's weight tile [128 x 256 B] and activation slice [Mp x 256 B]
// arrive by wave-wide direct-to-LDS buffer loads through a 3-stage ring, two
// units ahead of the MFMAs (v_mfma_f32_32x32x16_bf16: weight rows as the A
// operand, activation rows as the B operand, so the accumulator holds C^T).
// Out-of-range weight rows and activation rows read as zero (buffer range).
#pragma once
#include "stream_sum.h"

namespace mla {

namespace {
constexpr int SU_ROWB = SU_K * 2;       // bytes per tile row
constexpr int SU_NST = 3;               // LDS ring depth
constexpr int SU_WTILE = SU_N * SU_ROWB;  // 32 KB

MLA_DEV void su_dma16(unsigned m0, int voff, u32x4 rsrc) {
  // lane l's 16 bytes at rsrc.base + voff -> LDS byte m0 + 16 l; issued from
  // asm so that the compiler's wait counting stays out (explicit vmcnt below)
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
MLA_DEV u32x4 su_rsrc(const void* base, long bytes) {
  const unsigned long a = (unsigned long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)(bytes < 0 ? 0 : (bytes > 0x7fffffffL ? 0x7fffffffL : bytes)));
  r[3] = 0x00020000u;
  return r;
}
}  // namespace

// Products of one launch: the units of product 0 come first, then those of
// product 1 (n = 1: product 0 only).
struct StreamPair {
  GemmParams p[2];
  StreamInfo s[2];
  float* part[2];
  int n;
};

// LDS bytes of gemm_stream_body for MB 32-row activation blocks
template <int MB>
constexpr int stream_lds_bytes() { return SU_NST * (SU_WTILE + 32 * MB * SU_ROWB); }

// One workgroup of the stream (256 threads): workgroup index bid of the
// plan's G, ring in lds (stream_lds_bytes<MB>() bytes, 16-byte aligned).
template <int MB, int NP>
MLA_DEV void gemm_stream_body(const StreamPair& sp, int bid, char* lds) {
  constexpr int MP = 32 * MB;
  constexpr int ATILE = MP * SU_ROWB;
  constexpr int STAGE = SU_WTILE + ATILE;
  constexpr int W_DPW = SU_WTILE / 1024 / 4;   // weight DMAs per wave per unit (8)
  constexpr int A_DPW = ATILE / 1024 / 4;      // activation DMAs per wave per unit (MB * 2)
  constexpr int DPW = W_DPW + A_DPW;
  const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const StreamInfo& s0 = sp.s[0];
  const int u0 = su_start(s0, bid), u1 = su_start(s0, bid + 1);
  const int U0 = s0.NB * s0.KS;  // units of product 0
  const int NB0 = s0.NB, KS0 = s0.KS, KS1 = sp.s[1].KS;
  // global block index of unit u: product 0's blocks, then product 1's
  auto gblock = [&](int u) { return NP == 1 || u < U0 ? u / KS0 : NB0 + (u - U0) / KS1; };
  // both products' operands, read once (the issue below picks one per unit)
  const bf16_t* const A0 = sp.p[0].A;  const bf16_t* const A1 = sp.p[1].A;
  const bf16_t* const B0 = sp.p[0].B;  const bf16_t* const B1 = sp.p[1].B;
  const bf16_t* const B20 = sp.p[0].B2;
  const long lda0 = sp.p[0].lda, lda1 = sp.p[1].lda, ldb0 = sp.p[0].ldb, ldb1 = sp.p[1].ldb;
  const int N0 = sp.p[0].N, N1 = sp.p[1].N, M0 = sp.p[0].M, bs0 = sp.p[0].b_split;
  const int gb0 = gblock(u0);

  // Tiles hold rows of 256 B (16 chunks of 16 B); chunk c of row r sits at
  // chunk position c ^ (r & 15), so the 16 rows of a half-wave operand read
  // (same logical chunk) hit 16 different bank groups (unswizzled, all of
  // them would share one: measured 16-way conflicts).  DMA i of this wave
  // fills tile rows 4 i .. 4 i + 3: lane l -> row 4 i + l / 16, chunk position
  // l % 16, i.e. logical chunk (l % 16) ^ (row & 15); the rows are
  // multiplied by the product's row pitch at issue.
  int wrow[W_DPW], wco[W_DPW], arow[A_DPW], aco[A_DPW];
#pragma unroll
  for (int i = 0; i < W_DPW; ++i) {
    wrow[i] = 4 * (w * W_DPW + i) + (lane >> 4);
    wco[i] = 16 * ((lane & 15) ^ (wrow[i] & 15));
  }
#pragma unroll
  for (int i = 0; i < A_DPW; ++i) {
    arow[i] = 4 * (w * A_DPW + i) + (lane >> 4);
    aco[i] = 16 * ((lane & 15) ^ (arow[i] & 15));
  }

#define SU_ISSUE(uu)                                                                         \
  do {                                                                                       \
    const int u_ = (uu);                                                                     \
    const bool p1_ = NP == 2 && u_ >= U0;                                                    \
    const int ks_n = p1_ ? KS1 : KS0;                                                        \
    const int ul_ = u_ - (p1_ ? U0 : 0);                                                     \
    const int nb_ = ul_ / ks_n, ks_ = ul_ - nb_ * ks_n;                                      \
    const int n0_ = nb_ * SU_N;                                                              \
    const long ldb_ = p1_ ? ldb1 : ldb0, lda_ = p1_ ? lda1 : lda0;                           \
    const bf16_t* wb_;                                                                       \
    int rows_;                                                                               \
    if (!p1_ && bs0 > 0 && n0_ >= bs0) {                                                     \
      wb_ = B20 + (long)(n0_ - bs0) * ldb_;                                                  \
      rows_ = min(SU_N, N0 - n0_);                                                           \
    } else {                                                                                 \
      wb_ = (p1_ ? B1 : B0) + (long)n0_ * ldb_;                                              \
      rows_ = min(SU_N, (p1_ ? N1 : (bs0 > 0 ? bs0 : N0)) - n0_);                            \
    }                                                                                        \
    const u32x4 wr_ = su_rsrc(wb_ + ks_ * SU_K, (long)rows_ * ldb_ * 2 - (long)ks_ * SU_ROWB);  \
    const u32x4 ar_ = su_rsrc((p1_ ? A1 : A0) + ks_ * SU_K, (long)M0 * lda_ * 2 - (long)ks_ * SU_ROWB);  \
    const int wp_ = (int)(ldb_ * 2), ap_ = (int)(lda_ * 2);                                  \
    const unsigned st_ = lds_base + ((u_ - u0) % SU_NST) * STAGE;                            \
    _Pragma("unroll") for (int i = 0; i < W_DPW; ++i)                                        \
      su_dma16(st_ + (w * W_DPW + i) * 1024, wrow[i] * wp_ + wco[i], wr_);                  \
    _Pragma("unroll") for (int i = 0; i < A_DPW; ++i)                                        \
      su_dma16(st_ + SU_WTILE + (w * A_DPW + i) * 1024, arow[i] * ap_ + aco[i], ar_);        \
  } while (0)

  floatx16 acc0[MB], acc1[MB], acc2[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc0[mb][e] = acc1[mb][e] = acc2[mb][e] = 0.f;

  for (int u = u0; u < u1 && u < u0 + SU_NST - 1; ++u) SU_ISSUE(u);
  // operand reads: weight row 32 w + l % 32, activation row 32 mb + l % 32,
  // logical chunk 2 s + l / 32 (k-step s of 16); both rows are = l (mod 16)
  const int wrd = (32 * w + (lane & 31)) * SU_ROWB;
  const int ard = SU_WTILE + (lane & 31) * SU_ROWB;
  const int cx = lane & 15;
  for (int u = u0; u < u1; ++u) {
    const int ahead = min(SU_NST - 2, u1 - 1 - u);  // units issued after u
    if (ahead >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(DPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (u + SU_NST - 1 < u1) SU_ISSUE(u + SU_NST - 1);
    const char* st = lds + ((u - u0) % SU_NST) * STAGE;
#define SU_UNIT(ACC)                                                                          \
  _Pragma("unroll") for (int s = 0; s < SU_K / 16; ++s) {                                    \
    const int co = 16 * ((2 * s + (lane >> 5)) ^ cx);                                       \
    const bf16x8 a = *(const bf16x8*)(st + wrd + co);                                        \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                      \
      const bf16x8 b = *(const bf16x8*)(st + ard + mb * 32 * SU_ROWB + co);                  \
      ACC[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, ACC[mb], 0, 0, 0);             \
    }                                                                                        \
  }
    const int ai = gblock(u) - gb0;  // accumulator set of this unit's block
    if (ai == 0) {
      SU_UNIT(acc0)
    } else if (NP == 1 || ai == 1) {
      SU_UNIT(acc1)
    } else {
      SU_UNIT(acc2)
    }
#undef SU_UNIT
  }
#undef SU_ISSUE

  // partial block of accumulator set a: global block gb0 + a, slot su_slot of
  // its product; lane holds C[m][n0 + r] for m = 32 mb + l % 32,
  // r = 32 w + 8 i + 4 (l / 32) + jj (acc element 4 i + jj)
  const int na = u1 > u0 ? gblock(u1 - 1) - gb0 + 1 : 0;
#pragma unroll
  for (int a = 0; a < NP + 1; ++a) {
    if (a >= na) break;
    const int gb = gb0 + a;
    const int pr = NP == 1 || gb < NB0 ? 0 : 1;
    const StreamInfo& si = sp.s[pr];
    float* slot = sp.part[pr] + su_slot(si, bid, gb - (pr ? NB0 : 0)) * si.Mp * SU_N;
    const int M = sp.p[pr].M;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = 32 * mb + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const floatx16& acc = a == 0 ? acc0[mb] : (a == 1 ? acc1[mb] : acc2[mb]);
        const floatx4 v = {acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
        *(floatx4*)(slot + (long)m * SU_N + 32 * w + 8 * i + 4 * (lane >> 5)) = v;
      }
    }
  }
}

// Thread e4 of the fixed-order split sum: output row m = e4 / (N / 4),
// columns 4 (e4 % (N / 4)) .. + 3, plus the optional residual and bias.
template <typename T>
MLA_DEV void stream_reduce_body(const float* __restrict__ part, const StreamInfo& s, int M, int N,
                                T* __restrict__ out, long ldo, const bf16_t* __restrict__ R, long ldr,
                                const T* __restrict__ bias, long e4) {
  if (e4 >= (long)M * (N / 4)) return;
  const int m = (int)(e4 / (N / 4)), n = 4 * (int)(e4 % (N / 4));
  floatx4 v = stream_sum4(part, s, m, n);
  if (R) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += bf2f(R[(long)m * ldr + n + q]);
  }
  if (bias) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += to_f<T>(bias[n + q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) out[(long)m * ldo + n + q] = from_f<T>(v[q]);
}

}  // namespace mla
