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

template <int MB, int NP>
__global__ __launch_bounds__(256) void gemm_stream_kernel(StreamPair sp) {
  constexpr int MP = 32 * MB;
  constexpr int ATILE = MP * SU_ROWB;
  constexpr int STAGE = SU_WTILE + ATILE;
  constexpr int W_DPW = SU_WTILE / 1024 / 4;   // weight DMAs per wave per unit (8)
  constexpr int A_DPW = ATILE / 1024 / 4;      // activation DMAs per wave per unit (MB * 2)
  constexpr int DPW = W_DPW + A_DPW;
  __shared__ __attribute__((aligned(16))) char lds[SU_NST * STAGE];
  const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const StreamInfo& s0 = sp.s[0];
  const int u0 = su_start(s0, blockIdx.x), u1 = su_start(s0, blockIdx.x + 1);
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
    float* slot = sp.part[pr] + su_slot(si, blockIdx.x, gb - (pr ? NB0 : 0)) * si.Mp * SU_N;
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

template <typename T>
__global__ __launch_bounds__(256) void stream_reduce_kernel(const float* __restrict__ part, StreamInfo s,
                                                            int M, int N, T* __restrict__ out, long ldo,
                                                            const bf16_t* __restrict__ R, long ldr,
                                                            const T* __restrict__ bias) {
  const long e4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
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

bool stream_ok(const GemmParams& p) {
  const long nb = (p.N + SU_N - 1) / SU_N, units = nb * (p.K / SU_K);
  return p.M >= 1 && p.M <= 64 && p.K % SU_K == 0 && p.N % 4 == 0 && p.batch <= 1 &&
         (p.b_split <= 0 || p.b_split % SU_N == 0) && (long)p.ldb * 2 * SU_N < 0x7fffffffL &&
         (long)p.lda * 2 * 64 < 0x7fffffffL &&
         units * (nb > 256 ? nb : 256) < 0x7fffffffL;  // unit arithmetic stays in 32 bits
}

StreamInfo stream_info(int M, int N, int K) {
  StreamInfo s;
  s.KS = K / SU_K;
  s.NB = (N + SU_N - 1) / SU_N;
  s.U = s.NB * s.KS;
  s.G = s.NB > 256 ? s.NB : 256;
  if (s.G > s.U) s.G = s.U;
  s.Mp = M <= 32 ? 32 : 64;
  s.u0 = 0;
  s.w0 = 0;
  s.NS = 2;  // a run shorter than a block's KS units touches at most two
  return s;
}

// slots of the workgroups holding this product's units
size_t stream_part_floats(const StreamInfo& s) {
  const int ub = s.u0 + s.NB * s.KS - 1;  // this product's last unit
  const int wb = ((ub + 1) * s.G - 1) / s.U;
  return (size_t)(wb - s.w0 + 1) * s.NS * s.Mp * SU_N;
}

static hipError_t launch_stream(const StreamPair& sp, hipStream_t st) {
  const dim3 g(sp.s[0].G);
  if (sp.n == 1) {
    if (sp.s[0].Mp == 32) hipLaunchKernelGGL((gemm_stream_kernel<1, 1>), g, dim3(256), 0, st, sp);
    else hipLaunchKernelGGL((gemm_stream_kernel<2, 1>), g, dim3(256), 0, st, sp);
  } else {
    if (sp.s[0].Mp == 32) hipLaunchKernelGGL((gemm_stream_kernel<1, 2>), g, dim3(256), 0, st, sp);
    else hipLaunchKernelGGL((gemm_stream_kernel<2, 2>), g, dim3(256), 0, st, sp);
  }
  return hipGetLastError();
}

hipError_t gemm_stream_bf16(const GemmParams& p, float* part, const StreamInfo& s, hipStream_t st) {
  if (!stream_ok(p) || s.u0 != 0 || s.U != s.NB * s.KS) return hipErrorInvalidValue;
  StreamPair sp;
  sp.p[0] = sp.p[1] = p;
  sp.s[0] = sp.s[1] = s;
  sp.part[0] = sp.part[1] = part;
  sp.n = 1;
  return launch_stream(sp, st);
}

bool stream_pair_info(const GemmParams& a, const GemmParams& b, StreamInfo* sa, StreamInfo* sb) {
  if (!stream_ok(a) || !stream_ok(b) || a.M != b.M || b.b_split > 0) return false;
  StreamInfo x = stream_info(a.M, a.N, a.K), y = stream_info(b.M, b.N, b.K);
  const int U = x.U + y.U;
  const int G = 256 < U ? 256 : U;
  if ((long)U * G >= 0x7fffffffL) return false;
  // blocks per workgroup: at most three (three accumulator sets)
  for (int w = 0; w < G; ++w) {
    const int u0 = (int)((long)w * U / G), u1 = (int)((long)(w + 1) * U / G);
    if (u1 <= u0) return false;
    auto gb = [&](int u) { return u < x.U ? u / x.KS : x.NB + (u - x.U) / y.KS; };
    if (gb(u1 - 1) - gb(u0) + 1 > 3) return false;
  }
  x.G = y.G = G;
  x.U = y.U = U;
  x.u0 = 0;
  y.u0 = x.NB * x.KS;
  x.w0 = 0;
  y.w0 = ((y.u0 + 1) * G - 1) / U;
  x.NS = y.NS = 3;
  *sa = x;
  *sb = y;
  return true;
}

hipError_t gemm_stream_bf16_pair(const GemmParams& a, const GemmParams& b, float* part_a, float* part_b,
                                 const StreamInfo& sa, const StreamInfo& sb, hipStream_t st) {
  if (sa.U != sb.U || sa.G != sb.G || sa.Mp != sb.Mp || sb.u0 != sa.NB * sa.KS) return hipErrorInvalidValue;
  StreamPair sp;
  sp.p[0] = a;
  sp.p[1] = b;
  sp.s[0] = sa;
  sp.s[1] = sb;
  sp.part[0] = part_a;
  sp.part[1] = part_b;
  sp.n = 2;
  return launch_stream(sp, st);
}

template <typename T>
hipError_t stream_reduce(const float* part, const StreamInfo& s, int M, int N, T* out, long ldo,
                         const bf16_t* R, long ldr, hipStream_t st, const T* bias) {
  const long n = (long)M * (N / 4);
  if (n == 0) return hipSuccess;
  if (N % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_reduce_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     s, M, N, out, ldo, R, ldr, bias);
  return hipGetLastError();
}
template hipError_t stream_reduce<float>(const float*, const StreamInfo&, int, int, float*, long,
                                         const bf16_t*, long, hipStream_t, const float*);
template hipError_t stream_reduce<bf16_t>(const float*, const StreamInfo&, int, int, bf16_t*, long,
                                          const bf16_t*, long, hipStream_t, const bf16_t*);

}  // namespace mla
