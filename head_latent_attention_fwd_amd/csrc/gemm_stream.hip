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

template <int MB>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmParams p, StreamInfo si, float* part) {
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
  const int u0 = su_start(si, blockIdx.x), u1 = su_start(si, blockIdx.x + 1);
  const int nb0 = u0 / si.KS;

  // Tiles hold rows of 256 B (16 chunks of 16 B); chunk c of row r sits at
  // chunk position c ^ (r & 15), so the 16 rows of a half-wave operand read
  // (same logical chunk) hit 16 different bank groups (unswizzled, all of
  // them would share one: measured 16-way conflicts).  DMA i of this wave
  // fills tile rows 4 i .. 4 i + 3: lane l -> row 4 i + l / 16, chunk position
  // l % 16, i.e. logical chunk (l % 16) ^ (row & 15).
  int wv[W_DPW], av[A_DPW];
#pragma unroll
  for (int i = 0; i < W_DPW; ++i) {
    const int row = 4 * (w * W_DPW + i) + (lane >> 4);
    wv[i] = row * (int)(p.ldb * 2) + 16 * ((lane & 15) ^ (row & 15));
  }
#pragma unroll
  for (int i = 0; i < A_DPW; ++i) {
    const int row = 4 * (w * A_DPW + i) + (lane >> 4);
    av[i] = row * (int)(p.lda * 2) + 16 * ((lane & 15) ^ (row & 15));
  }

#define SU_ISSUE(uu)                                                                         \
  do {                                                                                       \
    const int u_ = (uu), nb_ = u_ / si.KS, ks_ = u_ - nb_ * si.KS;                          \
    const int n0_ = nb_ * SU_N;                                                              \
    const bf16_t* wb_;                                                                       \
    int rows_;                                                                               \
    if (p.b_split > 0 && n0_ >= p.b_split) {                                                 \
      wb_ = p.B2 + (long)(n0_ - p.b_split) * p.ldb;                                          \
      rows_ = min(SU_N, p.N - n0_);                                                          \
    } else {                                                                                 \
      wb_ = p.B + (long)n0_ * p.ldb;                                                         \
      rows_ = min(SU_N, (p.b_split > 0 ? p.b_split : p.N) - n0_);                            \
    }                                                                                        \
    const u32x4 wr_ = su_rsrc(wb_ + ks_ * SU_K, (long)rows_ * p.ldb * 2 - (long)ks_ * SU_ROWB);  \
    const u32x4 ar_ = su_rsrc(p.A + ks_ * SU_K, (long)p.M * p.lda * 2 - (long)ks_ * SU_ROWB);    \
    const unsigned st_ = lds_base + ((u_ - u0) % SU_NST) * STAGE;                            \
    _Pragma("unroll") for (int i = 0; i < W_DPW; ++i)                                        \
      su_dma16(st_ + (w * W_DPW + i) * 1024, wv[i], wr_);                                    \
    _Pragma("unroll") for (int i = 0; i < A_DPW; ++i)                                        \
      su_dma16(st_ + SU_WTILE + (w * A_DPW + i) * 1024, av[i], ar_);                         \
  } while (0)

  floatx16 acc0[MB], acc1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc0[mb][e] = acc1[mb][e] = 0.f;

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
    if (u / si.KS != nb0) {
      SU_UNIT(acc1)
    } else {
      SU_UNIT(acc0)
    }
#undef SU_UNIT
  }
#undef SU_ISSUE

  // partial slot (workgroup, j) = [Mp][128] fp32; lane holds C[m][n0 + r] for
  // m = 32 mb + l % 32, r = 32 w + 8 i + 4 (l / 32) + jj (acc element 4 i + jj)
  const int nb1 = (u1 - 1) / si.KS;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j == 1 && nb1 == nb0) break;
    float* slot = part + (long)(2 * blockIdx.x + j) * si.Mp * SU_N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = 32 * mb + (lane & 31);
      if (m >= p.M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const floatx16& a = j ? acc1[mb] : acc0[mb];
        const floatx4 v = {a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
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
  return p.M >= 1 && p.M <= 64 && p.K % SU_K == 0 && p.N % 4 == 0 && p.batch <= 1 &&
         (p.b_split <= 0 || p.b_split % SU_N == 0) && (long)p.ldb * 2 * SU_N < 0x7fffffffL &&
         (long)p.lda * 2 * 64 < 0x7fffffffL;
}

StreamInfo stream_info(int M, int N, int K) {
  StreamInfo s;
  s.KS = K / SU_K;
  s.NB = (N + SU_N - 1) / SU_N;
  s.U = s.NB * s.KS;
  s.G = s.NB > 256 ? s.NB : 256;
  if (s.G > s.U) s.G = s.U;
  s.Mp = M <= 32 ? 32 : 64;
  return s;
}

size_t stream_part_floats(const StreamInfo& s) { return (size_t)s.G * 2 * s.Mp * SU_N; }

hipError_t gemm_stream_bf16(const GemmParams& p, float* part, const StreamInfo& s, hipStream_t st) {
  if (!stream_ok(p)) return hipErrorInvalidValue;
  if (s.Mp == 32)
    hipLaunchKernelGGL((gemm_stream_kernel<1>), dim3(s.G), dim3(256), 0, st, p, s, part);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<2>), dim3(s.G), dim3(256), 0, st, p, s, part);
  return hipGetLastError();
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
