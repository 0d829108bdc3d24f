// Weight-streaming bf16 GEMM for decode-sized products (M <= 64 rows):
// C[M,N] = A[M,K] . B[N,K]^T.
//
// In a decode step every projection multiplies a handful of token rows by a
// full weight matrix, so the time is the weight stream from HBM.  Each
// workgroup owns 128 output columns (32 per wave) and one 512-wide K slice:
// the activation slice [M, 512] is staged once in LDS, and each wave issues
// all 32 of its 16-byte weight loads (its columns' K slice, already in the
// MFMA B-operand layout of v_mfma_f32_32x32x16_bf16) before the first MFMA,
// which keeps ~128 KB per workgroup in flight.  Slices write fp32 partials
// that a fixed-order reduction sums (deterministic); a single slice writes
// bf16 directly.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {
constexpr int SK_KS = 512;             // K slice per workgroup
constexpr int SK_CH = SK_KS / 8;       // 16-byte chunks per activation row
MLA_DEV int sk_swz(int r) { return r & 15; }  // 1 KB rows: spread 16 rows over the 64 banks
}  // namespace

template <int MB, bool BF16OUT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p) {
  __shared__ u32x4 As[MB * 32 * SK_CH];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int n0 = blockIdx.x * 128 + w * 32;
  const int bidx = blockIdx.z;
  const int split = blockIdx.y;
  const int k0 = split * p.kchunk;
  const int nsteps = min(p.K - k0, SK_KS) / 16;
  const bf16_t* __restrict__ A = p.A + (long)bidx * p.sA;

  // activation slice [M, 512] first (into registers; stored to LDS below),
  // then this wave's weight rows: 32 columns x the K slice, issued back to
  // back so the whole slice is in flight at once.  Loads retire in order, so
  // the LDS stores of the activations wait for those loads only.
  constexpr int A_PER = MB * 32 * SK_CH / 256;
  u32x4 av[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int e = tid + 256 * i, r = e / SK_CH, c = e % SK_CH;
    const int gr = min(r, p.M - 1);
    const int cc = min(c, 2 * nsteps - 1);  // past the slice end: reload a valid chunk, unused
    av[i] = *(const u32x4*)(A + (long)gr * p.lda + k0 + 8 * cc);
  }
  const int col = min(n0 + lr, p.N - 1);
  const bf16_t* brow = (p.b_split > 0 && col >= p.b_split)
                           ? p.B2 + (long)(col - p.b_split) * p.ldb
                           : p.B + (long)bidx * p.sB + (long)col * p.ldb;
  brow += k0 + 8 * lg;
  u32x4 bv[SK_KS / 16];
#pragma unroll
  for (int s = 0; s < SK_KS / 16; ++s) bv[s] = *(const u32x4*)(brow + 16 * min(s, nsteps - 1));
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int e = tid + 256 * i, r = e / SK_CH, c = e % SK_CH;
    As[r * SK_CH + (c ^ sk_swz(r))] = av[i];
  }
  __syncthreads();

  floatx16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;
#pragma unroll
  for (int s = 0; s < SK_KS / 16; ++s) {
    if (s < nsteps) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = 32 * mb + lr;
        const bf16x8 a = __builtin_bit_cast(bf16x8, As[r * SK_CH + ((2 * s + lg) ^ sk_swz(r))]);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bv[s]),
                                                           acc[mb], 0, 0, 0);
      }
    }
  }
  const int c = n0 + lr;
  if (c >= p.N) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 32 * mb + 8 * (e >> 2) + 4 * lg + (e & 3);
      if (row >= p.M) continue;
      if (BF16OUT) {
        bf16_t* C = (bf16_t*)p.C + (long)bidx * p.sC;
        C[(long)row * p.ldc + c] = f2bf(acc[mb][e] + (p.bias ? bf2f(p.bias[c]) : 0.f));
      } else {
        float* C = (float*)p.C + (long)bidx * p.sC + (long)split * p.split_stride;
        C[(long)row * p.ldc + c] = acc[mb][e];
      }
    }
}

int skinny_splits(int K) { return (K + SK_KS - 1) / SK_KS; }

// p.M <= 64, p.K % 64 == 0.  With more than one K slice (K > 512) the output
// is fp32 partials [slices][M][ldc] (p.split_stride apart); otherwise bf16
// when bf16_out is set.
hipError_t gemm_skinny_bf16(GemmParams p, bool bf16_out, hipStream_t s) {
  if (p.M > 64 || p.M <= 0 || p.K % 64) return hipErrorInvalidValue;
  if (p.batch <= 0) p.batch = 1;
  const int S = skinny_splits(p.K);
  if (S > 1 && bf16_out) return hipErrorInvalidValue;
  p.kchunk = SK_KS;
  p.ksplit = S;
  dim3 grid((p.N + 127) / 128, S, p.batch);
  if (p.M <= 32) {
    if (bf16_out) hipLaunchKernelGGL((gemm_skinny_kernel<1, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_skinny_kernel<1, false>), grid, dim3(256), 0, s, p);
  } else {
    if (bf16_out) hipLaunchKernelGGL((gemm_skinny_kernel<2, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((gemm_skinny_kernel<2, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
