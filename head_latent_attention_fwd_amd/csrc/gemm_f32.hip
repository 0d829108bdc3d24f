// fp32 GEMM for the float32 path (any M, N, K): C = R + A . op(B) (+ bias).
//
// The float32 configuration is the parity-precision form of the method
// (the tiny MLA workload and arbitrary head widths); it is small, so a plain
// LDS-tiled FMA kernel with bounds checks everywhere is enough.  op(B) = B^T
// for nn.Linear weights stored [N, K]; op(B) = B for [K, N] operands (the
// query absorption multiplies by W_UK along its rows).
#include "common.h"
#include "kernels.h"

namespace mla {

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Params p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const long b = blockIdx.z;
  const float* A = p.A + b * p.sA;
  const float* Bm = p.B + b * p.sB;
  float* C = p.C + b * p.sC;
  const float* R = p.R ? p.R + b * p.sC : nullptr;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += BK) {
    for (int e = tid; e < BM * BK; e += 256) {
      int r = e / BK, k = e % BK;
      int gm = m0 + r, gk = k0 + k;
      As[k][r] = (gm < p.M && gk < p.K) ? A[(long)gm * p.lda + gk] : 0.f;
    }
    for (int e = tid; e < BN * BK; e += 256) {
      int n, k;
      if (p.b_is_nk) { n = e / BK; k = e % BK; } else { k = e / BN; n = e % BN; }
      int gn = n0 + n, gk = k0 + k;
      float v = 0.f;
      if (gn < p.N && gk < p.K)
        v = p.b_is_nk ? Bm[(long)gn * p.ldb + gk] : Bm[(long)gk * p.ldb + gn];
      Bs[k][n] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int gm = m0 + ty * 4 + i, gn = n0 + tx * 4 + j;
      if (gm < p.M && gn < p.N) {
        float v = acc[i][j];
        if (R) v += R[(long)gm * p.ldr + gn];
        if (p.bias) v += p.bias[gn];
        C[(long)gm * p.ldc + gn] = v;
      }
    }
}

hipError_t gemm_f32(const GemmF32Params& p, hipStream_t s) {
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64, p.batch > 0 ? p.batch : 1);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
