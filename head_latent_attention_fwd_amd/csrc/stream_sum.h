// Partial-block bookkeeping of the balanced weight-streaming GEMM
// (gemm_stream.hip), shared with the kernels that consume its partials.
#pragma once
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int SU_N = 128;  // weight rows (output columns) per unit
constexpr int SU_K = 128;  // k per unit

// first unit of workgroup w: units are dealt out as equal contiguous runs
MLA_DEV inline int su_start(const StreamInfo& s, int w) { return (int)(((long)w * s.U) / s.G); }

// Sum of C[m][n .. n+3] over the partial slots of n's 128-column block, in
// workgroup order (deterministic).  Slot (w, j) is workgroup w's j-th block
// ([Mp][128] fp32).  Loads are issued 8 slots at a time.
MLA_DEV inline floatx4 stream_sum4(const float* __restrict__ part, const StreamInfo& s, int m, int n) {
  const int nb = n / SU_N, nl = n - nb * SU_N;
  const int ua = nb * s.KS, ub = ua + s.KS - 1;
  const int wa = (int)(((long)(ua + 1) * s.G - 1) / s.U);  // workgroup holding unit ua
  const int wb = (int)(((long)(ub + 1) * s.G - 1) / s.U);  // ... and unit ub
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w0 = wa; w0 <= wb; w0 += 8) {
    floatx4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int w = w0 + q;
      if (w <= wb) {
        const int j = su_start(s, w) / s.KS == nb ? 0 : 1;
        v[q] = *(const floatx4*)(part + ((long)(2 * w + j) * s.Mp + m) * SU_N + nl);
      } else {
        v[q] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += v[q];
  }
  return acc;
}

}  // namespace mla
