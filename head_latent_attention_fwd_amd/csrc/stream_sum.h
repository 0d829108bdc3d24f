// Partial-block bookkeeping of the balanced weight-streaming GEMM
// (gemm_stream.hip), shared with the kernels that consume its partials.
#pragma once
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int SU_N = 128;  // weight rows (output columns) per unit
constexpr int SU_K = 128;  // k per unit

// first unit of workgroup w: units are dealt out as equal contiguous runs
// (w U < 2^31: U is at most a few hundred thousand units)
MLA_DEV inline int su_start(const StreamInfo& s, int w) { return w * s.U / s.G; }

// Workgroups [wa, wb] hold the units of this product's 128-column block nb.
MLA_DEV inline void su_span(const StreamInfo& s, int nb, int& wa, int& wb) {
  const int ua = s.u0 + nb * s.KS, ub = ua + s.KS - 1;
  wa = ((ua + 1) * s.G - 1) / s.U;  // workgroup holding unit ua
  wb = ((ub + 1) * s.G - 1) / s.U;  // ... and unit ub
}

// Partial slot of workgroup w's part of block nb: its blocks of this
// product are numbered from the one holding its first unit of the product
// (w holds units of nb, so that one is nb, nb - 1 or nb - 2).
MLA_DEV inline long su_slot(const StreamInfo& s, int w, int nb) {
  const int f = max(su_start(s, w), s.u0);
  const int ua = s.u0 + nb * s.KS;
  const int j = f >= ua ? 0 : (f >= ua - s.KS ? 1 : 2);
  return (long)(w - s.w0) * s.NS + j;
}

// Sum of C[m][n .. n+3] over the partial slots of n's 128-column block, in
// workgroup order (deterministic).  Slot (w, j) is workgroup w's j-th block
// ([Mp][128] fp32).  Loads are issued 8 slots at a time.
MLA_DEV inline floatx4 stream_sum4(const float* __restrict__ part, const StreamInfo& s, int m, int n) {
  const int nb = n / SU_N, nl = n - nb * SU_N;
  int wa, wb;
  su_span(s, nb, wa, wb);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int w0 = wa; w0 <= wb; w0 += 8) {
    floatx4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int w = w0 + q;
      if (w <= wb) {
        v[q] = *(const floatx4*)(part + (su_slot(s, w, nb) * s.Mp + m) * SU_N + nl);
      } else {
        v[q] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += v[q];
  }
  return acc;
}

// R rows m[r] (ok[r] false: skipped, result zero) of the 8 columns n .. n+7
// (n % 8 == 0, so one 128-column block), summed over the block's partial
// slots in workgroup order like stream_sum4; the loads of 4 slots x R rows
// are issued together.
template <int R>
MLA_DEV inline void stream_sum8_rows(const float* __restrict__ part, const StreamInfo& s, const int (&m)[R],
                                     const bool (&ok)[R], int n, floatx4 (&out)[R][2]) {
  const int nb = n / SU_N, nl = n - nb * SU_N;
  int wa, wb;
  su_span(s, nb, wa, wb);
#pragma unroll
  for (int r = 0; r < R; ++r) out[r][0] = out[r][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int w0 = wa; w0 <= wb; w0 += 4) {
    floatx4 v[4][R][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = w0 + q;
      const float* base = part + (w <= wb ? su_slot(s, w, nb) : 0) * s.Mp * SU_N + nl;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool go = w <= wb && ok[r];
        v[q][r][0] = go ? *(const floatx4*)(base + (long)m[r] * SU_N) : floatx4{0.f, 0.f, 0.f, 0.f};
        v[q][r][1] = go ? *(const floatx4*)(base + (long)m[r] * SU_N + 4) : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        out[r][0] += v[q][r][0];
        out[r][1] += v[q][r][1];
      }
  }
}

}  // namespace mla
