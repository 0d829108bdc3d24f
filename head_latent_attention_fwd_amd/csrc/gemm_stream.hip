// Weight-streaming bf16 GEMM for decode-sized products (M <= 64 rows) and
// its fixed-order split sum: the kernels and their host launchers.  The
// device bodies, and the design, are in stream_body.h.
#include "stream_body.h"

namespace mla {

template <int MB, int NP>
__global__ __launch_bounds__(256) void gemm_stream_kernel(StreamPair sp) {
  __shared__ __attribute__((aligned(16))) char lds[stream_lds_bytes<MB>()];
  gemm_stream_body<MB, NP>(sp, blockIdx.x, lds);
}

template <typename T>
__global__ __launch_bounds__(256) void stream_reduce_kernel(const float* __restrict__ part, StreamInfo s,
                                                            int M, int N, T* __restrict__ out, long ldo,
                                                            const bf16_t* __restrict__ R, long ldr,
                                                            const T* __restrict__ bias) {
  stream_reduce_body<T>(part, s, M, N, out, ldo, R, ldr, bias, (long)blockIdx.x * blockDim.x + threadIdx.x);
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
