// Row-wise and elementwise kernels of the MLA forward: the latent RMSNorms
// with the shared-key RoPE, the block RMSNorms, the RoPE table, cache
// scatters and split-K reductions.  All arithmetic is fp32; T is the storage
// type (float or bf16).
//
// Sources (by page title and section):
//  "Kimi K2 · Dense transformer block": equation list (RMSNorm of the block
//    input and of the residual stream, RMSNorm of the query latent, RoPE of
//    the shared rotary key with the table R of the in/out line).
//  "Kimi K2 · Key-value compression": c^KV = x W_DKV, then RMSNorm; the joint
//    projection's 576 outputs are split into the 512 latent and the 64-wide
//    rotary key after the product (Explanation); the latent plus the rotary
//    key is the 576-value cache entry.
//  "Kimi K2 · Mix and project": code excerpt, where the cache update stores
//    each head's assembled key and value.
// RMSNorm is g * x / sqrt(mean(x^2) + eps); RoPE turns the consecutive pair
// (2i, 2i+1) by t * base^(-2i/d_rope).
#include "norm_body.h"

namespace mla {

// Sum over the 256 threads of a block (4 waves); every thread gets the total.
MLA_DEV float block_sum256(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <typename T, int NT>
__global__ __launch_bounds__(NT) void latent_norm_rope_kernel(LatentNormParams<T> p) {
  extern __shared__ __attribute__((aligned(16))) float row[];  // [q_lora + kv_lora + d_rope]
  __shared__ float red[NT / 64];
  latent_norm_rope_body<T, NT>(p, blockIdx.x, blockIdx.y, gridDim.y, row, red);
}

template <typename T>
hipError_t latent_norm_rope(const LatentNormParams<T>& p, hipStream_t s) {
  size_t shm = (size_t)(p.q_lora + p.kv_lora + p.d_rope) * sizeof(float);
  if (p.stream && (p.q_lora + p.kv_lora + p.d_rope) % 4) return hipErrorInvalidValue;
  // few rows (decode): a wide workgroup keeps the partial loads of a row in
  // flight together
  // the query and kv halves of a row in workgroups of their own when the
  // split falls on a 4-column boundary
  const dim3 g(p.M, p.q_lora % 4 == 0 ? 2 : 1);
  if (p.M <= 64)
    hipLaunchKernelGGL((latent_norm_rope_kernel<T, 1024>), g, dim3(1024), shm, s, p);
  else
    hipLaunchKernelGGL((latent_norm_rope_kernel<T, 256>), g, dim3(256), shm, s, p);
  return hipGetLastError();
}
template hipError_t latent_norm_rope<float>(const LatentNormParams<float>&, hipStream_t);
template hipError_t latent_norm_rope<bf16_t>(const LatentNormParams<bf16_t>&, hipStream_t);

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* __restrict__ x, long ldx,
                                                          const T* __restrict__ g, T* __restrict__ y,
                                                          long ldy, int D, float eps) {
  extern __shared__ float rowbuf[];
  __shared__ float red[4];
  const long m = blockIdx.x;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) {
    float v = to_f<T>(x[m * ldx + c]);
    rowbuf[c] = v;
    ss += v * v;
  }
  const float tot = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)D + eps);
  for (int c = threadIdx.x; c < D; c += 256)
    y[m * ldy + c] = from_f<T>(to_f<T>(g[c]) * (rowbuf[c] * r));
}

// bf16 rows of up to 8192 features: each thread keeps its (at most four)
// 16-byte chunks of the row in registers between the sum of squares and the
// scaled store, so the row is read once with coalesced 16-byte loads.
constexpr int RMS_VEC_CH = 4;  // chunks of 8 per thread: D <= 256 * 8 * 4
__global__ __launch_bounds__(256) void rmsnorm_rows_bf16_kernel(const bf16_t* __restrict__ x, long ldx,
                                                                const bf16_t* __restrict__ g,
                                                                bf16_t* __restrict__ y, long ldy, int D,
                                                                float eps) {
  __shared__ float red[4];
  const long m = blockIdx.x;
  const int nch = D / 8;
  u32x4 v[RMS_VEC_CH];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RMS_VEC_CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      v[i] = *(const u32x4*)(x + m * ldx + 8 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = lo_bf(v[i][q]), b = hi_bf(v[i][q]);
        ss += a * a + b * b;
      }
    }
  }
  const float r = 1.0f / sqrtf(block_sum256(ss, red) / (float)D + eps);
#pragma unroll
  for (int i = 0; i < RMS_VEC_CH; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nch) {
      const u32x4 gv = *(const u32x4*)(g + 8 * c);
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack2bf(lo_bf(gv[q]) * (lo_bf(v[i][q]) * r), hi_bf(gv[q]) * (hi_bf(v[i][q]) * r));
      *(u32x4*)(y + m * ldy + 8 * c) = o;
    }
  }
}

template <typename T>
hipError_t rmsnorm_rows(const T* x, long ldx, const T* g, T* y, long ldy, int M, int D, float eps,
                        hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    const bool vec = D % 8 == 0 && D <= 256 * 8 * RMS_VEC_CH && ldx % 8 == 0 && ldy % 8 == 0 &&
                     ((uintptr_t)x | (uintptr_t)g | (uintptr_t)y) % 16 == 0;
    if (vec) {
      hipLaunchKernelGGL(rmsnorm_rows_bf16_kernel, dim3(M), dim3(256), 0, s, x, ldx, g, y, ldy, D, eps);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(rmsnorm_rows_kernel<T>, dim3(M), dim3(256), (size_t)D * sizeof(float), s, x,
                     ldx, g, y, ldy, D, eps);
  return hipGetLastError();
}
template hipError_t rmsnorm_rows<float>(const float*, long, const float*, float*, long, int, int,
                                        float, hipStream_t);
template hipError_t rmsnorm_rows<bf16_t>(const bf16_t*, long, const bf16_t*, bf16_t*, long, int,
                                         int, float, hipStream_t);

// R [n_pos, n_pairs]: angle t * base^(-2i / (2 n_pairs)), evaluated in fp64
// and stored as fp32.
__global__ void rope_table_kernel(int n_pos, int n_pairs, double base, float* cs, float* sn) {
  long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long)n_pos * n_pairs) return;
  int t = (int)(e / n_pairs), i = (int)(e % n_pairs);
  double inv_freq = pow(base, -(2.0 * i) / (2.0 * n_pairs));
  double ang = (double)t * inv_freq;
  cs[e] = (float)cos(ang);
  sn[e] = (float)sin(ang);
}

hipError_t rope_table(int n_pos, int n_pairs, double base, float* cos_out, float* sin_out,
                      hipStream_t s) {
  long n = (long)n_pos * n_pairs;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n_pos,
                     n_pairs, base, cos_out, sin_out);
  return hipGetLastError();
}

// In-place RoPE of the rotary columns of each head (fp32 path).
__global__ void rope_inplace_f32_kernel(float* x, long ldx, int M, int nheads, int head_dim,
                                        int rope_start, const float* rcos, const float* rsin,
                                        int n_pairs, int rope_T, int rope_pos0, const int* seq_pos,
                                        int pos_max) {
  const int np = (head_dim - rope_start) / 2;
  long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long)M * nheads * np) return;
  int i = (int)(e % np);
  int h = (int)((e / np) % nheads);
  long m = e / ((long)np * nheads);
  const int pos = seq_pos ? seq_position(seq_pos, (int)(m / rope_T), 0, pos_max)
                          : (int)(m % rope_T) + rope_pos0;
  float* v = x + m * ldx + (long)h * head_dim + rope_start + 2 * i;
  float c = rcos[(long)pos * n_pairs + i], s = rsin[(long)pos * n_pairs + i];
  float a = v[0], b = v[1];
  v[0] = a * c - b * s;
  v[1] = a * s + b * c;
}

hipError_t rope_inplace_f32(float* x, long ldx, int M, int ncols, int head_dim, int rope_start,
                            const float* rcos, const float* rsin, int n_pairs, int rope_T,
                            int rope_pos0, hipStream_t s, const int* seq_pos, int pos_max) {
  int nheads = ncols / head_dim;
  long n = (long)M * nheads * ((head_dim - rope_start) / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_inplace_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     x, ldx, M, nheads, head_dim, rope_start, rcos, rsin, n_pairs, rope_T,
                     rope_pos0, seq_pos, pos_max);
  return hipGetLastError();
}

__global__ void swiglu_f32_kernel(const float* g, const float* u, float* h, long n) {
  long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float gv = g[e];
  h[e] = gv / (1.f + expf(-gv)) * u[e];
}

hipError_t swiglu_f32(const float* g, const float* u, float* h, long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, u,
                     h, n);
  return hipGetLastError();
}

template <typename T>
__global__ void scatter_full_cache_kernel(const T* __restrict__ kv, const T* __restrict__ kr,
                                          T* __restrict__ kc, T* __restrict__ vc, int T_, int pos0,
                                          int L_cap, int H, int dn, int dr, int dv, long total,
                                          const int* __restrict__ seq_pos, int pos_max) {
  long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int W = dn + dr + dv;
  int c = (int)(e % W);
  int h = (int)((e / W) % H);
  long m = e / ((long)W * H);
  long b = m / T_;
  const int slot = seq_pos ? seq_position(seq_pos, (int)b, 0, pos_max) : (int)(m % T_) + pos0;
  long base = ((b * H + h) * L_cap + slot);
  const T* src = kv + (m * H + h) * (dn + dv);
  if (c < dn) kc[base * (dn + dr) + c] = src[c];
  else if (c < dn + dr) kc[base * (dn + dr) + c] = kr[m * dr + (c - dn)];
  else vc[base * dv + (c - dn - dr)] = src[dn + (c - dn - dr)];
}

// bf16 form: one 16-byte chunk (8 features) per thread; chunk c of (row m,
// head h) is K^C (c < dn/8), k^R (next dr/8) or V (last dv/8).  Grid: x =
// token row m (its sequence and slot are uniform per workgroup), y covers
// the H * (dn + dr + dv) / 8 chunks of the row in blocks of 256, so the
// per-thread index arithmetic is 32-bit.
__global__ void scatter_full_cache_bf16x8_kernel(const bf16_t* __restrict__ kv,
                                                 const bf16_t* __restrict__ kr, bf16_t* __restrict__ kc,
                                                 bf16_t* __restrict__ vc, int T_, int pos0, int L_cap,
                                                 int H, int dn, int dr, int dv,
                                                 const int* __restrict__ seq_pos, int pos_max) {
  const int W8 = (dn + dr + dv) / 8;
  const int e = blockIdx.y * blockDim.x + threadIdx.x;  // chunk within the row: (h, c)
  if (e >= H * W8) return;
  const long m = blockIdx.x;
  const int b = (int)(blockIdx.x / (unsigned)T_);
  const int slot = seq_pos ? seq_position(seq_pos, b, 0, pos_max) : (int)(blockIdx.x - (unsigned)b * T_) + pos0;
  const int h = e / W8, c = e - h * W8;
  const long base = ((long)b * H + h) * L_cap + slot;
  const bf16_t* src = kv + (m * H + h) * (dn + dv);
  const int f = 8 * c;
  if (f < dn) *(u32x4*)(kc + base * (dn + dr) + f) = *(const u32x4*)(src + f);
  else if (f < dn + dr) *(u32x4*)(kc + base * (dn + dr) + f) = *(const u32x4*)(kr + m * dr + (f - dn));
  else *(u32x4*)(vc + base * dv + (f - dn - dr)) = *(const u32x4*)(src + dn + (f - dn - dr));
}

template <typename T>
hipError_t scatter_full_cache(const T* kv, const T* kr, T* k_cache, T* v_cache, int Bn, int T_,
                              int pos0, int L_cap, int H, int d_nope, int d_rope, int d_v,
                              hipStream_t s, const int* seq_pos, int pos_max) {
  if constexpr (sizeof(T) == 2) {
    const bool vec = d_nope % 8 == 0 && d_rope % 8 == 0 && d_v % 8 == 0 &&
                     ((uintptr_t)kv | (uintptr_t)kr | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16 == 0;
    const long rows = (long)Bn * T_;
    const long row8 = (long)H * ((d_nope + d_rope + d_v) / 8);  // chunks per token row
    if (vec && rows <= 0x7fffffffL && row8 <= 65535L * 256) {
      if (rows == 0 || row8 == 0) return hipSuccess;
      hipLaunchKernelGGL(scatter_full_cache_bf16x8_kernel, dim3((unsigned)rows, (unsigned)((row8 + 255) / 256)),
                         dim3(256), 0, s, (const bf16_t*)kv, (const bf16_t*)kr, (bf16_t*)k_cache,
                         (bf16_t*)v_cache, T_, pos0, L_cap, H, d_nope, d_rope, d_v, seq_pos, pos_max);
      return hipGetLastError();
    }
  }
  long total = (long)Bn * T_ * H * (d_nope + d_rope + d_v);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_full_cache_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, s, kv, kr, k_cache, v_cache, T_, pos0, L_cap, H, d_nope, d_rope, d_v, total,
                     seq_pos, pos_max);
  return hipGetLastError();
}
template hipError_t scatter_full_cache<float>(const float*, const float*, float*, float*, int, int,
                                              int, int, int, int, int, int, hipStream_t, const int*,
                                              int);
template hipError_t scatter_full_cache<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, bf16_t*, int,
                                               int, int, int, int, int, int, int, hipStream_t,
                                               const int*, int);

template <typename T>
__global__ void reduce_splits_kernel(const float* __restrict__ part, int nsplit, long stride, int M,
                                     int N, T* __restrict__ out, long ldo, const T* __restrict__ bias) {
  // 4 consecutive columns per thread (N % 4 == 0 checked by the launcher)
  long e4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e4 >= (long)M * N / 4) return;
  const long e = 4 * e4;
  const long m = e / N;
  const int n = (int)(e % N);
  const floatx4 v = sum_splits4(part + e, stride, nsplit);
#pragma unroll
  for (int q = 0; q < 4; ++q) out[m * ldo + n + q] = from_f<T>(v[q] + (bias ? to_f<T>(bias[n + q]) : 0.f));
}

template <typename T>
hipError_t reduce_splits(const float* part, int nsplit, long split_stride, int M, int N, T* out,
                         long ldo, hipStream_t s, const T* bias) {
  long n = (long)M * N / 4;
  if (n == 0) return hipSuccess;
  if (N % 4 || split_stride % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reduce_splits_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     part, nsplit, split_stride, M, N, out, ldo, bias);
  return hipGetLastError();
}
template hipError_t reduce_splits<float>(const float*, int, long, int, int, float*, long,
                                         hipStream_t, const float*);
template hipError_t reduce_splits<bf16_t>(const float*, int, long, int, int, bf16_t*, long,
                                          hipStream_t, const bf16_t*);

// ---------------------------------------------------------------------------
// Streaming-read yardstick: workgroup g reads the g-th of gridDim.x equal
// contiguous ranges of a buffer in 16-byte chunks, sixteen loads in flight per
// thread, and folds the values with XOR so the loads stay live; one word per
// workgroup goes to `sink`.  It measures the HBM read rate this chip reaches
// with plain vector loads, the second denominator next to the nominal 8 TB/s.
// (A probe of the forms: contiguous ranges with 16 loads in flight read 1 GiB
// at 6.2-6.3 TB/s from 2048 workgroups up; grid-stride loops over the whole
// buffer reached 4.8-6.2 TB/s.)
__global__ __launch_bounds__(256) void read_sweep_kernel(const u32x4* __restrict__ p, long n16,
                                                         unsigned* __restrict__ sink) {
  constexpr int U = 16;
  const long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long b0 = (long)blockIdx.x * per, b1 = min(b0 + per, n16);
  long i = b0 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < b1; i += 256) acc ^= p[i];
  const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ unsigned red[4];
  const unsigned w = __reduce_xor_sync(~0ull, x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t read_sweep(const void* buf, size_t bytes, unsigned* sink, int nwg, hipStream_t s) {
  hipLaunchKernelGGL(read_sweep_kernel, dim3(nwg), dim3(256), 0, s, (const u32x4*)buf, (long)(bytes / 16),
                     sink);
  return hipGetLastError();
}

}  // namespace mla
