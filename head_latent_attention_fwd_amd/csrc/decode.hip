// Decode-step attention kernels (one query per sequence), bf16, gfx950.
//
// Sources: "Kimi K2 · Mix and project" (decode mode: one query per sequence
// reads L = P + 1 keys of the cache, per-head values of 128 features; the
// code excerpt's scaled scores, float32 softmax and P.V) and "Kimi K2 ·
// Key-value compression" (the full cache holds 20,480 values per position,
// 192-feature keys and 128-feature values for each of 64 heads; the latent
// cache would hold 576: the 512 normalised latent plus the 64 rotary-key
// features).
//
//  decode_full    : streams each (sequence, head)'s K [L,192] and V [L,128]
//                   with coalesced 16-byte loads; fp32 VALU dot products,
//                   scores kept in LDS, exact two-pass
//                   softmax per key range, split-L partials merged by a
//                   combine kernel when one (sequence, head) is spread over
//                   several workgroups.
//  decode_latent  : absorbed form.  All 64 heads share one [L, 576] latent
//                   stream, so the heads become the MFMA N dimension:
//                   S^T = C . Q~^T (v_mfma_f32_16x16x32_bf16, 16 heads per
//                   wave), then o~^T = C^T . P^T with C^T staged transposed in
//                   LDS.  Split-L partials (m, l, o~) per head are merged by
//                   latent_combine.
//  absorb_q       : q~_h = Q^C_h . W_UK,h (W_UK folded into the query), an
//                   MFMA product whose weight operand is transposed into LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

// ------------------------------------------------------------------------
// full-cache decode
// ------------------------------------------------------------------------
constexpr int DF_CHUNK_MAX = 4096;  // keys per workgroup (scores live in LDS)

// 8-term dot product of an fp32 query slice with 8 packed bf16 key values.
MLA_DEV float dot8(const float* q, u32x4 k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(q[2 * i], lo_bf(k[i]), acc);
    acc = fmaf(q[2 * i + 1], hi_bf(k[i]), acc);
  }
  return acc;
}

__global__ __launch_bounds__(256) void decode_full_kernel(DecodeFullParams p) {
  __shared__ float sc[DF_CHUNK_MAX];
  __shared__ float ob[16][129];
  __shared__ float red[8];
  const int tid = threadIdx.x;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int j0 = split * p.chunk;
  const int j1 = min(p.L, j0 + p.chunk);
  const int n = j1 - j0;
  const bf16_t* K = p.k_cache + (long)bh * p.L_cap * 192;
  const bf16_t* V = p.v_cache + (long)bh * p.L_cap * 128;

  // phase 1: scores.  8 lanes per key; lane g8 holds query chunks g8, g8+8, g8+16
  const int g8 = tid & 7, grp = tid >> 3;
  const bf16_t* qp = p.q + (long)bh * 192;
  float qf[24];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    u32x4 v = *(const u32x4*)(qp + 64 * c + 8 * g8);
    // chunk 2 holds rotary features 8*g8 .. +8: rotate by the token's position
    if (c == 2) v = rope8_bf16(v, p.rcos, p.rsin, p.L - 1, 32, 4 * g8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[8 * c + 2 * i] = lo_bf(v[i]);
      qf[8 * c + 2 * i + 1] = hi_bf(v[i]);
    }
  }
  for (int jb = j0 + grp; jb < j1; jb += 128) {
    float part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(jb + 32 * u, j1 - 1);
      const bf16_t* kp = K + (long)j * 192 + 8 * g8;
      const u32x4 k0 = *(const u32x4*)kp;
      const u32x4 k1 = *(const u32x4*)(kp + 64);
      const u32x4 k2 = *(const u32x4*)(kp + 128);
      part[u] = dot8(qf + 16, k2, dot8(qf + 8, k1, dot8(qf, k0, 0.f)));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v = part[u];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int j = jb + 32 * u;
      if (g8 == 0 && j < j1) sc[j - j0] = v * p.scale_log2;
    }
  }
  __syncthreads();

  // phase 2: max and exp2 in place, sum
  float mx = -INFINITY;
  for (int i = tid; i < n; i += 256) mx = fmaxf(mx, sc[i]);
  mx = warp_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sum = 0.f;
  for (int i = tid; i < n; i += 256) {
    float e = exp2f(sc[i] - mx);
    sc[i] = e;
    sum += e;
  }
  sum = warp_sum(sum);
  __syncthreads();
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = sum;
  __syncthreads();
  const float l = red[4] + red[5] + red[6] + red[7];

  // phase 3: P.V.  16 lanes per key (8 value features each), 16 keys in flight
  const int c16 = tid & 15, kg = tid >> 4;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int jb = j0 + kg; jb < j1; jb += 64) {
    u32x4 vv[4];
    float pj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(jb + 16 * u, j1 - 1);
      vv[u] = *(const u32x4*)(V + (long)j * 128 + 8 * c16);
      pj[u] = (jb + 16 * u < j1) ? sc[j - j0] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = fmaf(pj[u], lo_bf(vv[u][i]), o[2 * i]);
        o[2 * i + 1] = fmaf(pj[u], hi_bf(vv[u][i]), o[2 * i + 1]);
      }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[kg][8 * c16 + i] = o[i];
  __syncthreads();
  if (tid < 128) {
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) acc += ob[g][tid];
    if (p.nsplit == 1) {
      p.out[(long)bh * 128 + tid] = f2bf(acc / l);
    } else {
      float* pp = p.part + ((long)bh * p.nsplit + split) * 130;
      if (tid == 0) {
        pp[0] = mx;
        pp[1] = l;
      }
      pp[2 + tid] = acc;
    }
  }
}

__global__ __launch_bounds__(128) void decode_full_combine_kernel(const float* part, int nsplit,
                                                                  bf16_t* out) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* pp = part + (long)bh * nsplit * 130;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[s * 130]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = exp2f(pp[s * 130] - M);
    L += f * pp[s * 130 + 1];
    acc += f * pp[s * 130 + 2 + t];
  }
  out[(long)bh * 128 + t] = f2bf(acc / L);
}

hipError_t decode_full_bf16(const DecodeFullParams& p, hipStream_t s) {
  if (p.chunk > DF_CHUNK_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_full_kernel, dim3(p.nsplit, p.B * p.H), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(decode_full_combine_kernel, dim3(p.B * p.H), dim3(128), 0, s, p.part,
                     p.nsplit, p.out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// latent-cache decode (absorbed)
// ------------------------------------------------------------------------
namespace {
constexpr int LT = 32;     // keys per tile
constexpr int LCH = 72;    // 16-byte chunks per cache row (576 bf16)

MLA_DEV int cphys(int c, int row) { return (c & ~7) | ((c ^ row) & 7); }
// position of key offset k (0..31) inside a C^T row
MLA_DEV int lpos(int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); }
MLA_DEV int ctswz(int f) { return ((f >> 1) ^ (f >> 3)) & 3; }
}  // namespace

__global__ __launch_bounds__(256) void decode_latent_kernel(DecodeLatentParams p) {
  __shared__ u32x4 Cs[2][LT * LCH];   // [key][576] row-major, swizzled
  __shared__ u32x4 Ct[2][512 * 4];    // [feature][32 keys], keys permuted

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x, b = blockIdx.y;
  const int j0 = split * p.chunk;
  const int j1 = min(p.L, j0 + p.chunk);
  const int head = 16 * w + l16;

  bf16x8 qf[18];
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    const int f = 32 * s + 8 * g4;
    const bf16_t* src = f < 512 ? p.q_abs + ((long)b * p.H + head) * 512 + f
                                : p.q + ((long)b * p.H + head) * 192 + 128 + (f - 512);
    u32x4 v = *(const u32x4*)src;
    if (f >= 512) v = rope8_bf16(v, p.rcos, p.rsin, p.L - 1, 32, (f - 512) / 2);
    qf[s] = __builtin_bit_cast(bf16x8, v);
  }
  const bf16_t* cb = p.cache + (long)b * p.L_cap * 576;

  // loader: item e = kp + 16 c (key pair kp, chunk c), up to 5 per thread
  u32x4 r0[5], r1[5];
#define DL_LOAD(kv0)                                                                      \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < 5; ++i) {                                       \
      const int e = min(tid + 256 * i, 16 * LCH - 1);                                     \
      const int kp = e & 15, c = e >> 4;                                                  \
      const int ka = min((kv0) + 2 * kp, j1 - 1), kb = min((kv0) + 2 * kp + 1, j1 - 1);   \
      r0[i] = *(const u32x4*)(cb + (long)ka * 576 + 8 * c);                               \
      r1[i] = *(const u32x4*)(cb + (long)kb * 576 + 8 * c);                               \
    }                                                                                     \
  } while (0)
#define DL_STORE(buf)                                                                     \
  do {                                                                                    \
    uint32_t* ct32 = (uint32_t*)&Ct[buf][0];                                              \
    _Pragma("unroll") for (int i = 0; i < 5; ++i) {                                       \
      const int e = tid + 256 * i;                                                        \
      if (e < 16 * LCH) {                                                                 \
        const int kp = e & 15, c = e >> 4;                                                \
        Cs[buf][(2 * kp) * LCH + cphys(c, 2 * kp)] = r0[i];                               \
        Cs[buf][(2 * kp + 1) * LCH + cphys(c, 2 * kp + 1)] = r1[i];                       \
        if (c < 64) {                                                                     \
          const int pos = lpos(2 * kp);                                                   \
          _Pragma("unroll") for (int q = 0; q < 8; ++q) {                                 \
            const int f = 8 * c + q;                                                      \
            const uint32_t w0 = r0[i][q >> 1], w1 = r1[i][q >> 1];                        \
            const uint32_t val = (q & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))              \
                                         : ((w0 & 0xffffu) | (w1 << 16));                 \
            const int ph = (((pos >> 3) ^ ctswz(f)) << 3) | (pos & 7);                    \
            ct32[(f * 32 + ph) >> 1] = val;                                               \
          }                                                                               \
        }                                                                                 \
      }                                                                                   \
    }                                                                                     \
  } while (0)

  floatx4 O[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) O[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int ntiles = (j1 - j0 + LT - 1) / LT;

  DL_LOAD(j0);
  DL_STORE(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1, kv0 = j0 + t * LT;
    if (t + 1 < ntiles) DL_LOAD(kv0 + LT);
    floatx4 S[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 18; ++s)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 16 * mb + l16;
        const bf16x8 a = __builtin_bit_cast(bf16x8, Cs[cur][row * LCH + cphys(4 * s + g4, row)]);
        S[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], S[mb], 0, 0, 0);
      }
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v = S[mb][jj] * p.scale_log2;
        if (kv0 + 16 * mb + 4 * g4 + jj >= j1) v = -INFINITY;
        S[mb][jj] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pv = exp2f(S[mb][jj] - m_new);
        psum += pv;
        pf[4 * mb + jj] = (__bf16)pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      O[i] *= alpha;
      const int f = 16 * i + l16;
      const bf16x8 a = __builtin_bit_cast(bf16x8, Ct[cur][f * 4 + (g4 ^ ctswz(f))]);
      O[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, O[i], 0, 0, 0);
    }
    if (t + 1 < ntiles) DL_STORE(cur ^ 1);
    __syncthreads();
  }
#undef DL_LOAD
#undef DL_STORE

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  // partial record: m, l, 2 pad, o~[512] (16-byte aligned)
  float* pp = p.part + (((long)b * p.nsplit + split) * p.H + head) * 516;
  if (g4 == 0) {
    pp[0] = m_run;
    pp[1] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i)
    *(floatx4*)(pp + 4 + 16 * i + 4 * g4) = O[i];
}

__global__ __launch_bounds__(256) void latent_combine_kernel(const float* part, int nsplit, int H,
                                                             bf16_t* o_lat) {
  const int bh = blockIdx.x;  // b * H + h
  const int b = bh / H, h = bh % H;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[(((long)b * nsplit + s) * H + h) * 516]);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* pp = part + (((long)b * nsplit + s) * H + h) * 516;
    const float f = exp2f(pp[0] - M);
    L += f * pp[1];
    a0 += f * pp[4 + threadIdx.x];
    a1 += f * pp[4 + 256 + threadIdx.x];
  }
  o_lat[(long)bh * 512 + threadIdx.x] = f2bf(a0 / L);
  o_lat[(long)bh * 512 + 256 + threadIdx.x] = f2bf(a1 / L);
}

hipError_t decode_latent_bf16(const DecodeLatentParams& p, hipStream_t s) {
  if (p.H != 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_latent_kernel, dim3(p.nsplit, p.B), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_combine_kernel, dim3(p.B * p.H), dim3(256), 0, s, p.part, p.nsplit,
                     p.H, p.o_lat);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// query absorption: q~[b,h,k] = sum_c q[b,h,c] * W_UK,h[c,k], c < 128, k < 512
// (the key rows of head h in kv_b_proj, rows h*256 + c).  Workgroup = (h,
// 64 latent features, 64 sequences); W_UK,h tile [128 c][64 k] is stored
// transposed in LDS so that the MFMA B operand is c-contiguous.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_q_kernel(const bf16_t* __restrict__ q,
                                                       const bf16_t* __restrict__ w_ukv,
                                                       bf16_t* __restrict__ q_abs, int B, int H) {
  __shared__ u32x4 Wt[64 * 16];    // [k 64][c 128] -> 16 chunks per row, swizzled
  __shared__ u32x4 Qs[64 * 16];    // [b 64][c 128]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int h = blockIdx.x, n0 = blockIdx.y * 64, b0 = blockIdx.z * 64;
  // W tile: 128 c x 64 k = 1024 chunks of 8 k; item = (c pair, k chunk): 64 x 8 = 512
  uint32_t* wt32 = (uint32_t*)Wt;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = tid + 256 * it;
    const int cp = e & 63, kc = e >> 6;  // c pair 0..63, k chunk 0..7
    const bf16_t* src = w_ukv + ((long)h * 256 + 2 * cp) * 512 + n0 + 8 * kc;
    const u32x4 a = *(const u32x4*)src;
    const u32x4 bb = *(const u32x4*)(src + 512);
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2) {
      const int k = 8 * kc + q2;
      const uint32_t w0 = a[q2 >> 1], w1 = bb[q2 >> 1];
      const uint32_t val = (q2 & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
      const int c = 2 * cp;
      const int ph = ((((c >> 3) ^ (k & 7)) & 15) << 3) | (c & 7);
      wt32[(k * 128 + ph) >> 1] = val;
    }
  }
  // Q tile: 64 rows x 16 chunks
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int e = tid + 256 * it;
    const int r = e >> 4, c = e & 15;
    const int bb = min(b0 + r, B - 1);
    Qs[r * 16 + (c ^ (r & 7))] = *(const u32x4*)(q + ((long)bb * H + h) * 192 + 8 * c);
  }
  __syncthreads();
  // wave w: rows 32*(w>>1), cols 32*(w&1)
  const int rm = 32 * (w >> 1), cn = 32 * (w & 1);
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int ra = rm + lr, rbk = cn + lr;
    const bf16x8 a = __builtin_bit_cast(bf16x8, Qs[ra * 16 + ((2 * s + lg) ^ (ra & 7))]);
    const bf16x8 bv = __builtin_bit_cast(bf16x8, Wt[rbk * 16 + (((2 * s + lg) ^ (rbk & 7)) & 15)]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = b0 + rm + 8 * (e >> 2) + 4 * lg + (e & 3);
    const int col = n0 + cn + lr;
    if (row < B) q_abs[((long)row * H + h) * 512 + col] = f2bf(acc[e]);
  }
}

hipError_t absorb_q_bf16(const bf16_t* q, const bf16_t* w_ukv, bf16_t* q_abs, int B, int H,
                         hipStream_t s) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H, 8, (B + 63) / 64), dim3(256), 0, s, q, w_ukv, q_abs,
                     B, H);
  return hipGetLastError();
}

}  // namespace mla
