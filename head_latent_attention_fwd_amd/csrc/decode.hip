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
//                   LDS.  Split-L partials (m, l in fp32, o~ in bf16) per
//                   head are merged by latent_out together with the W_UV
//                   product.
//  absorb_q       : q~_h = Q^C_h . W_UK,h (W_UK folded into the query), an
//                   MFMA product whose weight operand is transposed into LDS.
#include "latent_body.h"

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
  __shared__ u32x4 qs[24];  // the query, summed from its partial blocks (fused form)
  const int tid = threadIdx.x;
  const int split = blockIdx.x, bh = blockIdx.y;
  // live length of this sequence: keys 0 .. P, P its new token's position
  const int P = seq_position(p.seq_pos, bh / p.H, p.L - 1, p.L - 1);
  const int j0 = split * p.chunk;
  const int j1 = min(P + 1, j0 + p.chunk);
  const int n = j1 - j0;  // <= 0: a split past this sequence's keys (empty partial)
  bf16_t* Kw = p.k_cache + (long)bh * p.L_cap * 192;
  bf16_t* Vw = p.v_cache + (long)bh * p.L_cap * 128;
  const bf16_t* K = Kw;
  const bf16_t* V = Vw;

  if (p.qpart || (p.kvpart && j0 <= P && P < j1)) {
    const int b = bh / p.H, h = bh - b * p.H;
    if (p.qpart && tid < 48) {
      // 4 query features per thread, rounded to bf16 as the stored query is
      const floatx4 v = stream_sum4(p.qpart, p.qsi, b, h * 192 + 4 * tid);
      ((u32x2*)qs)[tid] = u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
    }
    if (p.kvpart && j0 <= P && P < j1) {
      // the new token's key [K^C | k^R] and value go to slot P of the caches
      if (tid >= 64 && tid < 128) {
        const int e = tid - 64;  // K^C features 4 e (e < 32), else V features 4 (e - 32)
        const floatx4 v = stream_sum4(p.kvpart, p.kvsi, b, h * 256 + 4 * e);
        const u32x2 o = {pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
        if (e < 32) *(u32x2*)(Kw + (long)P * 192 + 4 * e) = o;
        else *(u32x2*)(Vw + (long)P * 128 + 4 * (e - 32)) = o;
      } else if (tid >= 128 && tid < 136) {
        const int c = tid - 128;
        *(u32x4*)(Kw + (long)P * 192 + 128 + 8 * c) = *(const u32x4*)(p.kr + (long)b * 64 + 8 * c);
      }
    }
    __syncthreads();  // slot L-1 written (workgroup scope) before the key loop reads it
  }

  // phase 1: scores.  8 lanes per key; lane g8 holds query chunks g8, g8+8, g8+16
  const int g8 = tid & 7, grp = tid >> 3;
  const bf16_t* qp = p.q + (long)bh * 192;
  float qf[24];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    u32x4 v = p.qpart ? qs[8 * c + g8] : *(const u32x4*)(qp + 64 * c + 8 * g8);
    // chunk 2 holds rotary features 8*g8 .. +8: rotate by the token's position
    if (c == 2) v = rope8_bf16(v, p.rcos, p.rsin, P, 32, 4 * g8);
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
// latent-cache decode (absorbed): kernels over the bodies in latent_body.h
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decode_latent_kernel(DecodeLatentParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kLatentAttnLds];
  decode_latent_body(p, blockIdx.x, lds);
}

__global__ __launch_bounds__(256) void latent_out_kernel(DecodeLatentParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kLatentOutLds];
  latent_out_body(p, blockIdx.x, blockIdx.y, lds);
}

hipError_t decode_latent_bf16(const DecodeLatentParams& p, hipStream_t s) {
  if (p.H != 64 || !p.w_ukv) return hipErrorInvalidValue;
  if (p.plan && (p.G < p.B || p.G > max(p.B, LO_NSMAX) || p.B > LP_NS)) return hipErrorInvalidValue;
  if (!p.plan && (p.splits < 1 || p.splits > LO_NSMAX || p.G != p.B * p.splits ||
                  p.splits > (p.L + LT - 1) / LT))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_latent_kernel, dim3(p.G), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_out_kernel, dim3(p.H, (p.B + LO_BG - 1) / LO_BG), dim3(256), 0, s, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void absorb_q_kernel(AbsorbParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kAbsorbLds];
  absorb_q_body<true>(p, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

hipError_t absorb_q_bf16(const AbsorbParams& p, hipStream_t s) {
  if (p.H <= 0 || p.B <= 0) return hipErrorInvalidValue;
  if (p.plan && (p.B > LP_NS || p.G < p.B)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(absorb_q_kernel, dim3(p.H, 512 / AB_N, (p.B + 63) / 64), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
