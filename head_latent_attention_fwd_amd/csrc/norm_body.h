// Device body of the latent RMSNorms with the shared-key RoPE, shared by its
// own kernel (rows.hip) and by the persistent latent-decode kernel.
//
// Sources (by page title and section): "Kimi K2 · Dense transformer block",
// equation list (RMSNorm of the query latent, RoPE of the shared rotary key
// with the table R); "Kimi K2 · Key-value compression", c^KV = x W_DKV then
// RMSNorm, the joint projection's 576 outputs split into the 512 latent and
// the 64-wide rotary key after the product, the two together being the
// 576-value cache entry.  RMSNorm is g * x / sqrt(mean(x^2) + eps); RoPE
// turns the consecutive pair (2i, 2i+1) by t * base^(-2i/d_rope).
#pragma once
#include "common.h"
#include "kernels.h"
#include "stream_sum.h"

namespace mla {

// Sum of 4 consecutive fp32 columns over the split-K partials p[s * stride],
// s = 0..nsplit-1, in split order (deterministic).  Loads are issued 8 splits
// at a time so their latencies overlap instead of one round trip per split.
MLA_DEV floatx4 sum_splits4(const float* __restrict__ p, long stride, int nsplit) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    floatx4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = s0 + j < nsplit ? *(const floatx4*)(p + (long)(s0 + j) * stride) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
  }
  return acc;
}

template <int NT>
MLA_DEV float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}

// Bias of down-projection output column c ([q latent | kv latent | rotary
// key]), or 0 without the attention_bias variant.
template <typename T>
MLA_DEV float down_bias(const LatentNormParams<T>& p, int c) {
  if (c < p.q_lora) return p.bias_q ? to_f<T>(p.bias_q[c]) : 0.f;
  return p.bias_kvr ? to_f<T>(p.bias_kvr[c - p.q_lora]) : 0.f;
}

// Workgroups of NT threads per row: sum the down-projection partials of the
// row in a fixed order (deterministic) -- either nsplit fp32 K-slices or the
// weight-streaming GEMM's partial blocks -- then the RMSNorms and the RoPE of
// the shared key, with the optional cache writes.  With two workgroups per
// row, the first takes the query latent and its norm, the second the kv
// latent, its norm and the rotary key.
// One workgroup (NT threads) for row m, part `by` of `gy` (gy = 1: the
// whole row; gy = 2: by = 0 the query half, by = 1 the kv half).  row: LDS
// for q_lora + kv_lora + d_rope floats (16-byte aligned); red: NT / 64 floats.
template <typename T, int NT>
MLA_DEV void latent_norm_rope_body(const LatentNormParams<T>& p, int m, int by, int gy, float* row,
                                   float* red) {
  const int tid = threadIdx.x;
  const int N1 = p.q_lora + p.kv_lora + p.d_rope;
  const bool do_q = gy == 1 || by == 0;
  const bool do_kv = gy == 1 || by == 1;
  const int c_lo = do_q ? 0 : p.q_lora, c_hi = do_kv ? N1 : p.q_lora;
  float sq = 0.f, skv = 0.f;
  // 4 columns per thread and iteration, all splits' loads in flight together
  const bool vec = (N1 % 4 == 0) && (p.ld_part % 4 == 0) && (p.split_stride % 4 == 0) && (c_lo % 4 == 0);
  if (p.stream) {
    for (int c4 = c_lo / 4 + tid; c4 < c_hi / 4; c4 += NT) {
      const floatx4 v = stream_sum4(p.part, p.si, m, 4 * c4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        const float x = v[q] + down_bias(p, c);
        row[c] = x;
        if (c < p.q_lora) sq += x * x;
        else if (c < p.q_lora + p.kv_lora) skv += x * x;
      }
    }
  } else if (vec) {
    for (int c4 = c_lo / 4 + tid; c4 < c_hi / 4; c4 += NT) {
      const floatx4 v = sum_splits4(p.part + (long)m * p.ld_part + 4 * c4, p.split_stride, p.nsplit);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        const float x = v[q] + down_bias(p, c);
        row[c] = x;
        if (c < p.q_lora) sq += x * x;
        else if (c < p.q_lora + p.kv_lora) skv += x * x;
      }
    }
  } else {
    for (int c = c_lo + tid; c < c_hi; c += NT) {
      float v = 0.f;
      for (int s = 0; s < p.nsplit; ++s)
        v += p.part[(long)s * p.split_stride + (long)m * p.ld_part + c];
      v += down_bias(p, c);
      row[c] = v;
      if (c < p.q_lora) sq += v * v;
      else if (c < p.q_lora + p.kv_lora) skv += v * v;
    }
  }
  // bf16 outputs four columns at a time (8-byte gain loads and stores, one
  // 16-byte LDS read) when the widths and leading dimensions allow it
  constexpr bool BF = sizeof(T) == 2;
  const bool v4 = BF && p.q_lora % 4 == 0 && p.kv_lora % 4 == 0 && p.ld_cq % 4 == 0 && p.ld_ckv % 4 == 0 &&
                  (p.kv_lora + p.d_rope) % 4 == 0;
  if (do_q) {
    const float rq = 1.0f / sqrtf(block_sum<NT>(sq, red) / (float)p.q_lora + p.eps);
    if (v4) {
      for (int c4 = tid; c4 < p.q_lora / 4; c4 += NT) {
        const u32x2 g = *(const u32x2*)(p.g_q + 4 * c4);
        const floatx4 x = *(const floatx4*)(row + 4 * c4);
        *(u32x2*)(p.cq + (long)m * p.ld_cq + 4 * c4) =
            u32x2{pack2bf(lo_bf(g[0]) * (x[0] * rq), hi_bf(g[0]) * (x[1] * rq)),
                  pack2bf(lo_bf(g[1]) * (x[2] * rq), hi_bf(g[1]) * (x[3] * rq))};
      }
    } else {
      for (int c = tid; c < p.q_lora; c += NT)
        p.cq[(long)m * p.ld_cq + c] = from_f<T>(to_f<T>(p.g_q[c]) * (row[c] * rq));
    }
  }
  if (!do_kv) return;
  const float rkv = 1.0f / sqrtf(block_sum<NT>(skv, red) / (float)p.kv_lora + p.eps);

  const int t = m % p.rope_T;
  const int pos = p.seq_pos ? seq_position(p.seq_pos, m, 0, p.pos_max) : t + p.rope_pos0;
  const int bseq = m / p.rope_T;
  T* lat = p.latent_cache
               ? p.latent_cache + ((long)bseq * p.L_cap + pos) * (p.kv_lora + p.d_rope)
               : nullptr;

  if (v4) {
    for (int c4 = tid; c4 < p.kv_lora / 4; c4 += NT) {
      const u32x2 g = *(const u32x2*)(p.g_kv + 4 * c4);
      const floatx4 x = *(const floatx4*)(row + p.q_lora + 4 * c4);
      const u32x2 y = {pack2bf(lo_bf(g[0]) * (x[0] * rkv), hi_bf(g[0]) * (x[1] * rkv)),
                       pack2bf(lo_bf(g[1]) * (x[2] * rkv), hi_bf(g[1]) * (x[3] * rkv))};
      *(u32x2*)(p.ckv + (long)m * p.ld_ckv + 4 * c4) = y;
      if (lat) *(u32x2*)(lat + 4 * c4) = y;
    }
  } else {
    for (int c = tid; c < p.kv_lora; c += NT) {
      T y = from_f<T>(to_f<T>(p.g_kv[c]) * (row[p.q_lora + c] * rkv));
      p.ckv[(long)m * p.ld_ckv + c] = y;
      if (lat) lat[c] = y;
    }
  }
  const int npairs = p.d_rope / 2;
  const float* kp = row + p.q_lora + p.kv_lora;
  for (int i = tid; i < npairs; i += NT) {
    float cs = p.rcos[(long)pos * p.n_pairs + i], sn = p.rsin[(long)pos * p.n_pairs + i];
    float a = kp[2 * i], b = kp[2 * i + 1];
    T y0 = from_f<T>(a * cs - b * sn), y1 = from_f<T>(a * sn + b * cs);
    p.kr[(long)m * p.ld_kr + 2 * i] = y0;
    p.kr[(long)m * p.ld_kr + 2 * i + 1] = y1;
    if (lat) {
      lat[p.kv_lora + 2 * i] = y0;
      lat[p.kv_lora + 2 * i + 1] = y1;
    }
  }
}

}  // namespace mla
