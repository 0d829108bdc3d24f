// Generic attention for the float32 path: one wave per (sequence, head,
// query), online softmax over the visible keys.
//
// Sources: "Kimi K2 · Mix and project", code excerpt -- scores are the
// query/key products times the softmax scale, the additive causal mask
// removes keys after the query, softmax over keys in float32, then P.V.
// "Kimi K2 · Dense transformer block", equation list -- the query of a head
// is [Q^C ; Q^R] and its key [K^C ; k^R] with k^R shared by all heads.
//
// All three forms of the step use this kernel through strides:
//  * prefill: K^C and V inside the kv up-projection output, k^R shared;
//  * decode with the full cache: K = [K^C ; k^R] and V per head in the cache;
//  * decode with the latent cache (absorbed): query [q~ ; Q^R], the key is
//    the cache row [c ; k^R] and the value its first kv_lora features, with
//    zero head strides (one latent shared by every head).
#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int GEN_MAX = 16;  // per-lane elements: query/key and value widths up to 1024

__global__ __launch_bounds__(256) void attn_generic_kernel(AttnGenericParams p) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  if (i >= p.Tq) return;
  const int dqk = p.d_nope + p.d_rope;

  float q[GEN_MAX];
  const float* qn = p.q_nope + ((long)b * p.Tq + i) * p.q_row + (long)h * p.q_head;
  const float* qr = p.q_rope + ((long)b * p.Tq + i) * p.qr_row + (long)h * p.qr_head;
#pragma unroll
  for (int k = 0; k < GEN_MAX; ++k) {
    int e = lane + 64 * k;
    q[k] = e < p.d_nope ? qn[e] : (e < dqk ? qr[e - p.d_nope] : 0.f);
  }
  float o[GEN_MAX];
#pragma unroll
  for (int k = 0; k < GEN_MAX; ++k) o[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int jmax = p.seq_pos ? min(p.Tk - 1, seq_position(p.seq_pos, b, 0, p.pos_max))
                            : min(p.Tk - 1, i + p.causal_offset);
  for (int j = 0; j <= jmax; ++j) {
    const float* kn = p.k_nope + (long)b * p.kn_b + (long)j * p.kn_j + (long)h * p.kn_h;
    const float* kr = p.k_rope + (long)b * p.kr_b + (long)j * p.kr_j + (long)h * p.kr_h;
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < GEN_MAX; ++k) {
      int e = lane + 64 * k;
      float kv = e < p.d_nope ? kn[e] : (e < dqk ? kr[e - p.d_nope] : 0.f);
      part = fmaf(q[k], kv, part);
    }
    const float s = warp_sum(part) * p.scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);  // m = -inf on the first key: alpha = 0
    const float pj = expf(s - mn);
    l = l * alpha + pj;
    const float* vv = p.v + (long)b * p.v_b + (long)j * p.v_j + (long)h * p.v_h;
#pragma unroll
    for (int k = 0; k < GEN_MAX; ++k) {
      int e = lane + 64 * k;
      float x = e < p.d_v ? vv[e] : 0.f;
      o[k] = o[k] * alpha + pj * x;
    }
    m = mn;
  }
  float* out = p.out + ((long)b * p.Tq + i) * p.o_row + (long)h * p.o_head;
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < GEN_MAX; ++k) {
    int e = lane + 64 * k;
    if (e < p.d_v) out[e] = o[k] * inv;
  }
}

hipError_t attn_generic_f32(const AttnGenericParams& p, hipStream_t s) {
  dim3 grid((p.Tq + 3) / 4, p.B * p.H);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
