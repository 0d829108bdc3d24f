// Causal flash attention for the MLA prefill, bf16 with fp32 softmax, gfx950.
//
// What it computes ("Kimi K2 · Mix and project", code excerpt, and the
// query/key assembly of "Kimi K2 · Dense transformer block"): for every
// sequence b, head h and query i, scores s_ij = scale * [Q^C ; Q^R]_i .
// [K^C_h ; k^R]_j over keys j <= i, a float32 softmax over j, and
// O_i = sum_j p_ij V_h,j, written straight into the head-merged layout
// [B*T, H*128] (column h*128 + c) that o_proj reads.  RoPE of the query's
// rotary part is applied here, as the query fragments are loaded.
//
// Design (CDNA4):
//  * 512 threads = 8 waves, 256 queries per workgroup (32 per wave), key
//    tiles of 64.  Registers stay within 256 per lane so two waves share each
//    SIMD: one wave's softmax (VALU) overlaps the other's MFMAs.
//  * Scores are formed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16: K rows are the A operand (K-contiguous rows in
//    LDS) and the wave's queries are the B operand, held in registers for the
//    whole loop.  Each lane then owns one query column, so the softmax
//    statistics are lane-local (plus one cross-half shuffle).
//  * O^T = V^T . P^T reuses the score accumulator directly as the B operand
//    (8 consecutive accumulator values = 8 keys of one query).  V^T is the A
//    operand: V tiles are stored transposed in LDS, with keys permuted inside
//    each group of 16 so that a lane's 8 keys are one 16-byte read.
//  * The shared rotary key k^R is loaded once per key into the 64 rotary
//    columns of the K tile (never replicated per head in memory).
//  * Softmax in the log2 domain with the scale folded into one FMA before
//    v_exp_f32.  The running maximum is only raised when a tile's maximum
//    exceeds it by more than 2^8 (exact: numerator and denominator share the
//    reference point; values stay below 2^8 * 64 per tile), so the O rescale
//    is skipped for most tiles.
//  * LDS swizzles are for 64 banks (gfx950 serves ds_read_b128 16 lanes at a
//    time from 256 bytes).  Two LDS stages (K 24 KB + V^T 16 KB each): the
//    next tile's global loads are in flight during the MFMAs.  Query tiles are
//    issued longest-first; heads map to XCD h % 8, so all query tiles of a
//    head share one L2.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {
constexpr int KCH = 24;   // 16-byte chunks per K row (192 bf16)
constexpr int BQ = 256;   // queries per workgroup
constexpr int NW = 8;     // waves per workgroup
constexpr float LAZY = 8.0f;  // raise the running max only past this margin (log2 units)

// K row = 384 bytes = 1.5 lines of 256 bytes.  Rows r and r + 2 start on the
// same bank group offset parity; XOR the chunk's low 3 bits with (r >> 1) so
// the 16 rows a half-wave reads hit 16 distinct 16-byte bank groups.
MLA_DEV int kphys(int c, int row) { return (c & ~7) | ((c ^ (row >> 1)) & 7); }
// V^T row = 128 bytes: pairs of rows share a 256-byte line.
MLA_DEV int vswz(int dv) { return (dv >> 1) & 7; }

// position of key offset k (0..63) inside a V^T row (see header comment)
MLA_DEV int vpos(int k) {
  int g16 = k >> 4, kk = k & 15;
  return g16 * 16 + 8 * ((kk >> 2) & 1) + 4 * (kk >> 3) + (kk & 3);
}
}  // namespace

__global__ __launch_bounds__(512) void flash_prefill_kernel(FlashParams p) {
  __shared__ u32x4 Ks[2][64 * KCH];
  __shared__ u32x4 Vt[2][128 * 8];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int nqt = (p.T + BQ - 1) / BQ;
  const int HB = p.H * p.B;
  const int qt = nqt - 1 - (int)(blockIdx.x / HB);
  const int rem = blockIdx.x % HB;
  const int h = rem % p.H, b = rem / p.H;
  const int q0 = qt * BQ;
  const long rowbase = (long)b * p.T;
  const long HS = p.H;

  // this wave's queries as MFMA B fragments: features 16 s + 8 lg .. +8.
  // The rotary features (s >= 8) are rotated here by the RoPE table row of
  // the query's position: each fragment holds 4 whole (2i, 2i+1) pairs.
  bf16x8 qf[12];
  {
    const int qrow = min(q0 + 32 * w + lr, p.T - 1);
    const bf16_t* qp = p.q + ((rowbase + qrow) * HS + h) * 192 + 8 * lg;
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      u32x4 v = *(const u32x4*)(qp + 16 * s);
      if (s >= 8) v = rope8_bf16(v, p.rcos, p.rsin, qrow, 32, (16 * s + 8 * lg - 128) / 2);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int qlast = min(q0 + BQ - 1, p.T - 1);
  const int n_kv = qlast / 64 + 1;

  // loaders: K tile = 64 rows x 24 chunks (3 per thread); V tile = 32 key
  // pairs x 16 chunks (one pair per thread).  Source pointers are formed once
  // for key offset 0 and advanced by the tile's first key; only the last tile
  // (keys past T - 1) takes the clamped path.
  const long krow_stride = HS * 256;  // elements between consecutive keys in kv
  const bf16_t* kp0[3];
  long kstep[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int e = tid + 512 * i, row = e / KCH, c = e % KCH;
    kp0[i] = c < 16 ? p.kv + ((rowbase + row) * HS + h) * 256 + 8 * c : p.kr + (rowbase + row) * 64 + 8 * (c - 16);
    kstep[i] = c < 16 ? krow_stride : 64;
  }
  const int vkp = tid & 31, vc = tid >> 5;
  const bf16_t* vp0 = p.kv + ((rowbase + 2 * vkp) * HS + h) * 256 + 128 + 8 * vc;
  u32x4 rk[3], rv[2];
#define FP_LOAD(kv0)                                                                      \
  do {                                                                                    \
    if ((kv0) + 64 <= p.T) {                                                              \
      _Pragma("unroll") for (int i = 0; i < 3; ++i)                                       \
        rk[i] = *(const u32x4*)(kp0[i] + (long)(kv0) * kstep[i]);                          \
      rv[0] = *(const u32x4*)(vp0 + (long)(kv0) * krow_stride);                            \
      rv[1] = *(const u32x4*)(vp0 + (long)((kv0) + 1) * krow_stride);                      \
    } else {                                                                              \
      _Pragma("unroll") for (int i = 0; i < 3; ++i) {                                     \
        const int e = tid + 512 * i, row = e / KCH;                                       \
        rk[i] = *(const u32x4*)(kp0[i] + (long)(min((kv0) + row, p.T - 1) - row) * kstep[i]); \
      }                                                                                   \
      const int k0_ = min((kv0) + 2 * vkp, p.T - 1) - 2 * vkp;                            \
      const int k1_ = min((kv0) + 2 * vkp + 1, p.T - 1) - 2 * vkp;                        \
      rv[0] = *(const u32x4*)(vp0 + (long)k0_ * krow_stride);                              \
      rv[1] = *(const u32x4*)(vp0 + (long)k1_ * krow_stride);                              \
    }                                                                                     \
  } while (0)
#define FP_STORE(buf)                                                                     \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < 3; ++i) {                                       \
      const int e = tid + 512 * i, row = e / KCH, c = e % KCH;                            \
      Ks[buf][row * KCH + kphys(c, row)] = rk[i];                                         \
    }                                                                                     \
    uint32_t* vt32 = (uint32_t*)&Vt[buf][0];                                              \
    const int pos = vpos(2 * vkp);                                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                       \
      const int dv = 8 * vc + i;                                                          \
      const uint32_t w0 = rv[0][i >> 1], w1 = rv[1][i >> 1];                              \
      const uint32_t val = (i & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))                    \
                                   : ((w0 & 0xffffu) | (w1 << 16));                       \
      const int ph = (((pos >> 3) ^ vswz(dv)) << 3) | (pos & 7);                          \
      vt32[(dv * 64 + ph) >> 1] = val;                                                    \
    }                                                                                     \
  } while (0)

  floatx16 O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int qi = q0 + 32 * w + lr;
  const int wq_first = q0 + 32 * w, wq_last = wq_first + 31;

  // Fragment byte offsets inside a stage (tile-invariant).  K fragment
  // (s, mb): row 32 mb + lr, chunk 2 s + lg at kphys(); the row's (row >> 1)
  // & 7 equals (lr >> 1) & 7, so the position depends on s & 3 only.
  int k_off[4], v_off[4];
#pragma unroll
  for (int s3 = 0; s3 < 4; ++s3) {
    k_off[s3] = (lr * KCH + (((2 * s3 + lg) ^ (lr >> 1)) & 7)) * 16;
    v_off[s3] = (lr * 8 + ((2 * s3 + lg) ^ vswz(lr))) * 16;  // V^T row dv = 32 d + lr, k-step s3
  }

  FP_LOAD(0);
  FP_STORE(0);
  __syncthreads();
  for (int t = 0; t < n_kv; ++t) {
    const int cur = t & 1, kv0 = t * 64;
    if (t + 1 < n_kv) FP_LOAD(kv0 + 64);
    if (kv0 <= wq_last) {  // wave-uniform: some key of the tile is visible
      floatx16 S[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[mb][e] = 0.f;
      // 24 K fragments (x = 2 s + mb), read RQ ahead of their MFMA
      const char* kb = (const char*)&Ks[cur][0];
      constexpr int RQ = 8;
#define FP_KFRAG(x) (*(const bf16x8*)(kb + k_off[((x) >> 1) & 3] + 32 * KCH * 16 * ((x) & 1) + 128 * ((x) >> 3)))
      bf16x8 fk[RQ];
#pragma unroll
      for (int u = 0; u < RQ; ++u) fk[u] = FP_KFRAG(u);
#pragma unroll
      for (int x = 0; x < 24; ++x) {
        S[x & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[x % RQ], qf[x >> 1], S[x & 1], 0, 0, 0);
        if (x + RQ < 24) fk[x % RQ] = FP_KFRAG(x + RQ);
      }
#undef FP_KFRAG
      __builtin_amdgcn_sched_group_barrier(0x100, RQ, 0);
#pragma unroll
      for (int x = 0; x < 24; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x + RQ < 24) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // scores in log2 units: sl2 * S; masked keys (after the query) -> -inf
      const bool diag = kv0 + 63 > wq_first;
      float tmax = -INFINITY;
      if (diag) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kv0 + 32 * mb + 8 * (e >> 2) + 4 * lg + (e & 3);
            if (key > qi) S[mb][e] = -INFINITY;
            tmax = fmaxf(tmax, S[mb][e]);
          }
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, S[mb][e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * sl2;
      // lazy running max: only move it when the tile max is far above it
      const bool raise = tmax > m_run + LAZY;
      const float m_new = raise ? tmax : m_run;
      if (__any(raise)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 for unchanged lanes
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) O[d][e] *= alpha;
      }
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(S[mb][e], sl2, -m_new));
          S[mb][e] = pv;
          psum += pv;
        }
      l_run += psum;
      // 16 V^T fragments (y = 4 ks + d), all read ahead of the MFMAs
      const char* vb = (const char*)&Vt[cur][0];
      bf16x8 fv[16];
#pragma unroll
      for (int y = 0; y < 16; ++y) fv[y] = *(const bf16x8*)(vb + v_off[y >> 2] + 32 * 128 * (y & 3));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int ih = 0; ih < 2; ++ih) {
          bf16x8 pf;
#pragma unroll
          for (int m = 0; m < 8; ++m) pf[m] = (__bf16)S[mb][8 * ih + m];
          const int ks = 2 * mb + ih;
#pragma unroll
          for (int d = 0; d < 4; ++d) O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[4 * ks + d], pf, O[d], 0, 0, 0);
        }
    }
    if (t + 1 < n_kv) FP_STORE(cur ^ 1);
    __syncthreads();
  }
#undef FP_LOAD
#undef FP_STORE

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi < p.T) {
    const float inv = 1.f / l_tot;
    bf16_t* op = p.out + (rowbase + qi) * (HS * 128) + (long)h * 128 + 4 * lg;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 v;
        v[0] = pack2bf(O[d][4 * i + 0] * inv, O[d][4 * i + 1] * inv);
        v[1] = pack2bf(O[d][4 * i + 2] * inv, O[d][4 * i + 3] * inv);
        *(u32x2*)(op + 32 * d + 8 * i) = v;
      }
  }
}

hipError_t flash_prefill_bf16(const FlashParams& p, hipStream_t s) {
  const int nqt = (p.T + BQ - 1) / BQ;
  hipLaunchKernelGGL(flash_prefill_kernel, dim3(nqt * p.H * p.B), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
