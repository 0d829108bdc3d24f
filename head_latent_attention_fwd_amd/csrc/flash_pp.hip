// Causal flash attention for the MLA prefill, bf16 with fp32 softmax, gfx950:
// ping-pong form.
//
// What it computes ("Kimi K2 · Mix and project", code excerpt; query/key
// assembly of "Kimi K2 · Dense transformer block"):
// s_ij = scale * [Q^C ; Q^R]_i . [K^C_h ; k^R]_j over keys j <= i, a float32
// softmax over j, O_i = sum_j p_ij V_h,j, written into the
// head-merged layout [B*T, H*128].  RoPE of the query's rotary part is applied
// as the query fragments are loaded.
//
// Why ping-pong: with one barrier per key tile, all eight waves run the
// QK products, the softmax and the PV products in lockstep, so the two waves
// sharing a SIMD reach their softmax (VALU) together and the matrix pipe
// idles.  Here the waves of the second half (4..7) run the same work rotated
// by one phase: in segment k the first half runs QK(k), softmax(k), PV(k) and
// the second half runs softmax(k-1), PV(k-1), QK(k), so while one wave of a
// SIMD is in its softmax the other issues MFMAs.
//
// Data movement: per key tile (64 keys) the content key tile [64 x 256 B],
// the rotary key tile [64 x 128 B] and the value tile [64 x 256 B] (row-major,
// as in memory) arrive by wave-wide direct-to-LDS buffer loads into a ring of
// NST stages; keys past T read as zero (buffer range) and are masked anyway
// by causality.  A tile is live in three consecutive segments (loading; first
// half + second-half QK; second-half PV), so the ring holds NST >= 3 tiles and
// the loads of tile k + NST - 2 are issued at the start of segment k.
//
// Products (v_mfma_f32_32x32x16_bf16): S^T = K . Q^T with key rows as the A
// operand (from LDS) and the wave's 32 queries as the B operand (registers),
// so each lane owns one query column and the softmax statistics are
// lane-local (plus one cross-half shuffle).  O^T = V^T . P^T with the score
// accumulator converted to bf16 as the B operand, and the V^T operand read
// from the row-major value tile with ds_read_b64_tr_b16: within each 16-lane
// group, output lane i receives element i % 4 of the 8-byte rows addressed by
// lanes i / 4 + 4 j (j = 0..3), so lanes addressing 4 consecutive key rows x 4
// feature quads yield, per lane, one feature over 4 consecutive keys.
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {
constexpr int PP_BQ = 256;                   // queries per workgroup: 8 waves x 32
constexpr int PP_NST = 3;                    // LDS ring stages
constexpr int PP_KC = 64 * 256;              // content key tile (128 features)
constexpr int PP_KR = 64 * 128;              // rotary key tile (64 features)
constexpr int PP_V = 64 * 256;               // value tile (128 features)
constexpr int PP_STG = PP_KC + PP_KR + PP_V; // 40 KB
constexpr int PP_DPW = 5;                    // DMAs per wave per tile (2 + 1 + 2)
constexpr int PP_QROW = 192 * 2;             // bytes of one query row (one head)
constexpr int PP_QST = PP_BQ * PP_QROW;      // 96 KB: the tile's queries, staged in LDS
constexpr int PP_LDS = PP_NST * PP_STG > PP_STG + PP_QST ? PP_NST * PP_STG : PP_STG + PP_QST;
constexpr float PP_LAZY = 8.0f;              // raise the running max past this margin (log2)

MLA_DEV void pp_dma16(unsigned m0, int voff, u32x4 rsrc) {
  // lane l's 16 bytes at rsrc.base + voff -> LDS byte m0 + 16 l (explicit
  // vmcnt waits below; the compiler's counting cannot tell ring stages apart)
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// chunk swizzle of a value-tile row
MLA_DEV int pp_vswz(int row) { return (row & 3) << 2; }
// chunk swizzle of a staged query row (384 B = 96 banks): rows r and r + 1 sit
// 32 banks apart, and XOR (r >> 1) & 7 spreads the 16 rows of a fragment
// read over the remaining eight 16-byte positions
MLA_DEV int pp_qswz(int row) { return (row >> 1) & 7; }
MLA_DEV u32x4 pp_rsrc(const void* base, long bytes) {
  const unsigned long a = (unsigned long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)(bytes > 0x7fffffffL ? 0x7fffffffL : bytes));
  r[3] = 0x00020000u;
  return r;
}
}  // namespace

__global__ __launch_bounds__(512) void flash_pp_kernel(FlashParams p) {
  __shared__ __attribute__((aligned(16))) char lds[PP_LDS];
  const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const bool second = w >= 4;  // rotated phase
  const int nqt = (p.T + PP_BQ - 1) / PP_BQ;
  const int HB = p.H * p.B;
  const int sp = (int)(blockIdx.x % p.nsplit);           // key split
  const int wg = (int)(blockIdx.x / p.nsplit);
  const int qt = nqt - 1 - wg / HB;  // longest query tiles first
  const int rem = wg % HB;
  const int h = rem % p.H, b = rem / p.H;
  const int q0 = qt * PP_BQ;  // first query row of the tile (query positions are P0 + row)
  const long rowbase = (long)b * p.T;
  const long HS = p.H;

  // positions: this lane's query and the wave's first / last query
  const int qlast = p.P0 + min(q0 + PP_BQ - 1, p.T - 1);
  // key tiles [k_lo, k_hi) of the tile's qlast / 64 + 1: this split's share
  const int n_all = qlast / 64 + 1;
  const int k_lo = sp * n_all / p.nsplit, n_kv = (sp + 1) * n_all / p.nsplit;
  const int qrow_l = q0 + 32 * w + lr;  // query row in the chunk
  const int qi = p.P0 + qrow_l;
  const int wq_first = p.P0 + q0 + 32 * w, wq_last = wq_first + 31;

  // ---- loaders.  Wave w moves content-key rows 8 w .. 8 w + 7 (two DMAs of
  // 4 rows x 256 B), rotary-key rows 8 w .. 8 w + 7 (one DMA of 8 rows x
  // 128 B) and value rows 8 w .. 8 w + 7 (two DMAs).  LDS chunk swizzles:
  // content-key rows (256 B) XOR the 16-byte chunk with (row & 15), so the
  // 16 rows of a fragment read hit 16 chunk positions; rotary-key rows
  // (128 B) with ((row >> 1) & 7); value rows (256 B) with 4 (row & 3): a
  // transposed value read covers 4 consecutive rows x the same 4 logical
  // chunks per half-wave, and row & 15 would put all four rows on the same 4
  // chunk positions (a 4-way bank conflict), while 4 (row & 3) gives each
  // row its own group of 4.
  // source rows: key j of this (sequence, head) at byte j * *_kb of its base
  const int nkeys = p.P0 + p.T;
  int kc_vo[2], v_vo[2], kr_vo;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (2 * w + i) + (lane >> 4);
    kc_vo[i] = row * p.kc_kb + 16 * ((lane & 15) ^ (row & 15));
    v_vo[i] = row * p.v_kb + 16 * ((lane & 15) ^ pp_vswz(row));
  }
  {
    const int row = 8 * w + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    kr_vo = row * p.kr_kb + 16 * c;
  }
  // keys past the last one read as zero (buffer range); causality masks them
  const u32x4 rkc = pp_rsrc(p.kc + b * p.kc_b + h * p.kc_h, (long)nkeys * p.kc_kb);
  const u32x4 rkr = pp_rsrc(p.kr2 + b * p.kr_b + h * p.kr_h, (long)nkeys * p.kr_kb);
  const u32x4 rvv = pp_rsrc(p.vv + b * p.v_b + h * p.v_h, (long)nkeys * p.v_kb);
#define PP_ISSUE(tt)                                                                         \
  do {                                                                                       \
    const unsigned sb_ = lds_base + (((tt) - k_lo) % PP_NST) * PP_STG;                       \
    const int kk_ = 64 * (tt);                                                               \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                            \
      pp_dma16(sb_ + 1024 * (2 * w + i), kc_vo[i] + kk_ * p.kc_kb, rkc);                     \
    pp_dma16(sb_ + PP_KC + 1024 * w, kr_vo + kk_ * p.kr_kb, rkr);                            \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                            \
      pp_dma16(sb_ + PP_KC + PP_KR + 1024 * (2 * w + i), v_vo[i] + kk_ * p.v_kb, rvv);       \
  } while (0)

  // Prologue loads: the first key tile (ring slot 0: slots count from the
  // split's first tile), then the tile's 256 query rows by direct-to-LDS
  // loads into slots 1 and 2 and the 16 KB past the ring, and the RoPE rows
  // of this lane's query, all in flight together.  Staged rows cost about
  // three 128-byte lines each, where loading the MFMA fragments straight
  // from memory (each load instruction spans 32 rows) costs 32 per load.
  for (int tt = k_lo; tt < k_lo + PP_NST - 2 && tt < n_kv; ++tt) PP_ISSUE(tt);
  {
    // staged chunk i = 64 (12 w + d) + lane: row i / 24, 16-byte position
    // i % 24, holding logical chunk (i % 24) ^ pp_qswz(row)
    const u32x4 rq = pp_rsrc(p.q + (rowbase * HS + h) * 192, (long)p.T * HS * PP_QROW);
#pragma unroll
    for (int d = 0; d < PP_QST / 1024 / 8; ++d) {
      const int i = 64 * (12 * w + d) + lane, row = i / 24, c = (i % 24) ^ pp_qswz(row);
      pp_dma16(lds_base + PP_STG + 1024 * (12 * w + d), min(q0 + row, p.T - 1) * (int)HS * PP_QROW + 16 * c, rq);
    }
  }
  const int qrow = min(q0 + 32 * w + lr, p.T - 1);
  floatx4 rcs[4][2];  // RoPE (cos, sin) of the rotary fragments s = 8..11
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const long o = (long)(p.P0 + qrow) * 32 + (16 * s + 8 * lg) / 2;
    rcs[s][0] = *(const floatx4*)(p.rcos + o);
    rcs[s][1] = *(const floatx4*)(p.rsin + o);
  }
  bf16x8 qf[12];  // this wave's 32 queries as MFMA B fragments: features 16 s + 8 lg .. +8

  // ---- fragment offsets inside a stage (tile-invariant).
  // K fragment (s, mb): key row 32 mb + lr.  s < 8: content chunk 2 s + lg;
  // s >= 8: rotary chunk 2 (s - 8) + lg.  (row & 15) = (lr & 15) and
  // ((row >> 1) & 7) = ((lr >> 1) & 7) for both mb.
  int kc_off[8], kr_off[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) kc_off[s] = lr * 256 + 16 * ((2 * s + lg) ^ (lr & 15));
#pragma unroll
  for (int s = 0; s < 4; ++s) kr_off[s] = PP_KC + lr * 128 + 16 * ((2 * s + lg) ^ ((lr >> 1) & 7));
  // V^T fragment (k-step ks = 2 mb + ih, feature block d), read r = 0, 1:
  // in 16-lane group G, lane s16 addresses key row 32 mb + 16 ih + 8 r +
  // 4 (G >> 1) + (s16 >> 2) and features 32 d + 16 (G & 1) + 4 (s16 & 3).
  // The value swizzle depends on row & 3 only, so the offset is tile-invariant
  // per (d, r) up to the immediate (32 mb + 16 ih) * 256.
  int v_off[4][2];
  {
    const int G = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + 4 * (G >> 1) + (s16 >> 2);
        const int fb = 2 * (32 * d + 16 * (G & 1) + 4 * (s16 & 3));  // byte in row
        v_off[d][r] = PP_KC + PP_KR + row * 256 + 16 * ((fb >> 4) ^ pp_vswz(row)) + (fb & 15);
      }
  }

  floatx16 O[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[d][e] = 0.f;
  floatx16 S[2];
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

#define PP_QK(tt)                                                                            \
  do {                                                                                       \
    const char* sb_ = lds + (((tt) - k_lo) % PP_NST) * PP_STG;                               \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                         \
      _Pragma("unroll") for (int e = 0; e < 16; ++e) S[mb][e] = 0.f;                         \
    constexpr int RQ = 6;                                                                    \
    bf16x8 fk[RQ];                                                                           \
    _Pragma("unroll") for (int u = 0; u < RQ; ++u) fk[u] = PP_KFRAG(sb_, u);                 \
    _Pragma("unroll") for (int x = 0; x < 24; ++x) {                                         \
      S[x & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[x % RQ], qf[x >> 1], S[x & 1], 0, 0, 0); \
      if (x + RQ < 24) fk[x % RQ] = PP_KFRAG(sb_, x + RQ);                                   \
    }                                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x100, RQ, 0);                                      \
    _Pragma("unroll") for (int x = 0; x < 24; ++x) {                                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
      if (x + RQ < 24) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    \
    }                                                                                        \
  } while (0)
  // fragment x = 2 s + mb
#define PP_KFRAG(sb, x)                                                                      \
  (*(const bf16x8*)((sb) + (((x) >> 1) < 8 ? kc_off[((x) >> 1) & 7] + 8192 * ((x) & 1)     \
                                          : kr_off[((x) >> 1) & 3] + 4096 * ((x) & 1))))

  // transposed V^T fragment y = 4 ks + d (ks = 2 mb + ih): two 4-key reads
#define PP_VREAD(sb, y, dst)                                                                 \
  do {                                                                                       \
    const char* vb_ = (sb) + (32 * ((y) >> 3) + 16 * (((y) >> 2) & 1)) * 256;                \
    (dst)[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                      \
        (__attribute__((address_space(3))) s16x4*)(vb_ + v_off[(y) & 3][0]));                \
    (dst)[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                      \
        (__attribute__((address_space(3))) s16x4*)(vb_ + v_off[(y) & 3][1]));                \
  } while (0)
  // softmax of tile tt (scores in S) and O += V^T . P^T
#define PP_SMPV(tt)                                                                          \
  do {                                                                                       \
    const int kv0_ = 64 * (tt);                                                              \
    float tmax = -INFINITY;                                                                  \
    if (kv0_ + 63 > wq_first) {                                                              \
      _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                       \
        _Pragma("unroll") for (int e = 0; e < 16; ++e) {                                     \
          const int key = kv0_ + 32 * mb + 8 * (e >> 2) + 4 * lg + (e & 3);                  \
          if (key > qi) S[mb][e] = -INFINITY;                                                \
          tmax = fmaxf(tmax, S[mb][e]);                                                      \
        }                                                                                    \
    } else {                                                                                 \
      _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                       \
        _Pragma("unroll") for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, S[mb][e]);         \
    }                                                                                        \
    {                                                                                        \
      const auto x32_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),              \
                                                         __float_as_uint(tmax), false, false); \
      tmax = fmaxf(__uint_as_float(x32_[0]), __uint_as_float(x32_[1])) * sl2;               \
    }                                                                                        \
    const bool raise_ = tmax > m_run + PP_LAZY;                                              \
    const float m_new_ = raise_ ? tmax : m_run;                                              \
    /* a query whose keys so far are all masked keeps m = -inf; it subtracts 0 */           \
    const float m_sub_ = m_new_ == -INFINITY ? 0.f : m_new_;                                 \
    if (__any(raise_)) {                                                                     \
      const float alpha_ = __builtin_amdgcn_exp2f(m_run - m_sub_);                           \
      l_run *= alpha_;                                                                       \
      _Pragma("unroll") for (int d = 0; d < 4; ++d)                                          \
        _Pragma("unroll") for (int e = 0; e < 16; ++e) O[d][e] *= alpha_;                    \
    }                                                                                        \
    m_run = m_new_;                                                                          \
    float psum_ = 0.f;                                                                       \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                         \
      _Pragma("unroll") for (int e = 0; e < 16; ++e) {                                       \
        const float pv_ = __builtin_amdgcn_exp2f(fmaf(S[mb][e], sl2, -m_sub_));              \
        S[mb][e] = pv_;                                                                      \
        psum_ += pv_;                                                                        \
      }                                                                                      \
    l_run += psum_;                                                                          \
    const char* sb_ = lds + (((tt) - k_lo) % PP_NST) * PP_STG;                               \
    /* fragment y = 4 ks + d; a ring of 3 keeps the transposed reads 2 ahead */             \
    s16x4 tv_[3][2];                                                                         \
    _Pragma("unroll") for (int y = 0; y < 2; ++y) PP_VREAD(sb_, y, tv_[y]);                  \
    bf16x8 pf_;                                                                              \
    _Pragma("unroll") for (int y = 0; y < 16; ++y) {                                         \
      const int ks = y >> 2, d = y & 3;                                                      \
      if (d == 0) {                                                                          \
        _Pragma("unroll") for (int m = 0; m < 8; ++m)                                        \
          pf_[m] = (__bf16)S[ks >> 1][8 * (ks & 1) + m];                                     \
      }                                                                                      \
      if (y + 2 < 16) PP_VREAD(sb_, y + 2, tv_[(y + 2) % 3]);                                \
      const s16x4 lo_ = tv_[y % 3][0], hi_ = tv_[y % 3][1];                                  \
      const bf16x8 a_ = __builtin_bit_cast(                                                  \
          bf16x8, s16x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]});    \
      O[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_, pf_, O[d], 0, 0, 0);                \
    }                                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                       \
    _Pragma("unroll") for (int y = 0; y < 16; ++y) {                                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
      if (y + 2 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                     \
    }                                                                                        \
  } while (0)

  // Prologue: tile 0 landed (NST = 3 keeps one tile in flight per segment).
  // Segment boundaries: the first half crosses one after PV(k), the second
  // half after QK(k); both halves meet the same n_kv - 1 barriers.  At a
  // boundary a wave first makes its own loads of the next tile land, then
  // (after the barrier) issues its loads of the tile NST - 2 ahead into the
  // buffer whose last reader (PV of the second half) finished before it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    // the rotary features (s >= 8) are rotated by the RoPE row of the position
    const int r = 32 * w + lr;
    const char* qs = lds + PP_STG + r * PP_QROW;
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      u32x4 v = *(const u32x4*)(qs + 16 * ((2 * s + lg) ^ pp_qswz(r)));
      if (s >= 8) {
        const floatx4 c = rcs[s - 8][0], sn = rcs[s - 8][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = lo_bf(v[i]), bb = hi_bf(v[i]);
          v[i] = pack2bf(a * c[i] - bb * sn[i], a * sn[i] + bb * c[i]);
        }
      }
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();  // every wave's queries read: slots 1 and 2 take key tiles now
  if (k_lo + PP_NST - 2 < n_kv) PP_ISSUE(k_lo + PP_NST - 2);
  for (int k = k_lo; k < n_kv; ++k) {
    // The fragment offsets are loop-invariant, and left alone the compiler
    // hoists every (offset + immediate) sum out of the loop (over 50 live
    // registers); marking them as redefined here keeps those sums inside the
    // loop, where they fold into the reads' offset fields.
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(kc_off[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(kr_off[i]));
#pragma unroll
    for (int d = 0; d < 4; ++d) asm volatile("" : "+v"(v_off[d][0]), "+v"(v_off[d][1]));
    const bool live = 64 * k <= wq_last;
    const bool more = k + 1 < n_kv;
    if (live) PP_QK(k);
    if (second && more) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (k + PP_NST - 1 < n_kv) PP_ISSUE(k + PP_NST - 1);
    }
    if (live) PP_SMPV(k);
    if (!second && more) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (k + PP_NST - 1 < n_kv) PP_ISSUE(k + PP_NST - 1);
    }
  }
#undef PP_ISSUE
#undef PP_QK
#undef PP_KFRAG
#undef PP_SMPV
#undef PP_VREAD

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (p.nsplit > 1) {
    // split partial: unnormalised O^T columns and (m, l) of this query.  The
    // fp32 tile goes through the (now free) ring as 256 rows of 512 bytes,
    // 16-byte chunk c of row r at c ^ (r & 31), and leaves as whole row
    // records, 16 bytes per lane.
    if (qrow_l < p.T && lg == 0) {
      const long rec = ((long)sp * p.B * p.T + rowbase + qrow_l) * HS + h;
      *(floatx2*)(p.ostat + 2 * rec) = floatx2{m_run, l_tot};
    }
    __syncthreads();  // every wave's last key tile read
    {
      const int r = 32 * w + lr;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(floatx4*)(lds + r * 512 + 16 * ((8 * d + 2 * i + lg) ^ (r & 31))) =
              floatx4{O[d][4 * i + 0], O[d][4 * i + 1], O[d][4 * i + 2], O[d][4 * i + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PP_BQ * 32 / 512; ++it) {
      const int idx = tid + 512 * it, r = idx >> 5, c = idx & 31;
      const floatx4 v = *(const floatx4*)(lds + r * 512 + 16 * (c ^ (r & 31)));
      if (q0 + r < p.T) {
        const long rec = ((long)sp * p.B * p.T + rowbase + q0 + r) * HS + h;
        *(floatx4*)(p.opart + rec * 128 + 4 * c) = v;
      }
    }
    return;
  }
  // The normalised tile goes through the (now free) ring as 256 rows of
  // 256 bytes, 16-byte chunk c of row r at c ^ (r & 15), and leaves as whole
  // row segments, 16 bytes per lane (a lane's own outputs are 8-byte pieces
  // of 32 different rows per store).
  const float inv = 1.f / l_tot;
  __syncthreads();  // every wave's last key tile read
  {
    const int r = 32 * w + lr;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 v;
        v[0] = pack2bf(O[d][4 * i + 0] * inv, O[d][4 * i + 1] * inv);
        v[1] = pack2bf(O[d][4 * i + 2] * inv, O[d][4 * i + 3] * inv);
        *(u32x2*)(lds + r * 256 + 16 * ((4 * d + i) ^ (r & 15)) + 8 * lg) = v;
      }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < PP_BQ * 16 / 512; ++it) {
    const int idx = tid + 512 * it, r = idx >> 4, c = idx & 15;
    const u32x4 v = *(const u32x4*)(lds + r * 256 + 16 * (c ^ (r & 15)));
    if (q0 + r < p.T) *(u32x4*)(p.out + (rowbase + q0 + r) * (HS * 128) + (long)h * 128 + 8 * c) = v;
  }
}

void flash_set_prefill_layout(FlashParams& p) {
  const long kvrow = (long)p.H * 256;  // elements per token row of kv
  p.kc = p.kv;       p.kc_b = (long)p.T * kvrow; p.kc_h = 256; p.kc_kb = (int)(kvrow * 2);
  p.vv = p.kv + 128; p.v_b = p.kc_b;             p.v_h = 256;  p.v_kb = p.kc_kb;
  p.kr2 = p.kr;      p.kr_b = (long)p.T * 64;    p.kr_h = 0;   p.kr_kb = 128;
  p.P0 = 0;
  p.nsplit = 1; p.opart = p.ostat = nullptr;
}

bool flash_prefill_fits(int T, int H) {
  FlashParams p;
  memset(&p, 0, sizeof p);
  p.T = T; p.H = H; p.B = 1;
  p.kc_kb = p.v_kb = H * 256 * 2;  // the prefill layout's per-key strides
  p.kr_kb = 128;
  return flash_pp_ok(p);
}

bool flash_pp_ok(const FlashParams& p) {
  // per-key byte offsets (64 keys past the last tile included) stay below 2^31
  const long nk = (long)p.P0 + p.T + 64;
  // the staged query rows' byte offsets stay below 2^31 too
  return p.P0 >= 0 && nk * p.kc_kb < 0x7fffffffL && nk * p.kr_kb < 0x7fffffffL &&
         (long)p.T * p.H * PP_QROW < 0x7fffffffL &&
         nk * p.v_kb < 0x7fffffffL && p.kc_kb % 16 == 0 && p.kr_kb % 16 == 0 && p.v_kb % 16 == 0;
}

hipError_t flash_prefill_pp_bf16(const FlashParams& p, hipStream_t s) {
  if (!flash_pp_ok(p)) return hipErrorInvalidValue;
  if (p.nsplit < 1 || (p.nsplit > 1 && (!p.opart || !p.ostat))) return hipErrorInvalidValue;
  const int nqt = (p.T + PP_BQ - 1) / PP_BQ;
  hipLaunchKernelGGL(flash_pp_kernel, dim3(nqt * p.H * p.B * p.nsplit), dim3(512), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  return flash_combine_bf16(p, s);
}

// Merge of the key splits: one thread per (row, head, 4 features); split s
// weighs by 2^(m_s - max m) and the sum is divided by sum 2^(m_s - max m) l_s.
__global__ __launch_bounds__(256) void flash_combine_kernel(const float* __restrict__ opart,
                                                            const float* __restrict__ ostat, int nsplit,
                                                            long rows_h, bf16_t* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;  // (row, head) * 32 + feature quad
  if (idx >= rows_h * 32) return;
  const long rh = idx >> 5;
  const int f4 = (int)(idx & 31);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ostat[2 * (s * rows_h + rh)]);
  float L = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const floatx2 ml = *(const floatx2*)(ostat + 2 * (s * rows_h + rh));
    const float f = exp2f(ml[0] - M);
    L += f * ml[1];
    acc += f * *(const floatx4*)(opart + (s * rows_h + rh) * 128 + 4 * f4);
  }
  const float inv = 1.f / L;
  *(u32x2*)(out + rh * 128 + 4 * f4) = u32x2{pack2bf(acc[0] * inv, acc[1] * inv), pack2bf(acc[2] * inv, acc[3] * inv)};
}

hipError_t flash_combine_bf16(const FlashParams& p, hipStream_t s) {
  const long rows_h = (long)p.B * p.T * p.H;
  hipLaunchKernelGGL(flash_combine_kernel, dim3((unsigned)((rows_h * 32 + 255) / 256)), dim3(256), 0, s,
                     p.opart, p.ostat, p.nsplit, rows_h, p.out);
  return hipGetLastError();
}

}  // namespace mla
