// Device bodies of the absorbed latent-cache decode: the split-L attention
// over the shared [L, 576] latent, the merge of its splits fused with the
// W_UV product, and the query absorption.  Shared by their own kernels
// (decode.hip) and by the persistent latent-decode kernel.
//
// Sources: "Kimi K2 · Key-value compression" (the latent cache holds 576
// values per position: the 512 normalised latent plus the 64 rotary-key
// features; W_UK folded into the query, W_UV applied after the attention)
// and "Kimi K2 · Mix and project" (decode mode: one query per sequence over
// L = P + 1 keys; scaled scores, float32 softmax, P.V).
#pragma once
#include "common.h"
#include "kernels.h"
#include "stream_sum.h"

namespace mla {

// ------------------------------------------------------------------------
// latent-cache decode (absorbed)
// ------------------------------------------------------------------------
namespace {
constexpr int LT = 32;                  // keys per tile
constexpr int ROWB = 1152;              // bytes per cache row (576 bf16)
constexpr int STAGE = LT * ROWB;        // one tile in LDS
constexpr int NST = 4;                  // LDS ring depth: NST - 1 tiles in flight
constexpr int DMA_PER_WAVE = STAGE / 1024 / 4;  // 1 KB per wave-wide DMA, 4 waves
// A head's running max is raised only when a tile exceeds it by this many
// log2 units, so bf16 probabilities stay below 2^16.
constexpr float LAZY_L = 16.0f;

// Tile layout in LDS: 16-byte chunk c (0..71) of key row r sits at chunk slot
// r * 72 + ((c & ~7) | ((c ^ lat_fr(r)) & 7)), with lat_fr a permutation of
// the row pair index u = (r >> 1) & 7.  Rows are 1152 bytes (4.5 windows of
// 64 banks), so both reads of a tile depend on u alone: the QK read (16 rows,
// one chunk each per 16 lanes) and the transposed PV read (8 rows x 2
// chunks).  Of the 168 linear (GF(2)) permutations of u, this one was
// measured free of bank conflicts for both on gfx950 (hardware counters);
// u itself leaves the PV reads 2-way, a rotation of u the QK reads.
MLA_DEV int lat_fr(int r) {
  const int u = (r >> 1) & 7;
  return ((u << 1) ^ (0 - (u >> 2))) & 7;  // 0 2 4 6 7 5 3 1
}
MLA_DEV int lat_slot(int c, int r) { return (c & ~7) | ((c ^ lat_fr(r)) & 7); }

// Wave-wide direct-to-LDS load: lane l's 16 bytes at global
// rsrc.base + voff go to LDS byte m0 + 16 l; lanes past the resource's size
// write zeros.  Issued from asm so the compiler's wait counting, which cannot
// tell ring stages apart and would wait for every load in flight, stays out;
// the kernel waits with explicit vmcnt values instead.
MLA_DEV void dma16(unsigned m0, int voff, u32x4 rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
MLA_DEV u32x4 lat_rsrc(const char* base, int bytes) {
  const unsigned long a = (unsigned long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)max(bytes, 0));
  r[3] = 0x00020000u;  // raw buffer, 32-bit data format
  return r;
}
// wait until at most n tiles of this wave's DMAs are still in flight
MLA_DEV void wait_tiles(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * DMA_PER_WAVE) : "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(DMA_PER_WAVE) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
}  // namespace

// block-wide sum / max of one int per thread (256 threads)
MLA_DEV int block_sum_int(int x, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
MLA_DEV int block_max_int(int x, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

// Split plan of the absorbed-cache attention, computed by one workgroup of
// 256 threads.  The keys of sequence b (0 .. its position) form n_b 32-key
// tiles.  With c the smallest tile count such that sum_b ceil(n_b / c) <= G,
// sequence b gets s_b = ceil(n_b / c) workgroups, which split its tiles
// evenly (at most c tiles each, at least one), so the longest run is as short
// as whole-sequence runs allow.  Output (ints): plan[v] = sequence of
// workgroup v (-1: idle), plan[G + v] and plan[2 G + v] = its key range
// [j0, j1); plan[3 G + b] and plan[3 G + B + b] = first workgroup and count of
// sequence b.  Needs B <= G and B <= LP_NS.
constexpr int LP_NS = 1024;  // sequences the plan handles (tile counts kept in LDS)
MLA_DEV void latent_plan(int B, int L, const int* seq_pos, int G, int* plan) {
  __shared__ int red[4];
  __shared__ int ns[LP_NS], ss[LP_NS], fs[LP_NS];  // tiles, workgroups, first workgroup
  const int tid = threadIdx.x;
  int t = 0, mx = 0;
  for (int b = tid; b < B; b += 256) {
    const int n = (seq_position(seq_pos, b, L - 1, L - 1) + LT) / LT;
    ns[b] = n;
    t += n;
    mx = max(mx, n);
  }
  t = block_sum_int(t, red);
  mx = block_max_int(mx, red);
  // sum_b ceil(n_b / c) <= t / c + B, so c >= t / (G - B) always fits
  int lo = max(1, (t + G - 1) / G);
  int hi = G > B ? min(mx, (t + G - B - 1) / (G - B)) : mx;
  hi = max(lo, hi);
  while (lo < hi) {  // the same bounds in every thread
    const int c = (lo + hi) / 2;
    int k = 0;
    for (int b = tid; b < B; b += 256) k += (ns[b] + c - 1) / c;
    if (block_sum_int(k, red) <= G) hi = c;
    else lo = c + 1;
  }
  for (int b = tid; b < B; b += 256) ss[b] = (ns[b] + lo - 1) / lo;
  __syncthreads();
  if (tid == 0) {
    int v = 0;
    for (int b = 0; b < B; ++b) {
      fs[b] = v;
      v += ss[b];
    }
    red[0] = v;
  }
  __syncthreads();
  const int used = red[0];
  for (int b = tid; b < B; b += 256) {
    plan[3 * G + b] = fs[b];
    plan[3 * G + B + b] = ss[b];
  }
  for (int v = tid; v < G; v += 256) {
    if (v >= used) {
      plan[v] = -1;
      continue;
    }
    int bl = 0, bh = B - 1;  // last sequence whose first workgroup is <= v
    while (bl < bh) {
      const int m = (bl + bh + 1) / 2;
      if (fs[m] <= v) bl = m;
      else bh = m - 1;
    }
    const int k = v - fs[bl], s = ss[bl], n = ns[bl];
    const int Lb = seq_position(seq_pos, bl, L - 1, L - 1) + 1;
    plan[v] = bl;
    plan[G + v] = LT * (k * n / s);
    plan[2 * G + v] = min(Lb, LT * ((k + 1) * n / s));
  }
}

// One workgroup = one run of key tiles of one sequence (latent_plan); 4 waves
// x 16 heads.  Per tile of
// 32 cache rows: S^T[key, head] = C[key, 0:576] . q~[head]^T (16x16x32 MFMA,
// key rows read from LDS, the absorbed query held in registers), exp2 in
// registers, O~^T[feature, head] += C^T[feature, key] . P^T with the C^T
// operand read straight from the row-major tile by ds_read_b64_tr_b16 (two
// 4-key reads per MFMA).  Tiles stream through an NST-stage LDS ring by
// direct-to-LDS buffer loads, NST - 1 tiles ahead of the compute.
//
// k-slot order of the PV product: the QK accumulator holds keys
// 16 mb + 4 g + j in lane group g, so slot 8 g + 4 mb + j; a transposed read
// of rows 16 mb + 4 g + (0..3) yields slots 8 g + 4 mb + (0..3).
//
// The running max is raised lazily.  When a head's tile max clears its
// current max by LAZY_L after the first tile, the workgroup restarts its
// split with the higher max rather than rescaling 128 accumulators per lane,
// so the hot loop carries no rescale at all.  Each restart needs a jump of
// 2^16 in some head's probabilities; splits with ordinary score ranges never
// restart.
// LDS bytes of decode_latent_body
constexpr int kLatentAttnLds = NST * STAGE + 32;

// Workgroup v of the split-L attention (256 threads); lds: kLatentAttnLds
// bytes, 16-byte aligned.
MLA_DEV void decode_latent_body(const DecodeLatentParams& p, int v, char* lds) {
  int* rflag = (int*)(lds + NST * STAGE);
  const unsigned lds_base = (unsigned)(unsigned long)(__attribute__((address_space(3))) char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int head = 16 * w + l16;
  // this workgroup's sequence and key range: from latent_plan, or (one
  // length for all) split k of sequence v / splits, an even share of its tiles
  int b, j0, j1;
  if (p.plan) {
    b = p.plan[v];
    if (b < 0) return;  // idle: fewer runs than workgroups
    j0 = p.plan[p.G + v];
    j1 = p.plan[2 * p.G + v];
  } else {
    b = v / p.splits;
    const int k = v - b * p.splits, n = (p.L + LT - 1) / LT;
    j0 = LT * (k * n / p.splits);
    j1 = min(p.L, LT * ((k + 1) * n / p.splits));
  }
  const int ntiles = (j1 - j0 + LT - 1) / LT;  // >= 1
  const char* cb = (const char*)(p.cache + ((long)b * p.L_cap + j0) * 576);

  // DMA k of this wave fills LDS bytes [1024 (w * DMA_PER_WAVE + k), +1024) of
  // a stage: chunk slot P = 64 (w * DMA_PER_WAVE + k) + lane holds row P / 72,
  // logical chunk lat_slot(P % 72, row) (the swizzle is an involution).
  int voff[DMA_PER_WAVE];
#pragma unroll
  for (int k = 0; k < DMA_PER_WAVE; ++k) {
    const int P = 64 * (w * DMA_PER_WAVE + k) + lane, row = P / 72;
    voff[k] = row * ROWB + 16 * lat_slot(P % 72, row);
  }
#define LAT_ISSUE(tt)                                                                       \
  do {                                                                                      \
    const u32x4 rs_ = lat_rsrc(cb + (long)(tt) * LT * ROWB, (j1 - j0 - (tt) * LT) * ROWB);   \
    const unsigned m0_ = lds_base + ((tt) % NST) * STAGE + w * DMA_PER_WAVE * 1024;         \
    _Pragma("unroll") for (int k = 0; k < DMA_PER_WAVE; ++k) dma16(m0_ + 1024 * k, voff[k], rs_); \
  } while (0)

  // QK fragment (s, mb): row 16 mb + l16, chunk 4 s + g4
  //   -> qk_off[s & 1] + 16 ROWB mb + 128 (s >> 1)
  int qk_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    qk_off[par] = l16 * ROWB + 16 * (((4 * par + g4) ^ lat_fr(l16)) & 7);
  // PV transposed read (n, mb): source row 16 mb + 4 g4 + (l16 >> 2), features
  // 16 n + 4 (l16 & 3) .. + 3  ->  pv_off[n & 3] + 16 ROWB mb + 128 (n >> 2)
  int pv_off[4];
#pragma unroll
  for (int n3 = 0; n3 < 4; ++n3) {
    const int row = 4 * g4 + (l16 >> 2);
    const int c = 2 * n3 + ((l16 >> 1) & 1);
    pv_off[n3] = row * ROWB + 16 * ((c ^ lat_fr(row)) & 7) + 8 * (l16 & 1);
  }

  // The first tiles are issued before the query is loaded, so the two are in
  // flight together.
  for (int tt = 0; tt < NST - 1 && tt < ntiles; ++tt) LAT_ISSUE(tt);
  // [q~ | roped q^R] of this head, laid out like a cache row
  bf16x8 qf[18];
#pragma unroll
  for (int s = 0; s < 18; ++s)
    qf[s] = *(const bf16x8*)(p.q_abs + ((long)b * p.H + head) * 576 + 32 * s + 8 * g4);

  const float sl2 = p.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  floatx4 O[32];
  bool restart = true, first_pass = true;
  while (restart) {
    restart = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      O[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(O[i]));  // keep the accumulators in AGPRs across both loops
    }
    l_run = 0.f;
    if (!first_pass)
      for (int tt = 0; tt < NST - 1 && tt < ntiles; ++tt) LAT_ISSUE(tt);
    first_pass = false;
    for (int t = 0;; ++t) {
      wait_tiles(min(NST - 2, ntiles - 1 - t));
      __syncthreads();
      if (t > 0) {
        const int4 fl = *(const int4*)&rflag[4 * ((t - 1) & 1)];
        if (fl.x | fl.y | fl.z | fl.w) {
          restart = true;
          break;
        }
      }
      if (t == ntiles) break;
      if (t + NST - 1 < ntiles) LAT_ISSUE(t + NST - 1);
#pragma unroll
      for (int i = 0; i < 32; ++i) asm volatile("" : "+a"(O[i]));
      const char* cs = lds + (t % NST) * STAGE;
      const int kv0 = j0 + t * LT;

      // QK: 36 fragments read RQ ahead of their MFMA, four accumulation chains
      constexpr int RQ = 8, RP = 8;
#define QK_FRAG(x) (*(const bf16x8*)(cs + qk_off[((x) >> 1) & 1] + 16 * ROWB * ((x) & 1) + 128 * ((x) >> 2)))
#define PV_FRAG(y)                                                                          \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                                  \
      (__attribute__((address_space(3))) s16x4*)(cs + pv_off[((y) >> 1) & 3] +             \
                                                  16 * ROWB * ((y) & 1) + 128 * ((y) >> 3)))
      bf16x8 fa[RQ];
#pragma unroll
      for (int u = 0; u < RQ; ++u) fa[u] = QK_FRAG(u);
      floatx4 S4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) S4[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 36; ++x) {
        const int s = x >> 1, mb = x & 1;
        S4[mb + 2 * (s & 1)] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[x % RQ], qf[s], S4[mb + 2 * (s & 1)], 0, 0, 0);
        if (x + RQ < 36) fa[x % RQ] = QK_FRAG(x + RQ);
      }
      // PV operand halves y = 2 n + mb; the first ones do not depend on the
      // softmax, so they are read under the tail of the QK products
      s16x4 fp[2 * RP];
#pragma unroll
      for (int u = 0; u < 2 * RP; ++u) fp[u] = PV_FRAG(u);
      __builtin_amdgcn_sched_group_barrier(0x100, RQ, 0);
#pragma unroll
      for (int x = 0; x < 36; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x < 36 - RQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      floatx4 S[2] = {S4[0] + S4[2], S4[1] + S4[3]};
      // S[mb][jj]: key 16 mb + 4 g4 + jj of the tile, head `head`
      if (kv0 + LT > j1) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (kv0 + 16 * mb + 4 * g4 + jj >= j1) S[mb][jj] = -INFINITY;
      }
      float tmax = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                         fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
      {  // max over the four lane groups (same head): lanes l ^ 16, l ^ 32
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1])) * sl2;
      }
      const bool raise = tmax > m_run + LAZY_L;
      if (raise) m_run = tmax;
      // the accumulators are still zero on the first tile: no restart needed
      const bool redo = __any(raise) && t > 0;
      float psum = 0.f;
      bf16x8 pf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(S[mb][jj], sl2, -m_run));
          psum += pv;
          pf[4 * mb + jj] = (__bf16)pv;
        }
      l_run += psum;
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        const s16x4 lo = fp[(2 * n) % (2 * RP)], hi = fp[(2 * n + 1) % (2 * RP)];
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        O[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, O[n], 0, 0, 0);
        if (n + RP < 32) {
          fp[(2 * n) % (2 * RP)] = PV_FRAG(2 * (n + RP));
          fp[(2 * n + 1) % (2 * RP)] = PV_FRAG(2 * (n + RP) + 1);
        }
      }
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (n + RP < 32) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#undef QK_FRAG
#undef PV_FRAG
      if (lane == 0) rflag[4 * (t & 1) + w] = redo ? 1 : 0;
    }
    if (restart) {
      // drain the ring before it is refilled from the first tile
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

#undef LAT_ISSUE
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  // split record: (m, l) in fp32 and o~[512] rounded to bf16 (the merge
  // weights it by 2^(m - max m) / L and rounds the merged o~ to bf16 again for
  // the W_UV product)
  const long rec = (long)v * p.H + head;
  if (g4 == 0) *(floatx2*)(p.stats + 2 * rec) = floatx2{m_run, l_tot};
  // o~ goes through the (drained) ring as 64 records of 1 KB, 16-byte chunk
  // c of record r at c ^ (r & 63) (a lane's own values are 8-byte pieces of
  // 16 records per store), and leaves as whole records, 16 bytes per lane
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave's last tile read
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    // features 16 i + 4 g4 .. + 3: chunk 2 i + (g4 >> 1), half g4 & 1
    const int c = 2 * i + (g4 >> 1);
    *(u32x2*)(lds + head * 1024 + 16 * (c ^ (head & 63)) + 8 * (g4 & 1)) =
        u32x2{pack2bf(O[i][0], O[i][1]), pack2bf(O[i][2], O[i][3])};
  }
  __syncthreads();
  bf16_t* ob = p.opart + (long)v * p.H * 512;
#pragma unroll
  for (int it = 0; it < 64 * 64 / 256; ++it) {
    const int idx = tid + 256 * it, r = idx >> 6, c = idx & 63;
    *(u32x4*)(ob + (long)r * 512 + 8 * c) = *(const u32x4*)(lds + r * 1024 + 16 * (c ^ (r & 63)));
  }
}

// Merge of the split partials fused with the value up-projection: one
// workgroup per (head h, group of LO_BG = 8 sequences).  The merged latent
// outputs o~ [8][512] go to LDS as bf16 (the precision of the W_UV product's
// operand), and O[b, h*128 + c] = o~[b] . W_UV,h[c] is one
// v_mfma_f32_32x32x16_bf16 chain per wave: rows = the 8 sequences (rows 8..31
// of the A operand are zero), columns = 32 of the head's 128 values (wave w:
// 32 w .. 32 w + 31), k = the 512 latent features.  Each lane's B operand,
// row c of W_UV,h (kv_b_proj row h*256 + 128 + c), is loaded into registers
// first, in flight while the splits are merged.  The workgroups of one head
// run on one XCD (grid x = head), so its 128 KB of W_UV rows come from HBM
// once.
namespace {
constexpr int LO_BG = 8;        // sequences per workgroup
constexpr int LO_NSMAX = 256;   // workgroups per sequence (latent_plan: at most 256)
}

// LDS bytes of latent_out_body: o~ rows, split weights and sums, record ranges
constexpr int kLatentOutLds = LO_BG * 1024 + 2 * LO_BG * LO_NSMAX * 4 + 2 * LO_BG * 4;

// Workgroup (head h, sequences LO_BG by .. LO_BG by + LO_BG - 1), 256
// threads; lds: kLatentOutLds bytes, 16-byte aligned.
MLA_DEV void latent_out_body(const DecodeLatentParams& p, int h, int by, char* lds) {
  char* otb = lds;  // o~ bf16, 16-byte chunk c of row r at c ^ r
  float(*wsc)[LO_NSMAX] = (float(*)[LO_NSMAX])(lds + LO_BG * 1024);  // f_s / L per (sequence, split record)
  float(*lsum)[LO_NSMAX] = (float(*)[LO_NSMAX])(lds + LO_BG * 1024 + LO_BG * LO_NSMAX * 4);
  int* wfirst = (int*)(lds + LO_BG * 1024 + 2 * LO_BG * LO_NSMAX * 4);
  int* wcount = wfirst + LO_BG;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int H = p.H, G = p.G;
  const int b0 = by * LO_BG;
  const int nb = min(LO_BG, p.B - b0);
  // B operand of k-step s: W_UV,h[c][16 s + 8 lg .. + 7], c = 32 w + lr
  const bf16_t* wr = p.w_ukv + ((long)h * 256 + 128 + 32 * w + lr) * 512 + 8 * lg;
  bf16x8 wv[32];
#pragma unroll
  for (int s2 = 0; s2 < 32; ++s2) wv[s2] = *(const bf16x8*)(wr + 16 * s2);
  // the attention kernel's records of sequence b0 + j: wcount[j] of them,
  // from slot wfirst[j] on
  if (tid < LO_BG) {
    const int bb = b0 + tid;
    wfirst[tid] = tid >= nb ? 0 : p.plan ? p.plan[3 * G + bb] : bb * p.splits;
    wcount[tid] = tid >= nb ? 0 : p.plan ? p.plan[3 * G + p.B + bb] : p.splits;
  }
  __syncthreads();
  int nsplit = 0;
#pragma unroll
  for (int j = 0; j < LO_BG; ++j) nsplit = max(nsplit, wcount[j]);
  // split statistics (m, l) of every (sequence, record), loaded in parallel
  for (int idx = tid; idx < LO_BG * nsplit; idx += 256) {
    const int j = idx / nsplit, sp = idx - j * nsplit;
    const bool ok = sp < wcount[j];
    const floatx2 ml = ok ? *(const floatx2*)(p.stats + 2 * (((long)wfirst[j] + sp) * H + h))
                          : floatx2{-INFINITY, 0.f};
    wsc[j][sp] = ml[0];
    lsum[j][sp] = ml[1];
  }
  __syncthreads();
  // split weights f_s / L of sequence j: f_s = 2^(m_s - max m), L = sum f_s l_s
  if (tid < nb) {
    const int j = tid;
    float M = -INFINITY;
    for (int sp = 0; sp < wcount[j]; ++sp) M = fmaxf(M, wsc[j][sp]);
    float L = 0.f;
    for (int sp = 0; sp < wcount[j]; ++sp) {
      const float f = exp2f(wsc[j][sp] - M);
      wsc[j][sp] = f;
      L += f * lsum[j][sp];
    }
    const float inv = 1.f / L;
    for (int sp = 0; sp < wcount[j]; ++sp) wsc[j][sp] *= inv;
  }
  __syncthreads();
  // merged o~: thread (k4, jq) merges features 4 k4 .. +3 of sequences
  // jq + 2 i (i < 4), loading 8 splits of all four at once
  {
    constexpr int NI = LO_BG / 2;
    const int k4 = tid & 127, jq = tid >> 7;
    floatx4 m[NI];
    const bf16_t* pp[NI];
    int cnt[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = jq + 2 * i;
      m[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      cnt[i] = j < nb ? wcount[j] : 0;
      pp[i] = p.opart + ((long)wfirst[j] * H + h) * 512 + 4 * k4;
    }
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      u32x2 v[NI][8];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          v[i][q] = s0 + q < cnt[i] ? *(const u32x2*)(pp[i] + (long)(s0 + q) * H * 512) : u32x2{0u, 0u};
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (s0 + q < cnt[i]) {
            const float f = wsc[jq + 2 * i][s0 + q];
            m[i] += f * floatx4{lo_bf(v[i][q][0]), hi_bf(v[i][q][0]), lo_bf(v[i][q][1]), hi_bf(v[i][q][1])};
          }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = jq + 2 * i, ch = k4 >> 1;
      *(u32x2*)(otb + r * 1024 + 16 * (ch ^ r) + 8 * (k4 & 1)) =
          u32x2{pack2bf(m[i][0], m[i][1]), pack2bf(m[i][2], m[i][3])};
    }
  }
  __syncthreads();
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < 32; ++s2) {
    const int ch = 2 * s2 + lg;
    const bf16x8 a = lr < LO_BG ? *(const bf16x8*)(otb + lr * 1024 + 16 * (ch ^ lr)) : bf16x8{};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wv[s2], acc, 0, 0, 0);
  }
  // rows 4 lg + e (e < 4) of the first 8-row block are the sequences
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * lg + e;
    if (j < nb) p.out[(long)(b0 + j) * H * 128 + (long)h * 128 + 32 * w + lr] = f2bf(acc[e]);
  }
}

// ------------------------------------------------------------------------
// query absorption: q~[b,h,k] = sum_c q[b,h,c] * W_UK,h[c,k], c < 128, k < 512
// (the key rows of head h in kv_b_proj, rows h*256 + c), written with the
// roped rotary query into qa[b][h][576] = [q~ (512) | RoPE(q^R, L-1) (64)], the
// same layout as a latent-cache row.  Workgroup = (h, 256 latent features,
// 64 sequences); the W_UK,h tile [128 c][256 k] is stored transposed in LDS
// so that the MFMA B operand is c-contiguous.  The query comes either as
// bf16 q [B][H][192] or as the q up-projection's weight-stream partial blocks
// (summed here in workgroup order).
// ------------------------------------------------------------------------
namespace {
constexpr int AB_N = 64;  // latent features per workgroup
}

// 8 consecutive query features f .. f+7 of head h for R rows b[r] (rows with
// ok[r] false give zeros), as packed bf16
template <int R>
MLA_DEV void absorb_q8(const AbsorbParams& p, int h, const int (&b)[R], const bool (&ok)[R], int f,
                       u32x4 (&o)[R]) {
  if (!p.qpart) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      o[r] = ok[r] ? *(const u32x4*)(p.q + ((long)b[r] * p.H + h) * 192 + f) : u32x4{0u, 0u, 0u, 0u};
    return;
  }
  floatx4 v[R][2];
  stream_sum8_rows<R>(p.qpart, p.qsi, b, ok, h * 192 + f, v);
#pragma unroll
  for (int r = 0; r < R; ++r)
    o[r] = u32x4{pack2bf(v[r][0][0], v[r][0][1]), pack2bf(v[r][0][2], v[r][0][3]),
                 pack2bf(v[r][1][0], v[r][1][1]), pack2bf(v[r][1][2], v[r][1][3])};
}

// LDS bytes of absorb_q_body (the transposed W tile and the query tile)
constexpr int kAbsorbLds = (AB_N * 16 + 64 * 16) * 16;

// Workgroup (head h, latent features AB_N by .., sequences 64 bz ..), 256
// threads; lds: kAbsorbLds bytes, 16-byte aligned.  PLAN: the ragged form's
// split plan may be requested (p.plan), made by workgroup (0, 0, 0).
template <bool PLAN>
MLA_DEV void absorb_q_body(const AbsorbParams& p, int h, int by, int bz, char* lds) {
  u32x4* Wt = (u32x4*)lds;          // [k AB_N][c 128] -> 16 chunks per row, swizzled
  u32x4* Qs = Wt + AB_N * 16;       // [b 64][c 128]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  // the attention kernel's split plan, made by the first workgroup
  if constexpr (PLAN) {
    if (p.plan && h == 0 && by == 0 && bz == 0) latent_plan(p.B, p.L, p.seq_pos, p.G, p.plan);
  }
  const int n0 = by * AB_N, b0 = bz * 64;
  // W tile: 128 c x AB_N k; item = (c pair, k chunk of 8): 64 x AB_N / 8,
  // all of a thread's loads in flight together
  uint32_t* wt32 = (uint32_t*)Wt;
  constexpr int WIT = 64 * AB_N / 8 / 256;
  u32x4 wa_[WIT], wb_[WIT];
#pragma unroll
  for (int it = 0; it < WIT; ++it) {
    const int e = tid + 256 * it;
    const int cp = e & 63, kc = e >> 6;
    const bf16_t* src = p.w_ukv + ((long)h * 256 + 2 * cp) * 512 + n0 + 8 * kc;
    wa_[it] = *(const u32x4*)src;
    wb_[it] = *(const u32x4*)(src + 512);
  }
  // Q tile: 64 rows x 16 chunks of the content query (rows past B are zero);
  // a thread's four rows share chunk c, so their partial loads go together
  {
    const int c = tid & 15;
    int rb[4];
    bool ok[4];
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rb[i] = b0 + (tid >> 4) + 16 * i;
      ok[i] = rb[i] < p.B;
    }
    absorb_q8<4>(p, h, rb, ok, 8 * c, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      Qs[r * 16 + (c ^ (r & 7))] = v[i];
    }
  }
  // rotary query of these rows, roped at position L-1 (64 rows x 8 chunks)
  if (by == 0) {
    const int c = tid & 7;
    int rb[2];
    bool ok[2];
    u32x4 v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rb[i] = b0 + (tid >> 3) + 32 * i;
      ok[i] = rb[i] < p.B;
    }
    absorb_q8<2>(p, h, rb, ok, 128 + 8 * c, v);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (ok[i])
        *(u32x4*)(p.qa + ((long)rb[i] * p.H + h) * 576 + 512 + 8 * c) =
            rope8_bf16(v[i], p.rcos, p.rsin, seq_position(p.seq_pos, rb[i], p.L - 1, p.L - 1), 32, 4 * c);
  }
  // transpose the W tile into LDS last: its loads, issued first, have landed
  // by the time the query sums (issued after them) have
#pragma unroll
  for (int it = 0; it < WIT; ++it) {
    const int e = tid + 256 * it;
    const int cp = e & 63, kc = e >> 6;  // c pair 0..63, k chunk
    const u32x4 a = wa_[it], bb = wb_[it];
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
  __syncthreads();
  // wave w: rows 32 (w >> 1), columns AB_N / 2 (w & 1) + 32 j
  constexpr int NJ = AB_N / 64;
  const int rm = 32 * (w >> 1), cn = (AB_N / 2) * (w & 1);
  floatx16 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int ra = rm + lr;
    const bf16x8 a = __builtin_bit_cast(bf16x8, Qs[ra * 16 + ((2 * s + lg) ^ (ra & 7))]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rbk = cn + 32 * j + lr;
      const bf16x8 bv = __builtin_bit_cast(bf16x8, Wt[rbk * 16 + (((2 * s + lg) ^ (rbk & 7)) & 15)]);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = b0 + rm + 8 * (e >> 2) + 4 * lg + (e & 3);
      const int col = n0 + cn + 32 * j + lr;
      if (row < p.B) p.qa[((long)row * p.H + h) * 576 + col] = f2bf(acc[j][e]);
    }
}

}  // namespace mla
