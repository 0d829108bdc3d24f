// The bf16 latent-cache decode step as one persistent, cooperative kernel.
//
// Sources: "Kimi K2 · Mix and project" (decode mode: one new token per
// sequence at position P, attending to L = P + 1 keys; o_proj after the
// head merge) and "Kimi K2 · Key-value compression" (the 576-value latent
// cache entry, W_UK folded into the query and W_UV applied after the
// attention).
//
// The multi-launch step runs eight kernels.  Here one workgroup per CU (256
// threads, every workgroup resident: cooperative launch) runs the same eight
// phases in order, each over the virtual grid of its own kernel (workgroup v
// of the phase taken by workgroup v mod G, in turn), with a grid-wide barrier
// between consecutive phases:
//   1. down-projection weight stream        (gemm_stream_body)
//   2. latent RMSNorms, RoPE, cache write   (latent_norm_rope_body, 256 threads)
//   3. q up-projection weight stream        (gemm_stream_body)
//   4. query absorption                     (absorb_q_body)
//   5. split-L attention over the cache     (decode_latent_body)
//   6. merge of the splits with W_UV        (latent_out_body)
//   7. o_proj weight stream                 (gemm_stream_body)
//   8. o_proj split sum (+ bias)            (stream_reduce_body)
// The phases share one LDS buffer, sized for the largest (the attention's
// ring).  The grid barrier is two-level: the workgroups of an XCD count in
// locally and the last of them alone makes that XCD's L2 write its dirty
// lines back (one agent-scope release per XCD instead of one per workgroup:
// 352 -> 308 us per step at B = 32, P = 8192).  That relies on every wave
// having waited for its own stores (s_waitcnt vmcnt(0): acknowledged by its
// XCD's L2) before its workgroup counts in, and on the L2 being shared by all
// CUs of an XCD.  Results equal the multi-launch step's up to the latent norms'
// reduction order (256 threads here; the multi-launch step takes 1,024 for
// decode-sized batches).
#include <cstring>

#include "latent_body.h"
#include "norm_body.h"
#include "stream_body.h"

namespace mla {

namespace {
constexpr int pd_max(int a, int b) { return a > b ? a : b; }
// LDS of the largest phase (the attention ring; the 64-row weight stream is
// 32 bytes smaller)
constexpr int kPersistLds =
    pd_max(pd_max(kLatentAttnLds, stream_lds_bytes<2>()), pd_max(kAbsorbLds, kLatentOutLds));
// polls of a barrier wait before it gives up (about a second)
constexpr unsigned kPollLimit = 1u << 20;
}  // namespace

// Kernel-side parameters: the streams as one-product pairs, the virtual grids.
struct PersistKernelParams {
  StreamPair down, qup, oproj;
  LatentNormParams<bf16_t> norm;
  AbsorbParams ab;
  DecodeLatentParams at;
  unsigned* sync;
  int norm_gy;          // workgroups per row of the norms (1 or 2)
  int ab_gy, ab_gz;     // absorption grid (H, ab_gy, ab_gz)
  int lo_gy;            // merge grid (H, lo_gy)
  long red_n;           // threads of the split sum: M * N / 4
};

// Grid-wide barrier of the resident workgroups, two levels.  Each workgroup
// (thread 0, after the workgroup's own barrier) waits until its own stores
// have reached its XCD's L2 and counts in on its XCD's counter sync[8 + x];
// the last one of the XCD (the count registered at kernel start, sync[16 +
// x]) clears that counter, makes the XCD's L2 write its dirty lines back
// (agent-scope release fence, once per XCD) and counts in globally on
// sync[0]; the last XCD clears sync[0] and advances the generation sync[1].
// Every workgroup polls the generation, then drops stale lines (acquire
// fence).  A wait that sees no new generation after kPollLimit polls gives up
// and sets sync[2].
MLA_DEV unsigned pd_xcc() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7u; }

MLA_DEV void pd_barrier(unsigned* sync, unsigned nxcd) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every wave's stores are in the L2
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned x = pd_xcc();
    const unsigned gen = __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned nloc = __hip_atomic_load(sync + 16 + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned a = __hip_atomic_fetch_add(sync + 8 + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a == nloc - 1) {
      __hip_atomic_store(sync + 8 + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
      const unsigned g = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (g == nxcd - 1) {
        __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    for (unsigned n = 0; __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen; ++n) {
      if (n >= kPollLimit) {
        __hip_atomic_store(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __threadfence();
  }
  __syncthreads();
}

// Registration at kernel start: every workgroup counts in on its XCD's
// sync[16 + x]; the number of XCDs holding workgroups is counted on sync[3]
// by the first of each XCD; a plain one-level barrier then makes the counts
// final before the first phase barrier reads them.
MLA_DEV unsigned pd_register(unsigned* sync, unsigned nwg) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned x = pd_xcc();
    if (__hip_atomic_fetch_add(sync + 16 + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
      __hip_atomic_fetch_add(sync + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    const unsigned gen = __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned a = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a == nwg - 1) {
      __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      for (unsigned n = 0; __hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen; ++n) {
        if (n >= kPollLimit) {
          __hip_atomic_store(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __threadfence();
  }
  __syncthreads();
  return __hip_atomic_load(sync + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB>
__global__ __launch_bounds__(256) void decode_latent_persistent_kernel(PersistKernelParams p) {
  __shared__ __attribute__((aligned(16))) char lds[kPersistLds];
  const int G = (int)gridDim.x, wg = (int)blockIdx.x;
  const unsigned nxcd = pd_register(p.sync, G);
  // 1. down-projection: x . [W_DQ; W_DKVR]^T as weight-stream partials
  for (int v = wg; v < p.down.s[0].G; v += G) {
    gemm_stream_body<MB, 1>(p.down, v, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 2. partial sums, latent norms, RoPE of the shared key, latent-cache slot P
  {
    float* row = (float*)lds;
    float* red = (float*)(lds + (((p.norm.q_lora + p.norm.kv_lora + p.norm.d_rope) * 4 + 15) & ~15));
    for (int v = wg; v < p.norm.M * p.norm_gy; v += G) {
      latent_norm_rope_body<bf16_t, 256>(p.norm, v / p.norm_gy, v % p.norm_gy, p.norm_gy, row, red);
      __syncthreads();
    }
  }
  pd_barrier(p.sync, nxcd);
  // 3. q up-projection as weight-stream partials (summed by the absorption)
  for (int v = wg; v < p.qup.s[0].G; v += G) {
    gemm_stream_body<MB, 1>(p.qup, v, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 4. q~ = Q^C W_UK per head, with the roped rotary query
  for (int v = wg; v < p.ab.H * p.ab_gy * p.ab_gz; v += G) {
    const int h = v % p.ab.H, r = v / p.ab.H;
    absorb_q_body<false>(p.ab, h, r % p.ab_gy, r / p.ab_gy, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 5. split-L attention over the latent cache
  for (int v = wg; v < p.at.G; v += G) {
    decode_latent_body(p.at, v, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 6. merge of the splits fused with O_h = o~_h W_UV,h^T
  for (int v = wg; v < p.at.H * p.lo_gy; v += G) {
    latent_out_body(p.at, v % p.at.H, v / p.at.H, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 7. o_proj as weight-stream partials
  for (int v = wg; v < p.oproj.s[0].G; v += G) {
    gemm_stream_body<MB, 1>(p.oproj, v, lds);
    __syncthreads();
  }
  pd_barrier(p.sync, nxcd);
  // 8. fixed-order split sum of o_proj (+ bias) into the output rows
  const GemmParams& o = p.oproj.p[0];
  for (long e = (long)wg * 256 + threadIdx.x; e < p.red_n; e += (long)G * 256)
    stream_reduce_body<bf16_t>(p.oproj.part[0], p.oproj.s[0], o.M, o.N, (bf16_t*)o.C, o.ldc, nullptr, 0,
                               o.bias, e);
}

namespace {
StreamPair pd_pair(const GemmParams& g, const StreamInfo& s, float* part) {
  StreamPair sp;
  sp.p[0] = sp.p[1] = g;
  sp.s[0] = sp.s[1] = s;
  sp.part[0] = sp.part[1] = part;
  sp.n = 1;
  return sp;
}
bool pd_stream_ok(const GemmParams& g, const StreamInfo& s, const float* part) {
  return part && stream_ok(g) && s.u0 == 0 && s.U == s.NB * s.KS && s.G > 0 && s.Mp == (g.M <= 32 ? 32 : 64);
}
}  // namespace

hipError_t decode_latent_persistent_bf16(const PersistLatentParams& h, hipStream_t st) {
  // the checks of each phase's own launcher
  if (!h.sync || !pd_stream_ok(h.down, h.down_si, h.down_part) || !pd_stream_ok(h.qup, h.qup_si, h.qup_part) ||
      !pd_stream_ok(h.oproj, h.oproj_si, h.oproj_part))
    return hipErrorInvalidValue;
  const int Mp = h.down_si.Mp;
  if (h.qup_si.Mp != Mp || h.oproj_si.Mp != Mp || h.down.M != h.norm.M || h.oproj.N % 4) return hipErrorInvalidValue;
  const int n1 = h.norm.q_lora + h.norm.kv_lora + h.norm.d_rope;
  if (!h.norm.stream || n1 % 4 || ((n1 * 4 + 15) & ~15) + 16 > kPersistLds || h.norm.seq_pos) return hipErrorInvalidValue;
  if (h.ab.plan || h.ab.H <= 0 || h.ab.B <= 0 || !h.ab.qpart) return hipErrorInvalidValue;
  const DecodeLatentParams& a = h.at;
  if (a.plan || a.seq_pos || a.H != 64 || !a.w_ukv || a.splits < 1 || a.splits > LO_NSMAX ||
      a.G != a.B * a.splits || a.splits > (a.L + LT - 1) / LT)
    return hipErrorInvalidValue;

  PersistKernelParams p;
  memset(&p, 0, sizeof p);
  p.down = pd_pair(h.down, h.down_si, h.down_part);
  p.qup = pd_pair(h.qup, h.qup_si, h.qup_part);
  p.oproj = pd_pair(h.oproj, h.oproj_si, h.oproj_part);
  p.norm = h.norm;
  p.ab = h.ab;
  p.at = h.at;
  p.sync = h.sync;
  p.norm_gy = h.norm.q_lora % 4 == 0 ? 2 : 1;
  p.ab_gy = 512 / AB_N;
  p.ab_gz = (h.ab.B + 63) / 64;
  p.lo_gy = (a.B + LO_BG - 1) / LO_BG;
  p.red_n = (long)h.oproj.M * (h.oproj.N / 4);

  const void* kern = Mp == 32 ? (const void*)decode_latent_persistent_kernel<1>
                              : (const void*)decode_latent_persistent_kernel<2>;
  int dev = 0, ncu = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
  if (e != hipSuccess) return e;
  if (ncu <= 0 || per_cu <= 0) return hipErrorLaunchFailure;
  // one workgroup per CU: every phase's virtual grid is strided over them
  const int G = ncu;
  e = hipMemsetAsync(h.sync, 0, 96, st);
  if (e != hipSuccess) return e;
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(kern, dim3(G), dim3(256), args, 0, st);
}

}  // namespace mla
