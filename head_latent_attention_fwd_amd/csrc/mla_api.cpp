// C-ABI host layer of the MLA library: argument validation, workspace
// carving and the launch sequence of each entry point (see include/mla.h).
//
// Launch sequences (bf16; the float32 path mirrors them with the generic
// kernels):
//  prefill : [x W_DQ^T | x W_DKVR^T] (one GEMM over both weights, fp32 out)
//            -> latent RMSNorms + RoPE of the shared key (+ latent cache)
//            -> q up-projection with RoPE epilogue, kv up-projection
//            -> causal flash attention -> o_proj (+ residual in the block)
//            (+ full-cache scatter)
//  decode  : the same projections at M = B with split-K, cache slot P
//            update, decode attention (full or absorbed latent), o_proj.
//  block   : RMSNorm -> prefill with residual -> RMSNorm -> SwiGLU GEMM
//            (W1/W3 interleaved, silu(g)*u epilogue) -> W2 GEMM + residual.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "kernels.h"

using namespace mla;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

#define HIPCHK(expr)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail(MLA_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

// ---- opt-in kernel timing: a pair of HIP events around each named launch
//      on the caller's stream, read back by mla_profile_summary() ----
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
thread_local bool g_prof = false;
thread_local std::vector<ProfRec> g_prof_pending;
thread_local std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr;
  ProfScope(const char* n, hipStream_t s) : name(n), st(s) {
    if (g_prof && (a = prof_event()) && hipEventRecord(a, st) != hipSuccess) {
      g_prof_pool.push_back(a);  // not recorded: no sample for this launch
      a = nullptr;
    }
  }
  ~ProfScope() {
    if (!a) return;
    hipEvent_t b = prof_event();
    if (!b || hipEventRecord(b, st) != hipSuccess) {
      g_prof_pool.push_back(a);
      if (b) g_prof_pool.push_back(b);
      return;
    }
    g_prof_pending.push_back({name, a, b});
  }
};

#define LAUNCH(name, expr)        \
  do {                            \
    ProfScope ps_((name), st);    \
    HIPCHK(expr);                 \
  } while (0)

size_t esize(const mla_dims* d) { return d->dtype == MLA_BF16 ? 2 : 4; }
long rup(long x, long a) { return (x + a - 1) / a * a; }

// Workspace carving: regions aligned to 256 bytes.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (size_t)rup((long)off, 256);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

int check_dims(const mla_dims* d, bool need_ff) {
  if (!d) return fail(MLA_ERR_NULL, "dims is NULL");
  if (d->d_model <= 0 || d->n_heads <= 0 || d->q_lora_rank <= 0 || d->kv_lora_rank <= 0 ||
      d->qk_nope_dim <= 0 || d->qk_rope_dim <= 0 || d->v_head_dim <= 0)
    return fail(MLA_ERR_SHAPE, "every width of mla_dims must be positive");
  if (d->qk_rope_dim % 2) return fail(MLA_ERR_SHAPE, "qk_rope_dim must be even (RoPE pairs)");
  if (need_ff && d->d_ff <= 0) return fail(MLA_ERR_SHAPE, "d_ff must be positive for the block");
  if (!(d->rms_eps >= 0.f) || !std::isfinite(d->softmax_scale) || d->softmax_scale < 0.f)
    return fail(MLA_ERR_SHAPE, "rms_eps must be >= 0 and softmax_scale 0 (default) or positive and finite");
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d is neither MLA_F32 nor MLA_BF16", d->dtype);
  if (d->dtype == MLA_F32) {
    if (d->qk_nope_dim + d->qk_rope_dim > 1024 || d->v_head_dim > 1024 ||
        d->kv_lora_rank + d->qk_rope_dim > 1024)
      return fail(MLA_ERR_UNSUPPORTED, "float32 path: head widths up to 1024");
  } else {
    if (d->qk_nope_dim != 128 || d->qk_rope_dim != 64 || d->v_head_dim != 128)
      return fail(MLA_ERR_UNSUPPORTED,
                  "bf16 path serves the Kimi K2 head widths (nope 128, rope 64, value 128)");
    if (d->d_model % 64 || d->q_lora_rank % 64 || d->kv_lora_rank % 64 ||
        (need_ff && d->d_ff % 64))
      return fail(MLA_ERR_UNSUPPORTED, "bf16 path: d_model, q_lora, kv_lora, d_ff multiples of 64");
  }
  return MLA_OK;
}

// The score scale: softmax_scale when positive, else 1/sqrt(d_nope + d_rope)
// (the head width of the scaled scores in the code excerpt of "Kimi K2 · Mix
// and project"; the same value serves the absorbed form).
float scale_of(const mla_dims* d) {
  if (d->softmax_scale > 0.f) return d->softmax_scale;
  return (float)(1.0 / std::sqrt((double)(d->qk_nope_dim + d->qk_rope_dim)));
}
constexpr float kLog2e = 1.4426950408889634f;

// The bf16 flash kernel addresses keys by 32-bit byte offsets from each
// (sequence, head) base; a prefill whose kv rows do not fit is refused up
// front (no other attention kernel serves it).
int check_flash_prefill(const mla_dims* d, int T) {
  if (d->dtype == MLA_BF16 && !flash_prefill_fits(T, d->n_heads))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 prefill: T=%d with %d heads exceeds the attention kernel's "
                "32-bit key offsets", T, d->n_heads);
  return MLA_OK;
}

// The kernels move every tensor with 16-byte vector and direct-to-LDS
// accesses, so device pointers must be 16-byte aligned (NULL is allowed
// here: the NULL checks are separate).
int check_align(std::initializer_list<const void*> ps, const char* what) {
  for (const void* q : ps)
    if (q && ((uintptr_t)q & 15u))
      return fail(MLA_ERR_UNSUPPORTED, "%s: device pointer %p is not 16-byte aligned", what, q);
  return MLA_OK;
}

int check_weights(const mla_weights* w) {
  if (!w) return fail(MLA_ERR_NULL, "weights is NULL");
  if (!w->w_dq || !w->g_q || !w->w_uqr || !w->w_dkvr || !w->g_kv || !w->w_ukv || !w->w_o)
    return fail(MLA_ERR_NULL, "a weight pointer is NULL");
  return check_align({w->w_dq, w->g_q, w->w_uqr, w->w_dkvr, w->g_kv, w->w_ukv, w->w_o, w->b_dq,
                      w->b_dkvr, w->b_o}, "weights");
}

int check_rope(const float* c, const float* s, int rows, int need) {
  if (!c || !s) return fail(MLA_ERR_NULL, "rope table pointer is NULL");
  if (int r = check_align({c, s}, "rope table")) return r;
  if (rows < need) return fail(MLA_ERR_SHAPE, "rope_rows %d < %d positions needed", rows, need);
  return MLA_OK;
}

// 32-bit element offsets inside the GEMM kernels: every operand must have
// fewer than 2^31 elements.
int check_i32(long elems, const char* what) {
  if (elems >= (long)INT_MAX) return fail(MLA_ERR_UNSUPPORTED, "%s exceeds 2^31 elements", what);
  return MLA_OK;
}


GemmParams gp_base() {
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.ksplit = 1;
  return p;
}

// ----------------------------------------------------------------- layouts
struct ProjBufs {
  void* part;   // fp32 [S][M][N1]
  int S, kchunk;
  int cfg;      // tile config of the down-projection GEMM (prefill)
  bool decode;  // small-M weight-streaming products
  void* cq;     // [M][q_lora]
  void* ckv;    // [M][kv_lora]
  void* kr;     // [M][d_rope]
  void* q;      // [M][H*dqk]
  void* kv;     // [M][H*(dn+dv)]   (NULL when not needed)
  void* o;      // [M][H*dv]
  void* upart;  // fp32 split-K partials of the small-M q up-projection (or NULL)
  size_t upart_floats;
  void* ukvpart;  // ... and of the kv up-projection (its own buffer, so that both
  size_t ukvpart_floats;  // can stay unsummed until the attention kernel reads them)
  void* opart;    // fp32 K-split partials of o_proj for 64 < M <= 1024 rows (or NULL)
  size_t opart_floats;
};

void carve_proj(Carver& c, const mla_dims* d, int M, bool need_kv, bool splitk, ProjBufs* b) {
  const int N1 = d->q_lora_rank + d->kv_lora_rank + d->qk_rope_dim;
  const int H = d->n_heads, dqk = d->qk_nope_dim + d->qk_rope_dim;
  const size_t es = esize(d);
  b->S = 1;
  b->kchunk = d->d_model;
  b->cfg = GEMM_CFG_AUTO;
  b->decode = splitk && d->dtype == MLA_BF16 && M <= 64;
  if (b->decode) {
    b->S = skinny_splits(d->d_model);
  } else if (d->dtype == MLA_BF16) {
    // the down-projection writes fp32 partials that the latent norm sums, so
    // it may split K to balance its few tiles over the CUs
    const GemmPlan gp = M <= 1024 ? gemm_plan_small(M, N1, d->d_model, true, 8)
                                  : gemm_plan(M, N1, d->d_model, 1, 4);
    b->S = gp.ksplit;
    b->kchunk = gp.kchunk;
    b->cfg = gp.cfg;
  }
  size_t part_floats = (size_t)b->S * M * N1;
  if (b->decode) {
    const size_t sf = stream_part_floats(stream_info(M, N1, d->d_model));
    if (sf > part_floats) part_floats = sf;
  }
  b->part = c.take(part_floats * 4);
  b->cq = c.take((size_t)M * d->q_lora_rank * es);
  b->ckv = c.take((size_t)M * d->kv_lora_rank * es);
  b->kr = c.take((size_t)M * d->qk_rope_dim * es);
  b->q = c.take((size_t)M * H * dqk * es);
  b->kv = need_kv ? c.take((size_t)M * H * (d->qk_nope_dim + d->v_head_dim) * es) : nullptr;
  b->o = c.take((size_t)M * H * d->v_head_dim * es);
  b->upart = b->ukvpart = nullptr;
  b->upart_floats = b->ukvpart_floats = 0;
  if (d->dtype == MLA_BF16 && (splitk || M <= 64)) {
    // partials of the q and kv up-projections when M is small (decode, or a
    // prefill / chunk of at most 64 rows: the small-M products split K)
    const int shapes[2][2] = {{H * dqk, d->q_lora_rank},
                              {H * (d->qk_nope_dim + d->v_head_dim), d->kv_lora_rank}};
    // (decode with kv: both up-projections may stream in one launch)
    StreamInfo pair[2];
    bool paired = false;
    if (M <= 64 && need_kv) {
      GemmParams a = gp_base(), bb = gp_base();
      a.M = bb.M = M;
      a.N = shapes[0][0]; a.K = a.lda = a.ldb = shapes[0][1];
      bb.N = shapes[1][0]; bb.K = bb.lda = bb.ldb = shapes[1][1];
      paired = stream_pair_info(a, bb, &pair[0], &pair[1]);
    }
    for (int i = 0; i < 2; ++i) {
      if (i == 1 && !need_kv) break;
      const int S = skinny_splits(shapes[i][1]);
      size_t need = S > 1 ? (size_t)S * M * shapes[i][0] : 0;
      if (M <= 64) {
        size_t sf = stream_part_floats(stream_info(M, shapes[i][0], shapes[i][1]));
        if (paired) sf = std::max(sf, stream_part_floats(pair[i]));
        if (sf > need) need = sf;
      }
      if (!need) continue;
      void* buf = c.take(need * 4);
      if (i == 0) { b->upart = buf; b->upart_floats = need; }
      else { b->ukvpart = buf; b->ukvpart_floats = need; }
    }
  }
  b->opart = nullptr;
  b->opart_floats = 0;
  if (d->dtype == MLA_BF16 && M > 64 && M <= 1024) {
    const int D = d->d_model, K = d->n_heads * d->v_head_dim;
    const GemmPlan op = gemm_plan_small(M, D, K, false, 8);
    if (op.ksplit > 1) {
      b->opart_floats = (size_t)op.ksplit * M * D;
      b->opart = c.take(b->opart_floats * 4);
    }
  }
}

// bf16-output product.  Decode-sized products (M <= 64) go to the weight-
// streaming kernel: one K slice writes bf16 directly, several write fp32
// partials to `part` that a fixed-order reduction sums.
int gemm_bf16_out(const char* name, GemmParams g, void* part, size_t part_floats,
                  hipStream_t st) {
  if (g.M > 64) {
    LAUNCH(name, gemm_bf16(g, EPI_BF16, -1, st));
    return MLA_OK;
  }
  if (stream_ok(g)) {
    const StreamInfo si = stream_info(g.M, g.N, g.K);
    if (part && stream_part_floats(si) <= part_floats) {
      LAUNCH(name, gemm_stream_bf16(g, (float*)part, si, st));
      LAUNCH("stream_reduce", stream_reduce<bf16_t>((const float*)part, si, g.M, g.N, (bf16_t*)g.C,
                                                    g.ldc, nullptr, 0, st, g.bias));
      return MLA_OK;
    }
  }
  const int S = skinny_splits(g.K);
  if (S == 1) {
    LAUNCH(name, gemm_skinny_bf16(g, true, st));
    return MLA_OK;
  }
  if (!part || (size_t)S * g.M * g.N > part_floats || g.N % 4)
    return fail(MLA_ERR_HIP, "internal: split-K partial buffer too small for %s", name);
  GemmParams f = g;
  f.C = part;
  f.ldc = g.N;
  f.split_stride = (long)g.M * g.N;
  LAUNCH(name, gemm_skinny_bf16(f, false, st));
  LAUNCH("reduce_splits", reduce_splits<bf16_t>((const float*)part, S, (long)g.M * g.N, g.M, g.N,
                                                 (bf16_t*)g.C, g.ldc, st, g.bias));
  return MLA_OK;
}

// Weight-streaming product whose partial blocks are left unsummed for the
// consuming kernel; false (nothing launched) when the shape or the partial
// buffer does not allow it.
bool gemm_stream_deferred(const char* name, const GemmParams& g, void* part, size_t part_floats,
                          hipStream_t st, StreamInfo* si, int* rc) {
  si->G = 0;
  *rc = MLA_OK;
  if (!part || g.M > 64 || !stream_ok(g)) return false;
  const StreamInfo s = stream_info(g.M, g.N, g.K);
  if (stream_part_floats(s) > part_floats) return false;
  *si = s;
  *rc = [&]() -> int {
    LAUNCH(name, gemm_stream_bf16(g, (float*)part, s, st));
    return MLA_OK;
  }();
  return true;
}

// Parameters of the bf16 latent norms over the down-projection's partials
// (b.part: b.S fp32 K slices, or the weight stream's blocks when si is
// given): rows m at position m % rowsT + pos0 (or seq_pos[m], clamped into
// [0, pos_max]), with the optional latent-cache write.
LatentNormParams<bf16_t> latent_norm_params(const mla_dims* d, const mla_weights* w, const ProjBufs& b, int M,
                                            int rowsT, int pos0, const float* rc, const float* rs,
                                            const StreamInfo* si, void* latent_cache, int L_cap,
                                            const int* seq_pos, int pos_max) {
  const int ql = d->q_lora_rank, kl = d->kv_lora_rank, dr = d->qk_rope_dim, N1 = ql + kl + dr;
  LatentNormParams<bf16_t> n;
  memset(&n, 0, sizeof n);
  n.part = (const float*)b.part; n.nsplit = b.S;
  n.split_stride = (long)M * N1; n.ld_part = N1;
  n.stream = si ? 1 : 0;
  if (si) n.si = *si;
  n.seq_pos = seq_pos; n.pos_max = pos_max;
  n.bias_q = (const bf16_t*)w->b_dq; n.bias_kvr = (const bf16_t*)w->b_dkvr;
  n.M = M; n.q_lora = ql; n.kv_lora = kl; n.d_rope = dr;
  n.g_q = (const bf16_t*)w->g_q; n.g_kv = (const bf16_t*)w->g_kv; n.eps = d->rms_eps;
  n.cq = (bf16_t*)b.cq; n.ld_cq = ql; n.ckv = (bf16_t*)b.ckv; n.ld_ckv = kl;
  n.kr = (bf16_t*)b.kr; n.ld_kr = dr;
  n.rcos = rc; n.rsin = rs; n.n_pairs = dr / 2; n.rope_T = rowsT; n.rope_pos0 = pos0;
  n.latent_cache = (bf16_t*)latent_cache; n.L_cap = L_cap;
  return n;
}

// ---------------------------------------------------- shared launch steps
// Down-projections, latent norms and RoPE, query up-projection (roped) and,
// if kv is given, the kv up-projection.  Rows m = b*rowsT + t at position
// t + pos0.  With `defer` (decode), the q and kv up-projections may stay as
// weight-stream partials (b.upart, b.ukvpart) for the attention kernels to
// sum; defer[0] / defer[1] then hold their StreamInfo (G = 0: materialised
// in b.q / b.kv as usual).
// With `extra` (a bf16 product that depends only on the latent norms' outputs,
// e.g. the chunked latent form's per-head K/V expansion), the q up-projection,
// when it runs alone, shares one launch with it; *extra_done reports whether
// it did (otherwise the caller launches `extra` itself).
int run_projections(const mla_dims* d, const mla_weights* w, const void* x, int M, int rowsT,
                    int pos0, const float* rc, const float* rs, const ProjBufs& b,
                    void* latent_cache, int L_cap, hipStream_t st, StreamInfo* defer = nullptr,
                    const int* seq_pos = nullptr, int pos_max = 0, const GemmParams* extra = nullptr,
                    bool* extra_done = nullptr) {
  if (extra_done) *extra_done = false;
  if (defer) defer[0].G = defer[1].G = 0;
  const int H = d->n_heads, dn = d->qk_nope_dim, dr = d->qk_rope_dim, dv = d->v_head_dim;
  const int dqk = dn + dr, ql = d->q_lora_rank, kl = d->kv_lora_rank;
  const int N1 = ql + kl + dr, D = d->d_model;
  if (d->dtype == MLA_BF16) {
    GemmParams g = gp_base();
    g.A = (const bf16_t*)x; g.lda = D;
    g.B = (const bf16_t*)w->w_dq; g.B2 = (const bf16_t*)w->w_dkvr; g.ldb = D;
    g.b_split = ql;
    g.C = b.part; g.ldc = N1;
    g.M = M; g.N = N1; g.K = D;
    g.split_stride = (long)M * N1;
    bool streamed = false;
    StreamInfo si{};
    if (b.decode && stream_ok(g)) {
      // decode: balanced weight stream; the latent-norm kernel sums its
      // partial blocks
      si = stream_info(M, N1, D);
      LAUNCH("gemm_down", gemm_stream_bf16(g, (float*)b.part, si, st));
      streamed = true;
    } else if (b.decode) {
      LAUNCH("gemm_down", gemm_skinny_bf16(g, false, st));  // decode: K-sliced weight stream
    } else {
      g.ksplit = b.S;
      g.kchunk = b.kchunk;
      LAUNCH("gemm_down", gemm_bf16(g, EPI_F32, b.cfg, st));
    }
    const LatentNormParams<bf16_t> n = latent_norm_params(d, w, b, M, rowsT, pos0, rc, rs, streamed ? &si : nullptr,
                                                         latent_cache, L_cap, seq_pos, pos_max);
    LAUNCH("latent_norm_rope", latent_norm_rope<bf16_t>(n, st));
    GemmParams q = gp_base();
    q.A = (const bf16_t*)b.cq; q.lda = ql;
    q.B = (const bf16_t*)w->w_uqr; q.ldb = ql;
    q.C = b.q; q.ldc = (long)H * dqk;
    q.M = M; q.N = H * dqk; q.K = ql;
    // the query's rotary part is rotated by the attention kernels as they
    // load it (each 16-byte fragment holds four whole RoPE pairs)
    int r_ = MLA_OK;
    GemmParams k = gp_base();
    k.A = (const bf16_t*)b.ckv; k.lda = kl;
    k.B = (const bf16_t*)w->w_ukv; k.ldb = kl;
    k.C = b.kv; k.ldc = (long)H * (dn + dv);
    k.M = M; k.N = H * (dn + dv); k.K = kl;
    if (b.kv && M > 64) {
      // prefill: both up-projections in one launch when they take the same
      // tile shape (256 x 256, or 128 x 128 for the 512-row chunks), the q
      // tiles (longer K) scheduled first on every XCD, so the kv tiles fill
      // the CUs the q product's last partial wave leaves idle
      const int cfg = gemm_pick_cfg(M, q.N, q.K, 1);
      if (cfg == gemm_pick_cfg(M, k.N, k.K, 1) && (cfg == GEMM_CFG_256x256 || cfg == GEMM_CFG_128x128)) {
        hipError_t e;
        {
          ProfScope ps_("gemm_qkv_up", st);
          e = gemm_bf16_pair(q, k, EPI_BF16, cfg, st);
        }
        if (e == hipSuccess) return MLA_OK;
        if (e != hipErrorInvalidValue) return fail(MLA_ERR_HIP, "gemm_bf16_pair failed: %s", hipGetErrorString(e));
        (void)hipGetLastError();
      }
    }
    if (defer && b.kv && b.upart && b.ukvpart && stream_pair_info(q, k, &defer[0], &defer[1]) &&
        stream_part_floats(defer[0]) <= b.upart_floats && stream_part_floats(defer[1]) <= b.ukvpart_floats) {
      // decode: both up-projections stream in one launch and stay as partials
      LAUNCH("gemm_qkv_up", gemm_stream_bf16_pair(q, k, (float*)b.upart, (float*)b.ukvpart, defer[0],
                                                  defer[1], st));
      return MLA_OK;
    }
    if (extra && extra_done && !b.kv && M > 64 && extra->batch <= 1 &&
        gemm_pick_cfg(extra->M, extra->N, extra->K, 1) == GEMM_CFG_256x256) {
      // q (K = q_lora, the longer) first on every XCD, the extra product's
      // short-K tiles filling in behind it
      hipError_t e;
      {
        ProfScope ps_("gemm_q_up_kv_expand", st);
        e = gemm_bf16_pair(q, *extra, EPI_BF16, GEMM_CFG_256x256, st);
      }
      if (e == hipSuccess) {
        *extra_done = true;
        return MLA_OK;
      }
      if (e != hipErrorInvalidValue) return fail(MLA_ERR_HIP, "gemm_bf16_pair failed: %s", hipGetErrorString(e));
      (void)hipGetLastError();
    }
    if (defer) defer[0].G = defer[1].G = 0;
    if (!(defer && gemm_stream_deferred("gemm_q_up", q, b.upart, b.upart_floats, st, &defer[0], &r_)))
      r_ = gemm_bf16_out("gemm_q_up", q, b.upart, b.upart_floats, st);
    if (r_) return r_;
    if (b.kv) {
      if (!(defer && gemm_stream_deferred("gemm_kv_up", k, b.ukvpart, b.ukvpart_floats, st, &defer[1], &r_)))
        r_ = gemm_bf16_out("gemm_kv_up", k, b.ukvpart, b.ukvpart_floats, st);
      if (r_) return r_;
    }
    return MLA_OK;
  }
  // float32 path
  GemmF32Params g;
  memset(&g, 0, sizeof g);
  g.A = (const float*)x; g.lda = D; g.B = (const float*)w->w_dq; g.ldb = D;
  g.C = (float*)b.part; g.ldc = N1; g.M = M; g.N = ql; g.K = D; g.batch = 1; g.b_is_nk = 1;
  LAUNCH("gemm_down", gemm_f32(g, st));
  g.B = (const float*)w->w_dkvr; g.C = (float*)b.part + ql; g.N = kl + dr;
  LAUNCH("gemm_down", gemm_f32(g, st));
  LatentNormParams<float> n;
  memset(&n, 0, sizeof n);
  n.part = (const float*)b.part; n.nsplit = 1; n.split_stride = 0; n.ld_part = N1;
  n.M = M; n.q_lora = ql; n.kv_lora = kl; n.d_rope = dr;
  n.g_q = (const float*)w->g_q; n.g_kv = (const float*)w->g_kv; n.eps = d->rms_eps;
  n.cq = (float*)b.cq; n.ld_cq = ql; n.ckv = (float*)b.ckv; n.ld_ckv = kl;
  n.kr = (float*)b.kr; n.ld_kr = dr;
  n.rcos = rc; n.rsin = rs; n.n_pairs = dr / 2; n.rope_T = rowsT; n.rope_pos0 = pos0;
  n.latent_cache = (float*)latent_cache; n.L_cap = L_cap;
  n.seq_pos = seq_pos; n.pos_max = pos_max;
  n.bias_q = (const float*)w->b_dq; n.bias_kvr = (const float*)w->b_dkvr;
  LAUNCH("latent_norm_rope", latent_norm_rope<float>(n, st));
  GemmF32Params q;
  memset(&q, 0, sizeof q);
  q.A = (const float*)b.cq; q.lda = ql; q.B = (const float*)w->w_uqr; q.ldb = ql;
  q.C = (float*)b.q; q.ldc = (long)H * dqk; q.M = M; q.N = H * dqk; q.K = ql; q.batch = 1;
  q.b_is_nk = 1;
  LAUNCH("gemm_q_up", gemm_f32(q, st));
  LAUNCH("rope_q", rope_inplace_f32((float*)b.q, (long)H * dqk, M, H * dqk, dqk, dn, rc, rs, dr / 2, rowsT,
                          pos0, st, seq_pos, pos_max));
  if (b.kv) {
    GemmF32Params k;
    memset(&k, 0, sizeof k);
    k.A = (const float*)b.ckv; k.lda = kl; k.B = (const float*)w->w_ukv; k.ldb = kl;
    k.C = (float*)b.kv; k.ldc = (long)H * (dn + dv); k.M = M; k.N = H * (dn + dv); k.K = kl;
    k.batch = 1; k.b_is_nk = 1;
    LAUNCH("gemm_kv_up", gemm_f32(k, st));
  }
  return MLA_OK;
}

// out[M, d] = o[M, H*dv] . W_O^T (+ R).  Split-K for small M (decode).
// o_proj (+ bias b_o when given) (+ residual R when given).
int run_oproj(const mla_dims* d, const void* w_o, const void* b_o, const void* o, int M, const void* R,
              void* out, void* part, size_t part_floats, int S, hipStream_t st) {
  const int D = d->d_model, K = d->n_heads * d->v_head_dim;
  if (d->dtype == MLA_BF16) {
    GemmParams g = gp_base();
    g.A = (const bf16_t*)o; g.lda = K; g.B = (const bf16_t*)w_o; g.ldb = K;
    g.M = M; g.N = D; g.K = K;
    g.bias = (const bf16_t*)b_o;
    if (S > 1) {
      g.C = out; g.ldc = D;
      return gemm_bf16_out("gemm_o_proj", g, part, part_floats, st);
    }
    if (M > 64 && M <= 1024 && !R && part) {
      // a few hundred rows: K split over fp32 partials, summed into bf16
      const GemmPlan op = gemm_plan_small(M, D, K, false, 8);
      if (op.ksplit > 1 && (size_t)op.ksplit * M * D <= part_floats) {
        GemmParams f = g;
        f.C = part; f.ldc = D;
        f.ksplit = op.ksplit; f.kchunk = op.kchunk; f.split_stride = (long)M * D;
        f.bias = nullptr;
        LAUNCH("gemm_o_proj", gemm_bf16(f, EPI_F32, op.cfg, st));
        LAUNCH("reduce_splits", reduce_splits<bf16_t>((const float*)part, op.ksplit, (long)M * D, M, D,
                                                      (bf16_t*)out, D, st, (const bf16_t*)b_o));
        return MLA_OK;
      }
    }
    g.C = out; g.ldc = D;
    if (R) { g.R = (const bf16_t*)R; g.ldr = D; }
    LAUNCH("gemm_o_proj", gemm_bf16(g, R ? EPI_RESID : EPI_BF16, -1, st));
    return MLA_OK;
  }
  GemmF32Params g;
  memset(&g, 0, sizeof g);
  g.A = (const float*)o; g.lda = K; g.B = (const float*)w_o; g.ldb = K;
  g.C = (float*)out; g.ldc = D; g.R = (const float*)R; g.ldr = D;
  g.bias = (const float*)b_o;
  g.M = M; g.N = D; g.K = K; g.batch = 1; g.b_is_nk = 1;
  LAUNCH("gemm_o_proj", gemm_f32(g, st));
  return MLA_OK;
}

// Key splits of the flash attention: when the (query tile, head, sequence)
// workgroups are fewer than the CUs, each one's key tiles are shared out
// over up to 256 / workgroups splits of at least 8 tiles (64 keys each).
static int flash_splits(int B, int T, int H, int P0) {
  const long wgs = (long)((T + 255) / 256) * H * B;
  if (wgs >= 256) return 1;
  const int n_min = (P0 + std::min(255, T - 1)) / 64 + 1;  // tiles of the first query tile
  const int s = std::min((int)(256 / wgs), n_min / 8);
  return s < 1 ? 1 : s;
}
static size_t flash_split_floats(int B, int T, int H, int P0) {
  const int s = flash_splits(B, T, H, P0);
  return s > 1 ? (size_t)s * B * T * H * (128 + 2) : 0;
}

struct PrefillPlan {
  ProjBufs pb;
  float* fpart;  // flash key-split partials (NULL: no split): outputs, then (m, l)
};

size_t prefill_layout(const mla_dims* d, int B, int T, void* ws, PrefillPlan* pl) {
  Carver c(ws);
  carve_proj(c, d, B * T, true, false, &pl->pb);
  const size_t ff = d->dtype == MLA_BF16 ? flash_split_floats(B, T, d->n_heads, 0) : 0;
  pl->fpart = ff ? (float*)c.take(ff * 4) : nullptr;
  return c.off + 256;
}

int prefill_core(const mla_dims* d, const mla_weights* w, const void* x, int B, int T,
                 const float* rc, const float* rs, void* out, const void* resid, void* k_cache,
                 void* v_cache, void* latent_cache, int L_cap, const PrefillPlan& pl,
                 hipStream_t st) {
  const int M = B * T, H = d->n_heads, dn = d->qk_nope_dim, dr = d->qk_rope_dim;
  const int dv = d->v_head_dim, dqk = dn + dr;
  const ProjBufs& b = pl.pb;
  int rc_ = run_projections(d, w, x, M, T, 0, rc, rs, b, latent_cache, L_cap, st);
  if (rc_) return rc_;
  if (d->dtype == MLA_BF16) {
    FlashParams f;
    memset(&f, 0, sizeof f);
    f.q = (const bf16_t*)b.q; f.kv = (const bf16_t*)b.kv; f.kr = (const bf16_t*)b.kr;
    f.out = (bf16_t*)b.o; f.B = B; f.T = T; f.H = H; f.rcos = rc; f.rsin = rs;
    f.scale_log2 = scale_of(d) * kLog2e;
    flash_set_prefill_layout(f);
    f.nsplit = pl.fpart ? flash_splits(B, T, H, 0) : 1;
    f.opart = pl.fpart;
    f.ostat = pl.fpart ? pl.fpart + (size_t)f.nsplit * M * H * 128 : nullptr;
    if (!flash_pp_ok(f)) return fail(MLA_ERR_HIP, "internal: prefill outside the flash kernel's range");
    LAUNCH("flash_prefill", flash_prefill_pp_bf16(f, st));
  } else {
    AttnGenericParams a;
    memset(&a, 0, sizeof a);
    const long kvw = (long)H * (dn + dv);
    a.q_nope = (const float*)b.q; a.q_row = (long)H * dqk; a.q_head = dqk;
    a.q_rope = (const float*)b.q + dn; a.qr_row = (long)H * dqk; a.qr_head = dqk;
    a.k_nope = (const float*)b.kv; a.kn_b = (long)T * kvw; a.kn_j = kvw; a.kn_h = dn + dv;
    a.k_rope = (const float*)b.kr; a.kr_b = (long)T * dr; a.kr_j = dr; a.kr_h = 0;
    a.v = (const float*)b.kv + dn; a.v_b = (long)T * kvw; a.v_j = kvw; a.v_h = dn + dv;
    a.out = (float*)b.o; a.o_row = (long)H * dv; a.o_head = dv;
    a.B = B; a.Tq = T; a.Tk = T; a.H = H; a.d_nope = dn; a.d_rope = dr; a.d_v = dv;
    a.causal_offset = 0; a.scale = scale_of(d);
    LAUNCH("attn_generic", attn_generic_f32(a, st));
  }
  if (k_cache) {
    if (d->dtype == MLA_BF16)
      LAUNCH("scatter_cache", scatter_full_cache<bf16_t>((const bf16_t*)b.kv, (const bf16_t*)b.kr,
                                        (bf16_t*)k_cache, (bf16_t*)v_cache, B, T, 0, L_cap, H, dn,
                                        dr, dv, st));
    else
      LAUNCH("scatter_cache", scatter_full_cache<float>((const float*)b.kv, (const float*)b.kr, (float*)k_cache,
                                       (float*)v_cache, B, T, 0, L_cap, H, dn, dr, dv, st));
  }
  return run_oproj(d, w->w_o, w->b_o, b.o, M, resid, out, b.opart, b.opart_floats, 1, st);
}

// --------------------------------------------------------------- decode
struct DecodePlan {
  ProjBufs pb;
  void* q_abs;      // [B][H][kv_lora]
  void* o_lat;      // [B][H][kv_lora]
  void* apart;      // attention split partials
  int nsplit, chunk;
  int ns_cap;       // split count (latent form: workgroups) the partial buffer was sized for
  void* opart;      // o_proj split partials ([S2][B][d], or the stream GEMM's blocks)
  size_t opart_floats;
  int S2, kchunk2;
  void* sync;       // 256 bytes: the persistent latent decode's barrier words
};

// Full-cache attention splits.  The kernel holds six workgroups per CU
// (1536 on the chip), each streaming one (sequence, head)'s chunk of at most
// 4096 keys (its scores live in LDS) in equal chunks.  Candidates: from the
// fewest splits the 4096-key limit allows up to the most that keep chunks at
// least 1024 keys long (at most 8), or that give a small batch 512
// workgroups.  The choice minimises the launch's length in resident rounds
// of workgroups times (chunk + 80 keys of per-workgroup setup): measured on
// B = 32, P = 4096, three splits of 1366 keys took 884 us against 1054 us for
// one chunk of 4096 keys plus one of a single key, while cutting P = 1000
// into three cost 10 us more than one chunk.
constexpr int kFullResident = 256 * 6;
static void full_split_range(int B, int H, int L, int* smin, int* smax) {
  const long bh = (long)B * H;
  *smin = std::max(1, (L + 4095) / 4096);
  const int fill = (int)((512 + bh - 1) / bh);     // a small batch: 512 workgroups
  const int lng = std::min(L / 1024, 8);           // chunks of >= 1024 keys
  *smax = std::max(*smin, std::min((L + 127) / 128, std::max(fill, lng)));
}
int full_split_cap(int B, int H, int L) {
  int a, b;
  full_split_range(B, H, L, &a, &b);
  return b;
}
void plan_full_splits(int B, int H, int L, int* nsplit, int* chunk) {
  int smin, smax;
  full_split_range(B, H, L, &smin, &smax);
  const long bh = (long)B * H;
  long best = -1;
  int bs = smin;
  for (int s = smin; s <= smax; ++s) {
    const long rounds = (bh * s + kFullResident - 1) / kFullResident;
    const long cost = rounds * ((L + s - 1) / s + 80);
    if (best < 0 || cost < best) {
      best = cost;
      bs = s;
    }
  }
  *chunk = (L + bs - 1) / bs;
  *nsplit = (L + *chunk - 1) / *chunk;
}

// latent form: 256 workgroups (one per CU), fewer when the batch has fewer
// 32-key tiles at its longest length L, and at least one per sequence; the
// device-side plan (latent_plan) gives each a run of one sequence's tiles
int plan_latent_groups(int B, int L) {
  const long tiles = (long)B * ((L + 31) / 32);
  const int g = tiles < 256 ? (int)tiles : 256;
  return g > B ? g : B;
}
// one length for all sequences: splits per sequence (about 256 workgroups)
int plan_latent_splits(int B, int L) {
  int s = (256 + B - 1) / B;
  const int maxs = (L + 31) / 32;
  if (s > maxs) s = maxs;
  return s < 1 ? 1 : s;
}

size_t decode_layout(const mla_dims* d, int B, int L_cap, int form, void* ws, DecodePlan* pl) {
  Carver c(ws);
  const int H = d->n_heads, kl = d->kv_lora_rank;
  const size_t es = esize(d);
  carve_proj(c, d, B, form == 0, true, &pl->pb);
  pl->q_abs = c.take((size_t)B * H * (kl + d->qk_rope_dim) * es);  // bf16: [q~ | roped q^R]
  pl->o_lat = c.take((size_t)B * H * kl * es);
  // upper bounds of the split counts chosen for any live length L <= L_cap
  // the most splits plan_full_splits chooses for any live length <= L_cap
  const int cap_f = full_split_cap(B, H, L_cap);
  // workgroups for any live length <= L_cap, ragged or not
  const int cap_l = std::max(plan_latent_groups(B, L_cap), B * plan_latent_splits(B, L_cap));
  size_t fpart = (size_t)B * H * cap_f * 130 * 4;
  // latent form: the split plan (3 G + 2 B ints), then one record per workgroup
  size_t lpart = ((size_t)(3 * cap_l + 2 * B) * sizeof(int) + 255) / 256 * 256 +
                 (size_t)cap_l * H * (2 * 4 + (size_t)kl * 2);
  pl->apart = c.take(fpart > lpart ? fpart : lpart);
  pl->ns_cap = form == 0 ? cap_f : cap_l;
  pl->nsplit = 1;
  pl->chunk = L_cap;
  pl->S2 = 1;
  pl->kchunk2 = H * d->v_head_dim;
  if (d->dtype == MLA_BF16 && B <= 64) pl->S2 = skinny_splits(H * d->v_head_dim);
  size_t of = (size_t)pl->S2 * B * d->d_model;
  if (d->dtype == MLA_BF16 && B <= 64) {
    const size_t sf = stream_part_floats(stream_info(B, d->d_model, H * d->v_head_dim));
    if (sf > of) of = sf;
  }
  pl->opart = c.take(of * 4);
  pl->opart_floats = of;
  pl->sync = c.take(256);
  return c.off + 256;
}

int check_decode_args(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                      int L_cap, const float* rc, const float* rs, int rope_rows, const void* out,
                      const void* ws) {
  int r = check_dims(d, false);
  if (r) return r;
  if ((r = check_weights(w))) return r;
  if (!x || !out) return fail(MLA_ERR_NULL, "x or out is NULL");
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if ((r = check_align({x, out}, "x / out"))) return r;
  if (B <= 0 || L_cap <= 0) return fail(MLA_ERR_SHAPE, "B and L_cap must be positive");
  if (P < 0 || P >= L_cap) return fail(MLA_ERR_SHAPE, "P=%d outside [0, L_cap=%d)", P, L_cap);
  if ((r = check_rope(rc, rs, rope_rows, P + 1))) return r;
  return MLA_OK;
}

}  // namespace

// ===================================================================== ABI
extern "C" {

const char* mla_status_string(int s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size is non-positive or inconsistent";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not served";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch failed";
    default: return "unknown mla_status";
  }
}

const char* mla_last_error(void) { return g_err; }

int mla_profile_enable(int on) {
  g_prof = on != 0;
  return MLA_OK;
}

int mla_profile_summary(char* buf, size_t len, int* n_entries) {
  g_err[0] = 0;
  struct Acc {
    std::string name;
    int count;
    double ms;
  };
  std::vector<Acc> acc;
  for (auto& r : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      ms = -1.f;
    bool found = false;
    for (auto& a : acc)
      if (a.name == r.name) {
        a.count += 1;
        a.ms += ms;
        found = true;
      }
    if (!found) acc.push_back({r.name, 1, (double)ms});
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_pending.clear();
  if (n_entries) *n_entries = (int)acc.size();
  if (buf && len) {
    size_t off = 0;
    buf[0] = 0;
    for (auto& a : acc) {
      int w = snprintf(buf + off, len - off, "%s %d %.6f\n", a.name.c_str(), a.count, a.ms);
      if (w < 0 || (size_t)w >= len - off) return fail(MLA_ERR_SHAPE, "profile buffer too small");
      off += (size_t)w;
    }
  }
  return MLA_OK;
}

int mla_rope_table(int n_pos, int d_rope, double base, float* cos_out, float* sin_out,
                   void* stream) {
  g_err[0] = 0;
  if (!cos_out || !sin_out) return fail(MLA_ERR_NULL, "rope table output is NULL");
  if (int r = check_align({cos_out, sin_out}, "rope table output")) return r;
  if (n_pos <= 0 || d_rope <= 0 || d_rope % 2) return fail(MLA_ERR_SHAPE, "bad n_pos/d_rope");
  if (!(base > 0.0)) return fail(MLA_ERR_SHAPE, "base must be positive");
  hipStream_t st = (hipStream_t)stream;
  LAUNCH("rope_table", rope_table(n_pos, d_rope / 2, base, cos_out, sin_out, st));
  return MLA_OK;
}

int mla_read_sweep(const void* buf, size_t bytes, unsigned* sink, void* stream) {
  g_err[0] = 0;
  if (!buf || !sink) return fail(MLA_ERR_NULL, "buffer or sink is NULL");
  if (int r = check_align({buf, sink}, "buffer / sink")) return r;
  if (bytes == 0 || bytes % 16) return fail(MLA_ERR_SHAPE, "bytes must be a positive multiple of 16");
  hipStream_t st = (hipStream_t)stream;
  LAUNCH("read_sweep", read_sweep(buf, bytes, sink, kReadSweepWG, st));
  return MLA_OK;
}

size_t mla_prefill_workspace_size(const mla_dims* d, int B, int T) {
  if (check_dims(d, false) || B <= 0 || T <= 0) return 0;
  PrefillPlan pl;
  return prefill_layout(d, B, T, nullptr, &pl);
}

int mla_prefill(const mla_dims* d, const mla_weights* w, const void* x, int B, int T,
                const float* rc, const float* rs, int rope_rows, void* out, void* k_cache,
                void* v_cache, void* latent_cache, int L_cap, void* ws, size_t ws_bytes,
                void* stream) {
  g_err[0] = 0;
  int r = check_dims(d, false);
  if (r) return r;
  if ((r = check_weights(w))) return r;
  if (!x || !out) return fail(MLA_ERR_NULL, "x or out is NULL");
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if (B <= 0 || T <= 0) return fail(MLA_ERR_SHAPE, "B and T must be positive");
  if ((r = check_rope(rc, rs, rope_rows, T))) return r;
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(MLA_ERR_NULL, "k_cache and v_cache must be given together");
  if ((r = check_align({x, out, ws, k_cache, v_cache, latent_cache}, "x / out / workspace / caches")))
    return r;
  if ((k_cache || latent_cache) && L_cap < T)
    return fail(MLA_ERR_SHAPE, "L_cap=%d smaller than T=%d", L_cap, T);
  const long M = (long)B * T;
  if ((r = check_i32(M * d->d_model, "x")) || (r = check_i32(M * d->n_heads * 256, "kv")) ||
      (r = check_flash_prefill(d, T)))
    return r;
  PrefillPlan pl;
  size_t need = prefill_layout(d, B, T, nullptr, &pl);
  if (ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  prefill_layout(d, B, T, ws, &pl);
  return prefill_core(d, w, x, B, T, rc, rs, out, nullptr, k_cache, v_cache, latent_cache, L_cap,
                      pl, (hipStream_t)stream);
}

// ------------------------------------------------------ chunked prefill
// T new tokens per sequence at positions P0 .. P0+T-1 against a cache whose
// slots 0 .. P0-1 hold the history.  Workspace: the projections of the
// B*T new rows, plus (latent form) the per-head keys/values expanded from
// the cache rows 0 .. L_cap-1 (bf16) or the absorbed query and latent output
// (float32).
struct ChunkPlan {
  ProjBufs pb;
  float* fpart;  // flash key-split partials, sized for the largest P0 (NULL: no split)
  void* kv_exp;  // bf16 latent form: [B][L_cap][H*(dn+dv)]
  void* q_abs;   // float32 latent form: [B*T][H][kv_lora]
  void* o_lat;   // float32 latent form: [B*T][H][kv_lora]
};

static size_t chunk_layout(const mla_dims* d, int B, int T, int L_cap, int form, void* ws, ChunkPlan* pl) {
  Carver c(ws);
  const size_t es = esize(d);
  const int H = d->n_heads;
  carve_proj(c, d, B * T, form == 0, false, &pl->pb);
  // key splits only grow with P0: size them for the largest, L_cap - T
  const size_t ff = d->dtype == MLA_BF16 ? flash_split_floats(B, T, H, std::max(0, L_cap - T)) : 0;
  pl->fpart = ff ? (float*)c.take(ff * 4) : nullptr;
  pl->kv_exp = pl->q_abs = pl->o_lat = nullptr;
  if (form == 1 && d->dtype == MLA_BF16)
    pl->kv_exp = c.take((size_t)B * L_cap * H * (d->qk_nope_dim + d->v_head_dim) * es);
  if (form == 1 && d->dtype == MLA_F32) {
    pl->q_abs = c.take((size_t)B * T * H * d->kv_lora_rank * es);
    pl->o_lat = c.take((size_t)B * T * H * d->kv_lora_rank * es);
  }
  return c.off + 256;
}

static int chunk_impl(const mla_dims* d, const mla_weights* w, const void* x, int B, int T, int P0,
                      int L_cap, int form, void* k_cache, void* v_cache, void* latent_cache,
               const float* rc, const float* rs, int rope_rows, void* out, void* ws,
               size_t ws_bytes, void* stream) {
  int r = check_dims(d, false);
  if (r) return r;
  if ((r = check_weights(w))) return r;
  if (!x || !out) return fail(MLA_ERR_NULL, "x or out is NULL");
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if (form == 0 && (!k_cache || !v_cache)) return fail(MLA_ERR_NULL, "k_cache/v_cache is NULL");
  if (form == 1 && !latent_cache) return fail(MLA_ERR_NULL, "latent_cache is NULL");
  if ((r = check_align({x, out, ws, k_cache, v_cache, latent_cache}, "x / out / workspace / caches")))
    return r;
  if (B <= 0 || T <= 0 || L_cap <= 0) return fail(MLA_ERR_SHAPE, "B, T and L_cap must be positive");
  if (P0 < 0 || (long)P0 + T > L_cap)
    return fail(MLA_ERR_SHAPE, "chunk positions %d..%ld outside the cache [0, %d)", P0, (long)P0 + T - 1, L_cap);
  if ((r = check_rope(rc, rs, rope_rows, P0 + T))) return r;
  const long M = (long)B * T;
  const int H = d->n_heads, dn = d->qk_nope_dim, dr = d->qk_rope_dim, dv = d->v_head_dim;
  const int kl = d->kv_lora_rank, dqk = dn + dr;
  if ((r = check_i32(M * d->d_model, "x")) || (r = check_i32(M * H * 256, "kv")) ||
      (r = check_i32((long)L_cap * H * (dn + dv), "expanded cache rows")))
    return r;
  ChunkPlan pl;
  size_t need = chunk_layout(d, B, T, L_cap, form, nullptr, &pl);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  chunk_layout(d, B, T, L_cap, form, ws, &pl);
  hipStream_t st = (hipStream_t)stream;
  const ProjBufs& b = pl.pb;
  // projections of the new rows at positions P0 + t; the latent form's cache
  // entries are written by the latent-norm kernel
  const int Lk = P0 + T;  // keys per sequence
  // latent form, bf16: per-head keys/values of cache rows 0 .. Lk-1,
  // [K^C | V] = c^KV-hat W_UKV^T (the prefill's kv product applied to the
  // cached latents), launched together with the q up-projection when it can
  GemmParams kx = gp_base();
  kx.A = (const bf16_t*)latent_cache; kx.lda = kl + dr; kx.sA = (long)L_cap * (kl + dr);
  kx.B = (const bf16_t*)w->w_ukv; kx.ldb = kl; kx.sB = 0;
  kx.C = pl.kv_exp; kx.ldc = (long)H * (dn + dv); kx.sC = (long)L_cap * H * (dn + dv);
  kx.M = Lk; kx.N = H * (dn + dv); kx.K = kl; kx.batch = B;
  const bool with_exp = form == 1 && d->dtype == MLA_BF16;
  bool exp_done = false;
  if ((r = run_projections(d, w, x, (int)M, T, P0, rc, rs, b, form == 1 ? latent_cache : nullptr,
                           L_cap, st, nullptr, nullptr, 0, with_exp ? &kx : nullptr, &exp_done)))
    return r;
  if (d->dtype == MLA_BF16) {
    FlashParams f;
    memset(&f, 0, sizeof f);
    f.q = (const bf16_t*)b.q; f.out = (bf16_t*)b.o; f.B = B; f.T = T; f.H = H;
    f.rcos = rc; f.rsin = rs; f.scale_log2 = scale_of(d) * kLog2e;
    f.P0 = P0;
    if (form == 0) {
      LAUNCH("scatter_cache", scatter_full_cache<bf16_t>((const bf16_t*)b.kv, (const bf16_t*)b.kr,
                                                         (bf16_t*)k_cache, (bf16_t*)v_cache, B, T, P0,
                                                         L_cap, H, dn, dr, dv, st));
      // keys and values straight from the cache rows [K^C | k^R] and V
      f.kc = (const bf16_t*)k_cache;      f.kc_b = (long)H * L_cap * dqk; f.kc_h = (long)L_cap * dqk; f.kc_kb = dqk * 2;
      f.kr2 = (const bf16_t*)k_cache + dn; f.kr_b = f.kc_b; f.kr_h = f.kc_h; f.kr_kb = dqk * 2;
      f.vv = (const bf16_t*)v_cache;      f.v_b = (long)H * L_cap * dv; f.v_h = (long)L_cap * dv; f.v_kb = dv * 2;
    } else {
      if (!exp_done) LAUNCH("gemm_kv_expand", gemm_bf16(kx, EPI_BF16, -1, st));
      const bf16_t* kv = (const bf16_t*)pl.kv_exp;
      const long row = (long)H * (dn + dv);
      f.kc = kv;       f.kc_b = (long)L_cap * row; f.kc_h = dn + dv; f.kc_kb = (int)(row * 2);
      f.vv = kv + dn;  f.v_b = f.kc_b;             f.v_h = dn + dv; f.v_kb = (int)(row * 2);
      f.kr2 = (const bf16_t*)latent_cache + kl; f.kr_b = (long)L_cap * (kl + dr); f.kr_h = 0;
      f.kr_kb = (kl + dr) * 2;
    }
    if (!flash_pp_ok(f))
      return fail(MLA_ERR_UNSUPPORTED, "chunked prefill: cache rows too long for 32-bit offsets");
    f.nsplit = pl.fpart ? flash_splits(B, T, H, P0) : 1;
    f.opart = pl.fpart;
    f.ostat = pl.fpart ? pl.fpart + (size_t)f.nsplit * M * H * 128 : nullptr;
    LAUNCH("flash_prefill", flash_prefill_pp_bf16(f, st));
  } else if (form == 0) {
    LAUNCH("scatter_cache", scatter_full_cache<float>((const float*)b.kv, (const float*)b.kr, (float*)k_cache,
                                                      (float*)v_cache, B, T, P0, L_cap, H, dn, dr, dv, st));
    AttnGenericParams a;
    memset(&a, 0, sizeof a);
    a.q_nope = (const float*)b.q; a.q_row = (long)H * dqk; a.q_head = dqk;
    a.q_rope = (const float*)b.q + dn; a.qr_row = (long)H * dqk; a.qr_head = dqk;
    a.k_nope = (const float*)k_cache; a.kn_b = (long)H * L_cap * dqk; a.kn_j = dqk; a.kn_h = (long)L_cap * dqk;
    a.k_rope = (const float*)k_cache + dn; a.kr_b = a.kn_b; a.kr_j = dqk; a.kr_h = a.kn_h;
    a.v = (const float*)v_cache; a.v_b = (long)H * L_cap * dv; a.v_j = dv; a.v_h = (long)L_cap * dv;
    a.out = (float*)b.o; a.o_row = (long)H * dv; a.o_head = dv;
    a.B = B; a.Tq = T; a.Tk = Lk; a.H = H; a.d_nope = dn; a.d_rope = dr; a.d_v = dv;
    a.causal_offset = P0; a.scale = scale_of(d);
    LAUNCH("attn_generic", attn_generic_f32(a, st));
  } else {
    // absorbed form over the latent cache, T queries per sequence
    GemmF32Params g;
    memset(&g, 0, sizeof g);
    g.A = (const float*)b.q; g.lda = (long)H * dqk;
    g.B = (const float*)w->w_ukv; g.ldb = kl; g.b_is_nk = 0;
    g.C = (float*)pl.q_abs; g.ldc = (long)H * kl;
    g.M = (int)M; g.N = kl; g.K = dn; g.batch = H;
    g.sA = dqk; g.sB = (long)(dn + dv) * kl; g.sC = kl;
    LAUNCH("absorb_q", gemm_f32(g, st));
    AttnGenericParams a;
    memset(&a, 0, sizeof a);
    const long cw = kl + dr;
    a.q_nope = (const float*)pl.q_abs; a.q_row = (long)H * kl; a.q_head = kl;
    a.q_rope = (const float*)b.q + dn; a.qr_row = (long)H * dqk; a.qr_head = dqk;
    a.k_nope = (const float*)latent_cache; a.kn_b = (long)L_cap * cw; a.kn_j = cw; a.kn_h = 0;
    a.k_rope = (const float*)latent_cache + kl; a.kr_b = a.kn_b; a.kr_j = cw; a.kr_h = 0;
    a.v = (const float*)latent_cache; a.v_b = a.kn_b; a.v_j = cw; a.v_h = 0;
    a.out = (float*)pl.o_lat; a.o_row = (long)H * kl; a.o_head = kl;
    a.B = B; a.Tq = T; a.Tk = Lk; a.H = H; a.d_nope = kl; a.d_rope = dr; a.d_v = kl;
    a.causal_offset = P0; a.scale = scale_of(d);
    LAUNCH("attn_generic", attn_generic_f32(a, st));
    GemmF32Params u;
    memset(&u, 0, sizeof u);
    u.A = (const float*)pl.o_lat; u.lda = (long)H * kl;
    u.B = (const float*)w->w_ukv + (long)dn * kl; u.ldb = kl; u.b_is_nk = 1;
    u.C = (float*)b.o; u.ldc = (long)H * dv;
    u.M = (int)M; u.N = dv; u.K = kl; u.batch = H;
    u.sA = kl; u.sB = (long)(dn + dv) * kl; u.sC = dv;
    LAUNCH("gemm_uv", gemm_f32(u, st));
  }
  return run_oproj(d, w->w_o, w->b_o, b.o, (int)M, nullptr, out, b.opart, b.opart_floats, 1, st);
}

size_t mla_prefill_chunk_workspace_size(const mla_dims* d, int B, int T, int L_cap) {
  if (check_dims(d, false) || B <= 0 || T <= 0 || L_cap <= 0) return 0;
  ChunkPlan a, b;
  const size_t s0 = chunk_layout(d, B, T, L_cap, 0, nullptr, &a);
  const size_t s1 = chunk_layout(d, B, T, L_cap, 1, nullptr, &b);
  return s0 > s1 ? s0 : s1;
}

int mla_prefill_chunk_fullcache(const mla_dims* d, const mla_weights* w, const void* x, int B, int T,
                                int P0, int L_cap, void* k_cache, void* v_cache, const float* rc,
                                const float* rs, int rope_rows, void* out, void* ws, size_t ws_bytes,
                                void* stream) {
  g_err[0] = 0;
  return chunk_impl(d, w, x, B, T, P0, L_cap, 0, k_cache, v_cache, nullptr, rc, rs, rope_rows, out, ws,
                    ws_bytes, stream);
}

int mla_prefill_chunk_latentcache(const mla_dims* d, const mla_weights* w, const void* x, int B, int T,
                                  int P0, int L_cap, void* latent_cache, const float* rc,
                                  const float* rs, int rope_rows, void* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  g_err[0] = 0;
  return chunk_impl(d, w, x, B, T, P0, L_cap, 1, nullptr, nullptr, latent_cache, rc, rs, rope_rows, out,
                    ws, ws_bytes, stream);
}

size_t mla_decode_workspace_size(const mla_dims* d, int B, int L_cap) {
  if (check_dims(d, false) || B <= 0 || L_cap <= 0) return 0;
  DecodePlan a, b;
  size_t s0 = decode_layout(d, B, L_cap, 0, nullptr, &a);
  size_t s1 = decode_layout(d, B, L_cap, 1, nullptr, &b);
  return s0 > s1 ? s0 : s1;
}

// Full-cache decode step.  P is the new tokens' position, or with seq_pos
// (device, per sequence) an upper bound of the positions: the split plan,
// the workspace and the argument checks use it.
static int decode_full_impl(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                            const int* seq_pos, int L_cap, void* k_cache, void* v_cache,
                            const float* rc, const float* rs, int rope_rows, void* out, void* ws,
                            size_t ws_bytes, void* stream) {
  int r = check_decode_args(d, w, x, B, P, L_cap, rc, rs, rope_rows, out, ws);
  if (r) return r;
  if (!k_cache || !v_cache) return fail(MLA_ERR_NULL, "k_cache/v_cache is NULL");
  if ((r = check_align({k_cache, v_cache, ws}, "caches / workspace"))) return r;
  DecodePlan pl;
  size_t need = decode_layout(d, B, L_cap, 0, nullptr, &pl);
  if (ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  decode_layout(d, B, L_cap, 0, ws, &pl);
  // the attention split depends on the live length L = P + 1
  plan_full_splits(B, d->n_heads, P + 1, &pl.nsplit, &pl.chunk);
  if (pl.nsplit > pl.ns_cap) return fail(MLA_ERR_HIP, "internal: split plan exceeds workspace");
  hipStream_t st = (hipStream_t)stream;
  const int H = d->n_heads, dn = d->qk_nope_dim, dr = d->qk_rope_dim, dv = d->v_head_dim;
  const ProjBufs& b = pl.pb;
  StreamInfo def[2];
  if ((r = run_projections(d, w, x, B, 1, P, rc, rs, b, nullptr, L_cap, st,
                           d->dtype == MLA_BF16 ? def : nullptr, seq_pos, P)))
    return r;
  if (d->dtype == MLA_BF16) {
    // fused form: the attention kernel sums q and the new slot's k/v from the
    // stream partials and writes slot P itself
    const bool fused_kv = def[1].G > 0;
    if (!fused_kv)
      LAUNCH("scatter_cache", scatter_full_cache<bf16_t>((const bf16_t*)b.kv, (const bf16_t*)b.kr, (bf16_t*)k_cache,
                                        (bf16_t*)v_cache, B, 1, P, L_cap, H, dn, dr, dv, st, seq_pos, P));
    DecodeFullParams a;
    a.q = (const bf16_t*)b.q; a.k_cache = (bf16_t*)k_cache;
    a.v_cache = (bf16_t*)v_cache; a.out = (bf16_t*)b.o; a.part = (float*)pl.apart;
    a.qpart = def[0].G > 0 ? (const float*)b.upart : nullptr; a.qsi = def[0];
    a.kvpart = fused_kv ? (const float*)b.ukvpart : nullptr; a.kvsi = def[1];
    a.kr = (const bf16_t*)b.kr;
    a.rcos = rc; a.rsin = rs;
    a.B = B; a.H = H; a.L = P + 1; a.L_cap = L_cap; a.nsplit = pl.nsplit; a.chunk = pl.chunk;
    a.scale_log2 = scale_of(d) * kLog2e;
    a.seq_pos = seq_pos;
    LAUNCH("decode_full", decode_full_bf16(a, st));
  } else {
    LAUNCH("scatter_cache", scatter_full_cache<float>((const float*)b.kv, (const float*)b.kr, (float*)k_cache,
                                     (float*)v_cache, B, 1, P, L_cap, H, dn, dr, dv, st, seq_pos, P));
    const int dqk = dn + dr;
    AttnGenericParams a;
    memset(&a, 0, sizeof a);
    a.q_nope = (const float*)b.q; a.q_row = (long)H * dqk; a.q_head = dqk;
    a.q_rope = (const float*)b.q + dn; a.qr_row = (long)H * dqk; a.qr_head = dqk;
    a.k_nope = (const float*)k_cache; a.kn_b = (long)H * L_cap * dqk; a.kn_j = dqk;
    a.kn_h = (long)L_cap * dqk;
    a.k_rope = (const float*)k_cache + dn; a.kr_b = a.kn_b; a.kr_j = dqk; a.kr_h = a.kn_h;
    a.v = (const float*)v_cache; a.v_b = (long)H * L_cap * dv; a.v_j = dv; a.v_h = (long)L_cap * dv;
    a.out = (float*)b.o; a.o_row = (long)H * dv; a.o_head = dv;
    a.B = B; a.Tq = 1; a.Tk = P + 1; a.H = H; a.d_nope = dn; a.d_rope = dr; a.d_v = dv;
    a.causal_offset = P; a.scale = scale_of(d);
    a.seq_pos = seq_pos; a.pos_max = P;
    LAUNCH("attn_generic", attn_generic_f32(a, st));
  }
  return run_oproj(d, w->w_o, w->b_o, b.o, B, nullptr, out, pl.opart, pl.opart_floats, pl.S2, st);
}

int mla_decode_fullcache(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                         int L_cap, void* k_cache, void* v_cache, const float* rc, const float* rs,
                         int rope_rows, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return decode_full_impl(d, w, x, B, P, nullptr, L_cap, k_cache, v_cache, rc, rs, rope_rows, out,
                          ws, ws_bytes, stream);
}

int mla_decode_fullcache_ragged(const mla_dims* d, const mla_weights* w, const void* x, int B,
                                const int* positions, int P_max, int L_cap, void* k_cache,
                                void* v_cache, const float* rc, const float* rs, int rope_rows,
                                void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!positions) return fail(MLA_ERR_NULL, "positions is NULL");
  return decode_full_impl(d, w, x, B, P_max, positions, L_cap, k_cache, v_cache, rc, rs, rope_rows,
                          out, ws, ws_bytes, stream);
}

// Latent-cache decode step; P and seq_pos as for decode_full_impl.
// Every argument check of the latent-cache decode except the workspace
// (no HIP call).
static int decode_latent_check(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                               int L_cap, const void* latent_cache, const float* rc, const float* rs,
                               int rope_rows, const void* out) {
  int r = check_decode_args(d, w, x, B, P, L_cap, rc, rs, rope_rows, out, d);  // workspace checked later
  if (r) return r;
  if (!latent_cache) return fail(MLA_ERR_NULL, "latent_cache is NULL");
  if ((r = check_align({latent_cache}, "latent_cache"))) return r;
  if (d->dtype == MLA_BF16 && (d->kv_lora_rank != 512 || d->n_heads != 64))
    return fail(MLA_ERR_UNSUPPORTED, "bf16 latent decode serves kv_lora 512 and 64 heads");
  if (d->dtype == MLA_BF16 && B > 1024)
    return fail(MLA_ERR_UNSUPPORTED, "bf16 latent decode serves batches of up to 1024 sequences");
  return MLA_OK;
}

// Parameters of the bf16 query absorption ([q~ | roped q^R] per head, q
// summed from the q up-projection's weight-stream partials when qsi.G > 0)
// and of the split-L attention with its merge (o~ W_UV into b.o).  Uniform
// position P with `splits` workgroups per sequence, or (seq_pos) the device
// plan over pl.nsplit workgroups.
static void latent_attn_params(const mla_dims* d, const mla_weights* w, const DecodePlan& pl, int B, int P,
                               const int* seq_pos, int splits, int L_cap, const void* latent_cache,
                               const float* rc, const float* rs, const StreamInfo& qsi, AbsorbParams* abp,
                               DecodeLatentParams* ap) {
  const int H = d->n_heads;
  const ProjBufs& b = pl.pb;
  AbsorbParams& ab = *abp;
  memset(&ab, 0, sizeof ab);
  ab.q = (const bf16_t*)b.q;
  ab.qpart = qsi.G > 0 ? (const float*)b.upart : nullptr; ab.qsi = qsi;
  ab.w_ukv = (const bf16_t*)w->w_ukv; ab.qa = (bf16_t*)pl.q_abs;
  ab.rcos = rc; ab.rsin = rs; ab.B = B; ab.H = H; ab.L = P + 1; ab.seq_pos = seq_pos;
  // the attention's split plan, then its records: fp32 (m, l) and bf16 o~
  int* plan = (int*)pl.apart;
  char* recs = (char*)pl.apart + ((size_t)(3 * pl.ns_cap + 2 * B) * sizeof(int) + 255) / 256 * 256;
  ab.plan = seq_pos ? plan : nullptr; ab.G = pl.nsplit;
  DecodeLatentParams& a = *ap;
  memset(&a, 0, sizeof a);
  a.q_abs = (const bf16_t*)pl.q_abs;
  a.cache = (const bf16_t*)latent_cache;
  a.stats = (float*)recs;
  a.opart = (bf16_t*)(recs + (size_t)pl.ns_cap * H * 2 * sizeof(float));
  a.plan = ab.plan; a.splits = splits;
  a.rcos = rc; a.rsin = rs;
  a.B = B; a.H = H; a.L = P + 1; a.L_cap = L_cap; a.G = pl.nsplit;
  a.scale_log2 = scale_of(d) * kLog2e;
  a.seq_pos = seq_pos;
  // merge of the splits fused with O_h = o~_h W_UV,h^T
  a.w_ukv = (const bf16_t*)w->w_ukv; a.out = (bf16_t*)b.o;
}

static int decode_latent_impl(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                              const int* seq_pos, int L_cap, void* latent_cache, const float* rc,
                              const float* rs, int rope_rows, void* out, void* ws, size_t ws_bytes,
                              void* stream) {
  int r = decode_latent_check(d, w, x, B, P, L_cap, latent_cache, rc, rs, rope_rows, out);
  if (r) return r;
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if ((r = check_align({ws}, "workspace"))) return r;
  DecodePlan pl;
  size_t need = decode_layout(d, B, L_cap, 1, nullptr, &pl);
  if (ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  decode_layout(d, B, L_cap, 1, ws, &pl);
  const int splits = seq_pos ? 0 : plan_latent_splits(B, P + 1);
  pl.nsplit = seq_pos ? plan_latent_groups(B, P + 1) : B * splits;
  if (pl.nsplit > pl.ns_cap) return fail(MLA_ERR_HIP, "internal: split plan exceeds workspace");
  hipStream_t st = (hipStream_t)stream;
  const int H = d->n_heads, dn = d->qk_nope_dim, dr = d->qk_rope_dim, dv = d->v_head_dim;
  const int kl = d->kv_lora_rank, dqk = dn + dr;
  const ProjBufs& b = pl.pb;
  // bf16: the q up-projection stays as weight-stream partials, summed by the
  // absorption kernel as it loads q (no reduction launch)
  StreamInfo def[2];
  if ((r = run_projections(d, w, x, B, 1, P, rc, rs, b, latent_cache, L_cap, st,
                           d->dtype == MLA_BF16 ? def : nullptr, seq_pos, P)))
    return r;
  if (d->dtype == MLA_BF16) {
    AbsorbParams ab;
    DecodeLatentParams a;
    latent_attn_params(d, w, pl, B, P, seq_pos, splits, L_cap, latent_cache, rc, rs, def[0], &ab, &a);
    LAUNCH("absorb_q", absorb_q_bf16(ab, st));
    LAUNCH("decode_latent", decode_latent_bf16(a, st));
  } else {
    GemmF32Params g;
    memset(&g, 0, sizeof g);
    // q~ = Q^C . W_UK (W_UK,h rows of kv_b_proj used as a [d_nope, kv_lora] matrix)
    g.A = (const float*)b.q; g.lda = (long)H * dqk;
    g.B = (const float*)w->w_ukv; g.ldb = kl; g.b_is_nk = 0;
    g.C = (float*)pl.q_abs; g.ldc = (long)H * kl;
    g.M = B; g.N = kl; g.K = dn; g.batch = H;
    g.sA = dqk; g.sB = (long)(dn + dv) * kl; g.sC = kl;
    LAUNCH("absorb_q", gemm_f32(g, st));
    AttnGenericParams a;
    memset(&a, 0, sizeof a);
    const long cw = kl + dr;
    a.q_nope = (const float*)pl.q_abs; a.q_row = (long)H * kl; a.q_head = kl;
    a.q_rope = (const float*)b.q + dn; a.qr_row = (long)H * dqk; a.qr_head = dqk;
    a.k_nope = (const float*)latent_cache; a.kn_b = (long)L_cap * cw; a.kn_j = cw; a.kn_h = 0;
    a.k_rope = (const float*)latent_cache + kl; a.kr_b = a.kn_b; a.kr_j = cw; a.kr_h = 0;
    a.v = (const float*)latent_cache; a.v_b = a.kn_b; a.v_j = cw; a.v_h = 0;
    a.out = (float*)pl.o_lat; a.o_row = (long)H * kl; a.o_head = kl;
    a.B = B; a.Tq = 1; a.Tk = P + 1; a.H = H; a.d_nope = kl; a.d_rope = dr; a.d_v = kl;
    a.causal_offset = P; a.scale = scale_of(d);
    a.seq_pos = seq_pos; a.pos_max = P;
    LAUNCH("attn_generic", attn_generic_f32(a, st));
    // O_h = o~_h . W_UV,h^T
    GemmF32Params u;
    memset(&u, 0, sizeof u);
    u.A = (const float*)pl.o_lat; u.lda = (long)H * kl;
    u.B = (const float*)w->w_ukv + (long)dn * kl; u.ldb = kl; u.b_is_nk = 1;
    u.C = (float*)b.o; u.ldc = (long)H * dv;
    u.M = B; u.N = dv; u.K = kl; u.batch = H;
    u.sA = kl; u.sB = (long)(dn + dv) * kl; u.sC = dv;
    LAUNCH("gemm_uv", gemm_f32(u, st));
  }
  return run_oproj(d, w->w_o, w->b_o, b.o, B, nullptr, out, pl.opart, pl.opart_floats, pl.S2, st);
}

// Hooks of the allocation-free entry point (noalloc.hip): the argument
// checks of the latent decode, and an error report into this thread's
// message.
__attribute__((visibility("hidden"))) int mla_internal_decode_latent_check(const mla_dims* d, const mla_weights* w, const void* x, int B,
                                     int P, int L_cap, const void* latent_cache, const float* rc,
                                     const float* rs, int rope_rows, const void* out) {
  g_err[0] = 0;
  return decode_latent_check(d, w, x, B, P, L_cap, latent_cache, rc, rs, rope_rows, out);
}

__attribute__((visibility("hidden"))) int mla_internal_fail(int code, const char* msg) {
  return fail(code, "%s", msg);
}

int mla_decode_latentcache(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                           int L_cap, void* latent_cache, const float* rc, const float* rs,
                           int rope_rows, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return decode_latent_impl(d, w, x, B, P, nullptr, L_cap, latent_cache, rc, rs, rope_rows, out, ws,
                            ws_bytes, stream);
}

int mla_decode_latentcache_persistent(const mla_dims* d, const mla_weights* w, const void* x, int B, int P,
                                      int L_cap, void* latent_cache, const float* rc, const float* rs,
                                      int rope_rows, void* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int r = decode_latent_check(d, w, x, B, P, L_cap, latent_cache, rc, rs, rope_rows, out);
  if (r) return r;
  if (d->dtype != MLA_BF16) return fail(MLA_ERR_UNSUPPORTED, "the persistent latent decode is bf16 only");
  if (B > 64) return fail(MLA_ERR_UNSUPPORTED, "the persistent latent decode serves batches of up to 64 sequences");
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if ((r = check_align({ws}, "workspace"))) return r;
  DecodePlan pl;
  const size_t need = decode_layout(d, B, L_cap, 1, nullptr, &pl);
  if (ws_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  decode_layout(d, B, L_cap, 1, ws, &pl);
  const int splits = plan_latent_splits(B, P + 1);
  pl.nsplit = B * splits;
  if (pl.nsplit > pl.ns_cap) return fail(MLA_ERR_HIP, "internal: split plan exceeds workspace");
  const ProjBufs& b = pl.pb;
  const int H = d->n_heads, dqk = d->qk_nope_dim + d->qk_rope_dim, ql = d->q_lora_rank;
  const int N1 = ql + d->kv_lora_rank + d->qk_rope_dim, D = d->d_model, K = H * d->v_head_dim;
  PersistLatentParams pp;
  memset(&pp, 0, sizeof pp);
  // the multi-launch step's products and plans (run_projections, decode_latent_impl, run_oproj)
  GemmParams& g = pp.down;
  g = gp_base();
  g.A = (const bf16_t*)x; g.lda = D;
  g.B = (const bf16_t*)w->w_dq; g.B2 = (const bf16_t*)w->w_dkvr; g.ldb = D; g.b_split = ql;
  g.C = b.part; g.ldc = N1; g.M = B; g.N = N1; g.K = D; g.split_stride = (long)B * N1;
  GemmParams& q = pp.qup;
  q = gp_base();
  q.A = (const bf16_t*)b.cq; q.lda = ql; q.B = (const bf16_t*)w->w_uqr; q.ldb = ql;
  q.C = b.q; q.ldc = (long)H * dqk; q.M = B; q.N = H * dqk; q.K = ql;
  GemmParams& o = pp.oproj;
  o = gp_base();
  o.A = (const bf16_t*)b.o; o.lda = K; o.B = (const bf16_t*)w->w_o; o.ldb = K;
  o.C = out; o.ldc = D; o.M = B; o.N = D; o.K = K; o.bias = (const bf16_t*)w->b_o;
  if (!b.decode || !stream_ok(g) || !stream_ok(q) || !stream_ok(o))
    return fail(MLA_ERR_UNSUPPORTED, "the persistent latent decode needs the weight-streaming shapes of every projection");
  pp.down_si = stream_info(B, N1, D);
  pp.qup_si = stream_info(B, q.N, q.K);
  pp.oproj_si = stream_info(B, D, K);
  pp.down_part = (float*)b.part;
  pp.qup_part = (float*)b.upart;
  pp.oproj_part = (float*)pl.opart;
  if (!b.upart || stream_part_floats(pp.qup_si) > b.upart_floats || stream_part_floats(pp.oproj_si) > pl.opart_floats)
    return fail(MLA_ERR_HIP, "internal: weight-stream partial buffers too small");
  pp.norm = latent_norm_params(d, w, b, B, 1, P, rc, rs, &pp.down_si, latent_cache, L_cap, nullptr, P);
  latent_attn_params(d, w, pl, B, P, nullptr, splits, L_cap, latent_cache, rc, rs, pp.qup_si, &pp.ab, &pp.at);
  pp.sync = (unsigned*)pl.sync;
  hipStream_t st = (hipStream_t)stream;
  LAUNCH("decode_latent_persistent", decode_latent_persistent_bf16(pp, st));
  return MLA_OK;
}

int mla_decode_latentcache_persistent_status(const mla_dims* d, int B, int L_cap, const void* ws, int* status) {
  g_err[0] = 0;
  if (!d || !ws || !status) return fail(MLA_ERR_NULL, "dims, workspace or status is NULL");
  int r = check_dims(d, false);
  if (r) return r;
  if (B <= 0 || L_cap <= 0) return fail(MLA_ERR_SHAPE, "B and L_cap must be positive");
  DecodePlan pl;
  decode_layout(d, B, L_cap, 1, const_cast<void*>(ws), &pl);
  unsigned v = 0;
  const hipError_t e = hipMemcpy(&v, (const unsigned*)pl.sync + 2, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  *status = v ? 1 : 0;
  return MLA_OK;
}

int mla_decode_latentcache_ragged(const mla_dims* d, const mla_weights* w, const void* x, int B,
                                  const int* positions, int P_max, int L_cap, void* latent_cache,
                                  const float* rc, const float* rs, int rope_rows, void* out,
                                  void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!positions) return fail(MLA_ERR_NULL, "positions is NULL");
  return decode_latent_impl(d, w, x, B, P_max, positions, L_cap, latent_cache, rc, rs, rope_rows,
                            out, ws, ws_bytes, stream);
}

size_t dense_block_workspace_size(const mla_dims* d, int B, int T) {
  if (check_dims(d, true) || B <= 0 || T <= 0) return 0;
  const size_t es = esize(d);
  const size_t M = (size_t)B * T;
  PrefillPlan pl;
  size_t attn = prefill_layout(d, B, T, nullptr, &pl);
  size_t extra = 3 * rup((long)(M * d->d_model * es), 256);          // x_attn, x1, x_ffn
  size_t ff = d->dtype == MLA_BF16 ? M * d->d_ff * es : 3 * M * d->d_ff * es;  // h (+ g, u)
  return attn + extra + (size_t)rup((long)ff, 256) + 1024;
}

int dense_block_fwd(const mla_dims* d, const mla_block_weights* w, const void* x, int B, int T,
                    const float* rc, const float* rs, int rope_rows, void* out, void* ws,
                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int r = check_dims(d, true);
  if (r) return r;
  if (!w) return fail(MLA_ERR_NULL, "block weights is NULL");
  if ((r = check_weights(&w->attn))) return r;
  if (!w->g_attn || !w->g_ffn || !w->w1 || !w->w3 || !w->w2)
    return fail(MLA_ERR_NULL, "a block weight pointer is NULL");
  if (!x || !out) return fail(MLA_ERR_NULL, "x or out is NULL");
  if (!ws) return fail(MLA_ERR_NULL, "workspace is NULL");
  if ((r = check_align({w->g_attn, w->g_ffn, w->w1, w->w3, w->w2, x, out, ws},
                       "block weights / x / out / workspace")))
    return r;
  if (B <= 0 || T <= 0) return fail(MLA_ERR_SHAPE, "B and T must be positive");
  if ((r = check_rope(rc, rs, rope_rows, T))) return r;
  const long M = (long)B * T;
  if ((r = check_i32(M * d->d_ff, "ffn hidden")) || (r = check_i32(M * d->n_heads * 256, "kv")) ||
      (r = check_i32((long)d->d_ff * d->d_model, "W1")) || (r = check_flash_prefill(d, T)))
    return r;
  size_t need = dense_block_workspace_size(d, B, T);
  if (ws_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const size_t es = esize(d);
  const int D = d->d_model, F = d->d_ff;
  Carver c(ws);
  void* xa = c.take((size_t)M * D * es);
  void* x1 = c.take((size_t)M * D * es);
  void* xf = c.take((size_t)M * D * es);
  void* hbuf = c.take((size_t)M * F * es * (d->dtype == MLA_BF16 ? 1 : 3));
  PrefillPlan pl;
  prefill_layout(d, B, T, c.take(0), &pl);
  if (d->dtype == MLA_BF16) {
    LAUNCH("rmsnorm", rmsnorm_rows<bf16_t>((const bf16_t*)x, D, (const bf16_t*)w->g_attn, (bf16_t*)xa, D,
                                (int)M, D, d->rms_eps, st));
    if ((r = prefill_core(d, &w->attn, xa, B, T, rc, rs, x1, x, nullptr, nullptr, nullptr, 0, pl,
                          st)))
      return r;
    LAUNCH("rmsnorm", rmsnorm_rows<bf16_t>((const bf16_t*)x1, D, (const bf16_t*)w->g_ffn, (bf16_t*)xf, D,
                                (int)M, D, d->rms_eps, st));
    GemmParams g = gp_base();
    g.A = (const bf16_t*)xf; g.lda = D;
    g.B = (const bf16_t*)w->w1; g.B2 = (const bf16_t*)w->w3; g.ldb = D;
    g.C = hbuf; g.ldc = F; g.M = (int)M; g.N = 2 * F; g.K = D;
    LAUNCH("gemm_swiglu", gemm_bf16(g, EPI_SWIGLU, -1, st));
    GemmParams o = gp_base();
    o.A = (const bf16_t*)hbuf; o.lda = F; o.B = (const bf16_t*)w->w2; o.ldb = F;
    o.C = out; o.ldc = D; o.R = (const bf16_t*)x1; o.ldr = D;
    o.M = (int)M; o.N = D; o.K = F;
    LAUNCH("gemm_w2_resid", gemm_bf16(o, EPI_RESID, -1, st));
    return MLA_OK;
  }
  LAUNCH("rmsnorm", rmsnorm_rows<float>((const float*)x, D, (const float*)w->g_attn, (float*)xa, D, (int)M,
                             D, d->rms_eps, st));
  if ((r = prefill_core(d, &w->attn, xa, B, T, rc, rs, x1, x, nullptr, nullptr, nullptr, 0, pl,
                        st)))
    return r;
  LAUNCH("rmsnorm", rmsnorm_rows<float>((const float*)x1, D, (const float*)w->g_ffn, (float*)xf, D, (int)M,
                             D, d->rms_eps, st));
  float* hg = (float*)hbuf;
  float* hu = hg + M * F;
  float* hh = hu + M * F;
  GemmF32Params g;
  memset(&g, 0, sizeof g);
  g.A = (const float*)xf; g.lda = D; g.B = (const float*)w->w1; g.ldb = D; g.C = hg; g.ldc = F;
  g.M = (int)M; g.N = F; g.K = D; g.batch = 1; g.b_is_nk = 1;
  LAUNCH("gemm_w1", gemm_f32(g, st));
  g.B = (const float*)w->w3; g.C = hu;
  LAUNCH("gemm_w3", gemm_f32(g, st));
  LAUNCH("swiglu", swiglu_f32(hg, hu, hh, M * F, st));
  GemmF32Params o;
  memset(&o, 0, sizeof o);
  o.A = hh; o.lda = F; o.B = (const float*)w->w2; o.ldb = F; o.C = (float*)out; o.ldc = D;
  o.R = (const float*)x1; o.ldr = D; o.M = (int)M; o.N = D; o.K = F; o.batch = 1; o.b_is_nk = 1;
  LAUNCH("gemm_w2_resid", gemm_f32(o, st));
  return MLA_OK;
}

}  // extern "C"
