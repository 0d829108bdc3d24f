/*
 * mla.h -- C ABI of the MI355X (gfx950) multi-head latent attention library.
 *
 * The library computes the forward pass of multi-head latent attention (MLA)
 * and of the dense transformer block built on it, as described by three
 * pages on Kimi K2 (cited below by title and section):
 *
 *   [DB] "Kimi K2 · Dense transformer block": the step list of the block and
 *        of MLA (down-projections with RMSNorm, up-projections into heads,
 *        RoPE, query/key assembly, residual adds, SwiGLU MLP), its in/out line
 *        (x [B, T, 7168], R [T, 32 pairs], M [T, T] -> [B, T, 7168]) and the
 *        Parameters table.
 *   [MP] "Kimi K2 · Mix and project": decode mode (one query per sequence
 *        reads L = P + 1 keys), the attention-core code excerpt (scaled
 *        scores, causal mask, float32 softmax, P.V, head merge, o_proj) and the
 *        size checks that reject mismatched shapes.
 *   [KV] "Kimi K2 · Key-value compression": the joint down-projection that
 *        emits the 512-feature latent and the 64-feature rotary key, the
 *        latent RMSNorm, and the cache sizes per position (576 for the latent
 *        form, 20,480 for full per-head keys and values).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers are DEVICE pointers unless stated; all tensors are contiguous
 *    row-major.  Every tensor has the element type dims->dtype (MLA_F32 or
 *    MLA_BF16) except the RoPE tables, which are always float32.  Every
 *    device pointer (tensors, weights, gains, biases, RoPE tables, caches,
 *    outputs, workspace) must be 16-byte aligned: the kernels move data in
 *    16-byte vectors.  A misaligned pointer returns MLA_ERR_UNSUPPORTED
 *    (device allocations are 256-byte aligned; offsets into them must keep
 *    16-byte alignment).
 *  - Weights use the nn.Linear [out, in] layout and the fused orderings of
 *    the module code excerpt on [KV]:
 *      w_dq   [q_lora, d]                     query down-projection
 *      g_q    [q_lora]                        query-latent RMSNorm gain
 *      w_uqr  [H*(d_nope+d_rope), q_lora]     query up-projection; per head h
 *                                             rows h*(d_nope+d_rope) + [nope | rope]
 *      w_dkvr [kv_lora + d_rope, d]           joint kv down-projection; rows
 *                                             [latent (kv_lora) | rotary key (d_rope)]
 *      g_kv   [kv_lora]                       kv-latent RMSNorm gain
 *      w_ukv  [H*(d_nope+d_v), kv_lora]       kv up-projection; per head h rows
 *                                             h*(d_nope+d_v) + [key content | value]
 *      w_o    [d, H*d_v]                      output projection; input column h*d_v + c
 *    No biases by default (the pages' parameter totals hold only without
 *    them); the optional attention_bias biases are described at mla_weights.
 *  - RMSNorm is g * x / sqrt(mean(x^2) + eps).  RoPE turns the consecutive
 *    pair (2i, 2i+1) of each rotary slice by angle t * theta_i; the caller
 *    passes the table R as rope_cos/rope_sin [rope_rows, d_rope/2] (float32;
 *    mla_rope_table fills it), row t for position t.
 *  - Ownership: the caller allocates and owns every buffer (inputs, weights,
 *    caches, outputs and the workspace).  The compute calls never allocate
 *    or free device memory and keep no pointer after they return.  Library
 *    state: a thread-local error message; the opt-in kernel timer
 *    (mla_profile_enable) creates HIP events and keeps them, with its
 *    pending records, in thread-local pools until the process ends.
 *  - Asynchrony: calls only enqueue kernels on `stream` (a hipStream_t; NULL
 *    is the default stream) and return.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Errors: all arguments are validated on the host before any HIP call;
 *    a bad argument returns a negative mla_status and enqueues nothing.
 *    mla_last_error() describes the last failure of the calling thread.
 *  - Supported shapes: MLA_F32 accepts any positive widths (value and
 *    query/key head widths up to 1024).  MLA_BF16 requires the Kimi K2 head
 *    widths d_nope = 128, d_rope = 64, d_v = 128 and d_model, q_lora,
 *    kv_lora, H*d_v and d_ff multiples of 64; the latent-cache decode in
 *    bf16 also requires kv_lora = 512, H = 64 and B <= 1024.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL                     */
  MLA_ERR_SHAPE = -2,       /* a size is non-positive or inconsistent          */
  MLA_ERR_UNSUPPORTED = -3, /* valid, but not a shape/dtype the library serves */
  MLA_ERR_WORKSPACE = -4,   /* workspace smaller than the *_workspace_size     */
  MLA_ERR_HIP = -5          /* a HIP launch failed                             */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Hyper-parameters of one MLA layer (and its dense block). */
typedef struct {
  int d_model;       /* d: 7168 in [DB]                                   */
  int n_heads;       /* H: 64                                             */
  int q_lora_rank;   /* query latent width: 1536                          */
  int kv_lora_rank;  /* kv latent width: 512 ([KV])                       */
  int qk_nope_dim;   /* per-head key/query content width: 128             */
  int qk_rope_dim;   /* rotary width: 64 (32 pairs, [DB] in/out line)     */
  int v_head_dim;    /* per-head value width: 128 ([MP] in/out line)      */
  int d_ff;          /* SwiGLU inner width (block only): 18432            */
  float rms_eps;     /* RMSNorm epsilon (1e-6)                            */
  float softmax_scale; /* score scale; 0 selects 1/sqrt(qk_nope_dim +    */
                       /* qk_rope_dim) (the value adopted for the pages'   */
                       /* unstated scale), negative or NaN is rejected     */
  int dtype;         /* mla_dtype                                         */
} mla_dims;

typedef struct {
  const void *w_dq, *g_q, *w_uqr, *w_dkvr, *g_kv, *w_ukv, *w_o;
  /* Optional biases of the attention_bias variant ([KV] module code: the
   * query down-projection, the joint kv down-projection and o_proj take
   * bias=config.attention_bias; the two up-projections have none).  NULL =
   * no bias (the pinned configuration).  dtype as the weights:
   *   b_dq [q_lora], b_dkvr [kv_lora + d_rope] (latent | rotary key), b_o [d].
   * y = x W^T + b; the down-projection biases are added before the latent
   * RMSNorms and the rotary key's RoPE. */
  const void *b_dq, *b_dkvr, *b_o;
} mla_weights;

/* Dense block ([DB]): input RMSNorm gain, MLA, post-attention RMSNorm gain,
 * SwiGLU W1, W3 [d_ff, d] and W2 [d, d_ff]. */
typedef struct {
  const void *g_attn, *g_ffn;
  mla_weights attn;
  const void *w1, *w3, *w2;
} mla_block_weights;

/* The RoPE table R ([DB] in/out line): cos_out/sin_out [n_pos, d_rope/2]
 * float32, angle t * base^(-2i/d_rope) evaluated in float64 on the device.
 * d_rope must be even and positive, n_pos positive, base > 0. */
int mla_rope_table(int n_pos, int d_rope, double base, float *cos_out, float *sin_out,
                   void *stream);

/* ---- Prefill ([DB] steps 1-3 of MLA, [MP] attention core and o_proj) ----
 * out[B, T, d] = MLA(x[B, T, d]) at positions 0..T-1 with the causal mask
 * (key j visible to query i iff j <= i; the [T, T] mask M is implicit).
 * rope tables need rope_rows >= T.
 * Optional cache outputs (pass NULL to skip, then L_cap is ignored):
 *   k_cache [B, H, L_cap, d_nope + d_rope], v_cache [B, H, L_cap, d_v]
 *     (both or neither): slots 0..T-1 receive each head's assembled key
 *     [K^C ; k^R] and value, as the pinned implementation caches them;
 *   latent_cache [B, L_cap, kv_lora + d_rope]: slots 0..T-1 receive the
 *     576-value entries [c^KV-hat ; k^R].
 * Requires T <= L_cap when a cache is given.  bf16: the attention kernel
 * addresses each head's keys with 32-bit byte offsets, so (T + 64) * H * 512
 * must stay below 2^31 (T <= 65471 at 64 heads); a longer prefill returns
 * MLA_ERR_UNSUPPORTED (mla_prefill_chunk_fullcache below, whose keys are
 * 384-byte cache rows, serves longer contexts in pieces).  The same limit
 * holds for dense_block_fwd. */
size_t mla_prefill_workspace_size(const mla_dims *dims, int B, int T);
int mla_prefill(const mla_dims *dims, const mla_weights *w, const void *x, int B, int T,
                const float *rope_cos, const float *rope_sin, int rope_rows, void *out,
                void *k_cache, void *v_cache, void *latent_cache, int L_cap,
                void *workspace, size_t workspace_bytes, void *stream);

/* ---- Decode with the full per-head cache ([MP] decode mode) ----
 * x [B, d]: one new token per sequence at position P (0 <= P < L_cap).
 * k_cache [B, H, L_cap, d_nope + d_rope], v_cache [B, H, L_cap, d_v] hold the
 * history in slots 0..P-1; the call overwrites slot P with the new token's
 * key and value (the cache update of [MP]'s code excerpt) and attends over
 * the L = P + 1 keys 0..P.  out [B, d].  rope_rows > P. */
size_t mla_decode_workspace_size(const mla_dims *dims, int B, int L_cap);
int mla_decode_fullcache(const mla_dims *dims, const mla_weights *w, const void *x, int B, int P,
                         int L_cap, void *k_cache, void *v_cache, const float *rope_cos,
                         const float *rope_sin, int rope_rows, void *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ---- Decode with the latent cache, absorbed form ([KV] Why/Explanation) ----
 * latent_cache [B, L_cap, kv_lora + d_rope]: entry [c^KV-hat ; k^R] per
 * position; slot P is overwritten with the new token's entry.  W_UK is
 * folded into the query and W_UV into the output; the softmax scale is
 * unchanged.  Same x, P, out and workspace rules as the full-cache form. */
int mla_decode_latentcache(const mla_dims *dims, const mla_weights *w, const void *x, int B,
                           int P, int L_cap, void *latent_cache, const float *rope_cos,
                           const float *rope_sin, int rope_rows, void *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ---- Latent-cache decode that allocates nothing ----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * step as mla_decode_latentcache (same arguments, results bit for bit), with
 * the workspace in a library-owned device array of
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB; one per GPU that loads the library,
 * held until the process ends) instead of a caller buffer.  No call
 * allocates or frees memory; the first call on a device looks up the
 * array's device address once (hipGetSymbolAddress).
 *   - Limit: mla_decode_workspace_size(dims, B, L_cap) must be at most
 *     MLA_NOALLOC_SCRATCH_BYTES (e.g. the Kimi K2 shapes up to B = 32 at
 *     L_cap = 100,000); a larger step returns MLA_ERR_WORKSPACE and
 *     enqueues nothing.
 *   - Device: the calling thread's current device; `stream` (NULL = default)
 *     must belong to it, else MLA_ERR_UNSUPPORTED.
 *   - Sharing: every call on a GPU uses that GPU's one array and leaves its
 *     contents behind; the step writes every word it reads, so nothing needs
 *     clearing.  Calls that overlap on one GPU (other streams or threads)
 *     race on the array: serialise them. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mla_decode_latentcache_noalloc(const mla_dims *dims, const mla_weights *w, const void *x,
                                   int B, int P, int L_cap, void *latent_cache,
                                   const float *rope_cos, const float *rope_sin, int rope_rows,
                                   void *out, void *stream);

/* ---- Latent-cache decode as one persistent kernel ----
 * The step of mla_decode_latentcache ([MP] decode mode, [KV] Why and
 * Explanation) as a single cooperative launch: one workgroup per CU runs the
 * down-projection, the latent norms with the cache write, the q
 * up-projection, the query absorption, the split-L attention, the merge
 * with W_UV and o_proj in turn, with a grid-wide barrier between phases,
 * instead of eight kernel launches.  Same arguments, workspace size and
 * rules as mla_decode_latentcache; the result equals it up to the latent
 * norms' reduction order (within the bf16 tolerance, not bit for bit).
 *   - Shapes: bf16 only, B <= 64, 64 heads and kv_lora 512 (else
 *     MLA_ERR_UNSUPPORTED before any HIP call).
 *   - Launch: hipLaunchCooperativeKernel, preceded by a 96-byte
 *     hipMemsetAsync of the workspace's barrier words; a device that cannot
 *     keep one workgroup per CU resident returns MLA_ERR_HIP.  Not for HIP
 *     graph capture (the memset).
 *   - A barrier wait that sees no progress for about a second gives up (the
 *     kernel always ends) and marks the workspace; the step's output is then
 *     undefined, and mla_decode_latentcache_persistent_status reports it. */
int mla_decode_latentcache_persistent(const mla_dims *dims, const mla_weights *w, const void *x,
                                      int B, int P, int L_cap, void *latent_cache,
                                      const float *rope_cos, const float *rope_sin, int rope_rows,
                                      void *out, void *workspace, size_t workspace_bytes,
                                      void *stream);
/* Diagnostic: *status = 1 if a barrier of the last persistent step run in
 * this workspace (same dims, B, L_cap) gave up, else 0.  Synchronous: it
 * copies 4 bytes to the host with hipMemcpy, so call it after the step's
 * stream has finished.  MLA_ERR_NULL / MLA_ERR_SHAPE for bad arguments. */
int mla_decode_latentcache_persistent_status(const mla_dims *dims, int B, int L_cap,
                                             const void *workspace, int *status);

/* ---- Decode over a ragged batch (both cache forms) ----
 * As mla_decode_fullcache / mla_decode_latentcache, but sequence b's new
 * token sits at its own position positions[b] ([MP]'s decode mode per
 * sequence: it writes slot positions[b] and attends over the
 * positions[b] + 1 keys 0 .. positions[b] of its own cache rows).
 *   positions : DEVICE int32 [B], read by the kernels (it may be written by
 *               earlier work on the same stream).  Each entry is clamped into
 *               [0, P_max], so no value can address outside the cache; a
 *               value outside that range gives the result of the clamped
 *               position.
 *   P_max     : host upper bound of the positions, 0 <= P_max < L_cap, used
 *               for the argument checks (rope_rows > P_max), the workspace
 *               and the split plan (mla_decode_workspace_size is unchanged).
 * Ownership, asynchrony and errors as for the uniform forms; a NULL
 * positions pointer returns MLA_ERR_NULL. */
int mla_decode_fullcache_ragged(const mla_dims *dims, const mla_weights *w, const void *x, int B,
                                const int *positions, int P_max, int L_cap, void *k_cache,
                                void *v_cache, const float *rope_cos, const float *rope_sin,
                                int rope_rows, void *out, void *workspace, size_t workspace_bytes,
                                void *stream);
int mla_decode_latentcache_ragged(const mla_dims *dims, const mla_weights *w, const void *x,
                                  int B, const int *positions, int P_max, int L_cap,
                                  void *latent_cache, const float *rope_cos, const float *rope_sin,
                                  int rope_rows, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ---- Chunked prefill (both cache forms) ----
 * T new tokens per sequence at positions P0 .. P0+T-1 (x [B, T, d] ->
 * out [B, T, d]) against a cache whose slots 0 .. P0-1 hold the history:
 * the tokens' entries are written to slots P0 .. P0+T-1, and the token at
 * position P0 + t attends to keys 0 .. P0 + t (the causal mask of [MP]'s
 * code excerpt, shifted by the cached length; its size checks allow a query
 * length above 1 against a longer key length).  P0 = 0 is a prefill with
 * cache outputs; T = 1 is a decode step at P = P0.
 *   k_cache/v_cache or latent_cache: as for the decode forms, [B, ...,
 *   L_cap, ...]; requires P0 >= 0, P0 + T <= L_cap, rope_rows >= P0 + T.
 * The latent form (bf16) expands the per-head keys and values of cache rows
 * 0 .. P0+T-1 from the cached latents into the workspace (the unabsorbed
 * form suits many queries per sequence); the float32 latent form attends in
 * absorbed form.  The workspace size depends on L_cap. */
size_t mla_prefill_chunk_workspace_size(const mla_dims *dims, int B, int T, int L_cap);
int mla_prefill_chunk_fullcache(const mla_dims *dims, const mla_weights *w, const void *x, int B,
                                int T, int P0, int L_cap, void *k_cache, void *v_cache,
                                const float *rope_cos, const float *rope_sin, int rope_rows,
                                void *out, void *workspace, size_t workspace_bytes, void *stream);
int mla_prefill_chunk_latentcache(const mla_dims *dims, const mla_weights *w, const void *x, int B,
                                  int T, int P0, int L_cap, void *latent_cache,
                                  const float *rope_cos, const float *rope_sin, int rope_rows,
                                  void *out, void *workspace, size_t workspace_bytes, void *stream);

/* ---- Dense transformer block ([DB]) ----
 * out = x' + SwiGLU(RMSNorm(x'; g_ffn)), x' = x + MLA(RMSNorm(x; g_attn)),
 * SwiGLU(z) = (silu(z W1^T) * (z W3^T)) W2^T.  x, out [B, T, d]; causal
 * prefill positions 0..T-1; rope_rows >= T. */
size_t dense_block_workspace_size(const mla_dims *dims, int B, int T);
int dense_block_fwd(const mla_dims *dims, const mla_block_weights *w, const void *x, int B, int T,
                    const float *rope_cos, const float *rope_sin, int rope_rows, void *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* ---- Kernel timing (a tracing aid; off by default) ----
 * After mla_profile_enable(1), every later call on the calling thread
 * records a pair of HIP events around each of its kernel launches on the
 * caller's stream (the only case in which the library creates HIP runtime
 * objects: events, kept for reuse until the process ends).
 * mla_profile_summary() waits for the recorded events, writes one line
 * "<kernel name> <launches> <total milliseconds>\n" per kernel name into buf
 * (NUL-terminated; MLA_ERR_SHAPE if len is too small), stores the number of
 * lines in *n_entries (may be NULL) and clears the record. */
int mla_profile_enable(int on);
int mla_profile_summary(char *buf, size_t len, int *n_entries);

/* ---- Measurement yardstick (not a step of the forward pass) ----
 * Reads every byte of buf once with 16-byte vector loads (4096 workgroups,
 * each a contiguous range, sixteen loads in flight per thread) so that the
 * caller can time the HBM read rate this chip reaches: the achievable
 * denominator next to the nominal 8 TB/s for the decode kernels' bandwidth.
 * buf: device, bytes a multiple of 16 (a buffer much larger than the 256 MB
 * Infinity Cache measures HBM); sink: device, 4096 unsigned ints whose XOR
 * is the XOR of every 32-bit word read.
 * MLA_ERR_NULL / MLA_ERR_SHAPE / MLA_ERR_UNSUPPORTED (alignment) on bad
 * arguments; nothing is written to buf. */
int mla_read_sweep(const void *buf, size_t bytes, unsigned *sink, void *stream);

/* Static description of a status code, and the calling thread's last error
 * message (empty after a successful call). */
const char *mla_status_string(int status);
const char *mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
