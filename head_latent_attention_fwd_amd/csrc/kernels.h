// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;

// ------------------------------------------------------------------ GEMM
enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_RESID = 3, EPI_SWIGLU = 4 };
enum { GEMM_CFG_AUTO = -1, GEMM_CFG_256x256 = 0, GEMM_CFG_128x128 = 1, GEMM_CFG_64x128 = 2,
       GEMM_CFG_256x224 = 3 };  // 256x224: products 1792k columns wide (bf16, residual, fp32 K slices)

struct GemmParams {
  const bf16_t* A;   // [M, K] row-major, leading dim lda
  const bf16_t* B;   // [N, K] row-major (nn.Linear weight), leading dim ldb
  const bf16_t* B2;  // second weight: SwiGLU W3 (B is W1, both [N/2, K]); or,
                     // when b_split > 0, the rows n >= b_split of the product
  int b_split;       // rows [0, b_split) from B, [b_split, N) from B2 (0: off)
  void* C;           // output, leading dim ldc (fp32 for EPI_F32, else bf16)
  const bf16_t* R;   // residual [M, N] for EPI_RESID, leading dim ldr
  long lda, ldb, ldc, ldr;
  int M, N, K;       // SwiGLU: N = 2 * d_ff (output has N/2 columns)
  int ksplit;        // number of K slices (grid.y = batch * ksplit)
  int kchunk;        // K per slice, a multiple of 64
  long split_stride; // elements between the fp32 partial outputs of slices
  int batch;
  long sA, sB, sC;   // batch strides in elements
  int tiles_m, tiles_n;  // filled by the launcher
  int group_m;           // M tiles per group of the tile order (launcher)
  const bf16_t* bias;    // optional per-output-column bias [N] (bf16-output
                         // epilogues: EPI_BF16, EPI_RESID, the skinny kernel)
};

struct GemmPlan { int cfg, ksplit, kchunk; };
// tile config and K split (<= max_split; splits need fp32 partial outputs)
GemmPlan gemm_plan(int M, int N, int K, int batch, int max_split);
int gemm_pick_cfg(int M, int N, int K, int batch);
// plan for 64 < M <= 1024 rows (K split with fp32 partials when it pays)
GemmPlan gemm_plan_small(int M, int N, int K, bool fp32_out, int max_split);
hipError_t gemm_bf16(GemmParams p, int epi, int cfg, hipStream_t s);
// Two independent products in one launch (same epilogue and tile config,
// no batch or K split, at least 8 tiles each); product a's tiles are
// scheduled first on every XCD, so a should be the one with the longer K.
hipError_t gemm_bf16_pair(GemmParams a, GemmParams b, int epi, int cfg, hipStream_t s);

// Weight-streaming product for M <= 64 rows (decode): K is cut into 512-wide
// slices; more than one slice writes fp32 partials [slices][M][ldc]
// (split_stride apart), a single slice may write bf16.
int skinny_splits(int K);
hipError_t gemm_skinny_bf16(GemmParams p, bool bf16_out, hipStream_t s);

// Balanced weight-streaming GEMM (M <= 64): units of 128 weight rows x 128 k
// dealt out to G workgroups in equal runs; each writes its fp32 partial
// blocks [Mp][128] (at most NS per workgroup and product) to slots
// (w - w0) NS + j, summed per n-block in workgroup order by stream_reduce /
// stream_sum4.  One launch may stream two products (same rows M): the
// second's units follow the first's.
struct StreamInfo {
  int G;    // workgroups of the launch
  int U;    // units of the launch (both products)
  int KS;   // units per 128-column block of this product (K / 128)
  int NB;   // 128-column blocks of this product
  int Mp;   // padded rows per partial block (32 or 64)
  int u0;   // this product's first unit in the launch
  int w0;   // first workgroup holding this product's units
  int NS;   // partial slots per workgroup
};
bool stream_ok(const GemmParams& p);  // M <= 64, K % 128 == 0, N % 4 == 0, b_split % 128 == 0
StreamInfo stream_info(int M, int N, int K);
size_t stream_part_floats(const StreamInfo& s);
hipError_t gemm_stream_bf16(const GemmParams& p, float* part, const StreamInfo& s, hipStream_t st);
// Two products in one launch (same M; no b_split on the second): false when
// some workgroup would hold more than three 128-column blocks.
bool stream_pair_info(const GemmParams& a, const GemmParams& b, StreamInfo* sa, StreamInfo* sb);
hipError_t gemm_stream_bf16_pair(const GemmParams& a, const GemmParams& b, float* part_a, float* part_b,
                                 const StreamInfo& sa, const StreamInfo& sb, hipStream_t st);
// out[m, n] = sum of the partials (+ R[m, n] when R is not NULL) (+ bias[n]
// when bias is not NULL)
template <typename T>
hipError_t stream_reduce(const float* part, const StreamInfo& s, int M, int N, T* out, long ldo,
                         const bf16_t* R, long ldr, hipStream_t st, const T* bias = nullptr);

// fp32 generic GEMM: C[b] = (R ? R : 0) + A[b] . op(B[b]); op(B) = B^T when
// b_is_nk (B stored [N, K]) else B (stored [K, N]).
struct GemmF32Params {
  const float* A; const float* B; float* C; const float* R;
  long lda, ldb, ldc, ldr;
  int M, N, K, batch;
  long sA, sB, sC;
  int b_is_nk;
  const float* bias;  // optional per-output-column bias [N]
};
hipError_t gemm_f32(const GemmF32Params& p, hipStream_t s);

// -------------------------------------------------------- row kernels
// Sum the split-K partials of the joint down-projection row and produce the
// normalised query latent, normalised kv latent and roped shared key, with
// optional cache writes.
template <typename T> struct LatentNormParams {
  const float* part;  // [nsplit][M][ld_part] fp32 partials (nsplit >= 1)
  int nsplit; long split_stride; long ld_part;
  int M, q_lora, kv_lora, d_rope;
  const T* g_q; const T* g_kv;
  float eps;
  T* cq;  long ld_cq;    // [M, q_lora]
  T* ckv; long ld_ckv;   // [M, kv_lora]
  T* kr;  long ld_kr;    // [M, d_rope]
  const float* rcos; const float* rsin; int n_pairs;
  int rope_T, rope_pos0;  // position of row m = m % rope_T + rope_pos0
  // optional latent cache [B][L_cap][kv_lora + d_rope]: row m = b*rope_T + t
  // goes to slot t + rope_pos0 of sequence b
  T* latent_cache; int L_cap;
  // stream != 0: `part` holds the weight-streaming GEMM's partial blocks
  // (StreamInfo si), summed here instead of the nsplit fp32 slices
  int stream; StreamInfo si;
  // optional per-sequence positions (decode, rope_T = 1): row m is at
  // position seq_pos[m] clamped into [0, pos_max] instead of rope_pos0
  const int* seq_pos; int pos_max;
  // optional biases of the two down-projections, added to the summed row
  // before the norms and the RoPE: bias_q [q_lora], bias_kvr [kv_lora + d_rope]
  const T* bias_q; const T* bias_kvr;
};
template <typename T> hipError_t latent_norm_rope(const LatentNormParams<T>& p, hipStream_t s);

template <typename T>
hipError_t rmsnorm_rows(const T* x, long ldx, const T* g, T* y, long ldy, int M, int D, float eps,
                        hipStream_t s);

hipError_t rope_table(int n_pos, int n_pairs, double base, float* cos_out, float* sin_out,
                      hipStream_t s);

// fp32-path elementwise helpers
hipError_t rope_inplace_f32(float* x, long ldx, int M, int ncols, int head_dim, int rope_start,
                            const float* rcos, const float* rsin, int n_pairs, int rope_T,
                            int rope_pos0, hipStream_t s, const int* seq_pos = nullptr,
                            int pos_max = 0);
hipError_t swiglu_f32(const float* g, const float* u, float* h, long n, hipStream_t s);
// streaming-read yardstick: reads bytes / 16 chunks of buf, one word per
// workgroup into sink [nwg]
constexpr int kReadSweepWG = 4096;
hipError_t read_sweep(const void* buf, size_t bytes, unsigned* sink, int nwg, hipStream_t s);

// Scatter the per-head keys/values of new tokens into the full cache.
// kv [M][H][d_nope + d_v] (row m = b * T + t), kr [M][d_rope]; slot t + pos0,
// or (decode, T = 1) slot seq_pos[b] clamped into [0, pos_max].
template <typename T>
hipError_t scatter_full_cache(const T* kv, const T* kr, T* k_cache, T* v_cache, int Bn, int T_,
                              int pos0, int L_cap, int H, int d_nope, int d_rope, int d_v,
                              hipStream_t s, const int* seq_pos = nullptr, int pos_max = 0);

// Sum fp32 split partials [nsplit][M][N] into T out [M][ldo] (+ bias[n]).
template <typename T>
hipError_t reduce_splits(const float* part, int nsplit, long split_stride, int M, int N, T* out,
                         long ldo, hipStream_t s, const T* bias = nullptr);

// ------------------------------------------------------------ attention
// Generic attention (fp32 path and any head widths): one wave per query.
struct AttnGenericParams {
  const float* q_nope; long q_row; long q_head;    // query (b, i, h) at b*Tq*q_row... see below
  const float* q_rope; long qr_row; long qr_head;
  const float* k_nope; long kn_b, kn_j, kn_h;
  const float* k_rope; long kr_b, kr_j, kr_h;
  const float* v;      long v_b, v_j, v_h;
  float* out; long o_row; long o_head;
  int B, Tq, Tk, H, d_nope, d_rope, d_v;
  int causal_offset;  // query i sees keys j <= i + causal_offset
  float scale;
  // optional (decode, Tq = 1): sequence b sees keys j <= seq_pos[b] clamped
  // into [0, pos_max]
  const int* seq_pos; int pos_max;
};
hipError_t attn_generic_f32(const AttnGenericParams& p, hipStream_t s);

// bf16 flash prefill (Kimi head widths 128 + 64, value 128), causal.
struct FlashParams {
  const bf16_t* q;   // [B*T][H][192]   (rope part NOT yet rotated: RoPE is
                     // applied to the query fragments as they are loaded)
  const bf16_t* kv;  // [B*T][H][256]   ([k_nope 128 | v 128] per head)
  const bf16_t* kr;  // [B*T][64]       (rotated, shared by heads)
  bf16_t* out;       // [B*T][H*128]
  const float* rcos; const float* rsin;  // RoPE table [>= T][32]
  int B, T, H;
  float scale_log2;  // softmax scale * log2(e)
  // Key/value sources of the ping-pong kernel (flash_pp.hip), per sequence b
  // and head h: key j's content part (128) at kc + b kc_b + h kc_h (elements)
  // + j kc_kb (bytes), its rotary part (64) likewise from kr2, its value (128)
  // from vv.  Keys 0 .. P0 + T - 1 exist; query t sits at position P0 + t
  // and sees keys j <= P0 + t.  flash_set_prefill_layout() fills these for a
  // plain prefill (kv / kr above, P0 = 0).
  const bf16_t* kc;  long kc_b, kc_h; int kc_kb;
  const bf16_t* kr2; long kr_b, kr_h; int kr_kb;
  const bf16_t* vv;  long v_b, v_h;   int v_kb;
  int P0;
  // Key split (ping-pong kernel): with nsplit > 1, each (query tile, head)
  // is spread over nsplit workgroups, each over an even share of its key
  // tiles; they write unnormalised outputs opart [nsplit][B*T][H][128] and
  // (m, l) ostat [nsplit][B*T][H][2] (fp32), which flash_combine_bf16 merges
  // into out.  nsplit = 1: out written directly.
  int nsplit;
  float* opart; float* ostat;
};
// merge of the key-split partials of flash_prefill_pp_bf16 into p.out
hipError_t flash_combine_bf16(const FlashParams& p, hipStream_t s);
// the key/value source fields for the prefill layout (kv [B*T][H][256], kr [B*T][64])
void flash_set_prefill_layout(FlashParams& p);
// ping-pong form (flash_pp.hip); needs its byte offsets below 2^31
bool flash_pp_ok(const FlashParams& p);
// whether a plain prefill of T tokens with H heads fits flash_pp_ok (host
// check, before any launch)
bool flash_prefill_fits(int T, int H);
hipError_t flash_prefill_pp_bf16(const FlashParams& p, hipStream_t s);

// bf16 decode over the full per-head cache (one query per sequence).
struct DecodeFullParams {
  const bf16_t* q;       // [B][H][192] (rope part rotated here, at position L-1)
  bf16_t* k_cache;       // [B][H][L_cap][192]
  bf16_t* v_cache;       // [B][H][L_cap][128]
  // Optional fused inputs of a decode step (NULL: q is read from `q` and
  // slot L-1 of the caches is already written): the q and kv up-projections
  // as weight-stream partial blocks (summed here, in workgroup order) and the
  // roped shared key kr [B][64].  The workgroup whose key range holds slot
  // L-1 writes that slot of both caches before reading them.
  const float* qpart; StreamInfo qsi;
  const float* kvpart; StreamInfo kvsi; const bf16_t* kr;
  bf16_t* out;           // [B][H*128]
  float* part;           // split partials: [B*H][nsplit][128 + 2]
  const float* rcos; const float* rsin;  // RoPE table, row L-1 used
  int B, H, L, L_cap, nsplit, chunk;
  float scale_log2;
  // optional per-sequence positions: sequence b's new token sits at
  // seq_pos[b] (clamped into [0, L - 1]) and attends over that many + 1 keys
  const int* seq_pos;
};
hipError_t decode_full_bf16(const DecodeFullParams& p, hipStream_t s);

// bf16 absorbed decode over the latent cache.
struct DecodeLatentParams {
  const bf16_t* q_abs;   // [B][H][576]  [absorbed query q~ (W_UK folded in) | roped q^R]
  const bf16_t* cache;   // [B][L_cap][576]
  float* stats;          // [G][H][2]: running max m (log2 units) and sum l per workgroup
  bf16_t* opart;         // [G][H][512]: unnormalised o~ per workgroup
  const float* rcos; const float* rsin;  // RoPE table, row L-1 used
  // G workgroups.  With seq_pos, plan (3 G + 2 B ints, written by absorb_q;
  // G >= B) gives each a key range of one sequence and each sequence its
  // workgroups; without (one length L for all), plan is NULL and sequence b
  // has workgroups b * splits .. + splits - 1 (G = B * splits)
  int B, H, L, L_cap, G, splits;
  const int* plan;
  float scale_log2;
  const int* seq_pos;  // optional per-sequence positions, as for DecodeFullParams
  // the merge of the splits is fused with the value up-projection (W_UV rows
  // of kv_b_proj [H*256][512]), writing out [B][H*128] (head dims 128 + 128)
  const bf16_t* w_ukv; bf16_t* out;
};
hipError_t decode_latent_bf16(const DecodeLatentParams& p, hipStream_t s);

// bf16 query absorption q~[b,h,:] = q_nope[b,h,:] . W_UK,h  (W_UK,h = rows
// h*256 .. h*256+127 of kv_b_proj, each of 512 latent features), written with
// the rotary query roped at position L-1: qa[b][h] = [q~ (512) | q^R (64)].
struct AbsorbParams {
  const bf16_t* q;                    // [B][H][192], or NULL with qpart
  const float* qpart; StreamInfo qsi; // q as weight-stream partial blocks
  const bf16_t* w_ukv;                // [H*256][512]
  bf16_t* qa;                         // [B][H][576]
  const float* rcos; const float* rsin;
  int B, H, L;
  const int* seq_pos;                 // optional: row b roped at seq_pos[b] (clamped to [0, L-1])
  // optional: the latent attention's split plan for G workgroups, written
  // here (3 G + 2 B ints; G >= B)
  int* plan; int G;
};
hipError_t absorb_q_bf16(const AbsorbParams& p, hipStream_t s);

// The whole bf16 latent-cache decode step (uniform position, M <= 64 rows) as
// one cooperative launch: down-projection weight stream, latent norms with
// RoPE and the cache write, q up-projection weight stream, query absorption,
// split-L attention, merge fused with W_UV, o_proj weight stream and its split
// sum, with a grid-wide barrier between consecutive phases.  Each phase runs
// the same device body as its own kernel in the multi-launch step, over the
// same plans (StreamInfo of each stream, the attention's splits).
struct PersistLatentParams {
  GemmParams down; StreamInfo down_si; float* down_part;   // partials summed by the norms
  LatentNormParams<bf16_t> norm;
  GemmParams qup; StreamInfo qup_si; float* qup_part;      // partials summed by the absorption
  AbsorbParams ab;
  DecodeLatentParams at;
  GemmParams oproj; StreamInfo oproj_si; float* oproj_part;
  // barrier state (24 words, zeroed on the stream before the launch): [0]
  // XCD arrivals, [1] generation, [2] status (1: a barrier wait gave up), [3]
  // XCDs holding workgroups, [8 + x] arrivals and [16 + x] workgroups of XCD x
  unsigned* sync;
};
hipError_t decode_latent_persistent_bf16(const PersistLatentParams& p, hipStream_t s);

}  // namespace mla
