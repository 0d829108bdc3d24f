"""CPU oracle for the multi-head latent attention (MLA) forward and the dense block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it, and it shares no code, table or helper with the HIP path.

Everything is computed in float64 (``dtype`` may be lowered to float32 only
for the CPU timing baseline), with NumPy's matmul as the one library primitive.
No intermediate is rounded: the oracle consumes exactly the values the GPU is
given (bf16 inputs are passed here as their exact float values) and returns
the exact result up to float64 rounding.

Sources, cited by page title and section:

[DB] "Kimi K2 · Dense transformer block" -- the step-by-step equation list
     ("All 28 steps"), its in/out line (x [B,T,7168], R [T, 32 pairs],
     M [T,T]), the Parameters table and the decoder-layer code excerpt
     (pre-norm residual structure).
[MP] "Kimi K2 · Mix and project" -- the in/out line of decode mode
     (P = 1,000 cached positions, L = P + 1 keys), the Parameters table
     (o_proj 8,192 x 7,168), the Explanation (o_proj is the only step that
     mixes heads) and the attention-core code excerpt (RoPE, query/key
     assembly, scaled scores, additive causal mask, float32 softmax, P.V,
     head merge, o_proj).
[KV] "Kimi K2 · Key-value compression" -- the equations c^KV = x W_DKV and
     c^KV-hat = RMSNorm(c^KV), the Parameters table, the Explanation (576
     latent values per position against 20,480 for full per-head keys and
     values; one joint projection emits the latent and the rotary key and is
     split after the product) and the module/forward code excerpts.

Readings taken where the pages are silent (each one is also stated at the
function that uses it):

* RMSNorm is g * x / sqrt(mean(x^2) + eps), eps = 1e-6.
* RoPE rotates consecutive pairs (2i, 2i+1) by the angle t * base^(-2i/d_rope),
  base 10000, position t = 0..T-1 in prefill and t = P for a decode token.
  Any other fixed pairing is the same map up to one permutation applied to
  both queries and keys, which leaves every score unchanged.
* The softmax scale is 1/sqrt(d_nope + d_rope), also in the absorbed form.
* The causal mask sets scores of keys j > i to -inf (exact zeros after exp).
* No linear layer has a bias in the pinned configuration (the pages'
  parameter totals hold only then).  The module code on [KV] makes the
  query down-projection, the joint kv down-projection and o_proj carry a bias
  when the config asks for one (attention_bias); the optional b_dq, b_dkvr
  and b_o below are those biases, added to the products y = x W^T + b.
* The per-head row layouts of the fused up-projections are head-major:
  q rows h*(d_nope+d_rope) + [nope | rope], kv rows h*(d_nope+d_v) + [k | v].
* Decode: slots 0..P-1 of a cache are history; the new token's entries are
  written to slot P, and the token attends to keys 0..P.
* Dropout is the identity (inference forward).
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

__all__ = [
    "MLADims", "KIMI_K2", "TINY", "MLAWeights", "BlockWeights",
    "weight_shapes", "bias_shapes", "block_weight_shapes", "parameter_counts",
    "cache_values_per_position", "rms_norm", "rope_angles", "apply_rope",
    "silu", "mla_project", "attention", "mla_prefill",
    "mla_decode_fullcache", "mla_decode_latentcache", "dense_block",
]


@dataclass(frozen=True)
class MLADims:
    """Hyper-parameters of one MLA layer and its dense block.

    The Kimi K2 values come from [DB] (7,168 model width, 64 heads, R with
    32 rotary pairs), [KV] (512-feature latent, 64-feature rotary key,
    per-head keys of 192 features and values of 128) and the parameter
    totals of [DB]/[KV]/[MP], which fix the query latent (1,536) and the MLP
    inner width (18,432).
    """
    d_model: int
    n_heads: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_dim: int
    qk_rope_dim: int
    v_head_dim: int
    d_ff: int = 0
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def q_head_dim(self) -> int:
        return self.qk_nope_dim + self.qk_rope_dim

    @property
    def softmax_scale(self) -> float:
        # Reading: 1/sqrt of the per-head query/key width (the pages show the
        # multiplication by the scale in [MP], not its value).
        return 1.0 / math.sqrt(self.q_head_dim)


KIMI_K2 = MLADims(d_model=7168, n_heads=64, q_lora_rank=1536, kv_lora_rank=512,
                  qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128, d_ff=18432)
# The tiny float32 prefill workload: d=256, 4 heads, q latent 96, kv latent 64,
# 32 nope + 16 rope, v 32.  d_ff is only used by tiny block tests.
TINY = MLADims(d_model=256, n_heads=4, q_lora_rank=96, kv_lora_rank=64,
               qk_nope_dim=32, qk_rope_dim=16, v_head_dim=32, d_ff=512)


def weight_shapes(dims: MLADims) -> dict:
    """Shapes of the MLA weights in nn.Linear [out, in] layout ([KV] code
    excerpt of the module definitions): q_a_proj, its RMSNorm gain, q_b_proj,
    kv_a_proj_with_mqa (latent rows first, then the rotary-key rows), its
    latent RMSNorm gain, kv_b_proj and o_proj.  No biases."""
    H = dims.n_heads
    return {
        "w_dq": (dims.q_lora_rank, dims.d_model),
        "g_q": (dims.q_lora_rank,),
        "w_uqr": (H * dims.q_head_dim, dims.q_lora_rank),
        "w_dkvr": (dims.kv_lora_rank + dims.qk_rope_dim, dims.d_model),
        "g_kv": (dims.kv_lora_rank,),
        "w_ukv": (H * (dims.qk_nope_dim + dims.v_head_dim), dims.kv_lora_rank),
        "w_o": (dims.d_model, H * dims.v_head_dim),
    }


def block_weight_shapes(dims: MLADims) -> dict:
    """Dense-block weights ([DB] steps and Parameters): the two block RMSNorm
    gains and the SwiGLU matrices W1, W3 [d_ff, d] and W2 [d, d_ff]."""
    return {
        "g_attn": (dims.d_model,),
        "g_ffn": (dims.d_model,),
        "w1": (dims.d_ff, dims.d_model),
        "w3": (dims.d_ff, dims.d_model),
        "w2": (dims.d_model, dims.d_ff),
    }


def parameter_counts(dims: MLADims) -> dict:
    """Per-component parameter counts, summed from the shape tables above
    ([DB], [KV] and [MP] Parameters tables)."""
    mla = {k: int(np.prod(s)) for k, s in weight_shapes(dims).items()}
    blk = {k: int(np.prod(s)) for k, s in block_weight_shapes(dims).items()}
    kv_compression = dims.d_model * dims.kv_lora_rank + mla["g_kv"]
    mla_total = sum(mla.values())
    mlp_total = blk["w1"] + blk["w3"] + blk["w2"]
    return {
        "kv_compression": kv_compression,
        "mla": mla_total,
        "o_proj": mla["w_o"],
        "mlp": mlp_total,
        "attn_norm": blk["g_attn"],
        "mlp_norm": blk["g_ffn"],
        "block": blk["g_attn"] + mla_total + blk["g_ffn"] + mlp_total,
        "kv_a_output_features": weight_shapes(dims)["w_dkvr"][0],
    }


def cache_values_per_position(dims: MLADims) -> dict:
    """Values cached per position and layer ([KV] Explanation): the latent
    plus the shared rotary key, against full per-head keys and values."""
    return {
        "latent": dims.kv_lora_rank + dims.qk_rope_dim,
        "full": dims.n_heads * (dims.q_head_dim + dims.v_head_dim),
    }


@dataclass
class MLAWeights:
    w_dq: np.ndarray
    g_q: np.ndarray
    w_uqr: np.ndarray
    w_dkvr: np.ndarray
    g_kv: np.ndarray
    w_ukv: np.ndarray
    w_o: np.ndarray
    # optional biases of the attention_bias variant ([KV] module code):
    # q_a_proj [q_lora], kv_a_proj_with_mqa [kv_lora + d_rope], o_proj [d]
    b_dq: np.ndarray | None = None
    b_dkvr: np.ndarray | None = None
    b_o: np.ndarray | None = None

    def check(self, dims: MLADims) -> None:
        for name, shape in weight_shapes(dims).items():
            got = getattr(self, name).shape
            if got != shape:
                raise ValueError(f"{name}: shape {got}, expected {shape}")
        for name, shape in bias_shapes(dims).items():
            b = getattr(self, name)
            if b is not None and b.shape != shape:
                raise ValueError(f"{name}: shape {b.shape}, expected {shape}")


def bias_shapes(dims: MLADims) -> dict:
    """Biases of the attention_bias variant: the layers the [KV] module code
    builds with bias=config.attention_bias (q_b_proj and kv_b_proj have
    bias=False)."""
    return {"b_dq": (dims.q_lora_rank,), "b_dkvr": (dims.kv_lora_rank + dims.qk_rope_dim,),
            "b_o": (dims.d_model,)}


def _bias(b, dtype):
    return 0.0 if b is None else _f(b, dtype)


@dataclass
class BlockWeights:
    g_attn: np.ndarray
    g_ffn: np.ndarray
    attn: MLAWeights
    w1: np.ndarray
    w3: np.ndarray
    w2: np.ndarray

    def check(self, dims: MLADims) -> None:
        self.attn.check(dims)
        for name, shape in block_weight_shapes(dims).items():
            got = getattr(self, name).shape
            if got != shape:
                raise ValueError(f"{name}: shape {got}, expected {shape}")


def _f(a, dtype):
    return np.asarray(a, dtype=dtype)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis ([DB] steps x_attn = RMSNorm(x_n) and
    x_ffn = RMSNorm(x'_n); [KV] c^KV-hat = RMSNorm(c^KV); the query-latent
    norm of [DB]).  Reading: g * x / sqrt(mean(x^2) + eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def rope_angles(positions: np.ndarray, d_rope: int, base: float,
                dtype=np.float64) -> tuple[np.ndarray, np.ndarray]:
    """The rotary table R [positions, d_rope/2 pairs] of [DB]'s in/out line,
    as (cos, sin).  Reading: pair i turns by t * base^(-2i/d_rope)."""
    n_pairs = d_rope // 2
    i = np.arange(n_pairs, dtype=np.float64)
    inv_freq = base ** (-(2.0 * i) / d_rope)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """RoPE(x_t, R_t) ([DB] steps Q^R_t = RoPE(Q^pe_t, R_t) and
    k^R_t = RoPE(k^pe_t, R_t)).  ``x`` is [..., d_rope] and ``cos``/``sin``
    broadcast against [..., d_rope/2].  Pair (2i, 2i+1) becomes
    (a cos - b sin, a sin + b cos)."""
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """a = g * sigma(g) of [DB]'s SwiGLU steps, sigma the logistic function."""
    return z / (1.0 + np.exp(-z))


def mla_project(dims: MLADims, w: MLAWeights, x: np.ndarray,
                positions: np.ndarray, dtype=np.float64) -> dict:
    """Steps 1-3 of MLA for tokens ``x`` [B, T, d] at ``positions`` [T].

    [DB] equation list: c^Q = x W_DQ, c^Q-hat = RMSNorm(c^Q); c^KV = x W_DKV,
    c^KV-hat = RMSNorm(c^KV); q^C = c^Q-hat W_UQ and q^pe = c^Q-hat W_QR,
    reshaped per head; k^C = c^KV-hat W_UK, reshaped; k^pe = x W_KR (one
    rotary key shared by every head); v = c^KV-hat W_UV, reshaped; RoPE on
    Q^pe and k^pe.  [KV]: W_DKV and W_KR are one matrix whose product is split
    into the 512 latent and the 64 rotary features; W_UK and W_UV are one
    matrix whose per-head output is split into key content and value.
    """
    w.check(dims)
    H, dn, dr, dv = dims.n_heads, dims.qk_nope_dim, dims.qk_rope_dim, dims.v_head_dim
    B, T, _ = x.shape
    x = _f(x, dtype)
    # Query path: down-projection, latent RMSNorm, up-projection.
    c_q = x @ _f(w.w_dq, dtype).T + _bias(w.b_dq, dtype)           # [B,T,q_lora]
    c_q_hat = rms_norm(c_q, _f(w.g_q, dtype), dims.rms_eps)
    q = (c_q_hat @ _f(w.w_uqr, dtype).T).reshape(B, T, H, dn + dr)
    q_nope = q[..., :dn]                                            # Q^C
    q_pe = q[..., dn:]                                              # Q^pe
    # Joint KV down-projection, split after the product ([KV] Explanation).
    a = x @ _f(w.w_dkvr, dtype).T + _bias(w.b_dkvr, dtype)         # [B,T,kv_lora+dr]
    c_kv = a[..., :dims.kv_lora_rank]
    k_pe = a[..., dims.kv_lora_rank:]                               # [B,T,dr]
    c_kv_hat = rms_norm(c_kv, _f(w.g_kv, dtype), dims.rms_eps)
    kv = (c_kv_hat @ _f(w.w_ukv, dtype).T).reshape(B, T, H, dn + dv)
    k_nope = kv[..., :dn]                                           # K^C
    v = kv[..., dn:]                                                # V
    # RoPE with the table row of each token's position.
    cos, sin = rope_angles(positions, dr, dims.rope_base, dtype)    # [T, dr/2]
    q_rope = apply_rope(q_pe, cos[None, :, None, :], sin[None, :, None, :])
    k_rope = apply_rope(k_pe, cos[None, :, :], sin[None, :, :])
    return dict(c_q=c_q, c_q_hat=c_q_hat, c_kv=c_kv, c_kv_hat=c_kv_hat,
                k_pe=k_pe, q_nope=q_nope, q_pe=q_pe, q_rope=q_rope,
                k_nope=k_nope, k_rope=k_rope, v=v)


def attention(q_nope, q_rope, k_nope, k_rope, v, scale, q_pos, k_pos,
              return_probs=False):
    """Scaled dot-product attention of [MP]'s code excerpt for one batch row.

    q_nope [Tq,H,dn], q_rope [Tq,H,dr], k_nope [Tk,H,dn], k_rope [Tk,dr]
    (shared by every head), v [Tk,H,dv].  Q = [Q^C ; Q^R] and
    K_h = [K^C_h ; k^R] ([DB] steps); scores S = scale * Q K^T; the causal
    mask removes keys whose position exceeds the query's; softmax over keys;
    O = P V.  Returns O [Tq,H,dv] (and P [H,Tq,Tk] when asked).
    """
    Tq, H, _ = q_nope.shape
    Tk = k_nope.shape[0]
    dv = v.shape[-1]
    out = np.empty((Tq, H, dv), dtype=q_nope.dtype)
    probs = np.empty((H, Tq, Tk), dtype=q_nope.dtype) if return_probs else None
    masked = np.asarray(k_pos)[None, :] > np.asarray(q_pos)[:, None]   # [Tq,Tk]
    for h in range(H):
        Q = np.concatenate([q_nope[:, h, :], q_rope[:, h, :]], axis=-1)      # [Tq,dqk]
        K = np.concatenate([k_nope[:, h, :], k_rope], axis=-1)               # [Tk,dqk]
        S = (Q @ K.T) * scale
        S = np.where(masked, -np.inf, S)
        m = np.max(S, axis=-1, keepdims=True)
        E = np.exp(S - m)
        P = E / np.sum(E, axis=-1, keepdims=True)
        out[:, h, :] = P @ v[:, h, :]
        if return_probs:
            probs[h] = P
    return (out, probs) if return_probs else out


def _merge_heads(o: np.ndarray) -> np.ndarray:
    """[MP] head merge: [.., H, dv] -> [.., H*dv], column h*dv + c."""
    return o.reshape(*o.shape[:-2], o.shape[-2] * o.shape[-1])


def mla_prefill(dims: MLADims, w: MLAWeights, x: np.ndarray, rows=None,
                dtype=np.float64, return_intermediates=False):
    """MLA forward over a prefill of x [B, T, d] at positions 0..T-1, causal.

    Steps 1-3 by :func:`mla_project`, step 4 by :func:`attention`, step 5 is
    the head merge and o_proj ([MP]).  ``rows`` (optional) restricts the
    query rows whose outputs are computed; keys and values always cover all
    T positions.  Returns out [B, len(rows) or T, d].
    """
    B, T, _ = x.shape
    pos = np.arange(T)
    p = mla_project(dims, w, x, pos, dtype)
    qrows = np.arange(T) if rows is None else np.asarray(rows)
    o = np.empty((B, len(qrows), dims.n_heads, dims.v_head_dim), dtype=dtype)
    for b in range(B):
        o[b] = attention(p["q_nope"][b, qrows], p["q_rope"][b, qrows],
                         p["k_nope"][b], p["k_rope"][b], p["v"][b],
                         dims.softmax_scale, pos[qrows], pos)
    out = _merge_heads(o) @ _f(w.w_o, dtype).T + _bias(w.b_o, dtype)
    if return_intermediates:
        p["o"] = o
        return out, p
    return out


def full_cache_entries(dims: MLADims, proj: dict) -> tuple[np.ndarray, np.ndarray]:
    """Per-head key [K^C_h ; k^R] and value of each token, as the pinned
    implementation caches them ([MP] code excerpt: the assembled key and the
    value are what the cache update stores).  Returns K [B,H,T,dqk] and
    V [B,H,T,dv]."""
    k_nope, k_rope, v = proj["k_nope"], proj["k_rope"], proj["v"]
    B, T, H, _ = k_nope.shape
    kr = np.broadcast_to(k_rope[:, :, None, :], (B, T, H, dims.qk_rope_dim))
    K = np.concatenate([k_nope, kr], axis=-1).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(K), np.ascontiguousarray(v.transpose(0, 2, 1, 3))


def latent_cache_entries(dims: MLADims, proj: dict) -> np.ndarray:
    """The 576-value latent cache entry [c^KV-hat ; k^R] of each token
    ([KV] Explanation).  Returns [B, T, kv_lora + dr]."""
    return np.concatenate([proj["c_kv_hat"], proj["k_rope"]], axis=-1)


def mla_decode_fullcache(dims: MLADims, w: MLAWeights, x_new: np.ndarray, P: int,
                         k_cache: np.ndarray, v_cache: np.ndarray, dtype=np.float64):
    """One decode step with the full per-head cache ([MP] decode mode:
    one query per sequence over L = P + 1 keys; cache update as in [MP]'s
    code excerpt).

    x_new [B, d] is the token at position P.  k_cache [B,H,L_cap,dqk] and
    v_cache [B,H,L_cap,dv] hold the history in slots 0..P-1.  Returns
    (out [B, d], k_cache', v_cache') with slot P of the copies overwritten by
    the new token's key and value.
    """
    B = x_new.shape[0]
    p = mla_project(dims, w, x_new[:, None, :], np.array([P]), dtype)
    K_new, V_new = full_cache_entries(dims, p)                       # [B,H,1,*]
    kc = _f(k_cache, dtype).copy()
    vc = _f(v_cache, dtype).copy()
    kc[:, :, P, :] = K_new[:, :, 0, :]
    vc[:, :, P, :] = V_new[:, :, 0, :]
    L = P + 1
    o = np.empty((B, dims.n_heads, dims.v_head_dim), dtype=dtype)
    for b in range(B):
        # Every cached key 0..P precedes or is the query's own position, so
        # the causal mask removes nothing here.  Each head reads its own key
        # rows as stored (the rotary part of each copy is that token's k^R).
        for h in range(dims.n_heads):
            Q = np.concatenate([p["q_nope"][b, 0, h], p["q_rope"][b, 0, h]])
            S = (kc[b, h, :L, :] @ Q) * dims.softmax_scale
            m = np.max(S)
            E = np.exp(S - m)
            Pr = E / np.sum(E)
            o[b, h] = Pr @ vc[b, h, :L, :]
    out = _merge_heads(o) @ _f(w.w_o, dtype).T + _bias(w.b_o, dtype)
    return out, kc, vc


def absorbed_query(dims: MLADims, w: MLAWeights, q_nope: np.ndarray, dtype=np.float64):
    """W_UK folded into the query: q~_h[k] = sum_c Q^C_h[c] W_UK,h[c, k],
    with W_UK,h the key rows of head h in kv_b_proj.  (Associativity of
    q^C . (W_UK c) -- the latent-caching design that [KV]'s "Why" section
    describes; the pages do not print the folding itself.)
    q_nope [..., H, dn] -> [..., H, kv_lora]."""
    H, dn, dv = dims.n_heads, dims.qk_nope_dim, dims.v_head_dim
    W = _f(w.w_ukv, dtype).reshape(H, dn + dv, dims.kv_lora_rank)
    W_UK = W[:, :dn, :]                                              # [H, dn, r]
    return np.einsum("...hc,hck->...hk", q_nope, W_UK)


def absorbed_output(dims: MLADims, w: MLAWeights, o_lat: np.ndarray, dtype=np.float64):
    """W_UV folded into the output: O_h[c] = sum_k o~_h[k] W_UV,h[c, k],
    with W_UV,h the value rows of head h in kv_b_proj.
    o_lat [..., H, kv_lora] -> [..., H, dv]."""
    H, dn, dv = dims.n_heads, dims.qk_nope_dim, dims.v_head_dim
    W = _f(w.w_ukv, dtype).reshape(H, dn + dv, dims.kv_lora_rank)
    W_UV = W[:, dn:, :]                                              # [H, dv, r]
    return np.einsum("...hk,hck->...hc", o_lat, W_UV)


def mla_decode_latentcache(dims: MLADims, w: MLAWeights, x_new: np.ndarray, P: int,
                           latent_cache: np.ndarray, dtype=np.float64):
    """One decode step with the 576-value latent cache, in absorbed form.

    The cache entry of a token is [c^KV-hat ; k^R] ([KV] Explanation).  The
    new token's entry is written to slot P.  Per head: q~ = absorbed query,
    s_j = scale * (q~ . c_j + Q^R . k^R_j) over j = 0..P with the unchanged
    scale 1/sqrt(d_nope + d_rope), softmax, o~ = sum_j p_j c_j, then
    O_h = o~ W_UV,h^T; head merge and o_proj as in prefill ([MP]).
    Returns (out [B, d], latent_cache').
    """
    B = x_new.shape[0]
    r = dims.kv_lora_rank
    p = mla_project(dims, w, x_new[:, None, :], np.array([P]), dtype)
    entry = latent_cache_entries(dims, p)                            # [B,1,576]
    cc = _f(latent_cache, dtype).copy()
    cc[:, P, :] = entry[:, 0, :]
    L = P + 1
    q_t = absorbed_query(dims, w, p["q_nope"][:, 0], dtype)          # [B,H,r]
    q_r = p["q_rope"][:, 0]                                          # [B,H,dr]
    o_lat = np.empty((B, dims.n_heads, r), dtype=dtype)
    for b in range(B):
        C = cc[b, :L, :r]
        KR = cc[b, :L, r:]
        S = (q_t[b] @ C.T + q_r[b] @ KR.T) * dims.softmax_scale      # [H, L]
        m = np.max(S, axis=-1, keepdims=True)
        E = np.exp(S - m)
        Pr = E / np.sum(E, axis=-1, keepdims=True)
        o_lat[b] = Pr @ C
    o = absorbed_output(dims, w, o_lat, dtype)                       # [B,H,dv]
    out = _merge_heads(o) @ _f(w.w_o, dtype).T + _bias(w.b_o, dtype)
    return out, cc


def mla_prefill_chunk_fullcache(dims: MLADims, w: MLAWeights, x: np.ndarray, P0: int,
                                k_cache: np.ndarray, v_cache: np.ndarray, dtype=np.float64):
    """Chunked prefill with the full cache: the T tokens x [B, T, d] sit at
    positions P0 .. P0+T-1 and slots 0 .. P0-1 of k_cache [B,H,L_cap,dqk] /
    v_cache [B,H,L_cap,dv] hold the history.  The tokens' keys and values go
    to slots P0 .. P0+T-1 (the cache update of [MP]'s code excerpt); token t
    attends over keys 0 .. P0+t (its causal mask, [T, P0+T]), each head reading
    its own key rows as stored.  Returns (out [B, T, d], k_cache', v_cache')."""
    B, T, _ = x.shape
    H, dv = dims.n_heads, dims.v_head_dim
    pos = P0 + np.arange(T)
    p = mla_project(dims, w, x, pos, dtype)
    K_new, V_new = full_cache_entries(dims, p)                        # [B,H,T,*]
    kc = _f(k_cache, dtype).copy()
    vc = _f(v_cache, dtype).copy()
    kc[:, :, P0:P0 + T] = K_new
    vc[:, :, P0:P0 + T] = V_new
    L = P0 + T
    masked = np.arange(L)[None, :] > pos[:, None]                    # [T, L]
    o = np.empty((B, T, H, dv), dtype=dtype)
    for b in range(B):
        for h in range(H):
            Q = np.concatenate([p["q_nope"][b, :, h], p["q_rope"][b, :, h]], axis=-1)   # [T, dqk]
            S = np.where(masked, -np.inf, (Q @ kc[b, h, :L].T) * dims.softmax_scale)
            E = np.exp(S - np.max(S, axis=-1, keepdims=True))
            o[b, :, h] = (E / np.sum(E, axis=-1, keepdims=True)) @ vc[b, h, :L]
    out = _merge_heads(o) @ _f(w.w_o, dtype).T + _bias(w.b_o, dtype)
    return out, kc, vc


def mla_prefill_chunk_latentcache(dims: MLADims, w: MLAWeights, x: np.ndarray, P0: int,
                                  latent_cache: np.ndarray, dtype=np.float64):
    """Chunked prefill with the latent cache [B, L_cap, kv_lora + dr], in
    absorbed form (as mla_decode_latentcache, with T queries at positions
    P0 .. P0+T-1 and the causal mask of the full-cache form).
    Returns (out [B, T, d], latent_cache')."""
    B, T, _ = x.shape
    r = dims.kv_lora_rank
    pos = P0 + np.arange(T)
    p = mla_project(dims, w, x, pos, dtype)
    cc = _f(latent_cache, dtype).copy()
    cc[:, P0:P0 + T] = latent_cache_entries(dims, p)
    L = P0 + T
    masked = (np.arange(L)[None, :] > pos[:, None])[:, None, :]     # [T, 1, L]
    q_t = absorbed_query(dims, w, p["q_nope"], dtype)               # [B,T,H,r]
    o_lat = np.empty((B, T, dims.n_heads, r), dtype=dtype)
    for b in range(B):
        C, KR = cc[b, :L, :r], cc[b, :L, r:]
        S = (q_t[b] @ C.T + p["q_rope"][b] @ KR.T) * dims.softmax_scale    # [T,H,L]
        S = np.where(masked, -np.inf, S)
        E = np.exp(S - np.max(S, axis=-1, keepdims=True))
        o_lat[b] = (E / np.sum(E, axis=-1, keepdims=True)) @ C
    o = absorbed_output(dims, w, o_lat, dtype)                       # [B,T,H,dv]
    out = _merge_heads(o) @ _f(w.w_o, dtype).T + _bias(w.b_o, dtype)
    return out, cc


def mla_decode_fullcache_ragged(dims: MLADims, w: MLAWeights, x_new: np.ndarray, positions,
                                k_cache: np.ndarray, v_cache: np.ndarray, dtype=np.float64):
    """Decode over a ragged batch with the full cache: sequence b's new token
    sits at its own position positions[b] ([MP]'s decode mode, applied to
    each sequence on its own: the sequences of a batch share no state).
    Returns (out [B, d], k_cache', v_cache')."""
    outs, kcs, vcs = [], [], []
    for b, P in enumerate(positions):
        o, kc, vc = mla_decode_fullcache(dims, w, x_new[b:b + 1], int(P), k_cache[b:b + 1],
                                         v_cache[b:b + 1], dtype)
        outs.append(o)
        kcs.append(kc)
        vcs.append(vc)
    return np.concatenate(outs), np.concatenate(kcs), np.concatenate(vcs)


def mla_decode_latentcache_ragged(dims: MLADims, w: MLAWeights, x_new: np.ndarray, positions,
                                  latent_cache: np.ndarray, dtype=np.float64):
    """Absorbed latent-cache decode over a ragged batch, one sequence at a
    time at its own position (as mla_decode_fullcache_ragged).
    Returns (out [B, d], latent_cache')."""
    outs, ccs = [], []
    for b, P in enumerate(positions):
        o, cc = mla_decode_latentcache(dims, w, x_new[b:b + 1], int(P), latent_cache[b:b + 1], dtype)
        outs.append(o)
        ccs.append(cc)
    return np.concatenate(outs), np.concatenate(ccs)


def dense_block(dims: MLADims, bw: BlockWeights, x: np.ndarray, rows=None,
                dtype=np.float64):
    """Dense transformer block of [DB]: x_attn = RMSNorm(x); x' = x + MLA(x_attn);
    x_ffn = RMSNorm(x'); g = x_ffn W1, u = x_ffn W3, a = g sigma(g), h = a * u;
    out = x' + h W2 (nn.Linear layout, so the products are x W^T here).

    ``rows`` restricts the output rows computed (keys/values of the attention
    still cover every position).  Returns [B, len(rows) or T, d].
    """
    bw.check(dims)
    B, T, _ = x.shape
    x = _f(x, dtype)
    qrows = np.arange(T) if rows is None else np.asarray(rows)
    x_attn = rms_norm(x, _f(bw.g_attn, dtype), dims.rms_eps)
    d_attn = mla_prefill(dims, bw.attn, x_attn, rows=qrows, dtype=dtype)
    x1 = x[:, qrows, :] + d_attn
    x_ffn = rms_norm(x1, _f(bw.g_ffn, dtype), dims.rms_eps)
    g = x_ffn @ _f(bw.w1, dtype).T
    u = x_ffn @ _f(bw.w3, dtype).T
    h = silu(g) * u
    return x1 + h @ _f(bw.w2, dtype).T
