"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds none of the method's arithmetic: it only draws normal
numbers with NumPy's PCG64 generator and rounds them once to bfloat16
(round to nearest, ties to even) where a workload is bf16.  Both the oracle
and the GPU consume exactly the values returned here.

Recipe (the source pages measure on no dataset, so synthetic tensors of the
pages' shapes stand in): generator ``numpy.random.default_rng(seed)``;
float32 draws in the fixed order x, W_DQ, W_DKVR, W_UQR, W_UKV, W_O,
then (block) W1, W3, W2, then caches; x and caches ~ N(0, 1), weights
~ N(0, 0.02^2) (0.02 is the standard deviation), every RMSNorm gain = 1.
"""
from __future__ import annotations

import numpy as np

W_STD = 0.02


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 arrays holding exactly representable bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng, shape, std, bf16):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_round(a) if bf16 else a


def mla_weights(dims, rng, bf16: bool) -> dict:
    """W_DQ, W_DKVR, W_UQR, W_UKV, W_O in nn.Linear [out, in] layout (draw
    order as in the recipe) plus unit gains g_q, g_kv."""
    H = dims.n_heads
    dqk = dims.qk_nope_dim + dims.qk_rope_dim
    w = {}
    w["w_dq"] = _draw(rng, (dims.q_lora_rank, dims.d_model), W_STD, bf16)
    w["w_dkvr"] = _draw(rng, (dims.kv_lora_rank + dims.qk_rope_dim, dims.d_model), W_STD, bf16)
    w["w_uqr"] = _draw(rng, (H * dqk, dims.q_lora_rank), W_STD, bf16)
    w["w_ukv"] = _draw(rng, (H * (dims.qk_nope_dim + dims.v_head_dim), dims.kv_lora_rank), W_STD, bf16)
    w["w_o"] = _draw(rng, (dims.d_model, H * dims.v_head_dim), W_STD, bf16)
    w["g_q"] = np.ones(dims.q_lora_rank, np.float32)
    w["g_kv"] = np.ones(dims.kv_lora_rank, np.float32)
    return w


BIAS_STD = 0.5  # synthetic attention_bias values: the pages give none


def attention_biases(dims, rng, bf16: bool) -> dict:
    """Biases of the attention_bias variant: b_dq [q_lora], b_dkvr
    [kv_lora + d_rope], b_o [d], each N(0, BIAS_STD^2)."""
    return {"b_dq": _draw(rng, (dims.q_lora_rank,), BIAS_STD, bf16),
            "b_dkvr": _draw(rng, (dims.kv_lora_rank + dims.qk_rope_dim,), BIAS_STD, bf16),
            "b_o": _draw(rng, (dims.d_model,), BIAS_STD, bf16)}


def prefill_inputs(dims, B, T, seed, bf16=True):
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, T, dims.d_model), 1.0, bf16)
    return x, mla_weights(dims, rng, bf16)


def block_inputs(dims, B, T, seed, bf16=True):
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, T, dims.d_model), 1.0, bf16)
    w = mla_weights(dims, rng, bf16)
    blk = {
        "w1": _draw(rng, (dims.d_ff, dims.d_model), W_STD, bf16),
        "w3": _draw(rng, (dims.d_ff, dims.d_model), W_STD, bf16),
        "w2": _draw(rng, (dims.d_model, dims.d_ff), W_STD, bf16),
        "g_attn": np.ones(dims.d_model, np.float32),
        "g_ffn": np.ones(dims.d_model, np.float32),
    }
    return x, w, blk


def _cache(rng, shape, bf16):
    """N(0,1) cache drawn one leading slice at a time (so the host never
    holds a float32 copy of a multi-GB cache).  Returns uint16 bf16 bits
    when ``bf16`` (else float32)."""
    out = np.empty(shape, dtype=np.uint16 if bf16 else np.float32)
    for b in range(shape[0]):
        a = rng.standard_normal(size=shape[1:], dtype=np.float32)
        out[b] = bf16_bits(bf16_round(a)) if bf16 else a
    return out


def decode_full_inputs(dims, B, P, L_cap, seed, bf16=True):
    """x_new [B, d], K cache [B,H,L_cap,dqk], V cache [B,H,L_cap,dv]
    (caches as bf16 bits when ``bf16``)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, dims.d_model), 1.0, bf16)
    w = mla_weights(dims, rng, bf16)
    H = dims.n_heads
    kc = _cache(rng, (B, H, L_cap, dims.qk_nope_dim + dims.qk_rope_dim), bf16)
    vc = _cache(rng, (B, H, L_cap, dims.v_head_dim), bf16)
    return x, w, kc, vc


def decode_latent_inputs(dims, B, P, L_cap, seed, bf16=True):
    """x_new [B, d] and latent cache [B, L_cap, kv_lora + d_rope]."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, dims.d_model), 1.0, bf16)
    w = mla_weights(dims, rng, bf16)
    cc = _cache(rng, (B, L_cap, dims.kv_lora_rank + dims.qk_rope_dim), bf16)
    return x, w, cc


def as_f32(a, bf16):
    """Cache arrays come back as bf16 bits; give the float32 values."""
    return bits_to_f32(a) if bf16 and a.dtype == np.uint16 else np.asarray(a, np.float32)
