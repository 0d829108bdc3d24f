"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only (no GPU marker).  Each ``pin_*`` function raises AssertionError when
the oracle breaks the property; the tests call them on the real oracle, and
the mutation tests at the bottom plant plausible mistakes in the oracle (on
the CPU, through monkeypatching) and check that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import mla_ref as ref
from tests import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "kimi_k2_counts.json")))

# A micro shape for the fast pins; every width differs so that a transposed or
# mis-split operand changes the result or fails on shape.
MICRO = ref.MLADims(d_model=24, n_heads=3, q_lora_rank=12, kv_lora_rank=10,
                    qk_nope_dim=4, qk_rope_dim=6, v_head_dim=5, d_ff=14)
# Same but with equal nope/value widths, so that a swapped key/value split is
# shape-preserving (as it is at the Kimi K2 shape) and must be caught by value.
MICRO_EQ = ref.MLADims(d_model=20, n_heads=2, q_lora_rank=12, kv_lora_rank=10,
                       qk_nope_dim=4, qk_rope_dim=4, v_head_dim=4, d_ff=12)


def _weights(dims, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    w = synth.mla_weights(dims, rng, bf16=False)
    w = {k: (v.astype(np.float64) * (scale if k.startswith("w_") else 1.0)) for k, v in w.items()}
    # non-unit gains so that a gain applied to the wrong axis shows up
    w["g_q"] = 1.0 + 0.5 * rng.standard_normal(dims.q_lora_rank)
    w["g_kv"] = 1.0 + 0.5 * rng.standard_normal(dims.kv_lora_rank)
    return w


def _mw(w):
    return ref.MLAWeights(**w)


def _x(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- page values
def pin_parameter_counts():
    c = ref.parameter_counts(ref.KIMI_K2)
    g = GOLDEN["parameters"]
    for k in ("kv_compression", "mla", "o_proj", "mlp", "attn_norm", "mlp_norm", "block"):
        assert c[k] == g[k]["value"], (k, c[k], g[k]["value"])
    d = ref.KIMI_K2
    assert d.d_model * d.kv_lora_rank == g["kv_down_projection_latent_part"]["value"]
    assert c["o_proj"] * 60 == g["o_proj_times_60_moe_blocks"]["value"]
    assert c["kv_a_output_features"] == GOLDEN["cache_values_per_position"]["kv_a_output_features"]["value"]


def pin_cache_sizes():
    c = ref.cache_values_per_position(ref.KIMI_K2)
    g = GOLDEN["cache_values_per_position"]
    assert c["latent"] == g["latent"]["value"]
    assert c["full"] == g["full"]["value"]
    assert ref.KIMI_K2.q_head_dim == g["full_key_features"]["value"]


def pin_shapes():
    d, s = ref.KIMI_K2, GOLDEN["shapes"]
    assert d.d_model == s["d_model"]["value"]
    assert d.qk_rope_dim // 2 == s["rope_pairs"]["value"]
    assert d.kv_lora_rank == s["kv_latent"]["value"]
    assert d.n_heads == s["decode_heads"]["value"]
    assert d.v_head_dim == s["decode_value_dim"]["value"]
    assert s["decode_P"]["value"] + 1 == s["decode_keys_read"]["value"]


def test_parameter_counts():
    pin_parameter_counts()


def test_cache_sizes():
    pin_cache_sizes()


def test_shapes():
    pin_shapes()


def test_oracle_runs_at_page_shapes():
    """The oracle's products accept weights of exactly the counted shapes
    (a transposed operand would raise here) at the full Kimi K2 widths."""
    d = ref.KIMI_K2
    rng = np.random.default_rng(7)
    w = {k: (0.02 * rng.standard_normal(s, dtype=np.float32)) for k, s in ref.weight_shapes(d).items()}
    w["g_q"][:] = 1
    w["g_kv"][:] = 1
    x = rng.standard_normal((1, 2, d.d_model), dtype=np.float32)
    out, p = ref.mla_prefill(d, _mw(w), x, dtype=np.float32, return_intermediates=True)
    assert out.shape == (1, 2, d.d_model)
    assert p["q_nope"].shape == (1, 2, 64, 128) and p["q_rope"].shape == (1, 2, 64, 64)
    assert p["k_nope"].shape == (1, 2, 64, 128) and p["v"].shape == (1, 2, 64, 128)
    assert p["c_kv_hat"].shape == (1, 2, 512) and p["k_rope"].shape == (1, 2, 64)
    assert ref.latent_cache_entries(d, p).shape[-1] == 576
    K, V = ref.full_cache_entries(d, p)
    assert K.shape[1] * (K.shape[-1] + V.shape[-1]) == 20480


# ----------------------------------------------------------------- RMSNorm
def pin_rmsnorm():
    rng = np.random.default_rng(1)
    eps = 1e-6
    for scale in (1e-4, 1e-2, 1.0, 30.0):
        x = scale * rng.standard_normal((5, 37))
        y = ref.rms_norm(x, np.ones(37), eps)
        m = np.mean(x * x, axis=-1)
        # closed form: mean(y^2) = m / (m + eps)
        np.testing.assert_allclose(np.mean(y * y, axis=-1), m / (m + eps), rtol=1e-12)
        # direction is kept: y is a positive multiple of x per row
        cos = np.sum(x * y, -1) / np.linalg.norm(x, axis=-1) / np.linalg.norm(y, axis=-1)
        np.testing.assert_allclose(cos, 1.0, rtol=1e-12)
    # the gain multiplies elementwise after normalising
    x = rng.standard_normal((3, 8))
    g = rng.standard_normal(8)
    np.testing.assert_allclose(ref.rms_norm(x, g, eps), g * ref.rms_norm(x, np.ones(8), eps), rtol=1e-12)


def test_rmsnorm():
    pin_rmsnorm()


# -------------------------------------------------------------------- RoPE
def pin_rope():
    d, base = 64, 10000.0
    rng = np.random.default_rng(2)
    # position 0 is the identity
    c0, s0 = ref.rope_angles(np.array([0]), d, base)
    v = rng.standard_normal(d)
    np.testing.assert_array_equal(ref.apply_rope(v, c0[0], s0[0]), v)
    # worked value: pair 16 of 32 turns by base^(-32/64) = 1/100 rad per position,
    # so at t = 100 the unit vector e_32 becomes (cos 1, sin 1) on (32, 33)
    c, s = ref.rope_angles(np.array([100]), d, base)
    e = np.zeros(d)
    e[32] = 1.0
    r = ref.apply_rope(e, c[0], s[0])
    np.testing.assert_allclose(r[32:34], [math.cos(1.0), math.sin(1.0)], rtol=1e-12)
    assert np.count_nonzero(r) == 2
    # pair 0 turns by exactly t radians
    e0 = np.zeros(d)
    e0[0] = 1.0
    c, s = ref.rope_angles(np.array([3]), d, base)
    np.testing.assert_allclose(ref.apply_rope(e0, c[0], s[0])[:2], [math.cos(3.0), math.sin(3.0)], rtol=1e-12)
    # norm preservation and relative-position invariance
    pos = np.array([0, 1, 5, 17, 300, 4097])
    c, s = ref.rope_angles(pos, d, base)
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for a in range(len(pos)):
        np.testing.assert_allclose(np.linalg.norm(ref.apply_rope(q, c[a], s[a])), np.linalg.norm(q), rtol=1e-12)
        for b in range(len(pos)):
            lhs = ref.apply_rope(q, c[a], s[a]) @ ref.apply_rope(k, c[b], s[b])
            cd, sd = ref.rope_angles(np.array([pos[a] - pos[b]]), d, base)
            rhs = ref.apply_rope(q, cd[0], sd[0]) @ k
            np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-9)
    # group property: rotating by m then n equals rotating by m + n
    cm, sm = ref.rope_angles(np.array([7]), d, base)
    cn, sn = ref.rope_angles(np.array([11]), d, base)
    cmn, smn = ref.rope_angles(np.array([18]), d, base)
    np.testing.assert_allclose(ref.apply_rope(ref.apply_rope(q, cm[0], sm[0]), cn[0], sn[0]),
                               ref.apply_rope(q, cmn[0], smn[0]), rtol=1e-12, atol=1e-12)


def test_rope():
    pin_rope()


# ----------------------------------------------------------------- SwiGLU
def pin_silu():
    assert ref.silu(np.array([0.0]))[0] == 0.0
    z = np.linspace(-20, 20, 81)
    # silu(z) - silu(-z) = z for the logistic gate
    np.testing.assert_allclose(ref.silu(z) - ref.silu(-z), z, rtol=1e-12, atol=1e-12)
    # tends to z for large z and to 0 for very negative z
    assert abs(ref.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(ref.silu(np.array([-40.0]))[0]) < 1e-15
    # sigma(0) = 1/2 gives derivative 1/2 at 0
    h = 1e-6
    np.testing.assert_allclose((ref.silu(np.array([h])) - ref.silu(np.array([-h])))[0] / (2 * h), 0.5, rtol=1e-6)


def test_silu():
    pin_silu()


# -------------------------------------------------------- softmax / P.V
def pin_softmax_and_mix():
    d = MICRO
    w = _weights(d, 3)
    x = _x((1, 7, d.d_model), 4)
    p = ref.mla_project(d, _mw(w), x, np.arange(7))
    pos = np.arange(7)
    o, P = ref.attention(p["q_nope"][0], p["q_rope"][0], p["k_nope"][0], p["k_rope"][0],
                         p["v"][0], d.softmax_scale, pos, pos, return_probs=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=1e-13)
    assert np.all(P >= 0)
    iu = np.triu_indices(7, 1)
    assert np.all(P[:, iu[0], iu[1]] == 0.0)          # masked entries exactly zero
    # query row 0 sees only key 0: its output is exactly V[0]
    np.testing.assert_array_equal(o[0], p["v"][0, 0])
    # a zero query gives uniform weights: O[i] = mean of V[0..i]
    zq = np.zeros_like(p["q_nope"][0])
    zr = np.zeros_like(p["q_rope"][0])
    o0 = ref.attention(zq, zr, p["k_nope"][0], p["k_rope"][0], p["v"][0], d.softmax_scale, pos, pos)
    for i in range(7):
        np.testing.assert_allclose(o0[i], p["v"][0, :i + 1].mean(0), rtol=1e-12)


def test_softmax_and_mix():
    pin_softmax_and_mix()


# --------------------------------------------------------------- causality
def pin_causality():
    d = MICRO
    w = _mw(_weights(d, 5))
    x = _x((2, 9, d.d_model), 6)
    out = ref.mla_prefill(d, w, x)
    for t in (0, 3, 7):
        y = x.copy()
        y[:, t + 1:, :] += _x(y[:, t + 1:, :].shape, 60 + t)
        out2 = ref.mla_prefill(d, w, y)
        np.testing.assert_array_equal(out2[:, :t + 1], out[:, :t + 1])
        assert not np.array_equal(out2[:, t + 1:], out[:, t + 1:])


def test_causality():
    pin_causality()


# ------------------------------------------------------ brute-force parity
def _close(a, b, tol=1e-10):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b))
    assert err <= tol * max(1.0, np.max(np.abs(b))), err


def pin_brute_prefill(dims=MICRO, T=6, seed=8):
    w = _weights(dims, seed)
    x = _x((2, T, dims.d_model), seed + 1)
    _close(ref.mla_prefill(dims, _mw(w), x), brute.prefill(dims, w, x))


def pin_brute_decode_full(dims=MICRO, seed=10):
    rng = np.random.default_rng(seed)
    w = _weights(dims, seed)
    B, P, L_cap = 2, 5, 8
    x = rng.standard_normal((B, dims.d_model))
    kc = rng.standard_normal((B, dims.n_heads, L_cap, dims.q_head_dim))
    vc = rng.standard_normal((B, dims.n_heads, L_cap, dims.v_head_dim))
    out, kc2, vc2 = ref.mla_decode_fullcache(dims, _mw(w), x, P, kc, vc)
    _close(out, brute.decode_fullcache(dims, w, x, P, kc, vc))
    np.testing.assert_array_equal(kc2[:, :, :P], kc[:, :, :P])
    np.testing.assert_array_equal(kc2[:, :, P + 1:], kc[:, :, P + 1:])
    # the rotary part of the new key is the same in every head
    kr = kc2[:, :, P, dims.qk_nope_dim:]
    np.testing.assert_array_equal(kr, np.broadcast_to(kr[:, :1], kr.shape))


def pin_brute_decode_latent(dims=MICRO, seed=11):
    """Absorbed latent decode (oracle) against the unabsorbed loop version
    that expands every cached latent to per-head keys and values."""
    rng = np.random.default_rng(seed)
    w = _weights(dims, seed)
    B, P, L_cap = 2, 6, 9
    x = rng.standard_normal((B, dims.d_model))
    cc = rng.standard_normal((B, L_cap, dims.kv_lora_rank + dims.qk_rope_dim))
    out, cc2 = ref.mla_decode_latentcache(dims, _mw(w), x, P, cc)
    _close(out, brute.decode_latentcache(dims, w, x, P, cc))
    np.testing.assert_array_equal(cc2[:, :P], cc[:, :P])


def pin_brute_block(dims=MICRO, seed=12):
    rng = np.random.default_rng(seed)
    w = _weights(dims, seed)
    blk = {"w1": 0.3 * rng.standard_normal((dims.d_ff, dims.d_model)),
           "w3": 0.3 * rng.standard_normal((dims.d_ff, dims.d_model)),
           "w2": 0.3 * rng.standard_normal((dims.d_model, dims.d_ff)),
           "g_attn": 1 + 0.3 * rng.standard_normal(dims.d_model),
           "g_ffn": 1 + 0.3 * rng.standard_normal(dims.d_model)}
    x = _x((1, 5, dims.d_model), seed + 1)
    bw = ref.BlockWeights(attn=_mw(w), **blk)
    _close(ref.dense_block(dims, bw, x), brute.dense_block(dims, w, blk, x))


def _bias_weights(dims, seed):
    w = _weights(dims, seed)
    w.update({k: v.astype(np.float64) for k, v in
              synth.attention_biases(dims, np.random.default_rng(seed + 100), bf16=False).items()})
    return w


def pin_brute_bias(dims=MICRO, seed=31):
    """attention_bias variant: every path against the loop oracle with the
    three biases (q_a_proj, kv_a_proj_with_mqa, o_proj) present."""
    rng = np.random.default_rng(seed)
    w = _bias_weights(dims, seed)
    x = _x((2, 5, dims.d_model), seed + 1)
    _close(ref.mla_prefill(dims, _mw(w), x), brute.prefill(dims, w, x))
    B, P, L_cap = 2, 4, 6
    xd = rng.standard_normal((B, dims.d_model))
    kc = rng.standard_normal((B, dims.n_heads, L_cap, dims.q_head_dim))
    vc = rng.standard_normal((B, dims.n_heads, L_cap, dims.v_head_dim))
    _close(ref.mla_decode_fullcache(dims, _mw(w), xd, P, kc, vc)[0], brute.decode_fullcache(dims, w, xd, P, kc, vc))
    cc = rng.standard_normal((B, L_cap, dims.kv_lora_rank + dims.qk_rope_dim))
    _close(ref.mla_decode_latentcache(dims, _mw(w), xd, P, cc)[0], brute.decode_latentcache(dims, w, xd, P, cc))
    blk = {"w1": 0.3 * rng.standard_normal((dims.d_ff, dims.d_model)),
           "w3": 0.3 * rng.standard_normal((dims.d_ff, dims.d_model)),
           "w2": 0.3 * rng.standard_normal((dims.d_model, dims.d_ff)),
           "g_attn": 1 + 0.3 * rng.standard_normal(dims.d_model),
           "g_ffn": 1 + 0.3 * rng.standard_normal(dims.d_model)}
    xb = _x((1, 4, dims.d_model), seed + 2)
    _close(ref.dense_block(dims, ref.BlockWeights(attn=_mw(w), **blk), xb), brute.dense_block(dims, w, blk, xb))


def pin_bias_special_cases(dims=MICRO, seed=32):
    """Zero biases are no biases (bit for bit); with W_O = 0 the output is
    b_o in every row exactly."""
    w = _weights(dims, seed)
    x = _x((2, 4, dims.d_model), seed + 1)
    wz = dict(w, b_dq=np.zeros(dims.q_lora_rank), b_dkvr=np.zeros(dims.kv_lora_rank + dims.qk_rope_dim),
              b_o=np.zeros(dims.d_model))
    np.testing.assert_array_equal(ref.mla_prefill(dims, _mw(wz), x), ref.mla_prefill(dims, _mw(w), x))
    wb = _bias_weights(dims, seed)
    wb["w_o"] = np.zeros_like(wb["w_o"])
    out = ref.mla_prefill(dims, _mw(wb), x)
    np.testing.assert_array_equal(out, np.broadcast_to(wb["b_o"], out.shape))


def test_attention_bias_variant():
    pin_brute_bias()
    pin_brute_bias(MICRO_EQ, 33)
    pin_bias_special_cases()


def test_brute_prefill():
    pin_brute_prefill()
    pin_brute_prefill(MICRO_EQ)


def test_brute_prefill_tiny_config():
    """The tiny float32 prefill shape itself (d=256, 4 heads, ...), few tokens."""
    pin_brute_prefill(ref.TINY, T=3, seed=21)


def test_brute_decode_full():
    pin_brute_decode_full()
    pin_brute_decode_full(MICRO_EQ)


def test_brute_decode_latent():
    pin_brute_decode_latent()
    pin_brute_decode_latent(MICRO_EQ)


def test_brute_block():
    pin_brute_block()


# ------------------------------------------- cross-form invariants (fp64)
def pin_absorbed_equals_unabsorbed(dims=MICRO_EQ, seed=13):
    """Latent decode (absorbed) == full-cache decode on the cache expanded
    from the same latents (K^C = c W_UK^T, k^R copied per head, V = c W_UV^T)."""
    rng = np.random.default_rng(seed)
    w = _weights(dims, seed)
    B, P, L_cap = 3, 7, 8
    r, H, dn = dims.kv_lora_rank, dims.n_heads, dims.qk_nope_dim
    x = rng.standard_normal((B, dims.d_model))
    cc = rng.standard_normal((B, L_cap, r + dims.qk_rope_dim))
    out_l, cc2 = ref.mla_decode_latentcache(dims, _mw(w), x, P, cc)
    kv = (cc[..., :r] @ w["w_ukv"].T).reshape(B, L_cap, H, -1)
    K = np.concatenate([kv[..., :dn], np.broadcast_to(cc[:, :, None, r:], (B, L_cap, H, dims.qk_rope_dim))], -1)
    V = kv[..., dn:]
    out_f, _, _ = ref.mla_decode_fullcache(dims, _mw(w), x, P, K.transpose(0, 2, 1, 3), V.transpose(0, 2, 1, 3))
    _close(out_l, out_f, 1e-11)


def pin_prefill_last_row_equals_decode(dims=MICRO, seed=14):
    """The last row of a T-token prefill equals a decode step at P = T-1 whose
    cache holds the first T-1 positions, in both cache forms."""
    w = _weights(dims, seed)
    T = 6
    x = _x((2, T, dims.d_model), seed + 1)
    out, p = ref.mla_prefill(dims, _mw(w), x, return_intermediates=True)
    K, V = ref.full_cache_entries(dims, p)
    C = ref.latent_cache_entries(dims, p)
    junkK, junkV, junkC = np.full_like(K, 1e3), np.full_like(V, -1e3), np.full_like(C, 7.0)
    junkK[:, :, :T - 1], junkV[:, :, :T - 1], junkC[:, :T - 1] = K[:, :, :T - 1], V[:, :, :T - 1], C[:, :T - 1]
    of, kc, vc = ref.mla_decode_fullcache(dims, _mw(w), x[:, -1], T - 1, junkK, junkV)
    ol, cc = ref.mla_decode_latentcache(dims, _mw(w), x[:, -1], T - 1, junkC)
    _close(of, out[:, -1], 1e-11)
    _close(ol, out[:, -1], 1e-11)
    _close(kc, K, 1e-12)
    _close(vc, V, 1e-12)
    _close(cc, C, 1e-12)


def test_absorbed_equals_unabsorbed():
    pin_absorbed_equals_unabsorbed()
    pin_absorbed_equals_unabsorbed(MICRO, 15)


def test_prefill_last_row_equals_decode():
    pin_prefill_last_row_equals_decode()
    pin_prefill_last_row_equals_decode(MICRO_EQ, 16)


def pin_ragged_decode(dims=MICRO, seed=21):
    """Per-sequence positions: sequence b's result (output and cache rows) is
    that of a prefill of its own T_b = P_b + 1 tokens -- last output row,
    first T_b cache slots -- whatever the other sequences' lengths, in both
    cache forms; with equal positions it is the uniform decode step."""
    w = _weights(dims, seed)
    Ts = [1, 4, 7]
    L_cap = 8
    B = len(Ts)
    xs = [_x((1, T, dims.d_model), seed + 1 + i) for i, T in enumerate(Ts)]
    K = np.full((B, dims.n_heads, L_cap, dims.q_head_dim), 1e3)
    V = np.full((B, dims.n_heads, L_cap, dims.v_head_dim), -1e3)
    C = np.full((B, L_cap, dims.kv_lora_rank + dims.qk_rope_dim), 7.0)
    want, Kw, Vw, Cw = [], K.copy(), V.copy(), C.copy()
    for b, (T, x) in enumerate(zip(Ts, xs)):
        out, p = ref.mla_prefill(dims, _mw(w), x, return_intermediates=True)
        Kb, Vb = ref.full_cache_entries(dims, p)
        Cb = ref.latent_cache_entries(dims, p)
        K[b, :, :T - 1], V[b, :, :T - 1], C[b, :T - 1] = Kb[0, :, :T - 1], Vb[0, :, :T - 1], Cb[0, :T - 1]
        Kw[b, :, :T], Vw[b, :, :T], Cw[b, :T] = Kb[0], Vb[0], Cb[0]
        want.append(out[0, -1])
    x_new = np.stack([x[0, -1] for x in xs])
    pos = [T - 1 for T in Ts]
    of, kc, vc = ref.mla_decode_fullcache_ragged(dims, _mw(w), x_new, pos, K, V)
    ol, cc = ref.mla_decode_latentcache_ragged(dims, _mw(w), x_new, pos, C)
    _close(of, np.stack(want), 1e-11)
    _close(ol, np.stack(want), 1e-11)
    _close(kc, Kw, 1e-12)
    _close(vc, Vw, 1e-12)
    _close(cc, Cw, 1e-12)
    # equal positions: the uniform step
    of2, _, _ = ref.mla_decode_fullcache_ragged(dims, _mw(w), x_new, [5, 5, 5], K, V)
    of3, _, _ = ref.mla_decode_fullcache(dims, _mw(w), x_new, 5, K, V)
    _close(of2, of3, 1e-12)


def test_ragged_decode():
    pin_ragged_decode()
    pin_ragged_decode(MICRO_EQ, 22)


def pin_chunked_prefill(dims=MICRO, seed=41):
    """Chunked prefill, both cache forms: a prefill of 7 tokens done as
    chunks of 3 and 4 gives the prefill's output rows and cache entries; a
    chunk at P0 = 0 is the prefill itself; a chunk of one token is the decode
    step at P = P0."""
    w = _mw(_bias_weights(dims, seed))
    B, T1, T2, L_cap = 2, 3, 4, 9
    x = _x((B, T1 + T2, dims.d_model), seed + 1)
    want, p = ref.mla_prefill(dims, w, x, return_intermediates=True)
    K, V = ref.full_cache_entries(dims, p)
    C = ref.latent_cache_entries(dims, p)
    kc = np.full((B, dims.n_heads, L_cap, dims.q_head_dim), 1e3)
    vc = np.full((B, dims.n_heads, L_cap, dims.v_head_dim), -1e3)
    cc = np.full((B, L_cap, dims.kv_lora_rank + dims.qk_rope_dim), 7.0)
    o1, kc, vc = ref.mla_prefill_chunk_fullcache(dims, w, x[:, :T1], 0, kc, vc)
    o2, kc, vc = ref.mla_prefill_chunk_fullcache(dims, w, x[:, T1:], T1, kc, vc)
    l1, cc = ref.mla_prefill_chunk_latentcache(dims, w, x[:, :T1], 0, cc)
    l2, cc = ref.mla_prefill_chunk_latentcache(dims, w, x[:, T1:], T1, cc)
    for got in (np.concatenate([o1, o2], 1), np.concatenate([l1, l2], 1)):
        _close(got, want, 1e-11)
    _close(kc[:, :, :T1 + T2], K, 1e-12)
    _close(vc[:, :, :T1 + T2], V, 1e-12)
    _close(cc[:, :T1 + T2], C, 1e-12)
    assert np.all(kc[:, :, T1 + T2:] == 1e3) and np.all(cc[:, T1 + T2:] == 7.0)
    # one-token chunk = decode step, both forms
    P0 = T1 + T2
    xd = _x((B, 1, dims.d_model), seed + 2)
    of, _, _ = ref.mla_prefill_chunk_fullcache(dims, w, xd, P0, kc, vc)
    od, _, _ = ref.mla_decode_fullcache(dims, w, xd[:, 0], P0, kc, vc)
    _close(of[:, 0], od, 1e-12)
    ol, _ = ref.mla_prefill_chunk_latentcache(dims, w, xd, P0, cc)
    odl, _ = ref.mla_decode_latentcache(dims, w, xd[:, 0], P0, cc)
    _close(ol[:, 0], odl, 1e-12)


def test_chunked_prefill():
    pin_chunked_prefill()
    pin_chunked_prefill(MICRO_EQ, 42)


def pin_block_residual():
    """With o_proj and W2 zero the block is the identity on x (exactly)."""
    d = MICRO
    rng = np.random.default_rng(17)
    w = _weights(d, 17)
    w["w_o"] = np.zeros_like(w["w_o"])
    bw = ref.BlockWeights(attn=_mw(w), g_attn=np.ones(d.d_model), g_ffn=np.ones(d.d_model),
                          w1=rng.standard_normal((d.d_ff, d.d_model)),
                          w3=rng.standard_normal((d.d_ff, d.d_model)),
                          w2=np.zeros((d.d_model, d.d_ff)))
    x = _x((2, 4, d.d_model), 18)
    np.testing.assert_array_equal(ref.dense_block(d, bw, x), x)


def test_block_residual():
    pin_block_residual()


def test_rows_subset_matches_full():
    d = MICRO
    w = _mw(_weights(d, 19))
    x = _x((2, 8, d.d_model), 20)
    full = ref.mla_prefill(d, w, x)
    rows = [0, 3, 7]
    np.testing.assert_allclose(ref.mla_prefill(d, w, x, rows=rows), full[:, rows], rtol=1e-13)


# ----------------------------------------------------------- mutations
ALL_PINS = [pin_parameter_counts, pin_cache_sizes, pin_rmsnorm, pin_rope, pin_silu,
            pin_softmax_and_mix, pin_causality, pin_brute_prefill, pin_brute_decode_full,
            pin_brute_decode_latent, pin_brute_block, pin_absorbed_equals_unabsorbed,
            pin_prefill_last_row_equals_decode, pin_block_residual, pin_ragged_decode,
            pin_brute_bias, pin_bias_special_cases, pin_chunked_prefill,
            lambda: pin_brute_prefill(MICRO_EQ), lambda: pin_brute_decode_latent(MICRO_EQ),
            lambda: pin_absorbed_equals_unabsorbed(MICRO, 15)]


def _some_pin_fails():
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # any failure of a pin counts as caught
            return True
    return False


def _orig(name):
    return getattr(ref, name)


_rms = _orig("rms_norm")
_rope = _orig("apply_rope")
_angles = _orig("rope_angles")
_attn = _orig("attention")
_absq = _orig("absorbed_query")
_abso = _orig("absorbed_output")
_silu = _orig("silu")
_shapes = _orig("weight_shapes")


def _attention_scaled(value):
    def f(q_nope, q_rope, k_nope, k_rope, v, scale, q_pos, k_pos, return_probs=False):
        return _attn(q_nope, q_rope, k_nope, k_rope, v, value, q_pos, k_pos, return_probs)
    return f


def _attention_no_rope(q_nope, q_rope, k_nope, k_rope, v, scale, q_pos, k_pos, return_probs=False):
    return _attn(q_nope, 0 * q_rope, k_nope, 0 * k_rope, v, scale, q_pos, k_pos, return_probs)


def _attention_off_by_one(q_nope, q_rope, k_nope, k_rope, v, scale, q_pos, k_pos, return_probs=False):
    return _attn(q_nope, q_rope, k_nope, k_rope, v, scale, np.asarray(q_pos) + 1, k_pos, return_probs)


def _absq_value_rows(dims, w, q_nope, dtype=np.float64):
    H, dn, dv = dims.n_heads, dims.qk_nope_dim, dims.v_head_dim
    W = np.asarray(w.w_ukv, dtype).reshape(H, dn + dv, dims.kv_lora_rank)
    return np.einsum("...hc,hck->...hk", q_nope, W[:, dn:dn + dn, :])


def _abso_key_rows(dims, w, o_lat, dtype=np.float64):
    H, dn, dv = dims.n_heads, dims.qk_nope_dim, dims.v_head_dim
    W = np.asarray(w.w_ukv, dtype).reshape(H, dn + dv, dims.kv_lora_rank)
    return np.einsum("...hk,hck->...hc", o_lat, W[:, :dv, :])


def _angles_i_over_d(p, d, b, dtype=np.float64):
    """Plausible slip: base^(-i/d) instead of base^(-2i/d)."""
    ang = np.asarray(p, float)[:, None] * b ** (-np.arange(d // 2) / d)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


MUTATIONS = {
    "rmsnorm_without_eps": ("rms_norm", lambda x, g, eps: _rms(x, g, 0.0)),
    "rmsnorm_sum_not_mean": ("rms_norm", lambda x, g, eps: g * x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps)),
    "rmsnorm_gain_ignored": ("rms_norm", lambda x, g, eps: _rms(x, np.ones_like(g), eps)),
    "rope_sign_flip": ("apply_rope", lambda x, c, s: _rope(x, c, -s)),
    "rope_half_frequency": ("rope_angles", lambda p, d, b, dtype=np.float64: _angles(np.asarray(p) * 0.5, d, b, dtype)),
    "rope_base_exponent_i_over_d": ("rope_angles", lambda p, d, b, dtype=np.float64: _angles_i_over_d(p, d, b, dtype)),
    "silu_without_gate": ("silu", lambda z: z),
    "softmax_scale_missing": ("attention", _attention_scaled(1.0)),
    "rope_term_dropped_from_scores": ("attention", _attention_no_rope),
    "causal_mask_off_by_one": ("attention", _attention_off_by_one),
    "absorbed_query_uses_value_rows": ("absorbed_query", _absq_value_rows),
    "absorbed_output_uses_key_rows": ("absorbed_output", _abso_key_rows),
    "mla_has_bias_terms": ("weight_shapes", lambda dims: {**_shapes(dims), "b_o": (dims.d_model,)}),
    "attention_bias_ignored": ("_bias", lambda b, dtype: 0.0),
    "attention_bias_subtracted": ("_bias", lambda b, dtype: 0.0 if b is None else -np.asarray(b, dtype)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, fn)
    assert _some_pin_fails(), f"no pin caught the planted mistake {name!r}"


def test_pins_pass_unmutated():
    assert not _some_pin_fails()
