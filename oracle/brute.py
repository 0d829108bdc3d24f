"""Brute-force loop oracle for tiny shapes.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.mla_ref``: only tests,
``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may use it).

A second, independent spelling of the same definition written as explicit
Python loops over scalars: no matrix product, no vectorised softmax, no
helper shared with ``oracle.mla_ref``.  It exists to pin the vectorised
oracle on small inputs (a transposed operand, a wrong index or a dropped term
in either spelling makes the two disagree).

Equations followed, by page title and section:
  "Kimi K2 · Dense transformer block", equation list: the two down-projections
    with their RMSNorms, the up-projections W_UQ, W_QR, W_UK, W_UV, the
    shared rotary key x W_KR, RoPE, query/key assembly, the residual and
    SwiGLU steps.
  "Kimi K2 · Mix and project", code excerpt: scores times the scale, additive
    causal mask, softmax over keys, P.V, head merge and o_proj.
  "Kimi K2 · Key-value compression", Explanation: the joint projection is
    split into the latent and the rotary key after the product.
The silent points are read as in ``oracle.mla_ref``: RMSNorm
g*x/sqrt(mean(x^2)+eps); RoPE on consecutive pairs with angle
t*base^(-2i/d_rope); scale 1/sqrt(d_nope+d_rope); head-major per-head rows.
"""
from __future__ import annotations

import math


def _vec(a):
    return [float(v) for v in a]


def _mat(a):
    return [[float(v) for v in row] for row in a]


def _linear(xrow, W, bias=None):
    """y[o] = sum_i x[i] * W[o][i] (+ b[o]) (nn.Linear layout [out, in])."""
    out = []
    for o, wrow in enumerate(W):
        s = 0.0
        for xi, wi in zip(xrow, wrow):
            s += xi * wi
        out.append(s if bias is None else s + bias[o])
    return out


def _rmsnorm(v, g, eps):
    ss = 0.0
    for a in v:
        ss += a * a
    r = 1.0 / math.sqrt(ss / len(v) + eps)
    return [gi * a * r for a, gi in zip(v, g)]


def _rope(v, t, base):
    n = len(v)
    out = list(v)
    for i in range(n // 2):
        ang = t * base ** (-(2.0 * i) / n)
        c, s = math.cos(ang), math.sin(ang)
        a, b = v[2 * i], v[2 * i + 1]
        out[2 * i] = a * c - b * s
        out[2 * i + 1] = a * s + b * c
    return out


def _project_token(d, w, xrow, t):
    """Per-token steps 1-3.  Returns dict of per-head lists."""
    H, dn, dr, dv, r = d.n_heads, d.qk_nope_dim, d.qk_rope_dim, d.v_head_dim, d.kv_lora_rank
    cq = _linear(xrow, w["w_dq"], w.get("b_dq"))
    cqh = _rmsnorm(cq, w["g_q"], d.rms_eps)
    qfull = _linear(cqh, w["w_uqr"])
    a = _linear(xrow, w["w_dkvr"], w.get("b_dkvr"))
    ckv = a[:r]
    kpe = a[r:r + dr]
    ckvh = _rmsnorm(ckv, w["g_kv"], d.rms_eps)
    kvfull = _linear(ckvh, w["w_ukv"])
    qn, qr, kn, vv = [], [], [], []
    for h in range(H):
        base_q = h * (dn + dr)
        qn.append(qfull[base_q:base_q + dn])
        qr.append(_rope(qfull[base_q + dn:base_q + dn + dr], t, d.rope_base))
        base_kv = h * (dn + dv)
        kn.append(kvfull[base_kv:base_kv + dn])
        vv.append(kvfull[base_kv + dn:base_kv + dn + dv])
    kr = _rope(kpe, t, d.rope_base)
    return dict(c_q=cq, c_kv_hat=ckvh, q_nope=qn, q_rope=qr, k_nope=kn, k_rope=kr, v=vv)


def _softmax_mix(scores, values):
    """softmax over the listed scores (masked ones are absent), then the
    probability-weighted sum of the value rows."""
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = sum(e)
    dv = len(values[0])
    o = [0.0] * dv
    for p, vrow in zip(e, values):
        for c in range(dv):
            o[c] += (p / z) * vrow[c]
    return o


def _weights(w):
    return {k: (_vec(v) if getattr(v, "ndim", 2) == 1 else _mat(v)) for k, v in w.items() if v is not None}


def prefill(d, w, x):
    """Causal MLA prefill of x [B][T][d] at positions 0..T-1 (plain nested
    lists or arrays).  ``w`` maps the weight names of the library's layout
    (w_dq, g_q, w_uqr, w_dkvr, g_kv, w_ukv, w_o, and optionally the biases
    b_dq, b_dkvr, b_o of the attention_bias variant) to arrays."""
    W = _weights(w)
    H, dv = d.n_heads, d.v_head_dim
    scale = 1.0 / math.sqrt(d.qk_nope_dim + d.qk_rope_dim)
    out = []
    for xb in x:
        toks = [_project_token(d, W, _vec(xrow), t) for t, xrow in enumerate(xb)]
        ob = []
        for i, ti in enumerate(toks):
            merged = []
            for h in range(H):
                Q = ti["q_nope"][h] + ti["q_rope"][h]
                scores, vals = [], []
                for j in range(i + 1):            # causal: keys j <= i
                    tj = toks[j]
                    K = tj["k_nope"][h] + tj["k_rope"]
                    s = 0.0
                    for qa, ka in zip(Q, K):
                        s += qa * ka
                    scores.append(s * scale)
                    vals.append(tj["v"][h])
                merged += _softmax_mix(scores, vals)
            assert len(merged) == H * dv
            ob.append(_linear(merged, W["w_o"], W.get("b_o")))
        out.append(ob)
    return out


def decode_fullcache(d, w, x_new, P, k_cache, v_cache):
    """One decode token per sequence at position P against the full cache
    [B][H][L_cap][dqk] / [B][H][L_cap][dv]; slot P is replaced by the new
    token.  Returns out [B][d]."""
    W = _weights(w)
    H = d.n_heads
    scale = 1.0 / math.sqrt(d.qk_nope_dim + d.qk_rope_dim)
    out = []
    for b, xrow in enumerate(x_new):
        tk = _project_token(d, W, _vec(xrow), P)
        merged = []
        for h in range(H):
            Q = tk["q_nope"][h] + tk["q_rope"][h]
            scores, vals = [], []
            for j in range(P + 1):
                if j == P:
                    K = tk["k_nope"][h] + tk["k_rope"]
                    V = tk["v"][h]
                else:
                    K = _vec(k_cache[b][h][j])
                    V = _vec(v_cache[b][h][j])
                s = 0.0
                for qa, ka in zip(Q, K):
                    s += qa * ka
                scores.append(s * scale)
                vals.append(V)
            merged += _softmax_mix(scores, vals)
        out.append(_linear(merged, W["w_o"], W.get("b_o")))
    return out


def decode_latentcache(d, w, x_new, P, latent_cache):
    """One decode token per sequence at position P against the latent cache
    [B][L_cap][kv_lora + dr] WITHOUT absorption: each cached latent is
    expanded to per-head keys and values through W_UK and W_UV, exactly as a
    prefill would have produced them.  Returns out [B][d]."""
    W = _weights(w)
    H, dn, dv, r = d.n_heads, d.qk_nope_dim, d.v_head_dim, d.kv_lora_rank
    scale = 1.0 / math.sqrt(d.qk_nope_dim + d.qk_rope_dim)
    out = []
    for b, xrow in enumerate(x_new):
        tk = _project_token(d, W, _vec(xrow), P)
        ents = []
        for j in range(P + 1):
            if j == P:
                c, kr = tk["c_kv_hat"], tk["k_rope"]
            else:
                e = _vec(latent_cache[b][j])
                c, kr = e[:r], e[r:]
            ents.append((_linear(c, W["w_ukv"]), kr))
        merged = []
        for h in range(H):
            Q = tk["q_nope"][h] + tk["q_rope"][h]
            scores, vals = [], []
            for kvfull, kr in ents:
                base = h * (dn + dv)
                K = kvfull[base:base + dn] + kr
                s = 0.0
                for qa, ka in zip(Q, K):
                    s += qa * ka
                scores.append(s * scale)
                vals.append(kvfull[base + dn:base + dn + dv])
            merged += _softmax_mix(scores, vals)
        out.append(_linear(merged, W["w_o"], W.get("b_o")))
    return out


def dense_block(d, w, blk, x):
    """Dense block: RMSNorm, MLA, residual, RMSNorm, SwiGLU, residual.
    ``blk`` maps g_attn, g_ffn, w1, w3, w2 to arrays."""
    Bk = _weights(blk)
    xn = [[_rmsnorm(_vec(r), Bk["g_attn"], d.rms_eps) for r in xb] for xb in x]
    att = prefill(d, w, xn)
    out = []
    for xb, ab in zip(x, att):
        ob = []
        for xrow, arow in zip(xb, ab):
            x1 = [a + b for a, b in zip(_vec(xrow), arow)]
            xf = _rmsnorm(x1, Bk["g_ffn"], d.rms_eps)
            g = _linear(xf, Bk["w1"])
            u = _linear(xf, Bk["w3"])
            hh = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
            ob.append([a + b for a, b in zip(x1, _linear(hh, Bk["w2"]))])
        out.append(ob)
    return out
