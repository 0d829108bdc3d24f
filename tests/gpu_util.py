"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
calling the oracle and comparing within the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

from oracle import mla_ref as ref

# Tolerances: max|gpu - oracle| <= TOL * max|oracle|
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_of(mla, od: ref.MLADims, dtype: str):
    return mla.make_dims(od.d_model, od.n_heads, od.q_lora_rank, od.kv_lora_rank, od.qk_nope_dim,
                         od.qk_rope_dim, od.v_head_dim, d_ff=od.d_ff, rms_eps=od.rms_eps,
                         softmax_scale=od.softmax_scale, dtype=dtype)


def to_dev(a, dtype, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=dev, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def bits_to_dev(bits, dtype, dev):
    """Cache arrays from tests.synth: uint16 bf16 bits (or float32)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(dev)


def from_dev(t):
    return t.float().cpu().numpy().astype(np.float64)


def weights_to_dev(w: dict, dtype, dev):
    return {k: to_dev(v, dtype, dev) for k, v in w.items()}


def oracle_weights(w: dict) -> ref.MLAWeights:
    return ref.MLAWeights(**{k: np.asarray(v, np.float64) for k, v in w.items()})


def assert_close(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(got - want)))
    scale = float(np.max(np.abs(want)))
    log(f"  {what}: max|err| {err:.3e}  max|ref| {scale:.3e}  ratio {err / max(scale, 1e-30):.2e} (tol {tol:g})")
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol:g} * {scale:.3e}"
    return err / max(scale, 1e-30)
