"""The allocation-free latent-cache decode (mla_decode_latentcache_noalloc)
against the workspace entry point it mirrors, through the C ABI.

The allocation-free call keeps its workspace in one library-owned device
array per GPU that persists between calls, so two calls run in a row, the
second with a smaller batch and cache (it must not depend on what the first
left in the array).  Both entry points run the same kernels on the same
inputs, so the outputs and the written cache slot agree bit for bit; the
smaller call is also checked against the oracle on the bf16 bar.
"""
import ctypes

import numpy as np
import pytest

from oracle import mla_ref as ref
from tests import synth
from tests.gpu_util import (TOL_BF16, assert_close, bits_to_dev, dims_of, from_dev, log, oracle_weights,
                            to_dev, weights_to_dev)

torch = pytest.importorskip("torch")
mla = pytest.importorskip("head_latent_attention_fwd_amd")

DEV = "cuda:0"


def _both(od, B, P, L_cap, seed):
    x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, seed, bf16=True)
    d = dims_of(mla, od, "bf16")
    wd = weights_to_dev(w, "bf16", DEV)
    xd = to_dev(x, "bf16", DEV)
    rope = mla.mla_rope_table(P + 1, od.qk_rope_dim, od.rope_base, DEV)
    c_ref = bits_to_dev(cc, "bf16", DEV)
    c_na = c_ref.clone()
    want = mla.mla_decode_latentcache(d, wd, xd, P, c_ref, rope)
    got = torch.empty_like(want)
    mla.mla_decode_latentcache_noalloc(d, wd, xd, P, c_na, rope, got)
    torch.cuda.synchronize()
    return x, w, cc, got, want, c_na, c_ref


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()
    od = ref.KIMI_K2
    for B, P, L_cap, seed in ((32, 8192, 8193, 1041), (4, 700, 750, 1042)):
        log(f"[noalloc decode] B={B} P={P} L_cap={L_cap}")
        x, w, cc, got, want, c_na, c_ref = _both(od, B, P, L_cap, seed)
        assert torch.equal(got, want), "allocation-free output differs from the workspace entry point"
        assert torch.equal(c_na, c_ref), "written cache slot differs"
        bs = [0, B - 1]
        cf = synth.as_f32(cc[bs], True).astype(np.float64)
        ow, _ = ref.mla_decode_latentcache(od, oracle_weights(w), x[bs].astype(np.float64), P, cf)
        assert_close(from_dev(got)[bs], ow, TOL_BF16, f"noalloc decode B={B} P={P} vs oracle")


def test_noalloc_rejects_steps_beyond_the_array():
    """Host side: a step whose workspace exceeds the array is refused with
    MLA_ERR_WORKSPACE before any HIP call; bad arguments keep their codes."""
    L = mla.load()
    d = mla.make_dims(7168, 64, 1536, 512, 128, 64, 128)
    fake = ctypes.c_void_p(0x1000)
    w = mla.Weights(*[fake] * 7)
    need = L.mla_decode_workspace_size(ctypes.byref(d), 1024, 8193)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    st = L.mla_decode_latentcache_noalloc(ctypes.byref(d), ctypes.byref(w), fake, 1024, 8192, 8193, fake,
                                          fake, fake, 8193, fake, None)
    assert st == -4 and "scratch" in L.mla_last_error().decode()
    st = L.mla_decode_latentcache_noalloc(ctypes.byref(d), ctypes.byref(w), fake, 4, 16, 16, fake, fake,
                                          fake, 17, fake, None)
    assert st == -2                                  # P outside the cache
    st = L.mla_decode_latentcache_noalloc(ctypes.byref(d), ctypes.byref(w), fake, 4, 3, 16, None, fake,
                                          fake, 17, fake, None)
    assert st == -1                                  # no cache
