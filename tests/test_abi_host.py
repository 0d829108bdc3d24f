"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function that include/mla.h declares,
and reject bad arguments with the documented status codes before making any
HIP call (the size checks of the "Kimi K2 · Mix and project" code excerpt
become error codes here).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("head_latent_attention_fwd_amd")


def _lib():
    try:
        return mla.load()
    except mla.MLAError as e:
        pytest.fail(f"libmla.so not built: {e}")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+|dense_block_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mla_prefill", "mla_decode_fullcache", "mla_decode_latentcache", "dense_block_fwd",
              "mla_rope_table", "mla_status_string", "mla_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in mla.h but not exported"


def kimi(dtype="bf16"):
    return mla.make_dims(7168, 64, 1536, 512, 128, 64, 128, d_ff=18432, dtype=dtype)


def tiny(dtype="f32"):
    return mla.make_dims(256, 4, 96, 64, 32, 16, 32, d_ff=512, dtype=dtype)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _w(**over):
    w = mla.Weights(*[FAKE] * 7)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def _prefill(L, d, w=None, x=FAKE, B=1, T=16, rc=FAKE, rs=FAKE, rows=16, out=FAKE, kc=None,
             vc=None, lc=None, L_cap=0, ws=FAKE, wsb=None):
    w = w or _w()
    if wsb is None:
        wsb = L.mla_prefill_workspace_size(ctypes.byref(d), B, T) if B > 0 and T > 0 else 0
    return L.mla_prefill(ctypes.byref(d), ctypes.byref(w), x, B, T, rc, rs, rows, out, kc, vc, lc,
                         L_cap, ws, wsb, None)


def test_workspace_sizes_positive():
    L = _lib()
    for d in (kimi(), tiny()):
        assert L.mla_prefill_workspace_size(ctypes.byref(d), 1, 2048) > 0
        assert L.mla_decode_workspace_size(ctypes.byref(d), 64, 1001) > 0
        assert L.dense_block_workspace_size(ctypes.byref(d), 1, 128) > 0
    # bad shapes give 0
    assert L.mla_prefill_workspace_size(ctypes.byref(kimi()), 0, 16) == 0
    d = tiny()
    d.n_heads = 0
    assert L.mla_decode_workspace_size(ctypes.byref(d), 1, 16) == 0


def test_null_pointers_rejected():
    L = _lib()
    d = tiny()
    assert _prefill(L, d, x=None) == -1
    assert _prefill(L, d, out=None) == -1
    assert _prefill(L, d, ws=None) == -1
    assert _prefill(L, d, rc=None) == -1
    assert _prefill(L, d, w=_w(w_ukv=None)) == -1
    assert L.mla_prefill(None, ctypes.byref(_w()), FAKE, 1, 1, FAKE, FAKE, 1, FAKE, None, None, None,
                         0, FAKE, 1 << 30, None) == -1
    assert "NULL" in L.mla_last_error().decode() or "null" in L.mla_last_error().decode().lower()
    # k_cache without v_cache
    assert _prefill(L, d, kc=FAKE, L_cap=16) == -1


def test_bad_shapes_rejected():
    L = _lib()
    d = tiny()
    assert _prefill(L, d, B=0) == -2              # empty inputs are refused, not a silent no-op
    assert _prefill(L, d, T=0) == -2
    assert _prefill(L, d, T=-3) == -2
    assert _prefill(L, d, rows=15) == -2          # rope table shorter than T
    assert _prefill(L, d, kc=FAKE, vc=FAKE, L_cap=8) == -2   # cache smaller than T
    d2 = tiny()
    d2.qk_rope_dim = 15                             # odd rotary width
    assert _prefill(L, d2) == -2
    d3 = tiny()
    d3.softmax_scale = float("nan")
    assert _prefill(L, d3) == -2
    # decode: P outside the cache
    w = _w()
    for P in (-1, 16):
        st = L.mla_decode_fullcache(ctypes.byref(d), ctypes.byref(w), FAKE, 2, P, 16, FAKE, FAKE,
                                    FAKE, FAKE, 64, FAKE, FAKE, 1 << 40, None)
        assert st == -2
    st = L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 10, 16, FAKE, FAKE,
                                  FAKE, 5, FAKE, FAKE, 1 << 40, None)   # rope rows 5 <= P
    assert st == -2


def test_ragged_decode_arguments_rejected():
    """Per-sequence positions: a NULL table, P_max outside the cache and a
    rope table not covering P_max are rejected before any HIP call."""
    L = _lib()
    d = tiny()
    w = _w()
    st = L.mla_decode_fullcache_ragged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, None, 5, 16, FAKE,
                                       FAKE, FAKE, FAKE, 64, FAKE, FAKE, 1 << 40, None)
    assert st == -1 and "positions" in L.mla_last_error().decode()
    st = L.mla_decode_latentcache_ragged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, None, 5, 16, FAKE,
                                         FAKE, FAKE, 64, FAKE, FAKE, 1 << 40, None)
    assert st == -1
    for P_max in (-1, 16):
        st = L.mla_decode_fullcache_ragged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, FAKE, P_max, 16,
                                           FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 1 << 40, None)
        assert st == -2
        st = L.mla_decode_latentcache_ragged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, FAKE, P_max, 16,
                                             FAKE, FAKE, FAKE, 64, FAKE, FAKE, 1 << 40, None)
        assert st == -2
    st = L.mla_decode_latentcache_ragged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, FAKE, 10, 16, FAKE,
                                         FAKE, FAKE, 10, FAKE, FAKE, 1 << 40, None)  # rope rows 10 <= P_max
    assert st == -2


def test_unsupported_rejected():
    L = _lib()
    d = kimi()
    d.qk_nope_dim = 96                              # bf16 path: Kimi head widths only
    assert _prefill(L, d, wsb=1 << 40) == -3
    d = kimi()
    d.dtype = 7
    assert _prefill(L, d, wsb=1 << 40) == -3
    d = kimi()
    d.kv_lora_rank = 448                            # bf16 latent decode needs 512
    st = L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(_w()), FAKE, 2, 3, 16, FAKE, FAKE,
                                  FAKE, 16, FAKE, FAKE, 1 << 40, None)
    assert st == -3
    d = kimi()                                      # bf16 latent decode: at most 1024 sequences
    st = L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(_w()), FAKE, 1025, 3, 16, FAKE, FAKE,
                                  FAKE, 16, FAKE, FAKE, 1 << 40, None)
    assert st == -3 and "1024" in L.mla_last_error().decode()
    st = L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(_w()), FAKE, 1024, 3, 16, FAKE, FAKE,
                                  FAKE, 16, FAKE, FAKE, 1, None)
    assert st == -4                                 # 1024 passes the batch check, then the workspace one


def test_prefill_beyond_attention_offsets_rejected():
    """A bf16 prefill whose per-head key rows do not fit the flash kernel's
    32-bit byte offsets is refused up front (MLA_ERR_UNSUPPORTED), for the
    prefill and the dense block, whatever the workspace; the largest T that
    fits passes that check and stops at the workspace check."""
    L = _lib()
    d = kimi()
    T_bad = (1 << 31) // (64 * 256 * 2) - 64        # 65472: (T + 64) kv rows reach 2^31 bytes
    assert _prefill(L, d, T=T_bad, rows=T_bad, wsb=1 << 40) == -3
    assert "offsets" in L.mla_last_error().decode()
    bw = mla.BlockWeights(FAKE, FAKE, _w(), FAKE, FAKE, FAKE)
    st = L.dense_block_fwd(ctypes.byref(d), ctypes.byref(bw), FAKE, 1, T_bad, FAKE, FAKE, T_bad, FAKE,
                           FAKE, 1 << 40, None)
    assert st == -3
    assert _prefill(L, d, T=T_bad - 1, rows=T_bad, wsb=1) == -4


def test_softmax_scale_default_and_range():
    """softmax_scale 0 selects the default scale (accepted); a negative one
    is rejected."""
    L = _lib()
    d = tiny()
    d.softmax_scale = 0.0
    assert _prefill(L, d, wsb=1) == -4               # past the dims check
    d.softmax_scale = -0.5
    assert _prefill(L, d) == -2


def test_small_workspace_rejected():
    L = _lib()
    d = kimi()
    need = L.mla_prefill_workspace_size(ctypes.byref(d), 1, 64)
    assert _prefill(L, d, T=64, rows=64, wsb=need - 1) == -4
    assert "workspace" in L.mla_last_error().decode()
    need = L.mla_decode_workspace_size(ctypes.byref(d), 4, 100)
    st = L.mla_decode_fullcache(ctypes.byref(d), ctypes.byref(_w()), FAKE, 4, 5, 100, FAKE, FAKE,
                                FAKE, FAKE, 100, FAKE, FAKE, need - 1, None)
    assert st == -4


def test_status_strings():
    L = _lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.mla_status_string(s).decode().startswith("MLA_")


def test_binding_raises_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    d = tiny()
    with pytest.raises((ValueError, TypeError)):
        mla.mla_prefill(d, {}, torch.zeros(1, 4, 256), (torch.zeros(4, 8), torch.zeros(4, 8)))


def test_misaligned_pointers_are_rejected():
    """Every device pointer must be 16-byte aligned (the kernels move data in
    16-byte vectors): a misaligned tensor, weight, table or workspace pointer
    returns MLA_ERR_UNSUPPORTED (-3) before any HIP call."""
    L = _lib()
    d = kimi()
    odd = ctypes.c_void_p(0x1008)
    assert _prefill(L, d, x=odd) == -3
    assert b"16-byte" in L.mla_last_error()
    assert _prefill(L, d, out=odd) == -3
    assert _prefill(L, d, ws=odd) == -3
    assert _prefill(L, d, rc=odd) == -3
    assert _prefill(L, d, w=_w(w_o=odd)) == -3
    assert _prefill(L, d, kc=odd, vc=FAKE, L_cap=16) == -3
    w = _w()
    st = L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 10, 16, odd, FAKE,
                                  FAKE, 64, FAKE, FAKE, 1 << 40, None)
    assert st == -3
    st = L.mla_decode_fullcache(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 10, 16, FAKE, FAKE,
                                FAKE, FAKE, 64, FAKE, odd, 1 << 40, None)
    assert st == -3


def test_read_sweep_arguments_rejected():
    """The measurement yardstick validates its arguments like the compute
    calls: NULL pointers, sizes that are not a positive multiple of 16 bytes
    and misaligned pointers are refused before any HIP call."""
    L = _lib()
    assert L.mla_read_sweep(None, 1024, FAKE, None) == -1
    assert L.mla_read_sweep(FAKE, 1024, None, None) == -1
    assert L.mla_read_sweep(FAKE, 0, FAKE, None) == -2
    assert L.mla_read_sweep(FAKE, 1000, FAKE, None) == -2
    assert L.mla_read_sweep(ctypes.c_void_p(0x1008), 1024, FAKE, None) == -3


def test_persistent_latent_decode_arguments_rejected():
    """The persistent latent decode checks as the multi-launch form does, and
    serves bf16 batches of up to 64 sequences; every case fails before a HIP
    call."""
    L = _lib()
    d = kimi()

    def call(d, B=2, P=3, L_cap=16, lc=FAKE, x=FAKE, out=FAKE, ws=FAKE, wsb=1 << 40):
        return L.mla_decode_latentcache_persistent(ctypes.byref(d), ctypes.byref(_w()), x, B, P, L_cap, lc,
                                                   FAKE, FAKE, 16, out, ws, wsb, None)

    assert call(d, lc=None) == -1
    assert call(d, x=None) == -1
    assert call(d, ws=None) == -1
    assert call(d, P=16) == -2                      # P outside [0, L_cap)
    assert call(d, B=0) == -2
    assert call(d, B=65) == -3 and "64" in L.mla_last_error().decode()
    assert call(tiny()) == -3 and "bf16" in L.mla_last_error().decode()
    d2 = kimi()
    d2.kv_lora_rank = 448
    assert call(d2) == -3
    assert call(d, wsb=1) == -4                     # everything else valid: workspace too small
    odd = mla.make_dims(960, 64, 192, 512, 128, 64, 128, dtype="bf16")
    assert call(odd) == -3                          # d_model 960: no weight-stream form (K % 128)
    assert "weight-streaming" in L.mla_last_error().decode()
    st = ctypes.c_int(7)
    assert L.mla_decode_latentcache_persistent_status(ctypes.byref(d), 2, 16, FAKE, None) == -1
    assert L.mla_decode_latentcache_persistent_status(ctypes.byref(d), 0, 16, FAKE, ctypes.byref(st)) == -2
    assert st.value == 7
