"""Thin Python binding of the C ABI in include/mla.h (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmla.so``.  PyTorch supplies device memory and the current
stream.  The binding checks tensor shapes, dtypes and devices against the
layer dimensions before calling (the C ABI sees only pointers and sizes), and
raises ``MLAError`` with the library's message on any non-zero status.

There is no fallback: if ``libmla.so`` has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
W_NAMES = ("w_dq", "g_q", "w_uqr", "w_dkvr", "g_kv", "w_ukv", "w_o")
# optional biases of the attention_bias variant (absent = no bias)
BIAS_NAMES = ("b_dq", "b_dkvr", "b_o")
BLOCK_NAMES = ("g_attn", "g_ffn", "w1", "w3", "w2")


class MLAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("q_lora_rank", ctypes.c_int), ("kv_lora_rank", ctypes.c_int),
                ("qk_nope_dim", ctypes.c_int), ("qk_rope_dim", ctypes.c_int),
                ("v_head_dim", ctypes.c_int), ("d_ff", ctypes.c_int),
                ("rms_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int)]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == MLA_BF16 else torch.float32


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in W_NAMES + BIAS_NAMES]


class BlockWeights(ctypes.Structure):
    _fields_ = [("g_attn", ctypes.c_void_p), ("g_ffn", ctypes.c_void_p), ("attn", Weights),
                ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(Dims)


def load():
    """Load libmla.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MLAError(-100, f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    L.mla_rope_table.argtypes = [_I, _I, ctypes.c_double, _P, _P, _P]
    L.mla_prefill_workspace_size.argtypes = [_DP, _I, _I]
    L.mla_prefill_workspace_size.restype = _SZ
    L.mla_prefill.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _P, _P, _I, _P, _P, _P, _P,
                              _I, _P, _SZ, _P]
    L.mla_decode_workspace_size.argtypes = [_DP, _I, _I]
    L.mla_decode_workspace_size.restype = _SZ
    L.mla_decode_fullcache.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _P, _P, _P, _P,
                                       _I, _P, _P, _SZ, _P]
    L.mla_decode_latentcache.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _P, _P, _P,
                                         _I, _P, _P, _SZ, _P]
    L.mla_decode_latentcache_noalloc.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _P, _P,
                                                 _P, _I, _P, _P]
    L.mla_decode_latentcache_persistent.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _P, _P,
                                                    _P, _I, _P, _P, _SZ, _P]
    L.mla_decode_latentcache_persistent_status.argtypes = [_DP, _I, _I, _P, ctypes.POINTER(_I)]
    L.mla_decode_fullcache_ragged.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _P, _I, _I, _P,
                                              _P, _P, _P, _I, _P, _P, _SZ, _P]
    L.mla_decode_latentcache_ragged.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _P, _I, _I,
                                                _P, _P, _P, _I, _P, _P, _SZ, _P]
    L.mla_prefill_chunk_workspace_size.argtypes = [_DP, _I, _I, _I]
    L.mla_prefill_chunk_workspace_size.restype = _SZ
    L.mla_prefill_chunk_fullcache.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _I, _P, _P,
                                              _P, _P, _I, _P, _P, _SZ, _P]
    L.mla_prefill_chunk_latentcache.argtypes = [_DP, ctypes.POINTER(Weights), _P, _I, _I, _I, _I, _P,
                                                _P, _P, _I, _P, _P, _SZ, _P]
    L.dense_block_workspace_size.argtypes = [_DP, _I, _I]
    L.dense_block_workspace_size.restype = _SZ
    L.dense_block_fwd.argtypes = [_DP, ctypes.POINTER(BlockWeights), _P, _I, _I, _P, _P, _I, _P, _P,
                                  _SZ, _P]
    L.mla_read_sweep.argtypes = [_P, _SZ, _P, _P]
    L.mla_read_sweep.restype = _I
    L.mla_profile_enable.argtypes = [_I]
    L.mla_profile_enable.restype = _I
    L.mla_profile_summary.argtypes = [ctypes.c_char_p, _SZ, ctypes.POINTER(_I)]
    L.mla_profile_summary.restype = _I
    L.mla_status_string.argtypes = [_I]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    for name in ("mla_rope_table", "mla_prefill", "mla_decode_fullcache",
                 "mla_decode_latentcache", "mla_decode_latentcache_noalloc", "mla_decode_latentcache_persistent",
                 "mla_decode_latentcache_persistent_status", "mla_decode_fullcache_ragged",
                 "mla_decode_latentcache_ragged", "mla_prefill_chunk_fullcache",
                 "mla_prefill_chunk_latentcache", "dense_block_fwd"):
        getattr(L, name).restype = _I
    _lib = L
    return L


def _check(status):
    if status != 0:
        L = load()
        raise MLAError(status, L.mla_last_error().decode() or L.mla_status_string(status).decode())


def make_dims(d_model, n_heads, q_lora_rank, kv_lora_rank, qk_nope_dim, qk_rope_dim, v_head_dim,
              d_ff=0, rms_eps=1e-6, softmax_scale=None, dtype="bf16") -> Dims:
    """mla_dims of one layer.  softmax_scale None passes 0, for which the
    library uses its documented default."""
    if softmax_scale is None:
        softmax_scale = 0.0
    dt = MLA_BF16 if dtype in ("bf16", torch.bfloat16, MLA_BF16) else MLA_F32
    return Dims(d_model, n_heads, q_lora_rank, kv_lora_rank, qk_nope_dim, qk_rope_dim, v_head_dim,
                d_ff, rms_eps, softmax_scale, dt)


def weight_shapes(d: Dims) -> dict:
    H = d.n_heads
    return {"w_dq": (d.q_lora_rank, d.d_model), "g_q": (d.q_lora_rank,),
            "w_uqr": (H * (d.qk_nope_dim + d.qk_rope_dim), d.q_lora_rank),
            "w_dkvr": (d.kv_lora_rank + d.qk_rope_dim, d.d_model), "g_kv": (d.kv_lora_rank,),
            "w_ukv": (H * (d.qk_nope_dim + d.v_head_dim), d.kv_lora_rank),
            "w_o": (d.d_model, H * d.v_head_dim)}


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _tensor(t, name, shape, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device or 'a GPU'}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def bias_shapes(d: Dims) -> dict:
    """Shapes of the optional attention_bias biases."""
    return {"b_dq": (d.q_lora_rank,), "b_dkvr": (d.kv_lora_rank + d.qk_rope_dim,), "b_o": (d.d_model,)}


def _weights(d: Dims, w: dict, device) -> Weights:
    shapes = weight_shapes(d)
    bshapes = bias_shapes(d)
    ptrs = [_tensor(w[n], n, shapes[n], d.torch_dtype, device) for n in W_NAMES]
    ptrs += [_tensor(w[n], n, bshapes[n], d.torch_dtype, device) if w.get(n) is not None else None
             for n in BIAS_NAMES]
    return Weights(*ptrs)


def _rope(rope, rows_needed, d: Dims, device):
    cos, sin = rope
    for n, t in (("rope_cos", cos), ("rope_sin", sin)):
        if t.dim() != 2 or t.shape[1] != d.qk_rope_dim // 2 or t.shape[0] < rows_needed:
            raise ValueError(f"{n}: shape {tuple(t.shape)}, need [>= {rows_needed}, {d.qk_rope_dim // 2}]")
        _tensor(t, n, t.shape, torch.float32, device)
    return ctypes.c_void_p(cos.data_ptr()), ctypes.c_void_p(sin.data_ptr()), cos.shape[0]


def _ws(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def mla_profile_enable(on: bool = True):
    """Record HIP events around every kernel launch of later calls (this thread)."""
    _check(load().mla_profile_enable(1 if on else 0))


def mla_profile_summary() -> dict:
    """{kernel name: (launches, total ms)} for the launches recorded since the
    last summary (waits for them to finish)."""
    L = load()
    buf = ctypes.create_string_buffer(1 << 16)
    n = _I(0)
    _check(L.mla_profile_summary(buf, len(buf), ctypes.byref(n)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def mla_rope_table(n_pos, d_rope, base=10000.0, device="cuda"):
    """The RoPE table R as float32 (cos, sin) [n_pos, d_rope/2], built on the GPU."""
    L = load()
    device = torch.device(device)
    cos = torch.empty(n_pos, d_rope // 2, dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(L.mla_rope_table(n_pos, d_rope, float(base), ctypes.c_void_p(cos.data_ptr()),
                            ctypes.c_void_p(sin.data_ptr()), _stream(device)))
    return cos, sin


def mla_read_sweep(buf, sink=None):
    """Read every byte of the device tensor buf once (the HBM read-rate
    yardstick); returns the sink tensor (4096 int32 words whose XOR is the
    XOR of every word read; allocated when not given)."""
    L = load()
    dev = buf.device
    if not buf.is_contiguous():
        raise MLAError(-2, "buf must be contiguous")
    if sink is None:
        sink = torch.empty(4096, dtype=torch.int32, device=dev)
    _check(L.mla_read_sweep(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                            ctypes.c_void_p(sink.data_ptr()), _stream(dev)))
    return sink


def prefill_workspace_size(d: Dims, B, T):
    return int(load().mla_prefill_workspace_size(ctypes.byref(d), B, T))


def decode_workspace_size(d: Dims, B, L_cap):
    return int(load().mla_decode_workspace_size(ctypes.byref(d), B, L_cap))


def block_workspace_size(d: Dims, B, T):
    return int(load().dense_block_workspace_size(ctypes.byref(d), B, T))


def mla_prefill(d: Dims, w: dict, x, rope, out=None, k_cache=None, v_cache=None,
                latent_cache=None, workspace=None):
    """out [B, T, d] = causal MLA of x [B, T, d]; optional cache outputs."""
    L = load()
    dev = x.device
    B, T = x.shape[0], x.shape[1]
    _tensor(x, "x", (B, T, d.d_model), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, T, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    L_cap = 0
    kc = vc = lc = None
    if k_cache is not None or v_cache is not None:
        L_cap = k_cache.shape[2]
        kc = _tensor(k_cache, "k_cache", (B, d.n_heads, L_cap, d.qk_nope_dim + d.qk_rope_dim), d.torch_dtype, dev)
        vc = _tensor(v_cache, "v_cache", (B, d.n_heads, L_cap, d.v_head_dim), d.torch_dtype, dev)
    if latent_cache is not None:
        if L_cap and latent_cache.shape[1] != L_cap:
            raise ValueError("latent_cache and k_cache must have the same capacity")
        L_cap = latent_cache.shape[1]
        lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    n = prefill_workspace_size(d, B, T)
    ws = _ws(n, dev, workspace)
    _check(L.mla_prefill(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()), B, T,
                         rc, rs, rows, ctypes.c_void_p(out.data_ptr()), kc, vc, lc, L_cap,
                         ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev)))
    return out


def mla_decode_fullcache(d: Dims, w: dict, x, P, k_cache, v_cache, rope, out=None, workspace=None):
    """One decode token per sequence at position P; slot P of the caches is
    overwritten with the new key/value.  x [B, d] -> out [B, d]."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = k_cache.shape[2]
    kc = _tensor(k_cache, "k_cache", (B, d.n_heads, L_cap, d.qk_nope_dim + d.qk_rope_dim), d.torch_dtype, dev)
    vc = _tensor(v_cache, "v_cache", (B, d.n_heads, L_cap, d.v_head_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P + 1, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(decode_workspace_size(d, B, L_cap), dev, workspace)
    _check(L.mla_decode_fullcache(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                  B, int(P), L_cap, kc, vc, rc, rs, rows,
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                  ws.numel(), _stream(dev)))
    return out


def mla_decode_latentcache(d: Dims, w: dict, x, P, latent_cache, rope, out=None, workspace=None):
    """Absorbed decode over the latent cache [B, L_cap, kv_lora + d_rope];
    slot P is overwritten with the new token's entry.  x [B, d] -> out [B, d]."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = latent_cache.shape[1]
    lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P + 1, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(decode_workspace_size(d, B, L_cap), dev, workspace)
    _check(L.mla_decode_latentcache(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                    B, int(P), L_cap, lc, rc, rs, rows,
                                    ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                    ws.numel(), _stream(dev)))
    return out


def mla_decode_latentcache_persistent(d: Dims, w: dict, x, P, latent_cache, rope, out=None, workspace=None):
    """mla_decode_latentcache as one persistent cooperative kernel (bf16,
    B <= 64): same arguments and workspace."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = latent_cache.shape[1]
    lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P + 1, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(decode_workspace_size(d, B, L_cap), dev, workspace)
    _check(L.mla_decode_latentcache_persistent(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                               B, int(P), L_cap, lc, rc, rs, rows,
                                               ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                               ws.numel(), _stream(dev)))
    return out


def mla_decode_latentcache_persistent_status(d: Dims, B, L_cap, workspace):
    """1 if a grid barrier of the last persistent step in `workspace` gave up,
    else 0 (synchronous: call after the step's stream has finished)."""
    L = load()
    st = ctypes.c_int(-1)
    _check(L.mla_decode_latentcache_persistent_status(ctypes.byref(d), int(B), int(L_cap),
                                                      ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(st)))
    return st.value


NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES of include/mla.h


def mla_decode_latentcache_noalloc(d: Dims, w: dict, x, P, latent_cache, rope, out):
    """mla_decode_latentcache with the library's own device scratch array
    instead of a workspace (no device allocation by the library; `out` must be
    given).  Steps whose workspace exceeds the array raise MLAError."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = latent_cache.shape[1]
    lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P + 1, d, dev)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    _check(L.mla_decode_latentcache_noalloc(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                            B, int(P), L_cap, lc, rc, rs, rows,
                                            ctypes.c_void_p(out.data_ptr()), _stream(dev)))
    return out


def _positions(positions, B, P_max, L_cap, dev):
    """Device int32 [B] per-sequence positions and their host upper bound."""
    pp = _tensor(positions, "positions", (B,), torch.int32, dev)
    P_max = int(P_max)
    if not 0 <= P_max < L_cap:
        raise ValueError(f"P_max={P_max} outside [0, L_cap={L_cap})")
    return pp, P_max


def mla_decode_fullcache_ragged(d: Dims, w: dict, x, positions, P_max, k_cache, v_cache, rope,
                                out=None, workspace=None):
    """Decode over a ragged batch: sequence b's new token sits at
    positions[b] (device int32 [B], each <= P_max); slot positions[b] of its
    cache rows is overwritten and keys 0..positions[b] are attended.
    x [B, d] -> out [B, d]."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = k_cache.shape[2]
    kc = _tensor(k_cache, "k_cache", (B, d.n_heads, L_cap, d.qk_nope_dim + d.qk_rope_dim), d.torch_dtype, dev)
    vc = _tensor(v_cache, "v_cache", (B, d.n_heads, L_cap, d.v_head_dim), d.torch_dtype, dev)
    pp, P_max = _positions(positions, B, P_max, L_cap, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P_max + 1, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(decode_workspace_size(d, B, L_cap), dev, workspace)
    _check(L.mla_decode_fullcache_ragged(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                         B, pp, P_max, L_cap, kc, vc, rc, rs, rows,
                                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel(), _stream(dev)))
    return out


def mla_decode_latentcache_ragged(d: Dims, w: dict, x, positions, P_max, latent_cache, rope,
                                  out=None, workspace=None):
    """Absorbed decode over the latent cache for a ragged batch (positions as
    in mla_decode_fullcache_ragged).  x [B, d] -> out [B, d]."""
    L = load()
    dev = x.device
    B = x.shape[0]
    _tensor(x, "x", (B, d.d_model), d.torch_dtype, dev)
    L_cap = latent_cache.shape[1]
    lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    pp, P_max = _positions(positions, B, P_max, L_cap, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, P_max + 1, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(decode_workspace_size(d, B, L_cap), dev, workspace)
    _check(L.mla_decode_latentcache_ragged(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                           B, pp, P_max, L_cap, lc, rc, rs, rows,
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel(), _stream(dev)))
    return out


def chunk_workspace_size(d: Dims, B, T, L_cap):
    return load().mla_prefill_chunk_workspace_size(ctypes.byref(d), B, T, L_cap)


def mla_prefill_chunk_fullcache(d: Dims, w: dict, x, P0, k_cache, v_cache, rope, out=None, workspace=None):
    """Chunked prefill with the full cache: x [B, T, d] holds the tokens at
    positions P0 .. P0+T-1; cache slots 0 .. P0-1 are the history, slots
    P0 .. P0+T-1 are written.  Returns out [B, T, d]."""
    L = load()
    dev = x.device
    B, T = x.shape[0], x.shape[1]
    _tensor(x, "x", (B, T, d.d_model), d.torch_dtype, dev)
    L_cap = k_cache.shape[2]
    kc = _tensor(k_cache, "k_cache", (B, d.n_heads, L_cap, d.qk_nope_dim + d.qk_rope_dim), d.torch_dtype, dev)
    vc = _tensor(v_cache, "v_cache", (B, d.n_heads, L_cap, d.v_head_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, int(P0) + T, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(chunk_workspace_size(d, B, T, L_cap), dev, workspace)
    _check(L.mla_prefill_chunk_fullcache(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                         B, T, int(P0), L_cap, kc, vc, rc, rs, rows,
                                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel(), _stream(dev)))
    return out


def mla_prefill_chunk_latentcache(d: Dims, w: dict, x, P0, latent_cache, rope, out=None, workspace=None):
    """Chunked prefill with the latent cache [B, L_cap, kv_lora + d_rope]
    (positions as in mla_prefill_chunk_fullcache).  Returns out [B, T, d]."""
    L = load()
    dev = x.device
    B, T = x.shape[0], x.shape[1]
    _tensor(x, "x", (B, T, d.d_model), d.torch_dtype, dev)
    L_cap = latent_cache.shape[1]
    lc = _tensor(latent_cache, "latent_cache", (B, L_cap, d.kv_lora_rank + d.qk_rope_dim), d.torch_dtype, dev)
    wt = _weights(d, w, dev)
    rc, rs, rows = _rope(rope, int(P0) + T, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, d.torch_dtype, dev)
    ws = _ws(chunk_workspace_size(d, B, T, L_cap), dev, workspace)
    _check(L.mla_prefill_chunk_latentcache(ctypes.byref(d), ctypes.byref(wt), ctypes.c_void_p(x.data_ptr()),
                                           B, T, int(P0), L_cap, lc, rc, rs, rows,
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel(), _stream(dev)))
    return out


def dense_block_fwd(d: Dims, w: dict, blk: dict, x, rope, out=None, workspace=None):
    """Dense transformer block: out = x' + SwiGLU(RMSNorm(x')), x' = x + MLA(RMSNorm(x))."""
    L = load()
    dev = x.device
    B, T = x.shape[0], x.shape[1]
    _tensor(x, "x", (B, T, d.d_model), d.torch_dtype, dev)
    dt = d.torch_dtype
    bw = BlockWeights(_tensor(blk["g_attn"], "g_attn", (d.d_model,), dt, dev),
                      _tensor(blk["g_ffn"], "g_ffn", (d.d_model,), dt, dev),
                      _weights(d, w, dev),
                      _tensor(blk["w1"], "w1", (d.d_ff, d.d_model), dt, dev),
                      _tensor(blk["w3"], "w3", (d.d_ff, d.d_model), dt, dev),
                      _tensor(blk["w2"], "w2", (d.d_model, d.d_ff), dt, dev))
    rc, rs, rows = _rope(rope, T, d, dev)
    if out is None:
        out = torch.empty_like(x)
    _tensor(out, "out", x.shape, dt, dev)
    ws = _ws(block_workspace_size(d, B, T), dev, workspace)
    _check(L.dense_block_fwd(ctypes.byref(d), ctypes.byref(bw), ctypes.c_void_p(x.data_ptr()), B, T,
                             rc, rs, rows, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(dev)))
    return out
