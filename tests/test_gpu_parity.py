"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bars: max|gpu - oracle| <= 1e-4 * max|oracle| for float32 workloads and
<= 2e-2 * max|oracle| for bf16 workloads.  Sizes span several tiles with
ragged tails; full-size workloads are checked on sampled outputs.
"""
import numpy as np
import pytest

from oracle import mla_ref as ref
from tests import synth
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, bits_to_dev, dims_of, from_dev, log,
                            oracle_weights, to_dev, weights_to_dev)

torch = pytest.importorskip("torch")
mla = pytest.importorskip("head_latent_attention_fwd_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# Kimi K2 widths with smaller model/latent widths, for fast oracle runs that
# still exercise the bf16 kernels' fixed head shapes.
# Widths that are multiples of 64 but not of 128 (d_model 960, query latent
# 192): the decode projections with K = 960 or K = 192, and the joint
# down-projection split at 192, leave the 128-k weight stream for the K-sliced
# register-streamed kernel; the 960-wide outputs end in a partial tile.
KIMI_ODD = ref.MLADims(d_model=960, n_heads=64, q_lora_rank=192, kv_lora_rank=512,
                       qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128, d_ff=1536)
# the same with a 576-wide query latent: its decode up-projection takes two
# 512-wide K slices whose fp32 partials a separate launch sums into bf16
KIMI_ODD576 = ref.MLADims(d_model=960, n_heads=64, q_lora_rank=576, kv_lora_rank=512,
                          qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128, d_ff=1536)
KIMI_NARROW = ref.MLADims(d_model=1024, n_heads=64, q_lora_rank=256, kv_lora_rank=512,
                          qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128, d_ff=1536)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mla.load()
    yield
    torch.cuda.synchronize()


def _rope(od, n):
    return mla.mla_rope_table(n, od.qk_rope_dim, od.rope_base, DEV)


# ------------------------------------------------------------------ prefill
@pytest.mark.parametrize("case", [
    ("tiny_config", ref.TINY, 1, 16, "f32", 1001),
    ("tiny_ragged", ref.TINY, 2, 37, "f32", 7),
    ("kimi_narrow_bf16", KIMI_NARROW, 2, 200, "bf16", 11),
    ("odd_widths_bf16", KIMI_ODD, 1, 100, "bf16", 15),
    ("kimi_bf16_T130", ref.KIMI_K2, 1, 130, "bf16", 12),
    ("kimi_bf16_T20_small_rows", ref.KIMI_K2, 2, 20, "bf16", 13),
    # a one-token prompt per sequence: every product has 3 rows, and the
    # attention is one key per query
    ("kimi_bf16_T1", ref.KIMI_K2, 3, 1, "bf16", 14),
])
def test_prefill(case):
    name, od, B, T, dt, seed = case
    log(f"[prefill {name}] B={B} T={T} dtype={dt} seed={seed}")
    x, w = synth.prefill_inputs(od, B, T, seed, bf16=(dt == "bf16"))
    want = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64))
    d = dims_of(mla, od, dt)
    got = mla.mla_prefill(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got), want, TOL_F32 if dt == "f32" else TOL_BF16, name)


def test_prefill_kimi_full_size_sampled_rows():
    """The Kimi K2 prefill workload itself (B=1, T=2048, bf16) in the launch
    configuration the benchmark times; the oracle computes all keys/values
    and a sample of query rows (first, last, and random)."""
    od = ref.KIMI_K2
    B, T = 1, 2048
    log(f"[prefill kimi full] B={B} T={T} bf16")
    x, w = synth.prefill_inputs(od, B, T, 1002, bf16=True)
    rows = sorted(set([0, 1, 63, 64, 127, 128, 1000, T - 1] +
                      list(np.random.default_rng(5).choice(T, 24, replace=False))))
    want = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.mla_prefill(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi prefill T=2048 sampled rows")


def test_prefill_kimi_ragged_T2000_sampled_rows():
    """Kimi K2 widths at T=2000: 256-row tiles with a ragged last row tile in
    every GEMM and a ragged last query tile in the attention kernel."""
    od = ref.KIMI_K2
    B, T = 1, 2000
    log(f"[prefill kimi ragged] B={B} T={T} bf16")
    x, w = synth.prefill_inputs(od, B, T, 1012, bf16=True)
    rows = sorted(set([0, 255, 256, 1791, 1792, 1900, 1983, 1984, T - 2, T - 1] +
                      list(np.random.default_rng(6).choice(T, 12, replace=False))))
    want = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.mla_prefill(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi prefill T=2000 sampled rows")


def test_prefill_24_heads_T2300_sampled_rows():
    """24 heads at T=2300: the q and kv up-projections have 9 x 18 and 9 x 24
    tiles of 256 x 256, 378 in all with neither count a multiple of the 8
    XCDs, so the persistent tile loop splits them unevenly over the XCDs and
    its product-1 runs differ between XCDs (with Kimi widths every count is a
    multiple of 8).  One sampled query row in every 256-row block, so a tile
    computed twice or not at all shows up."""
    od = ref.MLADims(d_model=7168, n_heads=24, q_lora_rank=1536, kv_lora_rank=512,
                     qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128)
    B, T = 1, 2300
    log(f"[prefill 24 heads] B={B} T={T} bf16")
    x, w = synth.prefill_inputs(od, B, T, 1015, bf16=True)
    rows = sorted(set([0, 255, 256, 511, 700, 1023, 1100, 1400, 1535, 1800, 2047, 2048, 2200, T - 1] +
                      list(np.random.default_rng(8).choice(T, 8, replace=False))))
    want = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.mla_prefill(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "24-head prefill T=2300 sampled rows")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_writes_caches(dt):
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, T, L_cap = 2, 70, 80
    log(f"[prefill caches] dtype={dt} B={B} T={T} L_cap={L_cap}")
    x, w = synth.prefill_inputs(od, B, T, 21, bf16=(dt == "bf16"))
    _, p = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), return_intermediates=True)
    K, V = ref.full_cache_entries(od, p)
    C = ref.latent_cache_entries(od, p)
    d = dims_of(mla, od, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kc = torch.zeros(B, od.n_heads, L_cap, od.q_head_dim, dtype=tdt, device=DEV)
    vc = torch.zeros(B, od.n_heads, L_cap, od.v_head_dim, dtype=tdt, device=DEV)
    lc = torch.zeros(B, L_cap, od.kv_lora_rank + od.qk_rope_dim, dtype=tdt, device=DEV)
    mla.mla_prefill(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), _rope(od, T),
                    k_cache=kc, v_cache=vc, latent_cache=lc)
    torch.cuda.synchronize()
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(from_dev(kc)[:, :, :T], K, tol, "k_cache")
    assert_close(from_dev(vc)[:, :, :T], V, tol, "v_cache")
    assert_close(from_dev(lc)[:, :T], C, tol, "latent_cache")
    assert torch.count_nonzero(kc[:, :, T:]) == 0 and torch.count_nonzero(lc[:, T:]) == 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_causality_bitwise(dt):
    """Perturbing tokens after position t leaves outputs 0..t bitwise equal."""
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, T = 1, 150
    x, w = synth.prefill_inputs(od, B, T, 31, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    tw = weights_to_dev(w, dt, DEV)
    rope = _rope(od, T)
    a = mla.mla_prefill(d, tw, to_dev(x, dt, DEV), rope).clone()
    for t in (0, 63, 64, 129):
        y = x.copy()
        y[:, t + 1:] = synth.bf16_round(y[:, t + 1:] * -1.5 + 0.25) if dt == "bf16" else y[:, t + 1:] * -1.5 + 0.25
        b = mla.mla_prefill(d, tw, to_dev(y, dt, DEV), rope)
        torch.cuda.synchronize()
        assert torch.equal(a[:, :t + 1], b[:, :t + 1]), f"t={t}"
        assert not torch.equal(a[:, t + 1:], b[:, t + 1:])


def test_prefill_deterministic():
    od = KIMI_NARROW
    x, w = synth.prefill_inputs(od, 1, 300, 41, bf16=True)
    d = dims_of(mla, od, "bf16")
    tw = weights_to_dev(w, "bf16", DEV)
    rope = _rope(od, 300)
    xd = to_dev(x, "bf16", DEV)
    a = mla.mla_prefill(d, tw, xd, rope).clone()
    for _ in range(3):
        assert torch.equal(a, mla.mla_prefill(d, tw, xd, rope))


# ------------------------------------------------------------------- decode
def _decode_full_case(od, B, P, L_cap, dt, seed, sample=None):
    x, w, kc, vc = synth.decode_full_inputs(od, B, P, L_cap, seed, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    kd, vd = bits_to_dev(kc, dt, DEV), bits_to_dev(vc, dt, DEV)
    got = mla.mla_decode_fullcache(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P, kd, vd,
                                   _rope(od, P + 1))
    torch.cuda.synchronize()
    bs = list(range(B)) if sample is None else sample
    kf = synth.as_f32(kc[bs], dt == "bf16").astype(np.float64)
    vf = synth.as_f32(vc[bs], dt == "bf16").astype(np.float64)
    want, kc2, vc2 = ref.mla_decode_fullcache(od, oracle_weights(w), x[bs].astype(np.float64), P, kf, vf)
    return from_dev(got)[bs], want, kd, vd, kc2, vc2, bs


@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, 3, 20, 24, "f32", 51),
    ("tiny_f32_P0", ref.TINY, 2, 0, 4, "f32", 52),
    ("kimi_narrow_bf16", KIMI_NARROW, 3, 300, 320, "bf16", 53),
    ("odd_widths_bf16", KIMI_ODD, 3, 150, 160, "bf16", 55),
    ("odd_widths_q576_bf16", KIMI_ODD576, 2, 90, 96, "bf16", 56),
    ("kimi_bf16_long", ref.KIMI_K2, 2, 5000, 5001, "bf16", 54),
])
def test_decode_fullcache(case):
    name, od, B, P, L_cap, dt, seed = case
    log(f"[decode full {name}] B={B} P={P} L_cap={L_cap} dtype={dt}")
    got, want, kd, vd, kc2, vc2, bs = _decode_full_case(od, B, P, L_cap, dt, seed)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(got, want, tol, name)
    # slot P now holds the new token's key and value; other slots untouched
    assert_close(from_dev(kd[:, :, P]), kc2[:, :, P], tol, "k_cache slot P")
    assert_close(from_dev(vd[:, :, P]), vc2[:, :, P], tol, "v_cache slot P")
    if P > 0:
        np.testing.assert_array_equal(from_dev(kd[:, :, :P]), kc2[:, :, :P])


def test_decode_fullcache_kimi_full_size_sampled():
    """The full-cache decode workload: B=64, P=1000 (L=1001 keys), bf16;
    oracle on a sample of sequences."""
    od = ref.KIMI_K2
    log("[decode full kimi] B=64 P=1000 bf16")
    got, want, *_ = _decode_full_case(od, 64, 1000, 1001, "bf16", 1003, sample=[0, 17, 63])
    assert_close(got, want, TOL_BF16, "decode full B=64 P=1000 sampled")


def _decode_latent_case(od, B, P, L_cap, dt, seed, sample=None, fn=None):
    x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, seed, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    cd = bits_to_dev(cc, dt, DEV)
    got = (fn or mla.mla_decode_latentcache)(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P, cd,
                                              _rope(od, P + 1))
    torch.cuda.synchronize()
    bs = list(range(B)) if sample is None else sample
    cf = synth.as_f32(cc[bs], dt == "bf16").astype(np.float64)
    want, cc2 = ref.mla_decode_latentcache(od, oracle_weights(w), x[bs].astype(np.float64), P, cf)
    return from_dev(got)[bs], want, cd, cc2, bs


@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, 3, 20, 24, "f32", 61),
    ("tiny_f32_P0", ref.TINY, 2, 0, 3, "f32", 62),
    ("kimi_narrow_bf16", KIMI_NARROW, 3, 700, 701, "bf16", 63),
    ("odd_widths_bf16", KIMI_ODD, 4, 260, 300, "bf16", 65),
    ("odd_widths_q576_bf16", KIMI_ODD576, 3, 130, 140, "bf16", 66),
    ("kimi_bf16_ragged", ref.KIMI_K2, 5, 333, 400, "bf16", 64),
])
def test_decode_latentcache(case):
    name, od, B, P, L_cap, dt, seed = case
    log(f"[decode latent {name}] B={B} P={P} L_cap={L_cap} dtype={dt}")
    got, want, cd, cc2, bs = _decode_latent_case(od, B, P, L_cap, dt, seed)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(got, want, tol, name)
    assert_close(from_dev(cd[:, P]), cc2[:, P], tol, "latent cache slot P")


def test_decode_latentcache_kimi_full_size_sampled():
    """The latent-cache decode workload: B=32, P=8192 (L=8193), bf16."""
    od = ref.KIMI_K2
    log("[decode latent kimi] B=32 P=8192 bf16")
    got, want, *_ = _decode_latent_case(od, 32, 8192, 8193, "bf16", 1004, sample=[0, 13, 31])
    assert_close(got, want, TOL_BF16, "decode latent B=32 P=8192 sampled")


# ---------------------------------------------- persistent latent decode
@pytest.mark.parametrize("case", [
    ("kimi_narrow", KIMI_NARROW, 3, 700, 701, 81, None),
    ("kimi_narrow_P0", KIMI_NARROW, 2, 0, 3, 82, None),
    ("kimi", ref.KIMI_K2, 5, 333, 400, 85, None),
    ("kimi_B33", ref.KIMI_K2, 33, 70, 96, 86, [0, 16, 31, 32]),   # 64-row weight-stream tiles
    ("kimi_B64", ref.KIMI_K2, 64, 40, 41, 87, [0, 31, 32, 63]),
])
def test_decode_latentcache_persistent(case):
    """The latent-cache decode as one persistent cooperative kernel: output
    and written cache slot against the oracle (sampled sequences for the
    large batches), no grid barrier gave up, a second call in the same
    workspace reproduces the output bit for bit, and the multi-launch step
    agrees within the bf16 tolerance (only the latent norms' reduction order
    differs)."""
    name, od, B, P, L_cap, seed, sample = case
    log(f"[decode latent persistent {name}] B={B} P={P} L_cap={L_cap} bf16")
    x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, seed, bf16=True)
    d = dims_of(mla, od, "bf16")
    wd, xd, rope = weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, P + 1)
    ws = torch.empty(mla.decode_workspace_size(d, B, L_cap), dtype=torch.uint8, device=DEV)
    cd = bits_to_dev(cc, "bf16", DEV)
    got = mla.mla_decode_latentcache_persistent(d, wd, xd, P, cd, rope, workspace=ws)
    torch.cuda.synchronize()
    assert mla.mla_decode_latentcache_persistent_status(d, B, L_cap, ws) == 0
    bs = list(range(B)) if sample is None else sample
    cf = synth.as_f32(cc[bs], True).astype(np.float64)
    want, cc2 = ref.mla_decode_latentcache(od, oracle_weights(w), x[bs].astype(np.float64), P, cf)
    assert_close(from_dev(got)[bs], want, TOL_BF16, name)
    assert_close(from_dev(cd[bs, P]), cc2[:, P], TOL_BF16, "latent cache slot P")
    got2 = mla.mla_decode_latentcache_persistent(d, wd, xd, P, cd, rope, workspace=ws)
    torch.cuda.synchronize()
    assert mla.mla_decode_latentcache_persistent_status(d, B, L_cap, ws) == 0
    assert torch.equal(got, got2), "second persistent call differs"
    multi = mla.mla_decode_latentcache(d, wd, xd, P, bits_to_dev(cc, "bf16", DEV), rope)
    torch.cuda.synchronize()
    assert_close(from_dev(got), from_dev(multi).astype(np.float64), TOL_BF16, "persistent vs multi-launch")


def test_decode_latentcache_persistent_kimi_full_size_sampled():
    """The latent-cache decode workload (B=32, P=8192, L=8193, bf16) through
    the persistent kernel, oracle on sampled sequences."""
    od = ref.KIMI_K2
    log("[decode latent persistent kimi] B=32 P=8192 bf16")
    got, want, *_ = _decode_latent_case(od, 32, 8192, 8193, "bf16", 1004, sample=[0, 13, 31],
                                        fn=mla.mla_decode_latentcache_persistent)
    assert_close(got, want, TOL_BF16, "persistent decode latent B=32 P=8192 sampled")


# ------------------------------------------------------------ ragged decode
def _pos_dev(positions):
    return torch.tensor(positions, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, [0, 3, 20, 9], 24, "f32", 71),
    ("kimi_narrow_bf16", KIMI_NARROW, [0, 1, 300, 127, 319], 320, "bf16", 72),
    ("odd_widths_bf16", KIMI_ODD, [3, 0, 150, 77], 160, "bf16", 74),
    ("kimi_bf16_splits", ref.KIMI_K2, [0, 4999, 2500], 5001, "bf16", 73),
])
def test_decode_fullcache_ragged(case):
    """Per-sequence positions with the full cache: each sequence against the
    oracle's decode at its own position, the written slot of each, and the
    cache rows past each position left untouched."""
    name, od, pos, L_cap, dt, seed = case
    B, P_max = len(pos), max(pos)
    log(f"[decode full ragged {name}] positions={pos} L_cap={L_cap} dtype={dt}")
    x, w, kc, vc = synth.decode_full_inputs(od, B, P_max, L_cap, seed, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    kd, vd = bits_to_dev(kc, dt, DEV), bits_to_dev(vc, dt, DEV)
    got = mla.mla_decode_fullcache_ragged(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), _pos_dev(pos),
                                          P_max, kd, vd, _rope(od, P_max + 1))
    torch.cuda.synchronize()
    kf = synth.as_f32(kc, dt == "bf16").astype(np.float64)
    vf = synth.as_f32(vc, dt == "bf16").astype(np.float64)
    want, kc2, vc2 = ref.mla_decode_fullcache_ragged(od, oracle_weights(w), x.astype(np.float64), pos, kf, vf)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(from_dev(got), want, tol, name)
    kdf, vdf = from_dev(kd), from_dev(vd)
    for b, P in enumerate(pos):
        assert_close(kdf[b, :, P], kc2[b, :, P], tol, f"{name} key slot {P}")
        assert_close(vdf[b, :, P], vc2[b, :, P], tol, f"{name} value slot {P}")
        if P + 1 < L_cap:
            np.testing.assert_array_equal(kdf[b, :, P + 1:], kf[b, :, P + 1:].astype(np.float32))


@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, [5, 0, 20], 24, "f32", 81),
    ("kimi_narrow_bf16", KIMI_NARROW, [0, 700, 31, 32], 701, "bf16", 82),
    ("odd_widths_bf16", KIMI_ODD, [0, 259, 64, 129], 300, "bf16", 85),
    ("kimi_bf16_splits", ref.KIMI_K2, [8192, 5, 4000], 8193, "bf16", 83),
    # 40 sequences, most of them a few tiles long and one of 94 tiles: the
    # split plan gives the long one many workgroups and leaves some idle;
    # 40 is not a multiple of the merge kernel's 8-sequence groups
    ("kimi_narrow_bf16_plan", KIMI_NARROW, [(37 * i) % 300 for i in range(39)] + [2999], 3000, "bf16", 84),
])
def test_decode_latentcache_ragged(case):
    name, od, pos, L_cap, dt, seed = case
    B, P_max = len(pos), max(pos)
    log(f"[decode latent ragged {name}] positions={pos} L_cap={L_cap} dtype={dt}")
    x, w, cc = synth.decode_latent_inputs(od, B, P_max, L_cap, seed, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    cd = bits_to_dev(cc, dt, DEV)
    got = mla.mla_decode_latentcache_ragged(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), _pos_dev(pos),
                                            P_max, cd, _rope(od, P_max + 1))
    torch.cuda.synchronize()
    cf = synth.as_f32(cc, dt == "bf16").astype(np.float64)
    want, cc2 = ref.mla_decode_latentcache_ragged(od, oracle_weights(w), x.astype(np.float64), pos, cf)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(from_dev(got), want, tol, name)
    cdf = from_dev(cd)
    for b, P in enumerate(pos):
        assert_close(cdf[b, P], cc2[b, P], tol, f"{name} latent slot {P}")


def test_decode_latentcache_max_batch():
    """The largest batch the bf16 latent decode serves, 1024 sequences: one
    length for all, then ragged positions in [0, 40] (the device split plan
    then gives every sequence one workgroup and fills its 1024-entry tables).
    Sequences are independent, so the oracle runs on a sample of them."""
    od = KIMI_NARROW
    log("[decode latent max batch] B=1024 P=40 L_cap=48 bf16 uniform")
    got, want, *_ = _decode_latent_case(od, 1024, 40, 48, "bf16", 95, sample=[0, 1, 511, 1000, 1023])
    assert_close(got, want, TOL_BF16, "decode latent B=1024 sampled")
    pos = [(7 * i) % 41 for i in range(1024)]
    log("[decode latent max batch] B=1024 ragged positions in [0, 40] L_cap=48 bf16")
    x, w, cc = synth.decode_latent_inputs(od, 1024, 40, 48, 96, bf16=True)
    cd = bits_to_dev(cc, "bf16", DEV)
    got = mla.mla_decode_latentcache_ragged(dims_of(mla, od, "bf16"), weights_to_dev(w, "bf16", DEV),
                                            to_dev(x, "bf16", DEV), _pos_dev(pos), 40, cd, _rope(od, 41))
    torch.cuda.synchronize()
    bs = [0, 5, 40, 41, 512, 1023]
    cf = synth.as_f32(cc[bs], True).astype(np.float64)
    want, cc2 = ref.mla_decode_latentcache_ragged(od, oracle_weights(w), x[bs].astype(np.float64),
                                                  [pos[b] for b in bs], cf)
    assert_close(from_dev(got)[bs], want, TOL_BF16, "decode latent ragged B=1024 sampled")
    cdf = from_dev(cd)
    for i, b in enumerate(bs):
        assert_close(cdf[b, pos[b]], cc2[i, pos[b]], TOL_BF16, f"latent slot {pos[b]} of sequence {b}")


@pytest.mark.parametrize("form", ["full", "latent"])
def test_ragged_decode_uniform_and_clamped(form):
    """Equal positions give the uniform entry point's result bit for bit;
    positions outside [0, P_max] act as the clamped positions."""
    od, B, P, L_cap, dt = KIMI_NARROW, 3, 40, 48, "bf16"
    log(f"[decode ragged uniform/clamp {form}]")
    d = dims_of(mla, od, dt)
    if form == "full":
        x, w, kc, vc = synth.decode_full_inputs(od, B, P, L_cap, 91, bf16=True)
        wd = weights_to_dev(w, dt, DEV)
        run_u = lambda: mla.mla_decode_fullcache(d, wd, to_dev(x, dt, DEV), P, bits_to_dev(kc, dt, DEV),
                                                 bits_to_dev(vc, dt, DEV), _rope(od, P + 1))
        run_r = lambda pos, pm: mla.mla_decode_fullcache_ragged(d, wd, to_dev(x, dt, DEV), _pos_dev(pos), pm,
                                                                bits_to_dev(kc, dt, DEV), bits_to_dev(vc, dt, DEV),
                                                                _rope(od, pm + 1))
    else:
        x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, 92, bf16=True)
        wd = weights_to_dev(w, dt, DEV)
        run_u = lambda: mla.mla_decode_latentcache(d, wd, to_dev(x, dt, DEV), P, bits_to_dev(cc, dt, DEV),
                                                   _rope(od, P + 1))
        run_r = lambda pos, pm: mla.mla_decode_latentcache_ragged(d, wd, to_dev(x, dt, DEV), _pos_dev(pos), pm,
                                                                  bits_to_dev(cc, dt, DEV), _rope(od, pm + 1))
    u = from_dev(run_u())
    r = from_dev(run_r([P] * B, P))
    np.testing.assert_array_equal(r, u)
    c1 = from_dev(run_r([P + 7, -5, 3], P))
    c2 = from_dev(run_r([P, 0, 3], P))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c1, c2)


# ---------------------------------------------------------- chunked prefill
@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, 2, 5, 9, 16, "f32", 111),
    ("kimi_narrow_bf16", KIMI_NARROW, 2, 100, 150, 300, "bf16", 112),
    ("odd_widths_bf16", KIMI_ODD, 1, 120, 170, 300, "bf16", 120),
    ("kimi_bf16", ref.KIMI_K2, 1, 300, 700, 1024, "bf16", 113),
    ("kimi_bf16_P0_0", ref.KIMI_K2, 1, 130, 0, 200, "bf16", 114),
    ("kimi_bf16_one_token", ref.KIMI_K2, 2, 1, 777, 800, "bf16", 115),
    # few query tiles against a long history: the attention splits each
    # (query tile, head)'s keys over 4, 2 and 2 workgroups
    ("kimi_bf16_keysplit4", ref.KIMI_K2, 1, 200, 2000, 2200, "bf16", 116),
    ("kimi_bf16_keysplit2", ref.KIMI_K2, 1, 300, 1700, 2000, "bf16", 117),
    ("kimi_bf16_keysplit_one_token", ref.KIMI_K2, 2, 1, 4000, 4001, "bf16", 118),
    # 512 rows: o_proj on 256 x 224 tiles in four fp32 K slices (256
    # workgroups), summed by reduce_splits
    ("kimi_bf16_T512", ref.KIMI_K2, 1, 512, 512, 1024, "bf16", 119),
])
@pytest.mark.parametrize("form", ["full", "latent"])
def test_prefill_chunk(case, form):
    """T new tokens at positions P0 .. P0+T-1 against a cache holding
    positions 0 .. P0-1: outputs and written cache slots against the oracle."""
    name, od, B, T, P0, L_cap, dt, seed = case
    log(f"[chunk {form} {name}] B={B} T={T} P0={P0} L_cap={L_cap} dtype={dt}")
    bf = dt == "bf16"
    x, w = synth.prefill_inputs(od, B, T, seed, bf16=bf)
    d = dims_of(mla, od, dt)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    if form == "full":
        _, _, kc, vc = synth.decode_full_inputs(od, B, max(P0, 1), L_cap, seed + 1, bf16=bf)
        kd, vd = bits_to_dev(kc, dt, DEV), bits_to_dev(vc, dt, DEV)
        got = mla.mla_prefill_chunk_fullcache(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P0, kd, vd,
                                              _rope(od, P0 + T))
        torch.cuda.synchronize()
        want, kc2, vc2 = ref.mla_prefill_chunk_fullcache(od, oracle_weights(w), x.astype(np.float64), P0,
                                                         synth.as_f32(kc, bf).astype(np.float64),
                                                         synth.as_f32(vc, bf).astype(np.float64))
        assert_close(from_dev(got), want, tol, name)
        assert_close(from_dev(kd)[:, :, P0:P0 + T], kc2[:, :, P0:P0 + T], tol, f"{name} key slots")
        assert_close(from_dev(vd)[:, :, P0:P0 + T], vc2[:, :, P0:P0 + T], tol, f"{name} value slots")
    else:
        _, _, cc = synth.decode_latent_inputs(od, B, max(P0, 1), L_cap, seed + 1, bf16=bf)
        cd = bits_to_dev(cc, dt, DEV)
        got = mla.mla_prefill_chunk_latentcache(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P0, cd,
                                                _rope(od, P0 + T))
        torch.cuda.synchronize()
        want, cc2 = ref.mla_prefill_chunk_latentcache(od, oracle_weights(w), x.astype(np.float64), P0,
                                                      synth.as_f32(cc, bf).astype(np.float64))
        assert_close(from_dev(got), want, tol, name)
        assert_close(from_dev(cd)[:, P0:P0 + T], cc2[:, P0:P0 + T], tol, f"{name} latent slots")


# --------------------------------------------------- attention_bias variant
def _with_biases(w, od, seed, bf16):
    return dict(w, **synth.attention_biases(od, np.random.default_rng(seed), bf16))


@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, 2, 37, "f32", 101),
    ("kimi_narrow_bf16", KIMI_NARROW, 2, 200, "bf16", 102),
    ("odd_widths_bf16", KIMI_ODD, 1, 90, "bf16", 104),
    ("kimi_bf16_T130", ref.KIMI_K2, 1, 130, "bf16", 103),
])
def test_prefill_attention_bias(case):
    """q_a_proj, kv_a_proj_with_mqa and o_proj biases (prefill, with both
    cache outputs)."""
    name, od, B, T, dt, seed = case
    log(f"[prefill bias {name}] B={B} T={T} dtype={dt}")
    x, w = synth.prefill_inputs(od, B, T, seed, bf16=(dt == "bf16"))
    w = _with_biases(w, od, seed + 1, dt == "bf16")
    want, p = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), return_intermediates=True)
    d = dims_of(mla, od, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    L_cap = T + 3
    lc = torch.zeros(B, L_cap, od.kv_lora_rank + od.qk_rope_dim, dtype=tdt, device=DEV)
    got = mla.mla_prefill(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), _rope(od, T), latent_cache=lc)
    torch.cuda.synchronize()
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(from_dev(got), want, tol, name)
    assert_close(from_dev(lc)[:, :T], ref.latent_cache_entries(od, p), tol, f"{name} latent cache")


def test_prefill_attention_bias_kimi_T1100_sampled_rows():
    """Biases at Kimi K2 widths above 1024 rows: o_proj takes the 256 x 224
    tiles (bias added in their staged epilogue, including the gathered
    strips 224..255 of each 256-column block) with a ragged last row tile
    (1100 = 4 x 256 + 76)."""
    od = ref.KIMI_K2
    B, T = 1, 1100
    log(f"[prefill bias kimi T=1100] B={B} T={T} bf16")
    x, w = synth.prefill_inputs(od, B, T, 1021, bf16=True)
    w = _with_biases(w, od, 1022, True)
    rows = sorted(set([0, 1, 255, 256, 1023, 1024, 1087, T - 1] +
                      list(np.random.default_rng(8).choice(T, 8, replace=False))))
    want = ref.mla_prefill(od, oracle_weights(w), x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.mla_prefill(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi prefill with biases T=1100 sampled rows")


def test_decode_latentcache_persistent_attention_bias():
    """The persistent latent decode with the attention_bias biases (q_a, kv_a
    and o_proj): the down-projection biases enter where the norm phase sums
    the row, b_o in the final split sum."""
    od = KIMI_NARROW
    B, P, L_cap, seed = 3, 30, 40, 108
    log(f"[decode bias persistent bf16] B={B} P={P}")
    d = dims_of(mla, od, "bf16")
    x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, seed, bf16=True)
    w = _with_biases(w, od, seed + 1, True)
    ws = torch.empty(mla.decode_workspace_size(d, B, L_cap), dtype=torch.uint8, device=DEV)
    got = mla.mla_decode_latentcache_persistent(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), P,
                                                bits_to_dev(cc, "bf16", DEV), _rope(od, P + 1), workspace=ws)
    torch.cuda.synchronize()
    assert mla.mla_decode_latentcache_persistent_status(d, B, L_cap, ws) == 0
    want, _ = ref.mla_decode_latentcache(od, oracle_weights(w), x.astype(np.float64), P,
                                         synth.as_f32(cc, True).astype(np.float64))
    assert_close(from_dev(got), want, TOL_BF16, "decode bias persistent bf16")


@pytest.mark.parametrize("form", ["full", "latent"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_attention_bias(form, dt):
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, P, L_cap, seed = 3, 30, 40, 104
    log(f"[decode bias {form} {dt}] B={B} P={P}")
    d = dims_of(mla, od, dt)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    if form == "full":
        x, w, kc, vc = synth.decode_full_inputs(od, B, P, L_cap, seed, bf16=(dt == "bf16"))
        w = _with_biases(w, od, seed + 1, dt == "bf16")
        got = mla.mla_decode_fullcache(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P,
                                       bits_to_dev(kc, dt, DEV), bits_to_dev(vc, dt, DEV), _rope(od, P + 1))
        want, _, _ = ref.mla_decode_fullcache(od, oracle_weights(w), x.astype(np.float64), P,
                                              synth.as_f32(kc, dt == "bf16").astype(np.float64),
                                              synth.as_f32(vc, dt == "bf16").astype(np.float64))
    else:
        x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, seed, bf16=(dt == "bf16"))
        w = _with_biases(w, od, seed + 1, dt == "bf16")
        got = mla.mla_decode_latentcache(d, weights_to_dev(w, dt, DEV), to_dev(x, dt, DEV), P,
                                         bits_to_dev(cc, dt, DEV), _rope(od, P + 1))
        want, _ = ref.mla_decode_latentcache(od, oracle_weights(w), x.astype(np.float64), P,
                                             synth.as_f32(cc, dt == "bf16").astype(np.float64))
    torch.cuda.synchronize()
    assert_close(from_dev(got), want, tol, f"decode bias {form} {dt}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dense_block_attention_bias(dt):
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, T, seed = 1, 70, 105
    log(f"[block bias {dt}] B={B} T={T}")
    x, w, blk = synth.block_inputs(od, B, T, seed, bf16=(dt == "bf16"))
    w = _with_biases(w, od, seed + 1, dt == "bf16")
    bw = ref.BlockWeights(attn=oracle_weights(w), **{k: np.asarray(v, np.float64) for k, v in blk.items()})
    want = ref.dense_block(od, bw, x.astype(np.float64))
    d = dims_of(mla, od, dt)
    got = mla.dense_block_fwd(d, weights_to_dev(w, dt, DEV), weights_to_dev(blk, dt, DEV),
                              to_dev(x, dt, DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got), want, TOL_F32 if dt == "f32" else TOL_BF16, f"block bias {dt}")


def _spike_scale(od, w, x_b, P, cf_b, pos, floor_rows):
    """Power of two that lifts row `pos`'s score, for its best head, at least
    12 (natural-log units) above every score in `floor_rows`; oracle steps."""
    pr = ref.mla_project(od, oracle_weights(w), x_b[None, None, :].astype(np.float64), np.array([P]))
    q_t = ref.absorbed_query(od, oracle_weights(w), pr["q_nope"][0, 0])       # [H, r]
    q_r = pr["q_rope"][0, 0]                                                    # [H, dr]
    r = od.kv_lora_rank
    S = (q_t @ cf_b[:, :r].T + q_r @ cf_b[:, r:].T) * od.softmax_scale          # [H, L]
    h = int(np.argmax(S[:, pos]))
    assert S[h, pos] > 0
    need = (S[h, floor_rows].max() + 12.0) / S[h, pos]
    return 2.0 ** int(np.ceil(np.log2(max(need, 1.0))))


def test_decode_latentcache_max_jump_restart():
    """Cache rows whose scores jump far above the running max after the first
    key tile of their split (B=32, L=1501: 192-key splits of 32-key tiles).
    The latent kernel raises a head's running max lazily and restarts the
    split when a later tile clears it by 2^16 in probability; rows at 230
    (sequence 0) and at 1000 then 1100 (sequence 5, two restarts) exercise
    that path.  Oracle on sequences 0, 5, 7."""
    od = ref.KIMI_K2
    B, P = 32, 1500
    log(f"[decode latent restart] B={B} P={P} bf16")
    x, w, cc = synth.decode_latent_inputs(od, B, P, P + 1, 1005, bf16=True)
    cf = synth.as_f32(cc, True).astype(np.float64)
    cf[:, P] = 0.0  # slot P is overwritten by the step; keep it out of the floor
    everything = np.arange(P)
    k0 = _spike_scale(od, w, x[0], P, cf[0], 230, everything)
    cc[0, 230] = synth.bf16_bits(cf[0, 230] * k0)
    k1 = _spike_scale(od, w, x[5], P, cf[5], 1000, everything)
    cc[5, 1000] = synth.bf16_bits(cf[5, 1000] * k1)
    cf5 = synth.as_f32(cc[5], True).astype(np.float64)
    cf5[1100] = cf5[1000]
    k2 = _spike_scale(od, w, x[5], P, cf5, 1100, np.arange(P)[np.arange(P) != 1100])
    cc[5, 1100] = synth.bf16_bits(cf5[1000] * k2)
    log(f"  spike scales {k0} {k1} {k2}")
    assert max(k0, k1, k2) <= 2.0 ** 12
    d = dims_of(mla, od, "bf16")
    cd = bits_to_dev(cc, "bf16", DEV)
    got = mla.mla_decode_latentcache(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), P, cd,
                                     _rope(od, P + 1))
    torch.cuda.synchronize()
    bs = [0, 5, 7]
    cfs = synth.as_f32(cc[bs], True).astype(np.float64)
    want, _ = ref.mla_decode_latentcache(od, oracle_weights(w), x[bs].astype(np.float64), P, cfs)
    assert_close(from_dev(got)[bs], want, TOL_BF16, "decode latent with score jumps")


# ------------------------------------------- online-softmax running-max raise
# The prefill attention keeps a running score maximum per (query, head) and,
# when a later key tile's scores clear it, rescales what it has accumulated
# (the online form of the float32 softmax in the code excerpt of "Kimi K2 ·
# Mix and project").  With the N(0,1) / N(0,0.02^2) inputs the first tile a
# query sees already holds its largest scores within a few units, so these
# cases plant keys whose scores jump far above everything before them.
RAISE_MARGIN = 8.0 * np.log(2.0)   # natural-log units; 8 in log2 units


def _late_raises(P, q_pos, tile=64):
    """(head, query, tile) events in the oracle probabilities P [H, Tq, Tk]
    where the best key of a key tile after the first outscores every earlier
    key by more than RAISE_MARGIN (scores differ as log-probabilities do)."""
    with np.errstate(divide="ignore"):
        lp = np.log(P)
    n = 0
    for qi, pos in enumerate(q_pos):
        run = lp[:, qi, :tile].max(-1)
        for t0 in range(tile, pos + 1, tile):
            tm = lp[:, qi, t0:min(t0 + tile, pos + 1)].max(-1)
            n += int(np.sum(tm > run + RAISE_MARGIN))
            run = np.maximum(run, tm)
    return n


def _scaled_bf16(a, k):
    """bf16 values times a power of two (exact)."""
    return synth.bf16_round(np.asarray(a, np.float32) * np.float32(k))


def test_prefill_running_max_raise():
    """Kimi K2 widths, B=1, T=1024: tokens 300 and 700 have their input
    scaled by 8 and 32.  Their latent and query paths pass an RMSNorm and do
    not change; their shared rotary key k^R = x W_KR grows with the input, so
    the scores of keys 300 and 700 jump far above the first key tile for
    many (query, head) pairs, in two steps for queries after 700.  Oracle on
    sampled rows; the oracle's own probabilities confirm the raises."""
    od = ref.KIMI_K2
    B, T = 1, 1024
    log(f"[prefill running-max raise] B={B} T={T} bf16")
    x, w = synth.prefill_inputs(od, B, T, 1021, bf16=True)
    x[0, 300] = _scaled_bf16(x[0, 300], 8.0)
    x[0, 700] = _scaled_bf16(x[0, 700], 32.0)
    rows = sorted(set([0, 299, 300, 301, 363, 511, 512, 699, 700, 701, 767, 768, 900, T - 1] +
                      list(np.random.default_rng(7).choice(T, 10, replace=False))))
    ow = oracle_weights(w)
    want = ref.mla_prefill(od, ow, x.astype(np.float64), rows=rows)
    p = ref.mla_project(od, ow, x.astype(np.float64), np.arange(T))
    chk = [r for r in rows if r >= 320]
    _, P = ref.attention(p["q_nope"][0, chk], p["q_rope"][0, chk], p["k_nope"][0], p["k_rope"][0],
                         p["v"][0], od.softmax_scale, np.asarray(chk), np.arange(T), return_probs=True)
    n = _late_raises(P, chk)
    log(f"  raise events in the sample: {n}")
    assert n >= 100
    d = dims_of(mla, od, "bf16")
    got = mla.mla_prefill(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "prefill with score jumps, sampled rows")


@pytest.mark.parametrize("form", ["full", "latent"])
def test_prefill_chunk_running_max_raise(form):
    """Chunked prefill, B=1, 200 new tokens after 2000 cached positions: the
    attention splits each query tile's keys over several workgroups whose
    partial maxima and sums are merged.  Cached keys 330, 771, 1320 and 1927
    (one inside each key split) are scaled by 16 (the whole key in the full
    cache; the rotary part of the latent entry, which leaves values alone),
    and new token 100 (position 2100) has its input scaled by 16."""
    od = ref.KIMI_K2
    B, T, P0, L_cap, seed = 1, 200, 2000, 2200, 131
    spikes = [330, 771, 1320, 1927]
    log(f"[chunk running-max raise {form}] B={B} T={T} P0={P0}")
    x, w = synth.prefill_inputs(od, B, T, seed, bf16=True)
    x[0, 100] = _scaled_bf16(x[0, 100], 16.0)
    ow = oracle_weights(w)
    d = dims_of(mla, od, "bf16")
    r = od.kv_lora_rank
    pos = P0 + np.arange(T)
    chk = list(range(100, T, 9))
    if form == "full":
        _, _, kc, vc = synth.decode_full_inputs(od, B, P0, L_cap, seed + 1, bf16=True)
        kf = synth.as_f32(kc, True)
        for j in spikes:
            kf[:, :, j] = _scaled_bf16(kf[:, :, j], 16.0)
        kc = synth.bf16_bits(kf)
        vf = synth.as_f32(vc, True).astype(np.float64)
        want, kc2, vc2 = ref.mla_prefill_chunk_fullcache(od, ow, x.astype(np.float64), P0,
                                                         kf.astype(np.float64), vf)
        p = ref.mla_project(od, ow, x.astype(np.float64), pos)
        qf = np.concatenate([p["q_nope"][0], p["q_rope"][0]], -1)[chk]          # [Tq,H,192]
        kk = kc2[0].transpose(1, 0, 2)                                          # [L,H,192]
        _, P = ref.attention(qf, qf[..., :0], kk, kk[:, 0, :0], vc2[0].transpose(1, 0, 2),
                             od.softmax_scale, pos[chk], np.arange(L_cap), return_probs=True)
        kd, vd = bits_to_dev(kc, "bf16", DEV), bits_to_dev(vc, "bf16", DEV)
        got = mla.mla_prefill_chunk_fullcache(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), P0,
                                              kd, vd, _rope(od, P0 + T))
    else:
        _, _, cc = synth.decode_latent_inputs(od, B, P0, L_cap, seed + 1, bf16=True)
        cf = synth.as_f32(cc, True)
        for j in spikes:
            cf[:, j, r:] = _scaled_bf16(cf[:, j, r:], 16.0)
        cc = synth.bf16_bits(cf)
        want, cc2 = ref.mla_prefill_chunk_latentcache(od, ow, x.astype(np.float64), P0, cf.astype(np.float64))
        p = ref.mla_project(od, ow, x.astype(np.float64), pos)
        qt = ref.absorbed_query(od, ow, p["q_nope"][0, chk])                    # [Tq,H,r]
        C = cc2[0]
        Cb = np.broadcast_to(C[:, None, :r], (L_cap, od.n_heads, r))
        _, P = ref.attention(qt, p["q_rope"][0, chk], Cb, C[:, r:], Cb, od.softmax_scale, pos[chk],
                             np.arange(L_cap), return_probs=True)
        cd = bits_to_dev(cc, "bf16", DEV)
        got = mla.mla_prefill_chunk_latentcache(d, weights_to_dev(w, "bf16", DEV), to_dev(x, "bf16", DEV), P0,
                                                cd, _rope(od, P0 + T))
    n = _late_raises(P, list(pos[chk]))
    log(f"  raise events in the sample: {n}")
    assert n >= 100
    torch.cuda.synchronize()
    assert_close(from_dev(got), want, TOL_BF16, f"chunk {form} with score jumps")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_absorbed_equals_full_on_gpu(dt):
    """Latent decode and full-cache decode over the cache expanded from the
    same latents agree (associativity), on the GPU."""
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, P, L_cap = 2, 90, 96
    log(f"[absorbed==full] dtype={dt}")
    x, w, cc = synth.decode_latent_inputs(od, B, P, L_cap, 71, bf16=(dt == "bf16"))
    cf = synth.as_f32(cc, dt == "bf16").astype(np.float64)
    r, H, dn = od.kv_lora_rank, od.n_heads, od.qk_nope_dim
    kv = (cf[..., :r] @ np.asarray(w["w_ukv"], np.float64).T).reshape(B, L_cap, H, -1)
    K = np.concatenate([kv[..., :dn], np.broadcast_to(cf[:, :, None, r:], (B, L_cap, H, od.qk_rope_dim))], -1)
    V = kv[..., dn:]
    K = synth.bf16_round(K.astype(np.float32)) if dt == "bf16" else K.astype(np.float32)
    V = synth.bf16_round(V.astype(np.float32)) if dt == "bf16" else V.astype(np.float32)
    d = dims_of(mla, od, dt)
    tw = weights_to_dev(w, dt, DEV)
    rope = _rope(od, P + 1)
    xd = to_dev(x, dt, DEV)
    ol = mla.mla_decode_latentcache(d, tw, xd, P, bits_to_dev(cc, dt, DEV), rope)
    kd = to_dev(np.ascontiguousarray(K.transpose(0, 2, 1, 3)), dt, DEV)
    vd = to_dev(np.ascontiguousarray(V.transpose(0, 2, 1, 3)), dt, DEV)
    of = mla.mla_decode_fullcache(d, tw, xd, P, kd, vd, rope)
    torch.cuda.synchronize()
    assert_close(from_dev(ol), from_dev(of), TOL_F32 if dt == "f32" else TOL_BF16, "absorbed vs full")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_last_row_equals_decode(dt):
    """Decode at P = T-1 over caches written by a (T-1)-token prefill equals
    the last row of a T-token prefill, for both cache forms (GPU only)."""
    od = ref.TINY if dt == "f32" else KIMI_NARROW
    B, T = 2, 66
    log(f"[prefill==decode] dtype={dt}")
    x, w = synth.prefill_inputs(od, B, T, 81, bf16=(dt == "bf16"))
    d = dims_of(mla, od, dt)
    tw = weights_to_dev(w, dt, DEV)
    rope = _rope(od, T)
    xd = to_dev(x, dt, DEV)
    full = mla.mla_prefill(d, tw, xd, rope)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kc = torch.zeros(B, od.n_heads, T, od.q_head_dim, dtype=tdt, device=DEV)
    vc = torch.zeros(B, od.n_heads, T, od.v_head_dim, dtype=tdt, device=DEV)
    lc = torch.zeros(B, T, od.kv_lora_rank + od.qk_rope_dim, dtype=tdt, device=DEV)
    mla.mla_prefill(d, tw, xd[:, :T - 1].contiguous(), rope, k_cache=kc, v_cache=vc, latent_cache=lc)
    xl = xd[:, T - 1].contiguous()
    of = mla.mla_decode_fullcache(d, tw, xl, T - 1, kc, vc, rope)
    ol = mla.mla_decode_latentcache(d, tw, xl, T - 1, lc, rope)
    torch.cuda.synchronize()
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(from_dev(of), from_dev(full[:, -1]), tol, "full-cache decode vs prefill last row")
    assert_close(from_dev(ol), from_dev(full[:, -1]), tol, "latent decode vs prefill last row")


# -------------------------------------------------------------------- block
@pytest.mark.parametrize("case", [
    ("tiny_f32", ref.TINY, 2, 19, "f32", 91),
    ("kimi_narrow_bf16", KIMI_NARROW, 1, 150, "bf16", 92),
    ("odd_widths_bf16", KIMI_ODD, 1, 140, "bf16", 93),
])
def test_dense_block(case):
    name, od, B, T, dt, seed = case
    log(f"[block {name}] B={B} T={T} dtype={dt}")
    x, w, blk = synth.block_inputs(od, B, T, seed, bf16=(dt == "bf16"))
    bw = ref.BlockWeights(attn=oracle_weights(w), **{k: np.asarray(v, np.float64) for k, v in blk.items()})
    want = ref.dense_block(od, bw, x.astype(np.float64))
    d = dims_of(mla, od, dt)
    got = mla.dense_block_fwd(d, weights_to_dev(w, dt, DEV), weights_to_dev(blk, dt, DEV),
                              to_dev(x, dt, DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got), want, TOL_F32 if dt == "f32" else TOL_BF16, name)


def test_dense_block_kimi_sampled_rows():
    """Kimi K2 block widths (d_ff 18432) at T=256, sampled rows."""
    od = ref.KIMI_K2
    B, T = 1, 256
    log(f"[block kimi] B={B} T={T} bf16")
    x, w, blk = synth.block_inputs(od, B, T, 1005, bf16=True)
    rows = [0, 1, 100, 128, 200, T - 1]
    bw = ref.BlockWeights(attn=oracle_weights(w), **{k: np.asarray(v, np.float64) for k, v in blk.items()})
    want = ref.dense_block(od, bw, x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.dense_block_fwd(d, weights_to_dev(w, "bf16", DEV), weights_to_dev(blk, "bf16", DEV),
                              to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi block sampled rows")


def test_dense_block_kimi_T2048_sampled_rows():
    """Kimi K2 block at T=2048: o_proj and W2 on the 256 x 224 tiles (256 of
    them, seven 32-column strips each) with the residual epilogue."""
    od = ref.KIMI_K2
    B, T = 1, 2048
    log(f"[block kimi T=2048] B={B} T={T} bf16")
    x, w, blk = synth.block_inputs(od, B, T, 1015, bf16=True)
    rows = [0, 1, 255, 256, 1000, 1791, 2046, T - 1]
    bw = ref.BlockWeights(attn=oracle_weights(w), **{k: np.asarray(v, np.float64) for k, v in blk.items()})
    want = ref.dense_block(od, bw, x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.dense_block_fwd(d, weights_to_dev(w, "bf16", DEV), weights_to_dev(blk, "bf16", DEV),
                              to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi block T=2048 sampled rows")


def test_dense_block_kimi_T4096_sampled_rows():
    """The dense block workload itself (B=1, T=4096, Kimi K2 widths, d_ff
    18432) in the launch configuration the benchmark times: 16 query tiles
    per head in the attention, 448 output tiles in o_proj and W2.  The
    oracle computes every key/value and a sample of rows (tile edges, the
    last rows and random ones)."""
    od = ref.KIMI_K2
    B, T = 1, 4096
    log(f"[block kimi T=4096] B={B} T={T} bf16")
    x, w, blk = synth.block_inputs(od, B, T, 1025, bf16=True)
    rows = sorted(set([0, 1, 255, 256, 1023, 2047, 2048, 3071, 3072, 3583, 3840, 4000, T - 2, T - 1] +
                      list(np.random.default_rng(8).choice(T, 10, replace=False))))
    bw = ref.BlockWeights(attn=oracle_weights(w), **{k: np.asarray(v, np.float64) for k, v in blk.items()})
    want = ref.dense_block(od, bw, x.astype(np.float64), rows=rows)
    d = dims_of(mla, od, "bf16")
    got = mla.dense_block_fwd(d, weights_to_dev(w, "bf16", DEV), weights_to_dev(blk, "bf16", DEV),
                              to_dev(x, "bf16", DEV), _rope(od, T))
    torch.cuda.synchronize()
    assert_close(from_dev(got)[:, rows], want, TOL_BF16, "kimi block T=4096 sampled rows")


def test_rope_table_matches_definition():
    """The device-built table against the oracle's float64 angles (float32 storage)."""
    c, s = mla.mla_rope_table(8192, 64, 10000.0, DEV)
    oc, os_ = ref.rope_angles(np.arange(8192), 64, 10000.0)
    torch.cuda.synchronize()
    assert np.max(np.abs(c.cpu().numpy() - oc)) < 1e-6
    assert np.max(np.abs(s.cpu().numpy() - os_)) < 1e-6
