"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer outputs (codes, packed words, alpha*) and float32 quantiser outputs
(activation magnitudes, scales s, steps) must match bit for bit; per-alpha
losses within 1e-4 relative; W4A16 outputs within 2e-3 * max|Y|.
Sizes here are small enough for the oracle to finish in seconds but span
several 256x256 tiles and ragged tails.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import GEMM_TOL, LOSS_RTOL, dev_tensor, gemm_tolerance, say, tie_band
from weight_only_quantization_awq_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_quantization_awq_amd import awq as mod
    return mod


# ------------------------------------------------------------ act_stats ----

# the main kernel takes 1, 2, 4 or 8 column runs per workgroup (at least 128
# workgroups); the last four shapes give 8, 8, 8 and 2 with a ragged last workgroup
@pytest.mark.parametrize("N,D_in,dtype", [(1, 8, "f32"), (128, 256, "f32"), (300, 384, "bf16"),
                                          (77, 1000, "bf16"), (4096, 130, "bf16"), (33, 65, "f32"),
                                          (2000, 264, "bf16"), (1500, 100, "f32"), (300, 4104, "bf16"),
                                          (100, 4100, "f32"), (64, 16392, "bf16"), (300, 3000, "bf16")])
def test_act_stats_bit_exact(awq, N, D_in, dtype):
    say("act_stats", N, D_in, dtype)
    case = synth.make_layer(N, max(D_in, 8), 8, seed=N + D_in, dtype=dtype, n_salient=2, salient_lo=30.0)
    X = case.X[:, :D_in].copy()
    a = awq.act_stats(dev_tensor(X, dtype)).cpu().numpy()
    torch.cuda.synchronize()
    want = oracle.act_stats(X)
    assert np.array_equal(a, want), np.flatnonzero(a != want)[:10]


@pytest.mark.parametrize("N,D_in,dtype", [(1, 8, "f32"), (300, 384, "bf16"), (77, 1000, "bf16"),
                                          (4096, 130, "bf16"), (33, 65, "f32"), (2000, 264, "bf16"),
                                          (1030, 8200, "bf16")])
def test_act_stats_max_bit_exact(awq, N, D_in, dtype):
    say("act_stats max", N, D_in, dtype)
    case = synth.make_layer(N, max(D_in, 8), 8, seed=N + D_in + 1, dtype=dtype, n_salient=2, salient_lo=30.0)
    X = case.X[:, :D_in].copy()
    a = awq.act_stats(dev_tensor(X, dtype), statistic="max").cpu().numpy()
    torch.cuda.synchronize()
    want = oracle.act_stats(X, "max")
    assert np.array_equal(a, want), np.flatnonzero(a != want)[:10]


def test_act_stats_max_nan(awq):
    say("act_stats max nan")
    X = np.ones((50, 16), np.float32)
    X[17, 3] = np.nan
    X[40, 9] = -7.0
    a = awq.act_stats(dev_tensor(X, "f32"), statistic="max").cpu().numpy()
    torch.cuda.synchronize()
    assert np.isnan(a[3]) and a[9] == 7.0
    assert np.array_equal(np.delete(a, 3), np.delete(oracle.act_stats(X, "max"), 3))


@pytest.mark.parametrize("D_in,D_out,dtype", [(1, 1, "f32"), (256, 256, "bf16"), (384, 520, "f32"),
                                               (96, 28672, "bf16"), (4096, 300, "bf16"), (7, 1029, "f32")])
def test_weight_stats_bit_exact(awq, D_in, D_out, dtype):
    say("weight_stats", D_in, D_out, dtype)
    rng = np.random.default_rng(D_in * 7 + D_out)
    W = (rng.standard_normal((D_in, D_out), dtype=np.float32) * 0.02).astype(np.float32)
    W[0, :] = 0.0                                   # an all-zero row
    if dtype == "bf16":
        W = synth.to_bf16_values(W)
    b = awq.weight_stats(dev_tensor(W, dtype)).cpu().numpy()
    torch.cuda.synchronize()
    want = oracle.weight_stats(W)
    assert np.array_equal(b, want), np.flatnonzero(b != want)[:10]


# ---------------------------------------------------------------- search ----

SEARCH_CASES = [
    # name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal
    ("bf16_ragged", 300, 384, 520, "bf16", 4, 128, "salient", 4),
    ("bf16_heavy", 512, 512, 300, "bf16", 4, 128, "heavy", 0),
    ("bf16_int3_g64", 200, 256, 264, "bf16", 3, 64, "salient", 3),
    ("f32_cfg1_shape", 128, 256, 256, "f32", 4, 128, "salient", 3),
    ("f32_g32_int3", 70, 96, 40, "f32", 3, 32, "heavy", 0),
    ("bf16_g8_int2", 17, 64, 12, "bf16", 2, 8, "salient", 1),
    ("bf16_one_row", 1, 128, 36, "bf16", 4, 128, "salient", 1),
    ("bf16_int8", 64, 256, 48, "bf16", 8, 128, "heavy", 0),
    ("bf16_336_tiles", 1024, 512, 1024, "bf16", 4, 128, "salient", 8),
    # 9 row tiles x 6 column tiles of 256: a one-tile second row block and a
    # two-tile last column group in the contraction's tile walk
    ("bf16_rows9_cols6", 2300, 512, 1300, "bf16", 4, 128, "salient", 6),
    # D_in >= 2048: bf16 matrix cores with the 64 correction rows
    ("bf16c_ragged", 300, 2048, 520, "bf16", 4, 128, "salient", 6),
    ("bf16c_int3_g64", 400, 2112, 300, "bf16", 3, 64, "salient", 8),
    ("bf16c_heavy_g256", 256, 2304, 600, "bf16", 4, 256, "heavy", 0),
    ("bf16c_g96", 300, 2112, 300, "bf16", 4, 96, "salient", 4),
    # group-size sweep (32 / 64 / 256) on one shape
    ("bf16_g256", 600, 1024, 520, "bf16", 4, 256, "salient", 6),
    ("bf16_g32_sweep", 600, 1024, 520, "bf16", 4, 32, "salient", 6),
    ("bf16_g64_sweep", 600, 1024, 520, "bf16", 4, 64, "salient", 6),
    ("f32_g256_int3", 100, 768, 136, "f32", 3, 256, "heavy", 0),
    ("bf16_g256_cols100", 64, 512, 100, "bf16", 4, 256, "salient", 2),
]


def _matrix(name):
    """Cases named "...bf16c..." force the bf16 matrix path (with its 64
    correction rows), which the size rule picks only for layers of at least
    2^39 multiply-adds per alpha."""
    return "bf16" if "bf16c" in name else None


def _run_search(awq, case, alphas, want_codes=True, matrix=None):
    X = dev_tensor(case.X, case.dtype)
    W = dev_tensor(case.W, case.dtype)
    a = awq.act_stats(X)
    r = awq.search_layer(X, W, alphas=alphas, bits=case.bits, group=case.group, a=a, want_codes=want_codes,
                         matrix=matrix)
    torch.cuda.synchronize()
    return r, a.cpu().numpy()


@pytest.mark.parametrize("spec", SEARCH_CASES, ids=[c[0] for c in SEARCH_CASES])
def test_search_matches_oracle(awq, spec):
    name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal = spec
    say("search", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits, group=group,
                            x_kind=x_kind, n_salient=n_sal, salient_lo=10.0, salient_hi=100.0)
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True)
    r, a = _run_search(awq, case, case.alphas, matrix=_matrix(name))
    assert np.array_equal(a, ref["a"])
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / np.maximum(ref["losses"], 1e-300)
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    b = r.best_index()
    band = tie_band(ref["losses"])
    assert b == ref["best"] or (len(band) > 1 and b in band), (b, ref["best"], band)
    # quantiser outputs at the GPU's alpha must match the oracle's at that alpha bit for bit
    assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][b])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][b])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][b])


@pytest.mark.parametrize("n_sal,factor", [(1, 1000.0), (4, 100.0)])
def test_search_dominant_channels_bf16_path(awq, n_sal, factor):
    """A layer whose activation energy sits in one or a few channels, on the
    bf16 matrix-core path (D_in >= 2048): without the correction rows of the
    64 largest channels, bf16 rounding of their error weights alone moves
    L(alpha) by up to about 2e-4 on such layers (CPU emulation from the
    oracle's codes); with them the losses stay within the 1e-4 tolerance."""
    say("search dominant channels", n_sal, factor)
    case = synth.make_layer(512, 2048, 1024, seed=310 + n_sal, dtype="bf16", n_salient=n_sal, salient_lo=factor,
                            salient_hi=factor, w_std=0.02)
    ref = oracle.search_layer(case.X, case.W, case.alphas, 4, 128, keep_all=True)
    r, a = _run_search(awq, case, case.alphas, matrix="bf16")
    assert np.array_equal(a, ref["a"])
    rel = np.abs(r.losses.cpu().numpy() - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    b = r.best_index()
    assert b == ref["best"] or b in tie_band(ref["losses"])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][b])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][b])


@pytest.mark.parametrize("kind", ["dead", "equal"])
def test_search_bf16_path_tied_statistics(awq, kind):
    """Correction-row selection on ties: all but 10 channels dead (2038
    equal statistics of 0 fill the 64 rows, lowest indices first), or 40
    distinct dominant channels (x80) above 40 identical ones (x50), of which
    the 24 lowest-indexed take the remaining rows.  The search is
    repeated and must give the same losses bit for bit; the losses stay
    within tolerance of the oracle and the codes and steps at the chosen
    alpha match it."""
    say("search bf16 path tied statistics", kind)
    case = synth.make_layer(256, 2048, 520, seed=91, dtype="bf16", n_salient=0, w_std=0.02)
    X = case.X.copy()
    if kind == "dead":
        X[:, 10:] = 0.0
    else:
        X[:, 100:140] = synth.to_bf16_values(X[:, 400:440] * 80.0)
        X[:, 300:340] = synth.to_bf16_values(X[:, [7]] * 50.0)
    c2 = synth.LayerCase("ties", X, case.W, "bf16", 4, 128, case.alphas)
    ref = oracle.search_layer(X, case.W, c2.alphas, 4, 128, keep_all=True)
    r1, a = _run_search(awq, c2, c2.alphas, matrix="bf16")
    r2, _ = _run_search(awq, c2, c2.alphas, matrix="bf16")
    assert np.array_equal(a, ref["a"])
    l1, l2 = r1.losses.cpu().numpy(), r2.losses.cpu().numpy()
    assert np.array_equal(l1, l2)
    rel = np.abs(l1 - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    b = r1.best_index()
    assert b == ref["best"] or b in tie_band(ref["losses"])
    assert np.array_equal(r1.codes.cpu().numpy(), ref["codes_all"][b])
    assert np.array_equal(r1.scales.cpu().numpy(), ref["scales_all"][b])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_search_64_alphas(awq, dtype):
    """The largest grid (64 points, split into alpha slices by the quantiser
    launch with a ragged last slice): every loss against the oracle, the
    quantiser at the GPU's alpha bit for bit, and the losses of the 21 points
    it shares with the default grid identical to a 21-point search."""
    say("search 64 alphas", dtype)
    case = synth.make_layer(300, 384, 520, seed=64, dtype=dtype, bits=4, group=128, x_kind="salient", n_salient=4,
                            salient_lo=10.0, salient_hi=100.0)
    extra = np.random.default_rng(640).uniform(0.0, 1.0, 43).astype(np.float32)
    alphas = np.concatenate([case.alphas.astype(np.float32), extra])
    ref = oracle.search_layer(case.X, case.W, alphas, 4, 128, keep_all=True)
    r64, a = _run_search(awq, case, alphas)
    r21, _ = _run_search(awq, case, case.alphas)
    l64 = r64.losses.cpu().numpy()
    rel = np.abs(l64 - ref["losses"]) / np.maximum(ref["losses"], 1e-300)
    assert rel.max() <= LOSS_RTOL, (rel.max(), int(rel.argmax()))
    assert np.array_equal(l64[:len(case.alphas)], r21.losses.cpu().numpy())
    b = r64.best_index()
    band = tie_band(ref["losses"])
    assert b == ref["best"] or (len(band) > 1 and b in band), (b, ref["best"], band)
    assert np.array_equal(r64.scales.cpu().numpy(), ref["scales_all"][b])
    assert np.array_equal(r64.codes.cpu().numpy(), ref["codes_all"][b])


@pytest.mark.parametrize("spec", SEARCH_CASES[:4], ids=[c[0] for c in SEARCH_CASES[:4]])
def test_quantiser_every_alpha(awq, spec):
    """Codes, steps and s at every grid point (single-point grids)."""
    name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal = spec
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits, group=group,
                            x_kind=x_kind, n_salient=n_sal, salient_lo=10.0, salient_hi=100.0)
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True)
    X = dev_tensor(case.X, dtype)
    W = dev_tensor(case.W, dtype)
    a = awq.act_stats(X)
    for k, al in enumerate(case.alphas):
        say("quantiser", name, "alpha", float(al))
        r = awq.search_layer(X, W, alphas=np.array([al], np.float32), bits=bits, group=group, a=a)
        torch.cuda.synchronize()
        assert r.best_index() == 0
        assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][k]), k
        assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][k]), k
        assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][k]), k
        got = float(r.losses.cpu().numpy()[0])
        assert abs(got - ref["losses"][k]) <= LOSS_RTOL * ref["losses"][k], (k, got, ref["losses"][k])


WSCALE_CASES = [
    # name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal, statistic
    ("w_bf16_ragged", 300, 384, 520, "bf16", 4, 128, "salient", 4, "mean"),
    ("w_f32_int3_g32", 70, 96, 40, "f32", 3, 32, "heavy", 0, "mean"),
    ("w_bf16_tiles_max", 1024, 512, 1024, "bf16", 4, 128, "salient", 8, "max"),
    ("max_bf16_heavy", 512, 512, 300, "bf16", 4, 128, "heavy", 0, "max"),
    ("w_bf16c_ragged", 300, 2048, 520, "bf16", 4, 128, "salient", 4, "mean"),
    ("max_bf16c_heavy", 256, 2048, 600, "bf16", 4, 128, "heavy", 0, "max"),
]


@pytest.mark.parametrize("spec", WSCALE_CASES, ids=[c[0] for c in WSCALE_CASES])
def test_search_statistic_variants(awq, spec):
    """The max statistic and the weight-term candidates a^α / b^(1−α)."""
    name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal, stat = spec
    say("search variant", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits,
                            group=group, x_kind=x_kind, n_salient=n_sal, salient_lo=10.0, salient_hi=100.0)
    weighted = name.startswith("w_")
    a_ref = oracle.act_stats(case.X, stat)
    b_ref = oracle.weight_stats(case.W) if weighted else None
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True, a=a_ref, b=b_ref)
    X = dev_tensor(case.X, dtype)
    W = dev_tensor(case.W, dtype)
    a = awq.act_stats(X, statistic=stat)
    b = awq.weight_stats(W) if weighted else None
    r = awq.search_layer(X, W, alphas=case.alphas, bits=bits, group=group, a=a, b=b, matrix=_matrix(name))
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), a_ref)
    if weighted:
        assert np.array_equal(b.cpu().numpy(), b_ref)
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / np.maximum(ref["losses"], 1e-300)
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    k = r.best_index()
    band = tie_band(ref["losses"])
    assert k == ref["best"] or (len(band) > 1 and k in band), (k, ref["best"], band)
    assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][k])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][k])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][k])


def test_weighted_search_dead_weight_row(awq):
    """A zero weight row (b_j = 0) keeps s_j = 1 at every alpha."""
    say("weighted search dead row")
    case = synth.make_layer(64, 256, 40, seed=9, dtype="f32", n_salient=2, salient_lo=20.0)
    W = case.W.copy()
    W[5, :] = 0.0
    b_ref = oracle.weight_stats(W)
    a_ref = oracle.act_stats(case.X)
    Xd, Wd = dev_tensor(case.X, "f32"), dev_tensor(W, "f32")
    a, b = awq.act_stats(Xd), awq.weight_stats(Wd)
    for al in (0.0, 0.35, 1.0):
        r = awq.search_layer(Xd, Wd, alphas=np.array([al], np.float32), bits=4, group=128, a=a, b=b)
        torch.cuda.synchronize()
        s_ref = oracle.scales_for_alpha(a_ref, al, b_ref)
        assert s_ref[5] == 1.0
        assert np.array_equal(r.s_best.cpu().numpy(), s_ref)


def test_search_edge_cases(awq):
    """Dead channel (a_j = 0), all-zero group, D_in == group, single column."""
    say("search edge cases")
    case = synth.make_layer(40, 256, 20, seed=5, dtype="bf16", n_salient=2, salient_lo=40.0)
    X = case.X.copy()
    W = case.W.copy()
    X[:, 7] = 0.0                 # dead channel -> s = 1
    W[128:256, 3] = 0.0           # all-zero group -> step 0, codes 0
    c2 = synth.LayerCase("edge", X, W, "bf16", 4, 128, case.alphas)
    ref = oracle.search_layer(X, W, c2.alphas, 4, 128, keep_all=True)
    r, a = _run_search(awq, c2, c2.alphas)
    assert a[7] == 0.0
    b = r.best_index()
    assert b in tie_band(ref["losses"])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][b])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][b])
    assert r.scales.cpu().numpy()[1, 3] == 0.0
    assert r.s_best.cpu().numpy()[7] == 1.0
    rel = np.abs(r.losses.cpu().numpy() - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL
    # D_in == group, one output column
    c3 = synth.make_layer(50, 128, 1, seed=6, dtype="bf16", n_salient=1, salient_lo=20.0)
    ref3 = oracle.search_layer(c3.X, c3.W, c3.alphas, 4, 128, keep_all=True)
    r3, _ = _run_search(awq, c3, c3.alphas)
    b3 = r3.best_index()
    assert b3 in tie_band(ref3["losses"])
    assert np.array_equal(r3.codes.cpu().numpy(), ref3["codes_all"][b3])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_search_denormal_weights(awq, dtype):
    """Subnormal weights: a group of only subnormals (subnormal steps) and a
    group mixing one normal weight with subnormals (codes 0 beside it)."""
    say("search denormal weights", dtype)
    case = synth.make_layer(64, 256, 48, seed=13, dtype=dtype, n_salient=2, salient_lo=20.0)
    W = case.W.copy()
    rng = np.random.default_rng(14)
    W[0:128, 5] = (rng.standard_normal(128) * 1e-39).astype(np.float32)     # all subnormal
    W[128:256, 9] = (rng.standard_normal(128) * 1e-40).astype(np.float32)   # subnormal ...
    W[130, 9] = np.float32(0.03)                                             # ... with one normal weight
    if dtype == "bf16":
        W = synth.to_bf16_values(W)
    assert np.count_nonzero((np.abs(W) < np.finfo(np.float32).tiny) & (W != 0)) > 100
    c = synth.LayerCase("denormal", case.X, W, dtype, 4, 128, case.alphas)
    ref = oracle.search_layer(case.X, W, c.alphas, 4, 128, keep_all=True)
    r, _ = _run_search(awq, c, c.alphas)
    b = r.best_index()
    assert b in tie_band(ref["losses"])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][b])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][b])
    assert 0.0 < r.scales.cpu().numpy()[0, 5] < np.finfo(np.float32).tiny   # a subnormal step
    rel = np.abs(r.losses.cpu().numpy() - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL


def test_search_nonfinite_reports(awq):
    say("search non-finite")
    case = synth.make_layer(32, 128, 16, seed=9, dtype="f32")
    X = case.X.copy()
    X[3, 5] = np.inf
    c = synth.LayerCase("inf", X, case.W, "f32", 4, 128, case.alphas)
    r, _ = _run_search(awq, c, c.alphas)
    with pytest.raises(awq.AwqNonFinite):
        r.best_index()


def test_search_repeatable(awq):
    """Fixed-order reductions: two runs give identical bits."""
    say("search repeatable")
    case = synth.make_layer(300, 384, 520, seed=3, dtype="bf16", n_salient=4, salient_lo=10.0, salient_hi=100.0)
    r1, _ = _run_search(awq, case, case.alphas)
    r2, _ = _run_search(awq, case, case.alphas)
    assert np.array_equal(r1.losses.cpu().numpy(), r2.losses.cpu().numpy())
    assert np.array_equal(r1.codes.cpu().numpy(), r2.codes.cpu().numpy())


# ------------------------------------------------------------------ pack ----

@pytest.mark.parametrize("D_in,D_out,bits", [(8, 1, 4), (64, 33, 4), (256, 520, 3), (128, 4, 2), (1024, 1000, 4)])
def test_pack_bit_exact(awq, D_in, D_out, bits):
    say("pack", D_in, D_out, bits)
    qmax = 2 ** (bits - 1) - 1
    rng = np.random.default_rng(D_in * 7 + D_out)
    q = rng.integers(-qmax, qmax + 1, (D_in, D_out)).astype(np.int8)
    got = awq.pack(torch.from_numpy(q).cuda(), bits=bits).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.pack_int4(q))


# ------------------------------------------------------------------ gemm ----

GEMM_CASES = [
    # M, D_in, D_out, group, inv, out
    (1, 256, 64, 128, False, "f32"),
    (1, 1024, 520, 128, True, "f32"),
    (5, 512, 300, 64, True, "bf16"),
    (8, 384, 132, 128, False, "f32"),
    (16, 256, 256, 32, True, "f32"),
    (17, 512, 196, 128, True, "f32"),
    (32, 1024, 512, 128, True, "bf16"),
    (33, 256, 100, 256, False, "f32"),
    (64, 512, 128, 128, True, "f32"),
    (100, 256, 72, 128, True, "f32"),
    # long k: the k axis is split across workgroups (float32 partials, summed in split order)
    (1, 4096, 512, 128, True, "f32"),
    (8, 8192, 1000, 128, False, "bf16"),
    (40, 2048, 264, 64, True, "f32"),      # a 32-row pass split 2 ways and an 8-row split pass
    (1, 14336, 256, 128, True, "f32"),     # two batches in flight per wave, k split 8 ways
    (2, 6144, 1024, 128, True, "bf16"),    # the same, split 4 ways
    (36, 8192, 520, 128, True, "f32"),     # a 32-row pass split 8 ways, then a pipelined 4-row pass split 8 ways
    (32, 4096, 512, 128, True, "bf16"),    # one 32-row pass split 4 ways
    (27, 6144, 2056, 256, False, "f32"),   # a 27-row pass split 4 ways, ragged last strip
    (6, 8192, 8200, 128, True, "f32"),     # over 2^26 weights: pre-pass, pipelined, split 2 ways
    # wide layers: many 64-column workgroups, ragged last one
    (1, 1024, 8192, 128, True, "f32"),
    (20, 512, 16396, 128, True, "f32"),
    (5, 256, 65536, 256, False, "f32"),
    (3, 512, 40000, 128, True, "bf16"),
    # two 64-column strips per wave (>= 12 rows, >= 192 workgroups of 128
    # columns, groups of 128 or more); ragged last workgroups where the second
    # strip lies wholly (24600) or partly (30000) past the last column
    (13, 256, 24600, 128, True, "bf16"),
    (1, 2048, 24704, 128, True, "bf16"),   # staged activations, two strips
    (2, 1024, 30000, 256, False, "f32"),   # the same, 2 rows, ragged
    (7, 512, 24640, 128, True, "f32"),     # staged activations, two strips, 7 rows
    (8, 1024, 24576, 128, True, "bf16"),   # the same, 8 rows (the most that stage)
    (7, 9088, 24576, 128, True, "f32"),    # 7 rows staged in two rounds, the second partial
    (2, 16768, 24704, 128, False, "f32"),  # 2 rows staged in three rounds, no inv_s
    (9, 2816, 24576, 128, True, "f32"),    # ring-staged activations, 9 rows, last 1024-k chunk partial
    (24, 2816, 24576, 128, True, "bf16"),  # pre-pass activations, two row tiles, two strips
    (17, 1024, 24704, 128, False, "f32"),  # the same, no inv_s, ragged last workgroup
    (16, 256, 24576, 128, False, "bf16"),  # ring, one chunk of two batches: six waves without one
    (10, 9216, 24704, 256, True, "f32"),   # ring, nine chunks (an odd count), group 256
    (5, 8192, 24576, 128, True, "bf16"),   # staged activations, two strips, 5 rows of 8192
    (5, 2048, 30000, 256, False, "f32"),   # the same, ragged
    (16, 1024, 24576, 256, False, "f32"),
    (29, 512, 24704, 256, True, "f32"),
    (32, 1024, 30000, 128, False, "bf16"),
    (44, 256, 24832, 128, True, "f32"),    # a 32-row and a 12-row pass, both with two strips
    (40, 256, 24576, 128, True, "f32"),    # a 32-row pass with two strips, an 8-row pass with one
    # prefill shapes (M >= 192, >= 64 tiles of 256 x 256): the matrix-core product
    (300, 512, 8200, 128, True, "f32"),    # ragged rows and columns
    (1030, 1056, 4100, 32, False, "bf16"), # group 32 (two steps per 64-k stage), k padded to 1088
    (256, 2048, 16384, 256, True, "f32"),
    (777, 384, 5000, 64, True, "bf16"),
    # more tiles than CUs with a short last round: the last column tiles run
    # split 2 ways along k (the tail split)
    (500, 1024, 35800, 128, True, "bf16"), # 280 tiles: 12 of 140 column tiles split, ragged rows and columns
    (700, 1024, 24000, 64, False, "f32"),  # 282 tiles: 9 of 94 column tiles (3 row tiles) split, group 64
]


@pytest.mark.parametrize("M,D_in,D_out,group,inv,out", GEMM_CASES)
def test_w4a16_gemm(awq, M, D_in, D_out, group, inv, out):
    say("gemm", M, D_in, D_out, group, inv, out)
    rng = np.random.default_rng(M * 1000 + D_in + D_out)
    X = synth.to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))
    q = rng.integers(-7, 8, (D_in, D_out)).astype(np.int8)
    words = oracle.pack_int4(q)
    scales = rng.uniform(0.001, 0.01, (D_in // group, D_out)).astype(np.float32)
    inv_s = rng.uniform(0.1, 2.0, D_in).astype(np.float32) if inv else None
    Yref = oracle.w4a16_gemm(X, words, scales, group, inv_s=inv_s)
    Yg = awq.w4a16_gemm(dev_tensor(X, "bf16"), torch.from_numpy(words.view(np.int32)).cuda(),
                        torch.from_numpy(scales).cuda(), group=group,
                        inv_s=torch.from_numpy(inv_s).cuda() if inv else None,
                        out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    Y = Yg.float().cpu().numpy().astype(np.float64)
    excess = np.abs(Y - Yref) - gemm_tolerance(Yref, out)
    assert excess.max() <= 0, (np.abs(Y - Yref).max(), excess.max(), np.abs(Yref).max())


def test_w4a16_gemm_split_workspace_reuse(awq):
    """A dirty caller workspace, reused across calls: results identical each time."""
    say("gemm split workspace reuse")
    M, D_in, D_out, group = 4, 8192, 768, 128
    rng = np.random.default_rng(7)
    X = synth.to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))
    q = rng.integers(-7, 8, (D_in, D_out)).astype(np.int8)
    words = oracle.pack_int4(q)
    scales = rng.uniform(0.001, 0.01, (D_in // group, D_out)).astype(np.float32)
    inv_s = rng.uniform(0.1, 2.0, D_in).astype(np.float32)
    Yref = oracle.w4a16_gemm(X, words, scales, group, inv_s=inv_s)
    need = awq.w4a16_workspace_size(M, D_in, D_out, True)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    args = (dev_tensor(X, "bf16"), torch.from_numpy(words.view(np.int32)).cuda(), torch.from_numpy(scales).cuda())
    outs = []
    for _ in range(3):
        Yg = awq.w4a16_gemm(*args, group=group, inv_s=torch.from_numpy(inv_s).cuda(), out_dtype=torch.float32,
                            workspace=ws)
        torch.cuda.synchronize()
        outs.append(Yg.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    err = np.abs(outs[0].astype(np.float64) - Yref).max()
    assert err <= GEMM_TOL * np.abs(Yref).max(), err


def test_end_to_end_small(awq):
    """search -> pack -> W4A16 with inv_s = 1/s*, against the oracle chain."""
    say("end to end small")
    case = synth.make_layer(256, 512, 264, seed=77, dtype="bf16", n_salient=5, salient_lo=10.0, salient_hi=100.0)
    ref = oracle.search_layer(case.X, case.W, case.alphas, 4, 128)
    r, _ = _run_search(awq, case, case.alphas)
    assert r.best_index() in tie_band(ref["losses"])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes"])
    packed = awq.pack(r.codes, bits=4)
    torch.cuda.synchronize()
    words_ref = oracle.pack_int4(ref["codes"])
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), words_ref)
    inv_s = (1.0 / r.s_best).contiguous()
    Xd = synth.decode_x(8, 512, seed=5)
    Y = awq.w4a16_gemm(dev_tensor(Xd, "bf16"), packed, r.scales, group=128, inv_s=inv_s).cpu().numpy()
    Yref = oracle.w4a16_gemm(Xd, words_ref, ref["scales"], 128, inv_s=(1.0 / ref["s_best"]).astype(np.float32))
    assert np.abs(Y - Yref).max() <= GEMM_TOL * np.abs(Yref).max()


def test_quantiser_half_integer_ties(awq):
    """Values at and one ulp around half-integer multiples of the step: the
    quantiser's fast reciprocal path must fall back to true division there."""
    say("quantiser ties")
    rng = np.random.default_rng(99)
    D_in, D_out, N = 256, 64, 32
    W = np.zeros((D_in, D_out), np.float32)
    for g in range(2):
        for o in range(D_out):
            e = np.float32(2.0 ** rng.integers(-8, 2))
            col = (rng.integers(-7, 7, 128) + np.float32(0.5)).astype(np.float32) * e
            wiggle = rng.integers(-2, 3, 128)
            col = np.nextafter(col, np.where(wiggle > 0, np.inf, -np.inf).astype(np.float32))   # one ulp off
            col = np.where(wiggle == 0, (rng.integers(-7, 7, 128) + np.float32(0.5)) * e, col).astype(np.float32)  # exact ties
            col[0] = np.float32(7.0) * e * (1 if rng.random() < 0.5 else -1)   # absmax -> step = e exactly
            W[g * 128:(g + 1) * 128, o] = col
    X = np.ones((N, D_in), np.float32)          # a == 1 -> s == 1 for every alpha
    case = synth.LayerCase("ties", X, W, "f32", 4, 128, np.array([0.0, 0.5], np.float32))
    ref = oracle.search_layer(X, W, case.alphas, 4, 128, keep_all=True)
    r, _ = _run_search(awq, case, case.alphas)
    assert r.best_index() == 0
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][0])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][0])


# -------------------------------------------------------------- clipping ----

CLIP_CASES = [
    # name, N, D_in, D_out, dtype, bits, group
    ("clip_bf16_ragged", 300, 384, 520, "bf16", 4, 128),
    ("clip_f32_int3_g32", 70, 96, 40, "f32", 3, 32),
    ("clip_bf16_chunks", 1024, 512, 1024, "bf16", 4, 128),
    ("clip_one_row_g64", 1, 256, 36, "bf16", 4, 64),
    ("clip_f32_ragged_chunk", 517, 256, 130, "f32", 4, 64),
    ("clip_bf16_g256", 600, 768, 200, "bf16", 4, 256),
    ("clip_f32_g256_int3", 300, 512, 70, "f32", 3, 256),
]
CLIP_RTOL = 1e-4


@pytest.mark.parametrize("spec", CLIP_CASES, ids=[c[0] for c in CLIP_CASES])
def test_clip_search_matches_oracle(awq, spec):
    name, N, D_in, D_out, dtype, bits, group = spec
    say("clip", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits,
                            group=group, n_salient=3, salient_lo=10.0, salient_hi=60.0)
    s = oracle.scales_for_alpha(oracle.act_stats(case.X), 0.45)
    ratios = np.linspace(1.0, 0.5, 11).astype(np.float32)
    ref = oracle.clip_search(case.X, case.W, s, ratios, bits, group)
    r = awq.clip_search(dev_tensor(case.X, dtype), dev_tensor(case.W, dtype), torch.from_numpy(s).cuda(),
                        ratios=ratios, bits=bits, group=group, want_errors=True)
    torch.cuda.synchronize()
    E = r.errors.cpu().numpy().astype(np.float64)
    Er = ref["errors"]
    floor = 1e-6 * Er.max(axis=0, keepdims=True)            # per (group, column) scale
    assert np.all(np.abs(E - Er) <= CLIP_RTOL * Er + floor), np.abs(E - Er).max()
    idx = r.ratio_idx.cpu().numpy()
    chosen = np.take_along_axis(Er, idx[None].astype(np.int64), 0)[0]
    assert np.all(chosen <= Er.min(axis=0) * (1 + 2 * CLIP_RTOL) + 2 * floor[0])
    agree = (idx == ref["ratio_idx"]).mean()
    assert agree > 0.97, agree                              # disagreements only in near ties
    # codes and steps at the GPU's ratio, bit for bit
    Wp = (s[:, None] * case.W.astype(np.float32)).astype(np.float32)
    codes = r.codes.cpu().numpy()
    scales = r.scales.cpu().numpy()
    for k, rat in enumerate(ratios):
        sel = idx == k
        if not sel.any():
            continue
        q, d = oracle.quantize_group_clipped(Wp, bits, group, float(rat))
        assert np.array_equal(scales[sel], d[sel])
        rows = np.repeat(sel, group, axis=0)
        assert np.array_equal(codes[rows], q[rows])


def test_clip_search_ratio_one_is_plain(awq):
    """A one-point grid {1} gives the plain quantiser's codes and steps."""
    say("clip ratio one")
    case = synth.make_layer(200, 256, 72, seed=12, dtype="bf16", n_salient=2, salient_lo=20.0)
    s = oracle.scales_for_alpha(oracle.act_stats(case.X), 0.6)
    r = awq.clip_search(dev_tensor(case.X, "bf16"), dev_tensor(case.W, "bf16"), torch.from_numpy(s).cuda(),
                        ratios=[1.0], bits=4, group=128)
    torch.cuda.synchronize()
    q, d = oracle.quantize_group_absmax((s[:, None] * case.W).astype(np.float32), 4, 128)
    assert np.array_equal(r.codes.cpu().numpy(), q) and np.array_equal(r.scales.cpu().numpy(), d)
    assert (r.ratio_idx.cpu().numpy() == 0).all()


# ------------------------------------------------------------ zero point ----

ZP_SEARCH_CASES = [
    # name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal
    ("zp_bf16_ragged", 300, 384, 520, "bf16", 4, 128, "salient", 4),
    ("zp_f32_int3_g32", 70, 96, 40, "f32", 3, 32, "heavy", 0),
    ("zp_bf16_tiles", 1024, 512, 1024, "bf16", 4, 128, "salient", 8),
    ("zp_bf16_int2_g8", 17, 64, 12, "bf16", 2, 8, "salient", 1),
    ("zp_bf16_int8", 64, 256, 48, "bf16", 8, 128, "heavy", 0),
    ("zp_f32_g256", 90, 512, 72, "f32", 4, 256, "heavy", 0),
    ("zp_bf16_int3_g64", 300, 512, 264, "bf16", 3, 64, "salient", 3),
    ("zp_bf16c_ragged", 300, 2048, 520, "bf16", 4, 128, "salient", 4),
]


@pytest.mark.parametrize("spec", ZP_SEARCH_CASES, ids=[c[0] for c in ZP_SEARCH_CASES])
def test_zero_point_search_matches_oracle(awq, spec):
    name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal = spec
    say("zp search", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits,
                            group=group, x_kind=x_kind, n_salient=n_sal, salient_lo=10.0, salient_hi=100.0)
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True, asym=True)
    X = dev_tensor(case.X, dtype)
    W = dev_tensor(case.W, dtype)
    a = awq.act_stats(X)
    r = awq.search_layer(X, W, alphas=case.alphas, bits=bits, group=group, a=a, zero_point=True,
                         matrix=_matrix(name))
    torch.cuda.synchronize()
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / np.maximum(ref["losses"], 1e-300)
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    k = r.best_index()
    band = tie_band(ref["losses"])
    assert k == ref["best"] or (len(band) > 1 and k in band), (k, ref["best"], band)
    assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][k])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][k])
    assert np.array_equal(r.zeros.cpu().numpy(), ref["zeros_all"][k])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][k])
    if bits <= 4 and D_in % 8 == 0:
        words = awq.pack(r.codes, bits=bits).cpu().numpy().view(np.uint32)
        assert np.array_equal(words, oracle.pack_int4(ref["codes_all"][k], offset=0))


ZP_GEMM_CASES = [
    # M, D_in, D_out, group, inv, out  (decode regime, then prefill regime)
    (1, 1024, 520, 128, True, "f32"),
    (8, 8192, 1000, 128, False, "bf16"),
    (16, 256, 256, 32, True, "f32"),
    (40, 2048, 264, 64, True, "f32"),
    (20, 512, 16396, 128, True, "f32"),
    (3, 512, 40000, 128, True, "bf16"),
    (24, 512, 24608, 128, True, "f32"),    # two column strips per wave
    (24, 2048, 1000, 128, True, "f32"),    # a 24-row pass split 2 ways
    (12, 256, 25000, 256, False, "bf16"),  # the same, one row tile
    (1, 512, 24608, 128, True, "f32"),     # staged activations, two strips, zero points
    (8, 8192, 24640, 256, False, "bf16"),  # the same, 8 rows of 8192 (the largest that stage)
    (300, 512, 8200, 128, True, "f32"),
    (777, 384, 5000, 64, True, "bf16"),
    (256, 2048, 16384, 256, True, "f32"),
    (1030, 1056, 4100, 32, False, "bf16"),   # prefill-sized, group 32: decode regime
    (520, 1024, 35800, 128, True, "bf16"),   # prefill tail split
]


@pytest.mark.parametrize("M,D_in,D_out,group,inv,out", ZP_GEMM_CASES)
def test_w4a16_gemm_zero_point(awq, M, D_in, D_out, group, inv, out):
    say("zp gemm", M, D_in, D_out, group, inv, out)
    rng = np.random.default_rng(M * 977 + D_in + D_out)
    X = synth.to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))
    q = rng.integers(0, 16, (D_in, D_out)).astype(np.uint8)
    words = oracle.pack_int4(q, offset=0)
    scales = rng.uniform(0.001, 0.01, (D_in // group, D_out)).astype(np.float32)
    zeros = rng.integers(0, 16, (D_in // group, D_out)).astype(np.uint8)
    inv_s = rng.uniform(0.1, 2.0, D_in).astype(np.float32) if inv else None
    Yref = oracle.w4a16_gemm(X, words, scales, group, inv_s=inv_s, zeros=zeros)
    Yg = awq.w4a16_gemm(dev_tensor(X, "bf16"), torch.from_numpy(words.view(np.int32)).cuda(),
                        torch.from_numpy(scales).cuda(), group=group,
                        inv_s=torch.from_numpy(inv_s).cuda() if inv else None,
                        out_dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                        zeros=torch.from_numpy(zeros).cuda())
    Y = Yg.float().cpu().numpy().astype(np.float64)
    excess = np.abs(Y - Yref) - gemm_tolerance(Yref, out)
    assert excess.max() <= 0, (np.abs(Y - Yref).max(), excess.max(), np.abs(Yref).max())


F16_SEARCH_CASES = [
    # name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal, zero_point, weight_term
    ("f16_sym_ragged", 300, 384, 520, "bf16", 4, 128, "salient", 4, False, False),
    ("f16_zp_ragged", 300, 384, 520, "bf16", 4, 128, "salient", 4, True, False),
    ("f16_sym_tiles_g64", 1024, 512, 1024, "bf16", 4, 64, "salient", 8, False, False),
    ("f16_zp_f32_int3_g32", 70, 96, 40, "f32", 3, 32, "heavy", 0, True, False),
    ("f16_sym_wscale", 256, 512, 264, "bf16", 4, 128, "salient", 5, False, True),
    ("f16_zp_int8_g256", 64, 512, 48, "bf16", 8, 256, "heavy", 0, True, False),
    ("f16_sym_int2_g8", 17, 64, 12, "bf16", 2, 8, "salient", 1, False, False),
    ("f16_zp_bf16c", 300, 2048, 520, "bf16", 4, 128, "salient", 4, True, False),
]


@pytest.mark.parametrize("spec", F16_SEARCH_CASES, ids=[c[0] for c in F16_SEARCH_CASES])
def test_f16_step_search_matches_oracle(awq, spec):
    name, N, D_in, D_out, dtype, bits, group, x_kind, n_sal, zp, wterm = spec
    say("f16-step search", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits,
                            group=group, x_kind=x_kind, n_salient=n_sal, salient_lo=10.0, salient_hi=100.0)
    X = dev_tensor(case.X, dtype)
    W = dev_tensor(case.W, dtype)
    a = awq.act_stats(X)
    b = awq.weight_stats(W) if wterm else None
    b_ref = oracle.weight_stats(case.W) if wterm else None
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True, b=b_ref, asym=zp,
                              f16_steps=True)
    r = awq.search_layer(X, W, alphas=case.alphas, bits=bits, group=group, a=a, b=b, zero_point=zp,
                         f16_steps=True, matrix=_matrix(name))
    torch.cuda.synchronize()
    assert r.scales.dtype == torch.float16
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / np.maximum(ref["losses"], 1e-300)
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    k = r.best_index()
    band = tie_band(ref["losses"])
    assert k == ref["best"] or (len(band) > 1 and k in band), (k, ref["best"], band)
    assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][k])
    want = ref["scales_all"][k].astype(np.float16)          # exact: the oracle's steps are FP16 values
    assert np.array_equal(r.scales.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][k])
    if zp:
        assert np.array_equal(r.zeros.cpu().numpy(), ref["zeros_all"][k])


F16_GEMM_CASES = [
    # M, D_in, D_out, group, inv, out, zero_point  (decode regime, then prefill regime)
    (1, 1024, 520, 128, True, "f32", False),
    (8, 2048, 1000, 64, False, "bf16", True),
    (32, 4096, 264, 32, True, "f32", False),
    (300, 512, 8200, 128, True, "f32", False),
    (777, 384, 5000, 64, True, "bf16", True),
    (256, 2048, 16384, 256, True, "f32", True),
    (1030, 1056, 4100, 32, False, "bf16", True),   # prefill-sized, zero points, group 32: decode regime
    (3, 512, 40000, 128, True, "bf16", False),
    (16, 1024, 24600, 128, False, "bf16", True),   # two column strips per wave
    (4, 1024, 24576, 128, False, "bf16", True),    # staged activations, two strips
    (6, 2048, 24704, 128, True, "f32", False),     # pre-pass activations, two strips
    (7, 1024, 24576, 128, True, "bf16", True),     # staged activations, two strips, zero points
    (2, 1024, 24600, 256, True, "f32", False),
    (32, 512, 24576, 256, True, "f32", False),
    (32, 4096, 768, 128, False, "bf16", True),     # a 32-row pass split 4 ways, zero points
    (500, 1024, 35800, 256, True, "f32", False),   # prefill tail split
]


@pytest.mark.parametrize("M,D_in,D_out,group,inv,out,zp", F16_GEMM_CASES)
def test_w4a16_gemm_f16_steps(awq, M, D_in, D_out, group, inv, out, zp):
    say("f16-step gemm", M, D_in, D_out, group, inv, out, zp)
    rng = np.random.default_rng(M * 131 + D_in * 7 + D_out)
    X = synth.to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))
    if zp:
        q = rng.integers(0, 16, (D_in, D_out)).astype(np.uint8)
        words = oracle.pack_int4(q, offset=0)
        zeros = rng.integers(0, 16, (D_in // group, D_out)).astype(np.uint8)
    else:
        q = rng.integers(-7, 8, (D_in, D_out)).astype(np.int8)
        words = oracle.pack_int4(q)
        zeros = None
    s16 = rng.uniform(0.001, 0.01, (D_in // group, D_out)).astype(np.float16)
    inv_s = rng.uniform(0.1, 2.0, D_in).astype(np.float32) if inv else None
    Yref = oracle.w4a16_gemm(X, words, s16.astype(np.float32), group, inv_s=inv_s, zeros=zeros)
    Yg = awq.w4a16_gemm(dev_tensor(X, "bf16"), torch.from_numpy(words.view(np.int32)).cuda(),
                        torch.from_numpy(s16).cuda(), group=group,
                        inv_s=torch.from_numpy(inv_s).cuda() if inv else None,
                        out_dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                        zeros=torch.from_numpy(zeros).cuda() if zp else None)
    Y = Yg.float().cpu().numpy().astype(np.float64)
    excess = np.abs(Y - Yref) - gemm_tolerance(Yref, out)
    assert excess.max() <= 0, (np.abs(Y - Yref).max(), excess.max(), np.abs(Yref).max())


def test_f16_steps_end_to_end(awq):
    """FP16-step search (zero points) -> pack -> W4A16 with FP16 steps, against the oracle chain."""
    say("f16-step end to end")
    case = synth.make_layer(256, 512, 264, seed=91, dtype="bf16", n_salient=5, salient_lo=10.0, salient_hi=100.0)
    X = dev_tensor(case.X, "bf16")
    W = dev_tensor(case.W, "bf16")
    r = awq.search_layer(X, W, alphas=case.alphas, bits=4, group=128, zero_point=True, f16_steps=True)
    packed = awq.pack(r.codes, bits=4)
    inv_s = (1.0 / r.s_best).contiguous()
    Xd = synth.decode_x(8, 512, seed=6)
    Y = awq.w4a16_gemm(dev_tensor(Xd, "bf16"), packed, r.scales, group=128, inv_s=inv_s, zeros=r.zeros)
    torch.cuda.synchronize()
    k = r.best_index()
    ref = oracle.search_layer(case.X, case.W, case.alphas, 4, 128, keep_all=True, asym=True, f16_steps=True)
    words = oracle.pack_int4(ref["codes_all"][k], offset=0)
    inv_ref = (np.float32(1.0) / ref["s_all"][k]).astype(np.float32)
    Yref = oracle.w4a16_gemm(Xd, words, ref["scales_all"][k], 128, inv_s=inv_ref, zeros=ref["zeros_all"][k])
    err = np.abs(Y.cpu().numpy().astype(np.float64) - Yref).max()
    assert err <= GEMM_TOL * np.abs(Yref).max(), err


def test_zero_point_end_to_end(awq):
    """zero-point search -> pack -> W4A16 with inv_s = 1/s*, against the oracle chain."""
    say("zp end to end")
    case = synth.make_layer(256, 512, 264, seed=78, dtype="bf16", n_salient=5, salient_lo=10.0, salient_hi=100.0)
    X = dev_tensor(case.X, "bf16")
    W = dev_tensor(case.W, "bf16")
    r = awq.search_layer(X, W, alphas=case.alphas, bits=4, group=128, zero_point=True)
    packed = awq.pack(r.codes, bits=4)
    inv_s = (1.0 / r.s_best).contiguous()
    Xd = synth.decode_x(8, 512, seed=5)
    Y = awq.w4a16_gemm(dev_tensor(Xd, "bf16"), packed, r.scales, group=128, inv_s=inv_s, zeros=r.zeros)
    torch.cuda.synchronize()
    k = r.best_index()
    ref = oracle.search_layer(case.X, case.W, case.alphas, 4, 128, keep_all=True, asym=True)
    words = oracle.pack_int4(ref["codes_all"][k], offset=0)
    inv_ref = (np.float32(1.0) / ref["s_all"][k]).astype(np.float32)
    Yref = oracle.w4a16_gemm(Xd, words, ref["scales_all"][k], 128, inv_s=inv_ref, zeros=ref["zeros_all"][k])
    err = np.abs(Y.cpu().numpy().astype(np.float64) - Yref).max()
    assert err <= GEMM_TOL * np.abs(Yref).max(), err


# ------------------------------------------------ fp16-path prescale edges ----

@pytest.mark.parametrize("factor", [1e-10, 1e-36])
def test_search_tiny_live_channel(awq, factor):
    """One live channel far below its group-mates (a_j tiny but >= FLT_MIN) on
    the fp16 contraction path, alpha up to 1: the error-weight prescale must
    not depend on the within-group spread of s (1e-36 also caps the prescale
    so that 2^kd / s stays finite)."""
    say("search tiny live channel", factor)
    case = synth.make_layer(512, 256, 512, seed=41, dtype="bf16", n_salient=3, salient_lo=10.0, salient_hi=100.0)
    X = case.X.copy()
    X[:, 37] = synth.to_bf16_values(X[:, 37] * np.float32(factor))
    assert np.abs(X[:, 37]).max() > 0
    c = synth.LayerCase("tiny", X, case.W, "bf16", 4, 128, case.alphas)
    ref = oracle.search_layer(X, case.W, c.alphas, 4, 128, keep_all=True)
    assert 0.0 < ref["a"][37] < 1e-8
    r, a = _run_search(awq, c, c.alphas)
    assert np.array_equal(a, ref["a"])
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    b = r.best_index()
    band = tie_band(ref["losses"])
    assert b == ref["best"] or (len(band) > 1 and b in band), (b, ref["best"], band)
    assert np.array_equal(r.s_best.cpu().numpy(), ref["s_all"][b])
    assert np.array_equal(r.scales.cpu().numpy(), ref["scales_all"][b])
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][b])


def test_f16_steps_subnormal_range(awq):
    """Every group's step in the FP16 subnormal range: rounding the step to
    FP16 can shrink it by far more than half a code, so the quotient passes
    qmax + 1/2 and the codes clamp; the per-alpha losses must be those of the
    clamped codes."""
    say("f16 steps, subnormal range")
    case = synth.make_layer(512, 256, 512, seed=43, dtype="bf16", n_salient=3, salient_lo=2.0, salient_hi=4.0)
    W = synth.to_bf16_values(case.W * np.float32(1e-5))
    c = synth.LayerCase("f16sub", case.X, W, "bf16", 4, 128, case.alphas)
    ref = oracle.search_layer(case.X, W, c.alphas, 4, 128, keep_all=True, f16_steps=True)
    steps = ref["scales_all"][0]
    assert np.count_nonzero((steps > 0) & (steps < 2.0 ** -14)) > steps.size // 2   # subnormal FP16 steps
    Xd, Wd = dev_tensor(case.X, "bf16"), dev_tensor(W, "bf16")
    a = awq.act_stats(Xd)
    r = awq.search_layer(Xd, Wd, alphas=c.alphas, bits=4, group=128, a=a, f16_steps=True)
    torch.cuda.synchronize()
    losses = r.losses.cpu().numpy()
    rel = np.abs(losses - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    k = r.best_index()
    band = tie_band(ref["losses"])
    assert k == ref["best"] or (len(band) > 1 and k in band), (k, ref["best"], band)
    want = ref["scales_all"][k].astype(np.float16)
    assert np.array_equal(r.scales.cpu().numpy().view(np.uint16), want.view(np.uint16))
    assert np.array_equal(r.codes.cpu().numpy(), ref["codes_all"][k])


def test_search_nonfinite_c_abi(awq):
    """Through the raw C ABI: a NaN in W gives best = -1 from the (asynchronous)
    search call, which returns AWQ_OK, and AWQ_ERR_NONFINITE from the
    synchronising awq_search_status; a finite layer gives AWQ_OK there."""
    import ctypes
    say("search non-finite, raw C ABI")
    lib = awq.load()
    case = synth.make_layer(64, 256, 40, seed=12, dtype="bf16", n_salient=2, salient_lo=20.0)
    alphas = np.ascontiguousarray(case.alphas, dtype=np.float32)
    for poison in (False, True):
        W = case.W.copy()
        if poison:
            W[200, 17] = np.nan
        X, Wd = dev_tensor(case.X, "bf16"), dev_tensor(W, "bf16")
        a = awq.act_stats(X)
        need = awq.search_workspace_size(64, 256, 40, torch.bfloat16, 4, 128, alphas.size)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        losses = torch.empty(alphas.size, dtype=torch.float64, device="cuda")
        best = torch.full((1,), 123, dtype=torch.int32, device="cuda")
        s_best = torch.empty(256, dtype=torch.float32, device="cuda")
        scales = torch.full((2, 40), -1.0, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.awq_search_layer(X.data_ptr(), 1, 64, 256, Wd.data_ptr(), 1, 40, a.data_ptr(), alphas.ctypes.data,
                                  alphas.size, 4, 128, losses.data_ptr(), best.data_ptr(), s_best.data_ptr(),
                                  scales.data_ptr(), None, ws.data_ptr(), need, stream)
        assert st == 0
        out = ctypes.c_int32(99)
        st2 = lib.awq_search_status(best.data_ptr(), stream, ctypes.byref(out))
        if poison:
            assert st2 == -5 and out.value == -1, (st2, out.value)
            assert b"NaN" in lib.awq_last_error()
            assert torch.all(scales == -1.0).item()          # outputs left unwritten
        else:
            assert st2 == 0 and 0 <= out.value < alphas.size, (st2, out.value)
            assert int(best.item()) == out.value


# ------------------------------------------- column-chunked search (small workspace) ----

CHUNK_CASES = [
    # name, N, D_in, D_out, dtype, bits, group, zero_point, chunks of 256 columns per pass (0: the minimum)
    ("chunk_bf16_min", 600, 512, 1300, "bf16", 4, 128, False, 0),
    ("chunk_bf16_3tiles", 600, 512, 1300, "bf16", 4, 128, False, 3),
    ("chunk_f32_min", 100, 256, 700, "f32", 3, 64, False, 0),
    ("chunk_bf16_zp_g256", 300, 1024, 800, "bf16", 4, 256, True, 2),
    ("chunk_bf16_rows9_3tiles", 2300, 512, 1300, "bf16", 4, 128, False, 3),
    ("chunk_bf16c_3tiles", 600, 2048, 1300, "bf16", 4, 128, False, 3),
    ("chunk_bf16c_zp_g256", 300, 2048, 800, "bf16", 4, 256, True, 2),
]


@pytest.mark.parametrize("spec", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_search_column_chunks(awq, spec):
    """A workspace below the one-pass size: the error weights and the loss
    contraction run per column chunk; every output equals the one-pass
    search's bit for bit, and the losses are within tolerance of the oracle."""
    name, N, D_in, D_out, dtype, bits, group, zp, tiles_per_chunk = spec
    say("search column chunks", spec)
    case = synth.make_layer(N, D_in, D_out, seed=zlib.crc32(name.encode()) % 1000, dtype=dtype, bits=bits,
                            group=group, n_salient=4, salient_lo=10.0, salient_hi=100.0)
    X, W = dev_tensor(case.X, dtype), dev_tensor(case.W, dtype)
    tdt = X.dtype
    full = awq.search_workspace_size(N, D_in, D_out, tdt, bits, group, len(case.alphas))
    least = awq.search_workspace_min_size(N, D_in, D_out, tdt, bits, group, len(case.alphas))
    elt = 2 if (dtype == "bf16" and N * D_out >= 65536) else 4
    # rows of the error weights: D_in padded to 64, plus the 64 correction rows
    # on layers that may take the bf16 path (the workspace sizes cover them)
    rows = (D_in + 63) // 64 * 64 + (64 if (elt == 2 and 2048 <= D_in <= 16384) else 0)
    per_tile = len(case.alphas) * rows * 256 * elt   # error weights of 256 columns
    size = least if tiles_per_chunk == 0 else least + (tiles_per_chunk - 1) * per_tile
    assert least < size + 1 <= full
    a = awq.act_stats(X)
    runs = []
    for nbytes in (full, size):
        ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
        r = awq.search_layer(X, W, alphas=case.alphas, bits=bits, group=group, a=a, workspace=ws, zero_point=zp,
                             matrix=_matrix(name))
        torch.cuda.synchronize()
        runs.append({k: getattr(r, k).cpu().numpy() for k in ("losses", "s_best", "scales", "codes")})
        runs[-1]["best"] = r.best_index()
        if zp:
            runs[-1]["zeros"] = r.zeros.cpu().numpy()
        del ws
    one, chunked = runs
    for k in one:
        assert np.array_equal(one[k], chunked[k]), k
    ref = oracle.search_layer(case.X, case.W, case.alphas, bits, group, keep_all=True, asym=zp)
    rel = np.abs(chunked["losses"] - ref["losses"]) / ref["losses"]
    assert rel.max() <= LOSS_RTOL, (rel.max(), rel)
    b = chunked["best"]
    assert b == ref["best"] or b in tie_band(ref["losses"])
    assert np.array_equal(chunked["codes"], ref["codes_all"][b])
    assert np.array_equal(chunked["scales"], ref["scales_all"][b])
