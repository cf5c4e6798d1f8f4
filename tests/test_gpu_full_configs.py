"""GPU parity at the five benchmark layer sizes, in the launch configuration
bench.py times (act_stats -> search_layer with a caller workspace -> pack ->
w4a16_gemm with inv_s = 1/s*).

Layers 1-4 are checked against the complete oracle search.  The large layer
(8192 x 28672, N = 4096) runs the oracle's steps one alpha at a time (all 21,
keeping only the quantiser outputs at the GPU's alpha*) to bound host memory,
then checks the packed words and the W4A16 products at M = 1, 8, 32 (decode)
and 512 (prefill).
"""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import GEMM_TOL, LOSS_RTOL, dev_tensor, say, tie_band
from weight_only_quantization_awq_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.full]


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_quantization_awq_amd import awq as mod
    return mod


def _gpu_search(awq, case):
    """The benchmark's call sequence for one layer; returns host copies."""
    X = dev_tensor(case.X, case.dtype)
    W = dev_tensor(case.W, case.dtype)
    tdt = X.dtype
    ws = torch.empty(awq.search_workspace_size(case.N, case.D_in, case.D_out, tdt, case.bits, case.group,
                                               len(case.alphas)), dtype=torch.uint8, device="cuda")
    a = awq.act_stats(X)
    r = awq.search_layer(X, W, alphas=case.alphas, bits=case.bits, group=case.group, a=a, workspace=ws)
    packed = awq.pack(r.codes, bits=case.bits) if case.bits <= 4 else None
    torch.cuda.synchronize()
    out = {
        "a": a.cpu().numpy(),
        "losses": r.losses.cpu().numpy(),
        "best": r.best_index(),
        "s_best": r.s_best.cpu().numpy(),
        "scales": r.scales.cpu().numpy(),
        "codes": r.codes.cpu().numpy(),
        "packed": None if packed is None else packed.cpu().numpy().view(np.uint32),
        "scales_dev": r.scales,
        "s_best_dev": r.s_best,
        "packed_dev": packed,
    }
    del X, W, ws, a
    return out


def _check_losses(got, ref, idx):
    for k in idx:
        rel = abs(got[k] - ref[k]) / ref[k]
        assert rel <= LOSS_RTOL, (k, got[k], ref[k], rel)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_full_oracle(awq, cfg):
    t0 = time.time()
    case = synth.config_case(cfg)
    say(f"config {cfg}: {case.name} N={case.N} D_in={case.D_in} D_out={case.D_out} bits={case.bits}")
    g = _gpu_search(awq, case)
    say(f"  gpu done; oracle search ({time.time() - t0:.1f}s)")
    Xo, Wo = case.X, case.W      # float32 arrays holding the exact bf16 values the GPU received
    ref = oracle.search_layer(Xo, Wo, case.alphas, case.bits, case.group)
    say(f"  oracle done ({time.time() - t0:.1f}s): alpha*={case.alphas[ref['best']]:.2f}")
    assert np.array_equal(g["a"], ref["a"])
    _check_losses(g["losses"], ref["losses"], range(len(case.alphas)))
    b = g["best"]
    band = tie_band(ref["losses"])
    assert b == ref["best"] or (len(band) > 1 and b in band), (b, ref["best"], band)
    if b == ref["best"]:
        rq, rd, rs = ref["codes"], ref["scales"], ref["s_best"]
    else:  # near tie: compare the quantiser at the GPU's alpha
        rs = oracle.scales_for_alpha(ref["a"], case.alphas[b])
        rq, rd = oracle.quantize_group_absmax((rs[:, None] * Wo).astype(np.float32), case.bits, case.group)
    assert np.array_equal(g["s_best"], rs)
    assert np.array_equal(g["scales"], rd)
    assert np.array_equal(g["codes"], rq)
    if g["packed"] is not None and case.D_in % 8 == 0:
        assert np.array_equal(g["packed"], oracle.pack_int4(rq))
    say(f"  config {cfg} ok ({time.time() - t0:.1f}s)")


@pytest.mark.timeout(900)
def test_config_large_layer_and_decode(awq):
    t0 = time.time()
    case = synth.config_case(5)
    say(f"config 5: {case.name} N={case.N} D_in={case.D_in} D_out={case.D_out}")
    g = _gpu_search(awq, case)
    b = g["best"]
    n = len(case.alphas)
    say(f"  gpu done, alpha*={case.alphas[b]:.2f} ({time.time() - t0:.1f}s); oracle checks")
    Xo, Wo = case.X, case.W
    a = oracle.act_stats(Xo)
    assert np.array_equal(g["a"], a)
    X64 = Xo.astype(np.float64)
    Y = X64 @ Wo.astype(np.float64)
    del X64
    ref = {}
    for k in range(n):
        s = oracle.scales_for_alpha(a, case.alphas[k])
        q, d = oracle.quantize_group_absmax((s[:, None] * Wo).astype(np.float32), case.bits, case.group)
        ref[k] = oracle.search_loss(Xo, Wo, s, oracle.dequantize(q, d, case.group), Y)
        say(f"  alpha {case.alphas[k]:.2f}: oracle L={ref[k]:.9e} gpu L={g['losses'][k]:.9e} "
            f"({time.time() - t0:.1f}s)")
        if k == b:
            assert np.array_equal(g["s_best"], s)
            assert np.array_equal(g["scales"], d)
            assert np.array_equal(g["codes"], q)
            assert np.array_equal(g["packed"], oracle.pack_int4(q))
        del q, d
    del Y
    ref = np.array([ref[k] for k in range(n)])
    _check_losses(g["losses"], ref, range(n))
    rb = oracle.argmin_first(ref)
    band = tie_band(ref)
    assert b == rb or (len(band) > 1 and b in band), (b, rb, band)

    # decode shapes on the packed result, inv_s = 1/s*
    inv_s = (1.0 / g["s_best_dev"]).contiguous()
    inv_h = inv_s.cpu().numpy()
    for M in (1, 8, 32, 512):
        say(f"  w4a16 M={M}")
        Xd = synth.decode_x(M, case.D_in)
        Xt = torch.from_numpy(Xd).to(torch.bfloat16).cuda()
        ws = torch.empty(max(awq.w4a16_workspace_size(M, case.D_in, case.D_out, True), 16), dtype=torch.uint8,
                         device="cuda")
        Yg = awq.w4a16_gemm(Xt, g["packed_dev"], g["scales_dev"], group=case.group, inv_s=inv_s,
                            out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        Yr = oracle.w4a16_gemm(Xd, g["packed"], g["scales"], case.group, inv_h)
        err = np.abs(Yg.cpu().numpy().astype(np.float64) - Yr).max()
        assert err <= GEMM_TOL * np.abs(Yr).max(), (M, err, np.abs(Yr).max())
    # M = 2048 (the prefill benchmark size; its last 16 column tiles run split
    # along k): the first 512 columns and the last 4352, across that boundary
    M = 2048
    say(f"  w4a16 M={M} (sampled columns)")
    Xd = synth.decode_x(M, case.D_in)
    Xt = torch.from_numpy(Xd).to(torch.bfloat16).cuda()
    ws = torch.empty(awq.w4a16_workspace_size(M, case.D_in, case.D_out, True), dtype=torch.uint8, device="cuda")
    Yg = awq.w4a16_gemm(Xt, g["packed_dev"], g["scales_dev"], group=case.group, inv_s=inv_s,
                        out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    sel = np.r_[0:512, case.D_out - 4352:case.D_out]
    Yr = oracle.w4a16_gemm(Xd, np.ascontiguousarray(g["packed"][:, sel]), np.ascontiguousarray(g["scales"][:, sel]),
                           case.group, inv_h)
    err = np.abs(Yg.cpu().numpy()[:, sel].astype(np.float64) - Yr).max()
    assert err <= GEMM_TOL * np.abs(Yr).max(), (M, err, np.abs(Yr).max())
    say(f"  config 5 ok ({time.time() - t0:.1f}s)")


@pytest.mark.timeout(600)
def test_large_layer_search_under_2gb(awq):
    """The 8192 x 28672 search (N = 4096) with a 2 GB workspace, i.e. in column
    chunks, against the one-pass search (9.9 GB): identical outputs bit for
    bit (the one-pass search is checked against the oracle above)."""
    case = synth.config_case(5)
    say("large layer search in a 2 GB workspace")
    X = dev_tensor(case.X, case.dtype)
    W = dev_tensor(case.W, case.dtype)
    n = len(case.alphas)
    full = awq.search_workspace_size(case.N, case.D_in, case.D_out, X.dtype, 4, 128, n)
    cap = 2 * 10 ** 9
    assert awq.search_workspace_min_size(case.N, case.D_in, case.D_out, X.dtype, 4, 128, n) <= cap < full
    a = awq.act_stats(X)
    outs = []
    for nbytes in (full, cap):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        r = awq.search_layer(X, W, alphas=case.alphas, bits=4, group=128, a=a, workspace=ws)
        torch.cuda.synchronize()
        outs.append((r.losses.cpu().numpy(), r.best_index(), r.s_best.cpu().numpy(), r.scales.cpu().numpy(),
                     r.codes.cpu().numpy()))
        del ws, r
        torch.cuda.empty_cache()
    for x, y in zip(*outs):
        assert np.array_equal(x, y)
