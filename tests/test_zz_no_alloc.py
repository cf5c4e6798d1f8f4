"""The allocation-free W4A16 entry point, through the C ABI, against the
workspace entry point it shares its kernels with (and against the oracle).

Named to be collected last: the calls share the library's static scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import GEMM_TOL, dev_tensor, say
from weight_only_quantization_awq_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_quantization_awq_amd import awq
    return awq.load()


def _operands(M, D_in, D_out, group, seed):
    rng = np.random.default_rng(seed)
    X = synth.to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))
    q = rng.integers(-7, 8, (D_in, D_out)).astype(np.int8)
    words = oracle.pack_int4(q)
    scales = rng.uniform(0.001, 0.01, (D_in // group, D_out)).astype(np.float32)
    inv_s = rng.uniform(0.1, 2.0, D_in).astype(np.float32)
    return X, words, scales, inv_s


def _call_both(lib, M, D_in, D_out, group, seed):
    X, words, scales, inv_s = _operands(M, D_in, D_out, group, seed)
    Xd = dev_tensor(X, "bf16")
    Pd = torch.from_numpy(words.view(np.int32)).cuda()
    Sd = torch.from_numpy(scales).cuda()
    Id = torch.from_numpy(inv_s).cuda()
    stream = torch.cuda.current_stream().cuda_stream
    need = lib.awq_w4a16_workspace_size(M, D_in, D_out, 1)
    assert 0 < need <= lib.awq_w4a16_noalloc_scratch_bytes()
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    Y_ws = torch.empty(M, D_out, dtype=torch.float32, device="cuda")
    Y_na = torch.full((M, D_out), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.awq_w4a16_gemm(Xd.data_ptr(), M, D_in, D_out, Pd.data_ptr(), Sd.data_ptr(), group, Id.data_ptr(),
                            Y_ws.data_ptr(), 0, ws.data_ptr(), need, stream)
    assert st == 0, lib.awq_last_error()
    st = lib.awq_w4a16_gemm_noalloc(Xd.data_ptr(), M, D_in, D_out, Pd.data_ptr(), Sd.data_ptr(), group,
                                    Id.data_ptr(), Y_na.data_ptr(), 0, stream)
    assert st == 0, lib.awq_last_error()
    torch.cuda.synchronize()
    Yref = oracle.w4a16_gemm(X, words, scales, group, inv_s=inv_s)
    return Y_ws.cpu().numpy(), Y_na.cpu().numpy(), Yref


def test_noalloc_matches_workspace_entry_point_twice(lib):
    """Two calls in a row on the shared scratch, the second smaller; each uses
    the scratch (the activation pre-pass and split-k partials)."""
    for (M, D_in, D_out, group, seed) in [(6, 8192, 8200, 128, 1), (40, 2048, 264, 64, 2)]:
        say("noalloc gemm", M, D_in, D_out, group)
        Y_ws, Y_na, Yref = _call_both(lib, M, D_in, D_out, group, seed)
        assert np.array_equal(Y_ws, Y_na)                       # same kernels, same order
        err = np.abs(Y_na.astype(np.float64) - Yref).max()
        assert err <= GEMM_TOL * np.abs(Yref).max(), err


def test_noalloc_rejects_oversized_shape(lib):
    """A shape whose scratch exceeds the static array: AWQ_ERR_WORKSPACE, nothing launched."""
    say("noalloc oversized")
    M, D_in, D_out = 4096, 8192, 28672
    assert lib.awq_w4a16_workspace_size(M, D_in, D_out, 1) > lib.awq_w4a16_noalloc_scratch_bytes()
    Y = torch.full((1,), 7.0, device="cuda")
    X = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    st = lib.awq_w4a16_gemm_noalloc(X.data_ptr(), M, D_in, D_out, X.data_ptr(), X.data_ptr(), 128, None,
                                    Y.data_ptr(), 0, torch.cuda.current_stream().cuda_stream)
    assert st == -4
    assert b"static scratch" in lib.awq_last_error()
    torch.cuda.synchronize()
    assert Y.item() == 7.0
