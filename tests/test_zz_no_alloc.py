"""ttq_colstats_noalloc (the statistic with the library's fixed per-GPU
scratch, for callers that cannot allocate) against ttq_colstats (the same
kernels with a caller workspace), through the C ABI: bit for bit, on two calls
in a row, the second with a smaller input (a different shape and dtype, so a
stale partial from the first call would show), and both against the oracle
within the statistic's tolerance.  Sizes past the fixed scratch are refused
before anything is enqueued."""
import numpy as np
import pytest

import oracle
import workloads as wl

torch = pytest.importorskip("torch")
import test_activation_aware_amd as ttq  # noqa: E402
from test_activation_aware_amd import _capi  # noqa: E402

pytestmark = pytest.mark.gpu


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_noalloc_matches_workspace_form_two_calls():
    assert torch.cuda.is_available()
    for cfg, T in ((5, 16384), (1, 333)):   # Qwen3-32B shape, then a smaller fp32 prompt
        w = wl.CONFIGS[cfg]
        X, _ = wl.config_inputs(cfg, T=T, d_out=8)
        print(f"noalloc colstats cfg={cfg} T={T} d={X.shape[1]} dtype={X.dtype}", flush=True)
        Xd = torch.from_numpy(X).cuda()
        D1, R1 = ttq.ttq_colstats(Xd, w.p, w.lam, w.alpha)
        D2, R2 = ttq.ttq_colstats_noalloc(Xd, w.p, w.lam, w.alpha)
        D1, R1, D2, R2 = _host(D1), _host(R1), _host(D2), _host(R2)
        assert D2.tobytes() == D1.tobytes() and R2.tobytes() == R1.tobytes()
        D0 = oracle.colstats(X, w.p, w.lam, w.alpha)
        assert np.max(np.abs(D2.astype(np.float64) - D0) / D0) <= 1e-5


def test_noalloc_refuses_sizes_past_the_scratch():
    lib = ttq.load()
    X = torch.zeros((64, 16384 + 64), dtype=torch.float16, device="cuda")   # d past 16384
    D = torch.empty(16384 + 64, dtype=torch.float32, device="cuda")
    st = lib.ttq_colstats_noalloc(X.data_ptr(), _capi.TTQ_F16, 64, 16384 + 64, 16384 + 64, 2.0, 0.4, 0.5,
                                  D.data_ptr(), D.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == _capi.TTQ_ERR_SHAPE and b"scratch" in lib.ttq_last_error()
