"""The no-allocation forward (cce_forward_noalloc), called through the C ABI,
against cce_forward on the same inputs: loss, LSE and the valid count must be
bitwise equal (the same kernels on the same data), on two calls in a row, the
second with a smaller problem (the static device array keeps the first call's
contents), and the result also matches the oracle."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from helpers import check_loss, check_lse, dev, dev_targets

pytestmark = pytest.mark.gpu


def _noalloc(M, e, c, t, red, bias=None, ls=0.0, zl=0.0, cap=0.0):
    import torch
    N, D = e.shape
    V = c.shape[0]
    code = {"none": 0, "sum": 1, "mean": 2}[red]
    loss = torch.full((N if code == 0 else 1,), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    nv = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dt = 0 if e.dtype == torch.bfloat16 else 1
    st = M.lib().cce_forward_noalloc(e.data_ptr(), c.data_ptr(), None if bias is None else bias.data_ptr(),
                                     t.data_ptr(), N, D, V, dt, -100, code, cap, ls, zl, loss.data_ptr(),
                                     lse.data_ptr(), nv.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, M.lib().cce_status_string(st)
    torch.cuda.synchronize()
    return loss, lse, nv


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import linear_cross_entropy_forward_amd as M
    M.lib()
    return M


@pytest.mark.parametrize("red", ["mean", "none"])
def test_noalloc_forward_matches_forward(M, red):
    import torch
    cases = [
        (W.custom(900, 136, 2100, "bf16", seed=301, c_std=0.1, ignore_frac=0.05), dict()),
        (W.custom(300, 72, 513, "bf16", seed=302, c_std=0.5, ignore_frac=0.1), dict(ls=0.1, zl=1e-3, bias=True)),
    ]
    for k, (inp, terms) in enumerate(cases):
        print(f"[noalloc] call {k} N={inp['e'].shape[0]} V={inp['c'].shape[0]} red={red}", flush=True)
        e, c, t = dev(inp["e"], "bf16"), dev(inp["c"], "bf16"), dev_targets(inp["targets"])
        b = dev(W.bias(c.shape[0], "bf16", seed=303), "bf16") if terms.get("bias") else None
        ls, zl = terms.get("ls", 0.0), terms.get("zl", 0.0)
        got = _noalloc(M, e, c, t, red, bias=b, ls=ls, zl=zl)
        want = M.forward(e, c, t, reduction=red, bias=b, label_smoothing=ls, z_loss=zl)
        torch.cuda.synchronize()
        assert torch.equal(got[0].reshape(-1), want[0].reshape(-1)), "loss differs from cce_forward"
        assert torch.equal(got[1], want[1]), "LSE differs from cce_forward"
        assert int(got[2].item()) == int(want[2].item())
        bias_np = W.bias(c.shape[0], "bf16", seed=303) if b is not None else None
        f = O.forward(inp["e"], inp["c"], inp["targets"], reduction=red, bias=bias_np, label_smoothing=ls,
                      z_loss=zl)
        assert int(got[2].item()) == f.n_valid
        check_loss(got[0].cpu().numpy() if red == "none" else float(got[0][0]), f.loss, red, "noalloc", f.n_valid)
        check_lse(got[1].cpu().numpy(), f.lse, "noalloc")


def test_noalloc_refuses_oversized(M):
    import torch
    N, D, V = 8192, 64, 256000   # state of N x 2000 partial pairs: 131 MB > 64 MiB
    assert M.lib().cce_state_size(N, D, V, 0) > 64 << 20
    e = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    st = M.lib().cce_forward_noalloc(e.data_ptr(), e.data_ptr(), None, e.data_ptr(), N, D, V, 0, -100, 2, 0.0, 0.0,
                                     0.0, e.data_ptr(), e.data_ptr(), None, None)
    assert st == -3
