"""Shared helpers of the GPU parity tests: device upload of the seeded inputs
and the tolerance checks (numbers from the method's stated accuracy targets:
loss 1e-3 relative, per-row LSE 2e-3 absolute, gradients 5e-3 relative
Frobenius without filtering and 2e-2 with it, masks and counts exact)."""
import numpy as np

LOSS_RTOL = 1e-3
LSE_ATOL = 2e-3
GRAD_RTOL = 5e-3
GRAD_RTOL_FILTERED = 2e-2


def dev(arr, dtype_name):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype_name == "bf16":
        t = t.to(torch.bfloat16)       # exact: values are bf16-representable
    return t.cuda()


def dev_targets(t):
    import torch
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.int64)).cuda()


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def check_loss(got, want, reduction, label="", n_valid=1):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if reduction == "none":
        # vector reading: relative L2 error and the LSE's absolute bound per row
        assert rel_fro(got, want) <= LOSS_RTOL, (label, rel_fro(got, want))
        assert np.max(np.abs(got - want)) <= LSE_ATOL, (label, np.max(np.abs(got - want)))
    else:
        # relative bound; for a loss near zero (e.g. V = 1) the per-row LSE
        # bound applies instead (summed over the rows a 'sum' adds up)
        err = abs(float(got) - float(want))
        rows = max(n_valid, 1) if reduction == "sum" else 1
        assert err <= LOSS_RTOL * abs(float(want)) or err <= LSE_ATOL * rows, (label, float(got), float(want))


def check_lse(got, want, label=""):
    err = np.max(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64)))
    assert err <= LSE_ATOL, (label, err)


def check_grad(got, want, rtol, label=""):
    err = rel_fro(got, want)
    assert err <= rtol, (label, err)
    return err
