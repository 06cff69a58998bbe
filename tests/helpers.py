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
        # 1e-3 relative.  Only a reduced loss whose own size is below the
        # per-row LSE bound (times the rows a 'sum' adds up), e.g. V = 1 or a
        # softmax saturated on the targets, is held to that absolute bound:
        # its rows are differences of LSE and logit, each exact only to it.
        err = abs(float(got) - float(want))
        floor = LSE_ATOL * (max(n_valid, 1) if reduction == "sum" else 1)
        if abs(float(want)) < floor:
            assert err <= floor, (label, float(got), float(want))
        else:
            assert err <= LOSS_RTOL * abs(float(want)), (label, float(got), float(want), err / abs(float(want)))


# A kernel's tile keep decision may differ from the oracle's only on tiles
# whose oracle margin max_i (max_j z_ij - LSE_i) lies within this distance of
# ln 2^-12: the kernel's per-block maxima and LSE are fp32 values, each within
# the LSE bound of the exact ones.
KEEP_MARGIN_TOL = 2 * LSE_ATOL


def check_keep(got, margin, tgt, threshold, label=""):
    """Tile-by-tile keep map: equal to the oracle's (margin >= threshold or a
    target inside) except on tiles without a target whose margin is within
    KEEP_MARGIN_TOL of the threshold.  Returns the number of such tiles that
    differ."""
    got = np.asarray(got, dtype=bool)
    want = (margin >= threshold) | tgt
    assert got.shape == want.shape, (label, got.shape, want.shape)
    diff = got != want
    near = ~tgt & (np.abs(margin - threshold) <= KEEP_MARGIN_TOL)
    bad = diff & ~near
    assert not bad.any(), (label, "keep map differs on", int(bad.sum()), "tiles away from the threshold",
                           np.argwhere(bad)[:5].tolist())
    return int(diff.sum())


def check_lse(got, want, label=""):
    err = np.max(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64)))
    assert err <= LSE_ATOL, (label, err)


def check_grad(got, want, rtol, label=""):
    err = rel_fro(got, want)
    assert err <= rtol, (label, err)
    return err


def coarsen_keep(margin, tgt, k):
    """Margins and target flags of tiles made of k x k blocks, from those of
    the blocks: a tile's largest log-softmax value is the largest of its
    blocks', and it holds a target iff one of its blocks does (row blocks and
    tiles are both cut from the non-ignored rows in order, so tile rows are
    whole groups of k block rows)."""
    margin = np.asarray(margin, dtype=np.float64)
    tgt = np.asarray(tgt, dtype=bool)
    nb, nv = margin.shape
    NB, NV = -(-nb // k), -(-nv // k)
    m = np.full((NB * k, NV * k), -np.inf)
    m[:nb, :nv] = margin
    t = np.zeros((NB * k, NV * k), dtype=bool)
    t[:nb, :nv] = tgt
    return m.reshape(NB, k, NV, k).max(axis=(1, 3)), t.reshape(NB, k, NV, k).any(axis=(1, 3))
