"""Pins of the fp64 oracle to facts that do not come from the oracle itself:
closed forms, brute force in plain Python, finite differences, invariants and
the values printed by the pages' self-tests (tests/golden/).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a wrong index or count) fails it.
"""
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _rand(seed, N, D, V, scale=1.0):
    g = np.random.default_rng(seed)
    e = g.standard_normal((N, D)) * scale
    c = g.standard_normal((V, D)) * scale
    t = g.integers(0, V, N)
    return e, c, t


# --------------------------------------------------------------------------- golden
def test_golden_zero_logits_1000():
    (V, expect, dec), = _read_golden("zero_logits_1000.txt")
    V, dec = int(V), int(dec)
    e = np.ones((1, 3))
    c = np.zeros((V, 3))
    f = O.forward(e, c, [0], reduction="mean")
    assert round(float(f.loss), dec) == float(expect)
    assert abs(float(f.loss) - math.log(1000.0)) < 1e-12


def test_golden_large_logit_finite():
    (z0, z1, tgt, expect), = _read_golden("large_logit.txt")
    # e = [1], c = [[z0], [z1]] gives the logits (z0, z1).
    e = np.array([[1.0]])
    c = np.array([[float(z0)], [float(z1)]])
    f = O.forward(e, c, [int(tgt)], reduction="none")
    assert np.isfinite(f.nll).all() and np.isfinite(f.lse).all()
    assert abs(float(f.nll[0]) - float(expect)) < 1e-9
    b = O.backward(e, c, [int(tgt)], reduction="sum")
    assert np.isfinite(b.dE).all() and np.isfinite(b.dC).all()
    # p = (1, ~0); G = p - onehot(1) = (1, -1): dE = 1*z0 - 1*z1
    assert abs(b.dE[0, 0] - (float(z0) - float(z1))) < 1e-9


# --------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_zero_classifier_closed_form(reduction):
    """c = 0: every logit is 0, so LSE = ln V, loss = ln V on valid rows,
    G = (1/V - onehot) * scale, dE = 0, dC_j = sum_i scale_i (1/V - [t_i = j]) e_i."""
    N, D, V = 9, 5, 13
    g = np.random.default_rng(3)
    e = g.standard_normal((N, D))
    c = np.zeros((V, D))
    t = g.integers(0, V, N)
    t[[2, 7]] = -100
    nv = N - 2
    gl = g.standard_normal(N) if reduction == "none" else 0.7
    f = O.forward(e, c, t, reduction=reduction)
    assert np.allclose(f.lse, math.log(V), atol=1e-13, rtol=0)
    nll_expect = np.array([0.0 if ti == -100 else math.log(V) for ti in t])
    assert np.allclose(f.nll, nll_expect, atol=1e-13, rtol=0)
    if reduction == "mean":
        assert abs(float(f.loss) - math.log(V)) < 1e-13
    elif reduction == "sum":
        assert abs(float(f.loss) - nv * math.log(V)) < 1e-12
    b = O.backward(e, c, t, reduction=reduction, grad_loss=gl)
    assert np.array_equal(b.dE, np.zeros_like(e))
    dC = np.zeros((V, D))
    for i in range(N):
        if t[i] == -100:
            continue
        s = gl[i] if reduction == "none" else (gl / nv if reduction == "mean" else gl)
        for j in range(V):
            dC[j] += s * ((1.0 / V) - (1.0 if j == t[i] else 0.0)) * e[i]
    assert np.allclose(b.dC, dC, atol=1e-13, rtol=1e-12)


def test_single_class_vocab():
    """V = 1: softmax is 1 on the target, so loss and gradients vanish."""
    g = np.random.default_rng(4)
    e, c = g.standard_normal((6, 4)), g.standard_normal((1, 4))
    t = np.zeros(6, dtype=np.int64)
    f = O.forward(e, c, t, reduction="sum")
    assert abs(float(f.loss)) < 1e-12
    b = O.backward(e, c, t, reduction="mean")
    assert np.abs(b.dE).max() < 1e-15 and np.abs(b.dC).max() < 1e-15


def test_two_class_is_logistic():
    """V = 2 reduces to the logistic loss softplus(z_other - z_target) and its
    gradient sigmoid(z_other - z_target) on the other class."""
    g = np.random.default_rng(5)
    N, D = 11, 3
    e, c = g.standard_normal((N, D)) * 3, g.standard_normal((2, D))
    t = g.integers(0, 2, N)
    z = e @ c.T
    d = z[np.arange(N), 1 - t] - z[np.arange(N), t]
    f = O.forward(e, c, t, reduction="none")
    assert np.allclose(f.nll, np.logaddexp(0.0, d), rtol=1e-13, atol=1e-14)
    sig = 1.0 / (1.0 + np.exp(-d))
    # dE_i = sig*(c_other - c_target) for reduction sum
    b = O.backward(e, c, t, reduction="sum")
    dE = sig[:, None] * (c[1 - t] - c[t])
    assert np.allclose(b.dE, dE, rtol=1e-12, atol=1e-14)


def test_shift_invariance():
    """Appending a constant feature 1 to every e_i and k to every c_j shifts
    every logit by k: LSE shifts by k and the loss does not change."""
    e, c, t = _rand(6, 7, 4, 9)
    for k in (0.0, 3.5, -40.0):
        e2 = np.concatenate([e, np.ones((7, 1))], axis=1)
        c2 = np.concatenate([c, np.full((9, 1), k)], axis=1)
        f1 = O.forward(e, c, t, reduction="none")
        f2 = O.forward(e2, c2, t, reduction="none")
        assert np.allclose(f2.nll, f1.nll, rtol=1e-12, atol=1e-12)
        assert np.allclose(f2.lse, f1.lse + k, rtol=1e-12, atol=1e-12)


def test_translating_classifier_leaves_dE():
    """Each valid row of G sums to zero, so adding one vector u to every c_j
    changes no logit difference and leaves dE unchanged."""
    e, c, t = _rand(7, 6, 5, 8)
    u = np.random.default_rng(70).standard_normal(5)
    b1 = O.backward(e, c, t, reduction="mean")
    b2 = O.backward(e, c + u, t, reduction="mean")
    # dE depends on c through G C; with Z shifted by e_i.u per row G is unchanged
    # and G (C + u) = G C + (G 1) u^T = G C.
    assert np.allclose(b2.dE, b1.dE, rtol=1e-11, atol=1e-13)


def test_gradient_rows_sum_to_zero():
    e, c, t = _rand(8, 10, 6, 17)
    t[3] = -100
    z = e @ c.T
    lse = O.row_logsumexp(z)
    valid = t != -100
    s = O.grad_scale(valid, "sum")
    g = O.softmax_grad_rows(z, lse, t, s, valid)
    assert np.abs(g.sum(axis=1)).max() < 1e-14
    assert np.array_equal(g[3], np.zeros(17))
    # target column carries p - 1 < 0; others p > 0
    for i in np.nonzero(valid)[0]:
        assert g[i, t[i]] < 0 and (np.delete(g[i], t[i]) > 0).all()


# --------------------------------------------------------------------------- brute force
def _brute(e, c, t, reduction, gl, ignore=-100):
    """Loops in plain Python floats: probabilities by exp(z)/sum exp(z)
    (no max subtraction; the inputs are small), loss = -ln p_target."""
    N, D = len(e), len(e[0])
    V = len(c)
    z = [[sum(float(e[i][d]) * float(c[j][d]) for d in range(D)) for j in range(V)] for i in range(N)]
    valid = [int(t[i]) != ignore for i in range(N)]
    nv = sum(valid)
    nll, lse, p = [], [], []
    for i in range(N):
        den = sum(math.exp(z[i][j]) for j in range(V))
        lse.append(math.log(den))
        p.append([math.exp(z[i][j]) / den for j in range(V)])
        nll.append(-math.log(p[i][int(t[i])]) if valid[i] else 0.0)
    if reduction == "none":
        loss = nll
        sc = [gl[i] if valid[i] else 0.0 for i in range(N)]
    elif reduction == "sum":
        loss = sum(nll)
        sc = [gl if valid[i] else 0.0 for i in range(N)]
    else:
        loss = sum(nll) / max(nv, 1)
        sc = [gl / max(nv, 1) if valid[i] else 0.0 for i in range(N)]
    G = [[(p[i][j] - (1.0 if j == int(t[i]) else 0.0)) * sc[i] for j in range(V)] for i in range(N)]
    dE = [[sum(G[i][j] * float(c[j][d]) for j in range(V)) for d in range(D)] for i in range(N)]
    dC = [[sum(G[i][j] * float(e[i][d]) for i in range(N)) for d in range(D)] for j in range(V)]
    return loss, nll, lse, nv, np.array(dE), np.array(dC)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(reduction, seed):
    g = np.random.default_rng(100 + seed)
    N, D, V = int(g.integers(1, 9)), int(g.integers(1, 5)), int(g.integers(2, 17))
    e = g.standard_normal((N, D))
    c = g.standard_normal((V, D))
    t = g.integers(0, V, N)
    if N > 2:
        t[g.integers(0, N)] = -100
    gl = list(g.standard_normal(N)) if reduction == "none" else 1.3
    loss, nll, lse, nv, dE, dC = _brute(e, c, t, reduction, gl)
    f = O.forward(e, c, t, reduction=reduction)
    assert f.n_valid == nv
    assert np.allclose(f.nll, nll, rtol=1e-12, atol=1e-13)
    assert np.allclose(f.lse, lse, rtol=1e-12, atol=1e-13)
    assert np.allclose(f.loss, loss, rtol=1e-12, atol=1e-13)
    b = O.backward(e, c, t, reduction=reduction, grad_loss=np.array(gl) if reduction == "none" else gl)
    assert np.allclose(b.dE, dE, rtol=1e-11, atol=1e-13)
    assert np.allclose(b.dC, dC, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------- finite differences
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_finite_differences(reduction):
    """Central differences of the fp64 loss (h = 1e-6) against dE and dC; for
    `none` the objective is sum_i g_i loss_i with a random upstream g."""
    g = np.random.default_rng(11)
    N, D, V = 5, 3, 7
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D))
    t = g.integers(0, V, N)
    t[1] = -100
    gl = g.standard_normal(N) if reduction == "none" else 0.8

    def obj(ee, cc):
        f = O.forward(ee, cc, t, reduction=reduction)
        return float(np.dot(gl, f.loss)) if reduction == "none" else gl * float(f.loss)

    b = O.backward(e, c, t, reduction=reduction, grad_loss=gl)
    h = 1e-6
    for arr, grad in ((e, b.dE), (c, b.dC)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = obj(e, c)
            arr[idx] = old - h
            lm = obj(e, c)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7 + 1e-6 * abs(fd), (idx, fd, grad[idx])


# --------------------------------------------------------------------------- mask / counts
def test_ignore_rows_and_counts():
    e, c, t = _rand(12, 10, 4, 11)
    t[[0, 4, 9]] = -100
    f = O.forward(e, c, t, reduction="none")
    assert f.n_valid == 7
    assert (f.nll[[0, 4, 9]] == 0.0).all()
    fs = O.forward(e, c, t, reduction="sum")
    fm = O.forward(e, c, t, reduction="mean")
    assert abs(float(fs.loss) - f.nll.sum()) < 1e-12
    assert abs(float(fm.loss) - f.nll.sum() / 7) < 1e-12
    b = O.backward(e, c, t, reduction="mean")
    assert (b.dE[[0, 4, 9]] == 0.0).all()
    # ignored rows contribute nothing to dC: dropping them changes nothing
    keep = np.array([i not in (0, 4, 9) for i in range(10)])
    b2 = O.backward(e[keep], c, t[keep], reduction="sum", grad_loss=1.0 / 7)
    assert np.allclose(b.dC, b2.dC, rtol=1e-12, atol=1e-14)


def test_all_ignored_mean_is_zero():
    e, c, t = _rand(13, 4, 3, 5)
    t[:] = -100
    f = O.forward(e, c, t, reduction="mean")
    assert f.n_valid == 0 and float(f.loss) == 0.0
    b = O.backward(e, c, t, reduction="mean")
    assert not b.dE.any() and not b.dC.any()


def test_custom_ignore_index():
    e, c, t = _rand(14, 6, 3, 5)
    t[2] = 3
    f1 = O.forward(e, c, t, ignore_index=3, reduction="none")
    assert f1.nll[2] == 0.0 and f1.n_valid == 6 - int((t == 3).sum())


def test_out_of_range_target_raises():
    e, c, t = _rand(15, 4, 3, 5)
    t[1] = 5
    with pytest.raises(ValueError):
        O.forward(e, c, t)
    t[1] = -7
    with pytest.raises(ValueError):
        O.forward(e, c, t)


# --------------------------------------------------------------------------- filtering
def _brute_keep(e, c, t, Bn, Bv, ignore=-100):
    """Loops: the k-th non-ignored row (k = 0, 1, ...) is in row block k // Bn."""
    N, V = len(e), len(c)
    z = e @ c.T
    nb, nvb = -(-N // Bn), -(-V // Bv)
    keep = np.zeros((nb, nvb), dtype=bool)
    k = 0
    for i in range(N):
        if t[i] == ignore:
            continue
        den = sum(math.exp(z[i, j]) for j in range(V))
        for j in range(V):
            if math.exp(z[i, j]) / den >= 2.0 ** -12 or j == t[i]:
                keep[k // Bn, j // Bv] = True
        k += 1
    return keep


@pytest.mark.parametrize("Bn,Bv", [(2, 3), (4, 8), (3, 5)])
def test_filter_keep_brute_force(Bn, Bv):
    g = np.random.default_rng(21)
    N, D, V = 11, 4, 37
    e, c = g.standard_normal((N, D)) * 5.0, g.standard_normal((V, D)) * 2.5
    t = g.integers(0, V, N)
    t[5] = -100
    keep = O.filter_keep(e, c, t, Bn, Bv)
    assert np.array_equal(keep, _brute_keep(e, c, t, Bn, Bv))
    assert 0 < keep.sum() < keep.size       # the case exercises both outcomes
    lse, keep2 = O.lse_and_keep(e, c, t, Bn, Bv)
    assert np.array_equal(keep, keep2)


def test_filtered_backward_drops_exactly_the_dropped_tiles():
    g = np.random.default_rng(22)
    N, D, V, Bn, Bv = 12, 4, 40, 3, 8
    e, c = g.standard_normal((N, D)) * 2.5, g.standard_normal((V, D)) * 1.5
    t = g.integers(0, V, N)
    keep = O.filter_keep(e, c, t, Bn, Bv)
    full = O.backward(e, c, t, reduction="sum")
    filt = O.backward(e, c, t, reduction="sum", keep=keep, tile=(Bn, Bv))
    # independent: sum of the dropped G entries' contributions, with loops
    z = e @ c.T
    dE = full.dE.copy()
    dC = full.dC.copy()
    for i in range(N):
        den = np.exp(z[i]).sum()
        for j in range(V):
            if not keep[i // Bn, j // Bv]:
                gij = math.exp(z[i, j]) / den - (1.0 if j == t[i] else 0.0)
                assert abs(gij) < 2.0 ** -12      # only sub-threshold entries are dropped
                dE[i] -= gij * c[j]
                dC[j] -= gij * e[i]
    assert np.allclose(filt.dE, dE, rtol=1e-12, atol=1e-14)
    assert np.allclose(filt.dC, dC, rtol=1e-12, atol=1e-14)
    # keep everything -> exact
    allk = np.ones_like(keep)
    b = O.backward(e, c, t, reduction="sum", keep=allk, tile=(Bn, Bv))
    assert np.allclose(b.dE, full.dE, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------- sampled forms
def test_sampled_forms_match_full():
    g = np.random.default_rng(31)
    N, D, V, Bn, Bv = 40, 6, 50, 8, 16
    e, c = g.standard_normal((N, D)) * 2.0, g.standard_normal((V, D))
    t = g.integers(0, V, N)
    t[[3, 17]] = -100
    for red in ("mean", "sum", "none"):
        gl = g.standard_normal(N) if red == "none" else 1.7
        f = O.forward(e, c, t, reduction=red)
        b = O.backward(e, c, t, reduction=red, grad_loss=gl)
        rows = np.array([0, 3, 9, 39])
        fr = O.forward(e, c, t, reduction="none", rows=rows)
        assert np.allclose(fr.lse, f.lse[rows], rtol=1e-14)
        assert np.allclose(fr.nll, f.nll[rows], rtol=1e-14)
        assert np.allclose(O.dE_rows(e, c, t, rows, reduction=red, grad_loss=gl), b.dE[rows],
                           rtol=1e-12, atol=1e-15)
        vid = np.array([0, 7, 49, int(t[0])])
        lse = O.lse_all(e, c, chunk=7)
        assert np.allclose(lse, f.lse, rtol=1e-14)
        assert np.allclose(O.dC_rows(e, c, t, vid, lse, reduction=red, grad_loss=gl), b.dC[vid],
                           rtol=1e-12, atol=1e-15)
    lse, keep = O.lse_and_keep(e, c, t, Bn, Bv)
    bf = O.backward(e, c, t, reduction="mean", keep=keep, tile=(Bn, Bv))
    assert np.allclose(O.dE_rows(e, c, t, [1, 20], keep=keep, tile=(Bn, Bv)), bf.dE[[1, 20]],
                       rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dC_rows(e, c, t, [2, 33], lse, keep=keep, tile=(Bn, Bv)), bf.dC[[2, 33]],
                       rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------- classifier bias
# The bias b [V] (README "API": classifier bias) is added to every row of the
# logits; its gradient is db = G^T 1.


def test_bias_closed_form_zero_classifier():
    """c = 0 and b_j = ln(j + 1): every row's logits are b, so
    sum_j exp(b_j) = V (V + 1) / 2 exactly, LSE = ln(V (V + 1) / 2),
    loss_i = LSE - ln(y_i + 1), p_j = (j + 1) / (V (V + 1) / 2), dE = 0 and
    db_j = sum_i scale_i (p_j - [y_i = j])."""
    N, D, V = 6, 3, 9
    g = np.random.default_rng(41)
    e = g.standard_normal((N, D))
    c = np.zeros((V, D))
    b = np.log(np.arange(1, V + 1, dtype=np.float64))
    t = np.array([0, 8, 3, -100, 3, 5])
    tot = V * (V + 1) / 2.0
    f = O.forward(e, c, t, reduction="sum", bias=b)
    assert np.allclose(f.lse, math.log(tot), rtol=0, atol=1e-13)
    want = sum(math.log(tot) - math.log(y + 1) for y in t if y != -100)
    assert abs(float(f.loss) - want) < 1e-12
    bw = O.backward(e, c, t, reduction="sum", bias=b)
    assert not bw.dE.any()
    p = np.arange(1, V + 1) / tot
    db = np.zeros(V)
    for y in t:
        if y != -100:
            db += p
            db[y] -= 1.0
    assert np.allclose(bw.db, db, rtol=1e-12, atol=1e-14)


def test_bias_as_extra_feature():
    """(e, c, b) equals the bias-free problem with e' = [e, 1], c' = [c, b]:
    same loss and LSE, the same dE and dC in the first D columns, and db is
    the extra column of dC'."""
    g = np.random.default_rng(42)
    N, D, V = 9, 5, 13
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D))
    b = g.standard_normal(V) * 2.0
    t = g.integers(0, V, N)
    t[4] = -100
    ea = np.concatenate([e, np.ones((N, 1))], axis=1)
    ca = np.concatenate([c, b[:, None]], axis=1)
    for red in ("mean", "none"):
        gl = g.standard_normal(N) if red == "none" else 0.7
        f1 = O.forward(e, c, t, reduction=red, bias=b)
        f2 = O.forward(ea, ca, t, reduction=red)
        assert np.allclose(f1.lse, f2.lse, rtol=1e-13) and np.allclose(f1.loss, f2.loss, rtol=1e-13)
        b1 = O.backward(e, c, t, reduction=red, grad_loss=gl, bias=b)
        b2 = O.backward(ea, ca, t, reduction=red, grad_loss=gl)
        assert np.allclose(b1.dE, b2.dE[:, :D], rtol=1e-12, atol=1e-15)
        assert np.allclose(b1.dC, b2.dC[:, :D], rtol=1e-12, atol=1e-15)
        assert np.allclose(b1.db, b2.dC[:, D], rtol=1e-12, atol=1e-15)


def test_bias_constant_shift_and_sum():
    """A constant bias shifts every LSE by the constant and changes neither the
    loss nor any gradient; db sums to zero (each valid row of G sums to 0)."""
    e, c, t = _rand(43, 7, 4, 10)
    t[2] = -100
    f0 = O.forward(e, c, t, reduction="none")
    fk = O.forward(e, c, t, reduction="none", bias=np.full(10, 3.25))
    assert np.allclose(fk.lse, f0.lse + 3.25, rtol=1e-14)
    assert np.allclose(fk.nll, f0.nll, rtol=1e-12, atol=1e-14)
    b0 = O.backward(e, c, t, reduction="mean")
    bk = O.backward(e, c, t, reduction="mean", bias=np.full(10, 3.25))
    assert np.allclose(bk.dE, b0.dE, rtol=1e-12, atol=1e-15) and np.allclose(bk.dC, b0.dC, rtol=1e-12, atol=1e-15)
    bb = O.backward(e, c, t, reduction="mean", bias=np.linspace(-2, 2, 10))
    assert abs(bb.db.sum()) < 1e-14


def test_bias_finite_differences():
    g = np.random.default_rng(44)
    N, D, V = 5, 3, 8
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D))
    b = g.standard_normal(V)
    t = g.integers(0, V, N)
    t[0] = -100
    bw = O.backward(e, c, t, reduction="mean", bias=b)
    h = 1e-6
    for j in range(V):
        bp, bm = b.copy(), b.copy()
        bp[j] += h
        bm[j] -= h
        fd = (float(O.forward(e, c, t, reduction="mean", bias=bp).loss)
              - float(O.forward(e, c, t, reduction="mean", bias=bm).loss)) / (2 * h)
        assert abs(fd - bw.db[j]) < 1e-8 + 1e-6 * abs(fd), (j, fd, bw.db[j])


def test_bias_brute_force_filter_and_sampled():
    """Filtering with a bias: a strongly negative bias on one vocab block drops
    its tiles except where a target lies; the keep map matches loops over the
    biased softmax; sampled db / dC / dE forms match the full backward."""
    g = np.random.default_rng(45)
    N, D, V, Bn, Bv = 10, 4, 24, 5, 8
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D)) * 0.5
    b = np.zeros(V)
    b[8:16] = -40.0
    t = g.choice(np.r_[0:8, 16:24], N)        # targets outside the suppressed block ...
    t[1] = 9                                  # ... except one
    keep = O.filter_keep(e, c, t, Bn, Bv, bias=b)
    z = e @ c.T + b[None, :]
    want = np.zeros_like(keep)
    for i in range(N):
        den = sum(math.exp(z[i, j]) for j in range(V))
        for j in range(V):
            if math.exp(z[i, j]) / den >= 2.0 ** -12 or j == t[i]:
                want[i // Bn, j // Bv] = True
    assert np.array_equal(keep, want)
    assert keep[0, 1] and not keep[1, 1]      # block 1 kept only for row block 0 (target 9)
    lse, keep2 = O.lse_and_keep(e, c, t, Bn, Bv, bias=b)
    assert np.array_equal(keep, keep2)
    full = O.backward(e, c, t, reduction="sum", bias=b, keep=keep, tile=(Bn, Bv))
    vid = np.array([0, 9, 12, 23])
    assert np.allclose(O.db_rows(e, c, t, vid, lse, reduction="sum", bias=b, keep=keep, tile=(Bn, Bv)),
                       full.db[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dC_rows(e, c, t, vid, lse, reduction="sum", bias=b, keep=keep, tile=(Bn, Bv)),
                       full.dC[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dE_rows(e, c, t, [0, 7], reduction="sum", bias=b, keep=keep, tile=(Bn, Bv)),
                       full.dE[[0, 7]], rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------- label smoothing, z-loss
# Label smoothing eps replaces the one-hot target by (1 - eps) onehot + eps / V
# (tirogla "Loss functions", "How it works" step 3); the z-loss adds
# lam * LSE^2 per row (same page, "Implementation notes").


@pytest.mark.parametrize("eps", [0.0, 0.15])
@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_label_smoothing_matches_torch_cross_entropy(reduction, eps):
    """Loss and gradients equal PyTorch's cross_entropy (with label_smoothing
    eps, which spreads eps over all V classes, the true one included; eps = 0
    is the plain loss), differentiated by autograd in float64 on the CPU
    through Z = E C^T + b."""
    import torch
    g = np.random.default_rng(50)
    N, D, V = 11, 6, 17
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D))
    b = g.standard_normal(V)
    t = g.integers(0, V, N)
    t[[3, 8]] = -100
    gl = g.standard_normal(N) if reduction == "none" else 0.6
    te, tc, tb = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (e, c, b))
    z = te @ tc.T + tb
    ref = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=-100, reduction=reduction,
                                            label_smoothing=eps)
    ref.backward(torch.tensor(gl, dtype=torch.float64))
    f = O.forward(e, c, t, reduction=reduction, bias=b, label_smoothing=eps)
    assert np.allclose(f.loss, ref.detach().numpy(), rtol=1e-12, atol=1e-14)
    bw = O.backward(e, c, t, reduction=reduction, grad_loss=gl, bias=b, label_smoothing=eps)
    assert np.allclose(bw.dE, te.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(bw.dC, tc.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(bw.db, tb.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_full_smoothing_closed_form():
    """eps = 1 (uniform target), c = 0, b_j = ln(j + 1): loss_i is
    LSE - (1/V) sum_j b_j = ln(V (V + 1) / 2) - ln(V!) / V on every valid row,
    independent of the target, and db_j = sum_i scale_i (p_j - 1/V)."""
    N, D, V = 5, 3, 7
    e = np.random.default_rng(51).standard_normal((N, D))
    c = np.zeros((V, D))
    b = np.log(np.arange(1, V + 1, dtype=np.float64))
    t = np.array([0, 6, -100, 2, 2])
    tot = V * (V + 1) / 2.0
    f = O.forward(e, c, t, reduction="none", bias=b, label_smoothing=1.0)
    want = math.log(tot) - math.lgamma(V + 1) / V
    assert np.allclose(f.nll, [want, want, 0.0, want, want], rtol=1e-13, atol=0)
    bw = O.backward(e, c, t, reduction="sum", grad_loss=2.0, bias=b, label_smoothing=1.0)
    assert not bw.dE.any()
    p = np.arange(1, V + 1) / tot
    assert np.allclose(bw.db, 4 * 2.0 * (p - 1.0 / V), rtol=1e-12, atol=1e-15)


def test_z_loss_closed_form():
    """c = 0, b_j = ln(j + 1), z-loss lam: LSE = ln(V (V + 1) / 2) = L on every
    row, loss_i = L - ln(y_i + 1) + lam L^2, and
    db_j = sum_i scale_i (p_j (1 + 2 lam L) - [y_i = j])."""
    N, D, V, lam = 6, 2, 9, 0.03
    e = np.random.default_rng(52).standard_normal((N, D))
    c = np.zeros((V, D))
    b = np.log(np.arange(1, V + 1, dtype=np.float64))
    t = np.array([1, 8, 3, -100, 3, 0])
    L = math.log(V * (V + 1) / 2.0)
    f = O.forward(e, c, t, reduction="mean", bias=b, z_loss=lam)
    want = sum(L - math.log(y + 1) + lam * L * L for y in t if y != -100) / 5
    assert abs(float(f.loss) - want) < 1e-13
    bw = O.backward(e, c, t, reduction="mean", bias=b, z_loss=lam)
    p = np.arange(1, V + 1) / (V * (V + 1) / 2.0)
    db = np.zeros(V)
    for y in t:
        if y != -100:
            db += p * (1 + 2 * lam * L)
            db[y] -= 1.0
    assert np.allclose(bw.db, db / 5, rtol=1e-12, atol=1e-15)
    assert not bw.dE.any()


@pytest.mark.parametrize("eps,lam", [(0.0, 0.05), (0.2, 0.0), (0.2, 0.05)])
def test_smoothing_z_loss_finite_differences(eps, lam):
    """Central differences of the oracle's own forward loss against its
    backward, for every entry of e, c and b (so a dropped factor 2 in the
    z-loss gradient, or a smoothing term with the wrong sign, fails)."""
    g = np.random.default_rng(53)
    N, D, V = 4, 3, 6
    e, c = g.standard_normal((N, D)), g.standard_normal((V, D))
    b = g.standard_normal(V)
    t = g.integers(0, V, N)
    t[2] = -100
    kw = dict(reduction="mean", label_smoothing=eps, z_loss=lam)
    bw = O.backward(e, c, t, bias=b, **kw)

    def loss(e_, c_, b_):
        return float(O.forward(e_, c_, t, bias=b_, **kw).loss)
    h = 1e-6
    for arr, grad, which in ((e, bw.dE, 0), (c, bw.dC, 1), (b, bw.db, 2)):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            args_p, args_m = [e.copy(), c.copy(), b.copy()], [e.copy(), c.copy(), b.copy()]
            args_p[which][ix] += h
            args_m[which][ix] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[ix]) < 1e-8 + 1e-6 * abs(fd), (which, ix, fd, grad[ix])


def test_smoothing_filter_keeps_uniform_term():
    """Filtering with smoothing: a vocab block suppressed by a bias of -60 has
    softmax below e^-50 everywhere, so its tiles are dropped (but for the one
    that holds a target), yet the filtered gradients equal the unfiltered ones
    to 1e-12: the -eps/V term of those entries is kept.  The classifier rows of
    the block have mean 3, so dropping that term would move dE by about
    eps/V * 8 * 3 per unit scale.  The sampled forms agree with the full one."""
    g = np.random.default_rng(54)
    N, D, V, Bn, Bv, eps, lam = 10, 4, 24, 5, 8, 0.3, 0.01
    e, c = g.standard_normal((N, D)) * 0.5, g.standard_normal((V, D)) * 0.5
    c[8:16] += 3.0
    b = np.zeros(V)
    b[8:16] = -60.0
    t = g.choice(np.r_[0:8, 16:24], N)
    t[1] = 9
    kw = dict(reduction="sum", bias=b, label_smoothing=eps, z_loss=lam)
    keep = O.filter_keep(e, c, t, Bn, Bv, bias=b)
    assert keep[0, 1] and not keep[1, 1]
    flt = O.backward(e, c, t, keep=keep, tile=(Bn, Bv), **kw)
    full = O.backward(e, c, t, **kw)
    for a, w in ((flt.dE, full.dE), (flt.dC, full.dC), (flt.db, full.db)):
        assert np.allclose(a, w, rtol=0, atol=1e-12)
    assert np.abs(full.dE).max() > 0.05
    lse, _ = O.lse_and_keep(e, c, t, Bn, Bv, bias=b)
    vid = np.array([0, 9, 12, 23])
    kk = dict(keep=keep, tile=(Bn, Bv), **kw)
    assert np.allclose(O.db_rows(e, c, t, vid, lse, **kk), flt.db[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dC_rows(e, c, t, vid, lse, **kk), flt.dC[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dE_rows(e, c, t, [0, 7], **kk), flt.dE[[0, 7]], rtol=1e-12, atol=1e-15)


def test_smoothing_filtered_drops_only_softmax_part():
    """With ordinary logits some tiles are dropped; the filtered and unfiltered
    dE then differ by exactly the dropped softmax entries times C, each entry
    below 2^-12 (1 + 2 lam LSE) scale, computed here by loops over entries."""
    g = np.random.default_rng(55)
    N, D, V, Bn, Bv, eps, lam = 6, 3, 40, 3, 8, 0.1, 0.02
    e, c = g.standard_normal((N, D)) * 2.0, g.standard_normal((V, D)) * 2.0
    t = g.integers(0, V, N)
    keep = O.filter_keep(e, c, t, Bn, Bv)
    assert not keep.all()
    kw = dict(reduction="sum", label_smoothing=eps, z_loss=lam)
    flt = O.backward(e, c, t, keep=keep, tile=(Bn, Bv), **kw)
    full = O.backward(e, c, t, **kw)
    want = full.dE.copy()
    for i in range(N):
        zi = [float(np.dot(e[i], c[j])) for j in range(V)]
        mx = max(zi)
        L = mx + math.log(sum(math.exp(z - mx) for z in zi))
        for j in range(V):
            if not keep[i // Bn, j // Bv]:
                p = math.exp(zi[j] - L) * (1 + 2 * lam * L)
                assert p < 2.0 ** -12 * (1 + 2 * lam * L)
                want[i] -= p * c[j]
    assert np.allclose(flt.dE, want, rtol=1e-11, atol=1e-14)


def test_one_pass_lse_keep_nll_matches_separate_forms():
    """lse_keep_nll (the single pass full-size checks use) gives the same LSE,
    keep map and per-row loss as forward and filter_keep, with bias,
    smoothing and z-loss."""
    g = np.random.default_rng(56)
    N, D, V, Bn, Bv = 23, 5, 41, 8, 16
    e, c = g.standard_normal((N, D)) * 1.5, g.standard_normal((V, D))
    b = g.standard_normal(V)
    t = g.integers(0, V, N)
    t[[2, 19]] = -100
    lse, keep, nll = O.lse_keep_nll(e, c, t, Bn, Bv, bias=b, label_smoothing=0.2, z_loss=0.01)
    f = O.forward(e, c, t, reduction="none", bias=b, label_smoothing=0.2, z_loss=0.01)
    assert np.allclose(lse, f.lse, rtol=1e-14) and np.allclose(nll, f.nll, rtol=1e-13, atol=0)
    assert np.array_equal(keep, O.filter_keep(e, c, t, Bn, Bv, bias=b))


def test_keep_margins_brute_force():
    """The per-tile margins (largest log-softmax maximum over a tile's valid
    rows) and target-tile flags, against explicit loops over rows and
    entries; the keep map is exactly margin >= ln 2^-12 or a target inside."""
    g = np.random.default_rng(57)
    N, D, V, Bn, Bv = 19, 4, 45, 4, 8
    e, c = g.standard_normal((N, D)) * 3.0, g.standard_normal((V, D)) * 2.0
    t = g.integers(0, V, N)
    t[[3, 4, 11]] = -100
    lse, keep, nll, margin, tgt = O.lse_keep_nll(e, c, t, Bn, Bv, margins=True)
    nb, nvb = -(-N // Bn), -(-V // Bv)
    want_m = np.full((nb, nvb), -np.inf)
    want_t = np.zeros((nb, nvb), dtype=bool)
    k = 0
    for i in range(N):
        if t[i] == -100:
            continue
        zi = [sum(e[i, d] * c[j, d] for d in range(D)) for j in range(V)]
        logden = math.log(sum(math.exp(x) for x in zi))
        for j in range(V):
            want_m[k // Bn, j // Bv] = max(want_m[k // Bn, j // Bv], zi[j] - logden)
        want_t[k // Bn, t[i] // Bv] = True
        k += 1
    fin = np.isfinite(want_m)
    assert np.array_equal(fin, np.isfinite(margin))
    assert np.allclose(margin[fin], want_m[fin], rtol=0, atol=1e-11)
    assert np.array_equal(tgt, want_t)
    assert np.array_equal(keep, (margin >= O.FILTER_LOG_THRESHOLD) | tgt)
    assert 0 < keep.sum() < keep.size and (keep & ~tgt).any()
    # the same pass without margins returns the same three results
    lse2, keep2, nll2 = O.lse_keep_nll(e, c, t, Bn, Bv)
    assert np.array_equal(keep, keep2) and np.array_equal(lse, lse2) and np.array_equal(nll, nll2)


def test_keep_margins_coarsen_across_tile_sizes():
    """The filter at two granularities from one pass: the margins and target
    flags of 8x8-entry tiles equal the 4x4-entry blocks' coarsened two by two
    (tests.helpers.coarsen_keep), with ignored rows in the input (row blocks
    are cut from the non-ignored rows at both sizes)."""
    from helpers import coarsen_keep
    g = np.random.default_rng(58)
    N, D, V = 37, 4, 61
    e, c = g.standard_normal((N, D)) * 2.5, g.standard_normal((V, D)) * 2.0
    t = g.integers(0, V, N)
    t[[0, 9, 10, 30]] = -100
    _, keep4, _, m4, t4 = O.lse_keep_nll(e, c, t, 4, 4, margins=True)
    _, keep8, _, m8, t8 = O.lse_keep_nll(e, c, t, 8, 8, margins=True)
    mc, tc = coarsen_keep(m4, t4, 2)
    fin = np.isfinite(m8)
    assert np.array_equal(np.isfinite(mc), fin) and np.array_equal(mc[fin], m8[fin])
    assert np.array_equal(tc, t8)
    assert np.array_equal(keep8, (mc >= O.FILTER_LOG_THRESHOLD) | tc)
    assert keep4.sum() < 4 * keep8.sum()   # the finer map drops entries the coarser keeps


# --------------------------------------------------------------------------- logit soft-capping
# Not defined on the pages: the Gemma 2 form Z' = s tanh(Z / s), after the bias.


@pytest.mark.parametrize("reduction,eps,lam", [("mean", 0.0, 0.0), ("none", 0.1, 0.0), ("sum", 0.0, 0.02),
                                               ("mean", 0.2, 0.01)])
def test_softcap_matches_torch_autograd(reduction, eps, lam):
    """Capped loss and gradients equal PyTorch's cross_entropy on
    s * tanh((E C^T + b) / s), plus lam * logsumexp^2 on valid rows,
    differentiated by autograd in float64 on the CPU."""
    import torch
    g = np.random.default_rng(60)
    N, D, V, s = 12, 5, 19, 2.5
    e, c = g.standard_normal((N, D)) * 1.5, g.standard_normal((V, D)) * 1.5
    b = g.standard_normal(V)
    t = g.integers(0, V, N)
    t[[1, 7]] = -100
    gl = g.standard_normal(N) if reduction == "none" else 0.8
    te, tc, tb = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (e, c, b))
    zc = s * torch.tanh((te @ tc.T + tb) / s)
    tt = torch.tensor(t)
    ce = torch.nn.functional.cross_entropy(zc, tt, ignore_index=-100, reduction="none", label_smoothing=eps)
    valid = torch.tensor(t != -100, dtype=torch.float64)
    per = ce + lam * torch.logsumexp(zc, dim=1) ** 2 * valid
    nv = max(int(valid.sum()), 1)
    ref = per if reduction == "none" else (per.sum() if reduction == "sum" else per.sum() / nv)
    ref.backward(torch.tensor(gl, dtype=torch.float64))
    kw = dict(reduction=reduction, bias=b, label_smoothing=eps, z_loss=lam, softcap=s)
    f = O.forward(e, c, t, **kw)
    assert np.allclose(f.loss, ref.detach().numpy(), rtol=1e-12, atol=1e-14)
    bw = O.backward(e, c, t, grad_loss=gl, **kw)
    assert np.allclose(bw.dE, te.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(bw.dC, tc.grad.numpy(), rtol=1e-11, atol=1e-14)
    assert np.allclose(bw.db, tb.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_softcap_saturated_closed_form():
    """Logits of +-1e4 with s = 5 saturate: tanh(2000) is 1 in fp64, so every
    capped logit is +-5 exactly, LSE = ln(k e^5 + (V - k) e^-5) for k
    positive logits, and every gradient is exactly 0 (the cap's derivative
    1 - tanh^2 vanishes)."""
    N, D, V, s = 4, 2, 6, 5.0
    e = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 0.0]]) * 100.0
    c = np.array([[1, 1], [-1, 1], [1, -1], [-1, -1], [1, 0.5], [-1, 0.5]], dtype=np.float64) * 100.0
    # every product is +-1e4 or +-5e3 (or +-1.5e4 / 0 for row 2: keep only nonzero rows' logic simple)
    z = e @ c.T
    t = np.array([0, 3, -100, 5])
    f = O.forward(e, c, t, reduction="none", softcap=s)
    for i in range(N):
        zi = np.where(z[i] > 0, s, np.where(z[i] < 0, -s, 0.0))
        want = math.log(sum(math.exp(x) for x in zi))
        assert abs(f.lse[i] - want) < 1e-12
        if t[i] != -100:
            assert abs(f.nll[i] - (want - zi[t[i]])) < 1e-12
    bw = O.backward(e, c, t, reduction="sum", softcap=s)
    sat = np.abs(z[[0, 1, 3]]) >= 1e3
    assert sat.all()
    assert np.abs(bw.dE[[0, 1, 3]]).max() < 1e-300 and np.abs(bw.dC).max() < 1e-300


def test_softcap_large_cap_is_uncapped():
    e, c, t = _rand(61, 7, 4, 11)
    t[3] = -100
    a = O.forward(e, c, t, reduction="none", softcap=1e7)
    b = O.forward(e, c, t, reduction="none")
    assert np.allclose(a.nll, b.nll, rtol=1e-9) and np.allclose(a.lse, b.lse, rtol=1e-9)
    ga = O.backward(e, c, t, reduction="mean", softcap=1e7)
    gb = O.backward(e, c, t, reduction="mean")
    assert np.allclose(ga.dE, gb.dE, rtol=1e-8, atol=1e-14) and np.allclose(ga.dC, gb.dC, rtol=1e-8, atol=1e-14)


def test_softcap_filter_brute_force_and_sampled():
    """Keep map on the capped softmax against loops over entries (a block
    pushed down by the bias is dropped); sampled dE, dC and db forms against
    the full filtered backward, with z-loss."""
    g = np.random.default_rng(62)
    N, D, V, Bn, Bv, s = 10, 4, 48, 5, 8, 6.0
    e, c = g.standard_normal((N, D)) * 2.0, g.standard_normal((V, D)) * 2.0
    b = g.standard_normal(V)
    b[16:24] -= 40.0                            # capped to about -s: below 2^-12 for every row
    t = g.choice(np.r_[0:16, 24:48], N)
    t[4] = -100
    keep = O.filter_keep(e, c, t, Bn, Bv, bias=b, softcap=s)
    want = np.zeros_like(keep)
    k = 0                                       # rank among the non-ignored rows
    for i in range(N):
        if t[i] == -100:
            continue
        zi = [s * math.tanh((float(np.dot(e[i], c[j])) + b[j]) / s) for j in range(V)]
        den = sum(math.exp(x) for x in zi)
        for j in range(V):
            if math.exp(zi[j]) / den >= 2.0 ** -12 or j == t[i]:
                want[k // Bn, j // Bv] = True
        k += 1
    assert np.array_equal(keep, want)
    assert not keep.all()
    kw = dict(reduction="sum", bias=b, softcap=s, z_loss=0.01)
    full = O.backward(e, c, t, keep=keep, tile=(Bn, Bv), **kw)
    lse, keep2, _ = O.lse_keep_nll(e, c, t, Bn, Bv, bias=b, softcap=s, z_loss=0.01)
    assert np.array_equal(keep, keep2)
    assert np.allclose(lse, O.lse_all(e, c, bias=b, softcap=s), rtol=1e-14)
    vid = np.array([0, 9, 30, 47])
    kk = dict(keep=keep, tile=(Bn, Bv), **kw)
    assert np.allclose(O.db_rows(e, c, t, vid, lse, **kk), full.db[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dC_rows(e, c, t, vid, lse, **kk), full.dC[vid], rtol=1e-12, atol=1e-15)
    assert np.allclose(O.dE_rows(e, c, t, [0, 7], **kk), full.dE[[0, 7]], rtol=1e-12, atol=1e-15)
    with pytest.raises(NotImplementedError):
        O.backward(e, c, t, keep=keep, tile=(Bn, Bv), reduction="sum", softcap=s, label_smoothing=0.1)


# --------------------------------------------------------------------------- padded-row compaction
def test_filter_tiles_skip_ignored_rows():
    """Tiles are cut from the non-ignored rows (padding skipped, the Loss
    functions page's "Efficiency"): with ignored rows interleaved, the
    filtered gradients equal those of the same problem with the ignored rows
    deleted (their dE rows are 0), with 'sum' so the scales agree; the keep
    maps agree block for block."""
    g = np.random.default_rng(63)
    N, D, V, Bn, Bv = 23, 4, 45, 4, 8
    e, c = g.standard_normal((N, D)) * 2.0, g.standard_normal((V, D)) * 2.0
    t = g.integers(0, V, N)
    ign = np.array([1, 2, 7, 8, 9, 15, 22])
    t[ign] = -100
    keep = O.filter_keep(e, c, t, Bn, Bv)
    v = t != -100
    keep_d = O.filter_keep(e[v], c, t[v], Bn, Bv)
    nb = keep_d.shape[0]
    assert np.array_equal(keep[:nb], keep_d) and not keep[nb:].any()
    assert 0 < keep.sum() < keep.size
    kw = dict(reduction="sum", label_smoothing=0.1, z_loss=0.01)
    a = O.backward(e, c, t, keep=keep, tile=(Bn, Bv), **kw)
    b = O.backward(e[v], c, t[v], keep=keep_d, tile=(Bn, Bv), **kw)
    assert np.allclose(a.dE[v], b.dE, rtol=1e-12, atol=1e-15) and not a.dE[~v].any()
    assert np.allclose(a.dC, b.dC, rtol=1e-12, atol=1e-15) and np.allclose(a.db, b.db, rtol=1e-12, atol=1e-15)
    lse, keep2, _ = O.lse_keep_nll(e, c, t, Bn, Bv)
    assert np.array_equal(keep, keep2)
    vid = np.array([0, 13, 44])
    assert np.allclose(O.dC_rows(e, c, t, vid, lse, keep=keep, tile=(Bn, Bv), **kw), a.dC[vid], rtol=1e-12,
                       atol=1e-15)
    assert np.allclose(O.dE_rows(e, c, t, [0, 3, 21], keep=keep, tile=(Bn, Bv), **kw), a.dE[[0, 3, 21]],
                       rtol=1e-12, atol=1e-15)


def test_empty_batch_is_an_empty_sum():
    """N = 0: every reduction is an empty sum (the mean's count is floored at
    1, Loss functions page, "Code"), so the loss is 0 and dC, db are 0."""
    c = np.random.default_rng(3).standard_normal((50, 8))
    e0, t0 = np.zeros((0, 8)), np.zeros(0, np.int64)
    for red in ("mean", "sum"):
        f = O.forward(e0, c, t0, reduction=red)
        assert f.loss == 0.0 and f.n_valid == 0
    assert O.forward(e0, c, t0, reduction="none").loss.shape == (0,)
    b = O.backward(e0, c, t0, reduction="mean", label_smoothing=0.1, bias=np.zeros(50))
    assert b.dE.shape == (0, 8) and not b.dC.any() and not b.db.any()
