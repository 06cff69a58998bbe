"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Small cases span several 256x256 tiles with ragged edges in every dimension
(N, V and D not multiples of the tile sizes) and run the whole oracle;
full-size cases (marked slow) run the launch configuration the benchmark
times and compare sampled outputs the oracle computes row by row.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from helpers import (GRAD_RTOL, GRAD_RTOL_FILTERED, check_grad, check_keep, check_loss, check_lse, coarsen_keep,
                     dev, dev_targets, rel_fro)

# The filter's two levels: gradient tiles of 256 x 256 (decided from the
# forward's partials) and, inside kept tiles, blocks of 32 x 32 (decided from
# the recomputed softmax).  The oracle's filtered gradient applies the block
# rule; the tile map is the block map coarsened.
BLOCK = 32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import linear_cross_entropy_forward_amd as M
    M.lib()
    return M


def _grad_arg(reduction, N, seed=0):
    import torch
    if reduction == "none":
        g = np.random.default_rng(seed).standard_normal(N).astype(np.float32)
        return g, torch.from_numpy(g).cuda()
    return 1.0, torch.ones(1, dtype=torch.float32, device="cuda")


def run(M, inp, reduction="mean", filter=False, accum="deterministic", vocab_chunk=0, ignore_index=-100,
        backward=True, grad_seed=0, bias=None, want_db=False, ls=0.0, zl=0.0, cap=0.0, grad_dtype="float32"):
    import torch
    dt = inp.get("dtype") or inp["workload"].dtype
    e, c, t = dev(inp["e"], dt), dev(inp["c"], dt), dev_targets(inp["targets"])
    b = dev(bias, dt) if bias is not None else None
    N, V = e.shape[0], c.shape[0]
    loss, lse, nv, ws = M.forward(e, c, t, ignore_index=ignore_index, reduction=reduction,
                                  bias=b, label_smoothing=ls, z_loss=zl, softcap=cap)
    out = {"loss": None, "lse": None}
    torch.cuda.synchronize()
    out["stats_fwd"] = M.read_stats(ws, N, V)
    if backward:
        g_np, g = _grad_arg(reduction, N, grad_seed)
        D = e.shape[1]
        bws = torch.empty(M.workspace_size(N, D, V, e.dtype, vocab_chunk), dtype=torch.uint8, device="cuda")
        res = M.backward(e, c, t, lse, g, ws, ignore_index=ignore_index, reduction=reduction, filter=filter,
                         accum=accum, vocab_chunk=vocab_chunk, bias=b, want_dbias=want_db, label_smoothing=ls,
                         z_loss=zl, softcap=cap, grad_dtype=grad_dtype, ws=bws)
        torch.cuda.synchronize()
        out["keep"] = M.read_keep_map(bws, N, D, V, e.dtype, vocab_chunk)
        out["blocks"] = M.read_block_map(bws, N, D, V, e.dtype, vocab_chunk)
        del bws
        out["dE"], out["dC"], out["g"] = res[0].float().cpu().numpy(), res[1].float().cpu().numpy(), g_np
        if want_db:
            out["db"] = res[2].cpu().numpy()
        out["stats"] = M.read_stats(ws, N, V)
    out["loss"] = loss.cpu().numpy()
    out["lse"] = lse.cpu().numpy()
    out["n_valid"] = int(nv.cpu().item())
    return out


def filtered_bound(filtered_oracle, exact_oracle):
    """Bound on the filtered GPU result's distance from the exact gradient:
    2e-2, or, where the method's own filter already drops more than that (the
    2^-12 threshold on isotropic synthetic classifiers), the filtered oracle's
    distance from exact plus the unfiltered tolerance."""
    return max(GRAD_RTOL_FILTERED, rel_fro(filtered_oracle, exact_oracle) + GRAD_RTOL)


def full_check(M, inp, reduction, filter, accum="deterministic", vocab_chunk=0, ignore_index=-100, label="",
               bias=None, want_db=False, ls=0.0, zl=0.0, cap=0.0, grad_dtype="float32"):
    e, c, t = inp["e"], inp["c"], inp["targets"]
    r = run(M, inp, reduction, filter, accum, vocab_chunk, ignore_index, bias=bias, want_db=want_db, ls=ls, zl=zl,
            cap=cap, grad_dtype=grad_dtype)
    terms = dict(label_smoothing=ls, z_loss=zl, softcap=cap)
    f = O.forward(e, c, t, ignore_index=ignore_index, reduction=reduction, bias=bias, **terms)
    assert r["n_valid"] == f.n_valid, label
    assert r["stats_fwd"]["n_valid"] == f.n_valid
    check_loss(r["loss"], f.loss, reduction, label, f.n_valid)
    check_lse(r["lse"], f.lse, label)
    if reduction == "none":
        assert (r["loss"][~f.valid] == 0.0).all(), "ignored rows must give exactly 0"
    b = O.backward(e, c, t, ignore_index=ignore_index, reduction=reduction, grad_loss=r["g"], bias=bias, **terms)
    assert (r["dE"][~f.valid] == 0.0).all(), "ignored rows must give exactly 0 gradient"
    Bn, Bv, _ = M.tile_shape()
    if filter:
        lse_o, keep, _, margin, tgt = O.lse_keep_nll(e, c, t, BLOCK, BLOCK, ignore_index=ignore_index, bias=bias,
                                                     softcap=cap, margins=True)
        mt, tt = coarsen_keep(margin, tgt, Bn // BLOCK)
        check_keep(r["keep"], mt, tt, O.FILTER_LOG_THRESHOLD, label + " tiles")
        check_keep(r["blocks"], margin, tgt, O.FILTER_LOG_THRESHOLD, label + " blocks")
        assert r["stats"]["blocks_kept"] == int(r["blocks"].sum())
        bf = O.backward(e, c, t, ignore_index=ignore_index, reduction=reduction, grad_loss=r["g"], keep=keep,
                        tile=(BLOCK, BLOCK), bias=bias, **terms)
        check_grad(r["dE"], bf.dE, GRAD_RTOL, label + " dE vs filtered oracle")
        check_grad(r["dC"], bf.dC, GRAD_RTOL, label + " dC vs filtered oracle")
        check_grad(r["dE"], b.dE, filtered_bound(bf.dE, b.dE), label + " dE vs exact")
        check_grad(r["dC"], b.dC, filtered_bound(bf.dC, b.dC), label + " dC vs exact")
        if want_db:
            check_grad(r["db"], bf.db, GRAD_RTOL, label + " db vs filtered oracle")
            check_grad(r["db"], b.db, filtered_bound(bf.db, b.db), label + " db vs exact")
        assert r["stats"]["tiles_kept"] == int(r["keep"].sum())
    else:
        check_grad(r["dE"], b.dE, GRAD_RTOL, label + " dE")
        check_grad(r["dC"], b.dC, GRAD_RTOL, label + " dC")
        if want_db:
            check_grad(r["db"], b.db, GRAD_RTOL, label + " db")
        # every tile of the blocks of non-ignored rows (blocks of padding only drop out)
        nvb = -(-c.shape[0] // Bv)
        assert r["stats"]["tiles_kept"] == -(-f.n_valid // Bn) * nvb, (r["stats"], f.n_valid)
        want_keep = np.zeros_like(r["keep"])
        want_keep[:-(-f.n_valid // Bn)] = True
        assert np.array_equal(r["keep"], want_keep)
        # unfiltered: every block of the computed tiles is kept
        want_blocks = np.zeros_like(r["blocks"])
        want_blocks[:-(-f.n_valid // Bn) * (Bn // BLOCK)] = True
        assert np.array_equal(r["blocks"], want_blocks)
        assert r["stats"]["blocks_kept"] == int(r["blocks"].sum())
    return r


# ----------------------------------------------------------------------------- small, whole oracle
def test_tiny_workload_fp32(M):
    inp = W.get("tiny")
    for flt in (False, True):
        full_check(M, inp, "mean", flt, label=f"tiny filter={flt}")


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_ragged_bf16(M, reduction):
    inp = W.custom(600, 136, 1100, "bf16", seed=11, c_std=0.1, ignore_frac=0.05)
    full_check(M, inp, reduction, False, label=f"ragged {reduction}")


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ragged_fp32(M, reduction):
    inp = W.custom(300, 68, 513, "f32", seed=12, c_std=0.2, ignore_frac=0.1)
    full_check(M, inp, reduction, True, label=f"ragged fp32 {reduction}")


@pytest.mark.parametrize("mode", ["trained", "calibrated"])
def test_filtering_peaked(M, mode):
    inp = W.custom(777, 264, 2600, "bf16", seed=13, e_mode=mode, targets="zipf", ignore_frac=0.03)
    r = full_check(M, inp, "mean", True, label=f"filter {mode}")
    if mode == "trained":
        assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"], "peaked softmax should skip tiles"


@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_compact_chunks_sparse_keep(M, accum):
    # bf16 gradient tiles are stored compactly and the backward's chunks are
    # cut by kept tiles: with a 256-wide chunk basis a chunk holds at most
    # S + nb - 1 = 2 * 4 - 1 kept tiles (N = 777: 4 token blocks) but spans
    # as many vocab tiles as the peaked softmax leaves kept tiles for, so
    # chunks of very different widths (and empty chunk numbers) occur.
    inp = W.custom(777, 264, 9000, "bf16", seed=21, e_mode="trained", targets="zipf", ignore_frac=0.03)
    r = full_check(M, inp, "mean", True, accum=accum, vocab_chunk=256, label=f"compact sparse {accum}")
    assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"] // 2, "peaked softmax should skip most tiles"
    # the same with a bias gradient and label smoothing (every vocab row's
    # dC and db come from the chunk that owns it, kept tiles or not)
    bias = W.bias(9000, "bf16", seed=22)
    full_check(M, inp, "sum", True, accum=accum, vocab_chunk=512, label=f"compact sparse terms {accum}", bias=bias,
               want_db=True, ls=0.1)


@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_vocab_chunks_and_splits(M, accum):
    # 256-wide vocabulary chunks: many chunks, several dE splits, ragged last chunk
    inp = W.custom(530, 200, 1900, "bf16", seed=14, c_std=0.08, ignore_frac=0.05)
    full_check(M, inp, "sum", False, accum=accum, vocab_chunk=256, label=f"chunks {accum}")
    full_check(M, inp, "mean", True, accum=accum, vocab_chunk=512, label=f"chunks filtered {accum}")


def test_deterministic_bitwise(M):
    inp = W.custom(700, 256, 3000, "bf16", seed=15, c_std=0.05, ignore_frac=0.02)
    runs = [run(M, inp, "mean", True, "deterministic") for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r["loss"], runs[0]["loss"])
        assert np.array_equal(r["lse"], runs[0]["lse"])
        assert np.array_equal(r["dE"], runs[0]["dE"])
        assert np.array_equal(r["dC"], runs[0]["dC"])
    ra = run(M, inp, "mean", True, "atomic")
    assert rel_fro(ra["dE"], runs[0]["dE"]) < 1e-5
    assert np.array_equal(ra["dC"], runs[0]["dC"])


# ----------------------------------------------------------------------------- edge cases
def test_single_class_vocab(M):
    inp = W.custom(100, 64, 1, "bf16", seed=16, c_std=0.5)
    r = full_check(M, inp, "sum", False, label="V=1")
    assert np.abs(r["loss"]).max() < 1e-4   # 100 rows of LSE - z_y, each ~1e-6 from rounding order


def test_two_class_vocab(M):
    inp = W.custom(260, 40, 2, "bf16", seed=17, c_std=0.5)
    full_check(M, inp, "none", False, label="V=2")


def test_single_row(M):
    inp = W.custom(1, 32, 700, "bf16", seed=18, c_std=0.3)
    full_check(M, inp, "mean", True, label="N=1")


def test_all_ignored(M):
    inp = W.custom(300, 64, 900, "bf16", seed=19, c_std=0.1)
    inp["targets"][:] = -100
    r = run(M, inp, "mean", True)
    assert r["n_valid"] == 0 and float(r["loss"]) == 0.0
    assert not r["dE"].any() and not r["dC"].any()


def test_no_ignored_and_extreme_targets(M):
    inp = W.custom(513, 96, 1537, "bf16", seed=20, c_std=0.1)
    t = inp["targets"]
    t[::3] = 0
    t[1::3] = 1536
    full_check(M, inp, "mean", True, label="targets 0 and V-1")


def test_repeated_targets(M):
    inp = W.custom(400, 64, 1000, "bf16", seed=21, c_std=0.1)
    inp["targets"][:] = 777
    full_check(M, inp, "sum", False, label="repeated target")


def test_large_logits(M):
    # logits of order 1e3: the LSE must come out finite and within 2e-3
    inp = W.custom(256, 64, 600, "bf16", seed=22, c_std=0.1)
    inp["e"] = W.round_to_bf16(inp["e"] * 400.0)
    r = full_check(M, inp, "none", True, label="large logits")
    assert np.isfinite(r["lse"]).all() and np.isfinite(r["dE"]).all()


def test_custom_ignore_index(M):
    inp = W.custom(320, 64, 500, "bf16", seed=23, c_std=0.1)
    inp["targets"][::4] = 7
    full_check(M, inp, "mean", False, ignore_index=7, label="ignore_index=7")


def test_bad_target_is_loud(M):
    inp = W.custom(64, 32, 100, "bf16", seed=24, c_std=0.1)
    inp["targets"][5] = 100          # out of range, not the ignore index
    r = run(M, inp, "none", False)
    assert math.isnan(r["loss"][5]) and np.isfinite(np.delete(r["loss"], 5)).all()
    assert r["stats_fwd"]["bad_targets"] == 1
    assert np.isnan(r["dE"][5]).all()


# ----------------------------------------------------------------------------- padded-row compaction
@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_padding_compacted(M, accum):
    """40% of the rows ignored, as trailing padding and scattered: the
    backward works on the valid rows only (blocks of padding drop out of every
    contraction), dE rows of ignored rows are exactly 0, and results match
    the oracle, whose filter tiles are cut from the valid rows."""
    inp = W.custom(1100, 136, 1300, "bf16", seed=61, c_std=0.1)
    t = inp["targets"]
    t[700:] = -100
    t[::9] = -100
    r = full_check(M, inp, "mean", False, accum=accum, label=f"padding {accum}")
    assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"]
    full_check(M, inp, "none", True, accum=accum, vocab_chunk=512, label=f"padding filtered {accum}")


def test_padding_with_all_terms(M):
    inp = W.custom(900, 72, 1100, "bf16", seed=62, c_std=0.1, ignore_frac=0.3)
    bias = W.bias(1100, "bf16", seed=62)
    full_check(M, inp, "sum", True, label="padding smoothing", bias=bias, want_db=True, ls=0.1, zl=1e-4)
    full_check(M, inp, "mean", True, label="padding softcap", bias=bias, want_db=True, zl=1e-4, cap=5.0)


# ----------------------------------------------------------------------------- classifier bias
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_bias_ragged_bf16(M, reduction):
    inp = W.custom(600, 136, 1100, "bf16", seed=31, c_std=0.1, ignore_frac=0.05)
    bias = W.bias(1100, "bf16", seed=31)
    full_check(M, inp, reduction, False, label=f"bias {reduction}", bias=bias, want_db=True)


def test_bias_ragged_fp32_filtered(M):
    inp = W.custom(300, 68, 513, "f32", seed=32, c_std=0.2, ignore_frac=0.1)
    bias = W.bias(513, "f32", seed=32, std=1.0)
    full_check(M, inp, "mean", True, label="bias fp32", bias=bias, want_db=True)


def test_bias_suppressed_block_is_filtered(M):
    """A strongly negative bias on vocab block 1 makes the filter drop its
    tiles (except those holding a target); forward, dE, dC and db agree with
    the filtered oracle, and the kept count matches its keep map."""
    inp = W.custom(700, 136, 1300, "bf16", seed=33, c_std=0.1)
    t = inp["targets"]
    inp["targets"] = np.where((t >= 256) & (t < 512), t - 256, t)   # no target inside the suppressed block
    bias = W.bias(1300, "bf16", seed=33, block_offsets={(256, 512): -40.0})
    r = full_check(M, inp, "sum", True, label="bias suppressed block", bias=bias, want_db=True)
    assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"]


@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_bias_with_vocab_chunks(M, accum):
    inp = W.custom(520, 72, 1400, "bf16", seed=34, c_std=0.1, ignore_frac=0.02)
    bias = W.bias(1400, "bf16", seed=34)
    full_check(M, inp, "mean", False, accum=accum, vocab_chunk=512, label=f"bias chunks {accum}", bias=bias,
               want_db=True)


def test_no_bias_gradient_is_column_sum(M):
    """Without a bias, dbias is still the gradient at b = 0: G's column sums."""
    inp = W.custom(400, 64, 700, "bf16", seed=35, c_std=0.1)
    full_check(M, inp, "mean", False, label="db without bias", want_db=True)


def test_bias_autograd(M):
    import torch
    inp = W.custom(260, 64, 900, "bf16", seed=36, c_std=0.1, ignore_frac=0.05)
    bias = W.bias(900, "bf16", seed=36)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16").requires_grad_(True)
    b = dev(bias, "bf16").requires_grad_(True)
    t = dev_targets(inp["targets"]).reshape(20, 13)
    loss = M.linear_cross_entropy(e.reshape(20, 13, 64), c, t, bias=b)
    loss.backward()
    f = O.forward(inp["e"], inp["c"], inp["targets"], bias=bias)
    bo = O.backward(inp["e"], inp["c"], inp["targets"], bias=bias)
    check_loss(loss.detach().float().cpu().numpy(), f.loss, "mean", "autograd bias", f.n_valid)
    assert b.grad is not None and b.grad.dtype == torch.bfloat16
    # gradients come back in bf16 (the inputs' dtype): allow the rounding
    check_grad(b.grad.float().cpu().numpy(), bo.db, GRAD_RTOL * 2, "autograd db")
    check_grad(c.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL * 2, "autograd dC")
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL * 2, "autograd dE")


def test_autograd_per_token_loss(M):
    """reduction='none' through autograd: the loss shaped like the targets
    ([20, 13]), ignored positions exactly 0, and a non-uniform upstream
    gradient (a weighted sum of the per-token losses) reaching dE and dC."""
    import torch
    inp = W.custom(260, 64, 900, "bf16", seed=37, c_std=0.1, ignore_frac=0.1)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16").requires_grad_(True)
    t = dev_targets(inp["targets"]).reshape(20, 13)
    w_np = np.random.default_rng(38).standard_normal(260).astype(np.float32)
    w = torch.from_numpy(w_np).cuda().reshape(20, 13)
    loss = M.linear_cross_entropy(e.reshape(20, 13, 64), c, t, reduction="none", filter=False)
    assert loss.shape == (20, 13) and loss.dtype == torch.float32
    (loss * w).sum().backward()
    f = O.forward(inp["e"], inp["c"], inp["targets"], reduction="none")
    check_loss(loss.detach().reshape(-1).cpu().numpy(), f.loss, "none", "autograd none")
    assert (loss.detach().reshape(-1).cpu().numpy()[~f.valid] == 0.0).all()
    bo = O.backward(inp["e"], inp["c"], inp["targets"], reduction="none", grad_loss=w_np.astype(np.float64))
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL * 2, "autograd none dE")
    check_grad(c.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL * 2, "autograd none dC")


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_scaled_upstream_gradient(M, reduction):
    """A reduced loss scaled before backward (loss scaling): the upstream
    gradient 3.5 multiplies every gradient."""
    import torch
    inp = W.custom(300, 72, 700, "bf16", seed=39, c_std=0.1, ignore_frac=0.1)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16").requires_grad_(True)
    t = dev_targets(inp["targets"])
    (3.5 * M.linear_cross_entropy(e, c, t, reduction=reduction, filter=False)).backward()
    bo = O.backward(inp["e"], inp["c"], inp["targets"], reduction=reduction, grad_loss=3.5)
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL * 2, f"scaled {reduction} dE")
    check_grad(c.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL * 2, f"scaled {reduction} dC")


# ----------------------------------------------------------------------------- label smoothing, z-loss
@pytest.mark.parametrize("reduction,ls,zl", [("mean", 0.1, 1e-4), ("none", 0.1, 0.0), ("sum", 0.0, 0.05),
                                             ("mean", 1.0, 0.0)])
def test_smoothing_zloss_ragged_bf16(M, reduction, ls, zl):
    inp = W.custom(600, 136, 1100, "bf16", seed=41, c_std=0.1, ignore_frac=0.05)
    full_check(M, inp, reduction, False, label=f"terms {reduction} ls={ls} zl={zl}", ls=ls, zl=zl)


def test_smoothing_zloss_bias_fp32_filtered(M):
    inp = W.custom(300, 68, 513, "f32", seed=42, c_std=0.2, ignore_frac=0.1)
    bias = W.bias(513, "f32", seed=42, std=1.0)
    full_check(M, inp, "mean", True, label="terms fp32 bias", bias=bias, want_db=True, ls=0.2, zl=1e-3)


def test_smoothing_suppressed_block_keeps_uniform_term(M):
    """A bias of -40 on vocab block 1 makes the filter drop its tiles, while the
    block's classifier rows are shifted by +0.5 so that the uniform -eps/V
    term over them is far above the tolerance: filtered dE, dC and db must
    still carry it (the filtered oracle keeps it on every entry)."""
    inp = W.custom(700, 136, 1300, "bf16", seed=43, c_std=0.1)
    t = inp["targets"]
    inp["targets"] = np.where((t >= 256) & (t < 512), t - 256, t)
    inp["c"][256:512] = W.round_to_bf16(inp["c"][256:512] + 0.5)
    bias = W.bias(1300, "bf16", seed=43, block_offsets={(256, 512): -40.0})
    r = full_check(M, inp, "sum", True, label="terms suppressed block", bias=bias, want_db=True, ls=0.3, zl=1e-4)
    assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"]


@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_smoothing_vocab_chunks(M, accum):
    # several chunks and dE splits: the smoothing term enters dE once (chunk 0,
    # split 0, or the atomic mode's initial fill)
    inp = W.custom(530, 200, 1900, "bf16", seed=44, c_std=0.08, ignore_frac=0.05)
    full_check(M, inp, "mean", False, accum=accum, vocab_chunk=256, label=f"terms chunks {accum}", ls=0.1,
               zl=1e-4)
    full_check(M, inp, "none", True, accum=accum, vocab_chunk=512, label=f"terms chunks filtered {accum}",
               ls=0.1, zl=1e-4)


def test_smoothing_deterministic_bitwise(M):
    inp = W.custom(700, 256, 3000, "bf16", seed=45, c_std=0.05, ignore_frac=0.02)
    runs = [run(M, inp, "mean", True, "deterministic", ls=0.1, zl=1e-4) for _ in range(2)]
    for k in ("loss", "lse", "dE", "dC"):
        assert np.array_equal(runs[1][k], runs[0][k]), k


def test_smoothing_autograd(M):
    import torch
    inp = W.custom(260, 64, 900, "bf16", seed=46, c_std=0.1, ignore_frac=0.05)
    bias = W.bias(900, "bf16", seed=46)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16").requires_grad_(True)
    b = dev(bias, "bf16").requires_grad_(True)
    t = dev_targets(inp["targets"]).reshape(20, 13)
    loss = M.linear_cross_entropy(e.reshape(20, 13, 64), c, t, bias=b, label_smoothing=0.1, z_loss=1e-3)
    loss.backward()
    kw = dict(bias=bias, label_smoothing=0.1, z_loss=1e-3)
    f = O.forward(inp["e"], inp["c"], inp["targets"], **kw)
    bo = O.backward(inp["e"], inp["c"], inp["targets"], **kw)
    check_loss(loss.detach().float().cpu().numpy(), f.loss, "mean", "autograd terms", f.n_valid)
    check_grad(b.grad.float().cpu().numpy(), bo.db, GRAD_RTOL * 2, "autograd terms db")
    check_grad(c.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL * 2, "autograd terms dC")
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL * 2, "autograd terms dE")


# ----------------------------------------------------------------------------- logit soft-capping
# (not defined on the pages: the Gemma 2 form s tanh(z / s))
@pytest.mark.parametrize("reduction", ["mean", "none", "sum"])
def test_softcap_ragged_bf16(M, reduction):
    # logit std about 3.5 against a cap of 4: the cap bends most logits
    inp = W.custom(600, 136, 1100, "bf16", seed=51, c_std=0.3, ignore_frac=0.05)
    full_check(M, inp, reduction, False, label=f"softcap {reduction}", cap=4.0)


@pytest.mark.skip(reason="soft-capping with fp32 operands is switched off: this case hung the GPU once and "
                         "no cause has been found in the code; the library rejects it (CCE_ERR_UNSUPPORTED)")
def test_softcap_bias_zloss_fp32_filtered(M):
    inp = W.custom(300, 68, 513, "f32", seed=52, c_std=0.5, ignore_frac=0.1)
    bias = W.bias(513, "f32", seed=52, std=1.0)
    full_check(M, inp, "mean", True, label="softcap fp32 bias zloss", bias=bias, want_db=True, zl=1e-3, cap=6.0)


def test_softcap_fp32_is_rejected(M):
    inp = W.custom(64, 32, 100, "f32", seed=58, c_std=0.1)
    with pytest.raises(M.CCEError):
        run(M, inp, "mean", backward=False, cap=5.0)


def test_softcap_bias_zloss_bf16_filtered(M):
    inp = W.custom(300, 72, 513, "bf16", seed=52, c_std=0.5, ignore_frac=0.1)
    bias = W.bias(513, "bf16", seed=52, std=1.0)
    full_check(M, inp, "mean", True, label="softcap bf16 bias zloss", bias=bias, want_db=True, zl=1e-3, cap=6.0)


def test_softcap_filtering_peaked(M):
    """Peaked (trained-like) logits capped at 30 still leave most tiles below
    2^-12: the capped softmax decides, as in the filtered oracle."""
    inp = W.custom(777, 264, 2600, "bf16", seed=53, e_mode="trained", targets="zipf", ignore_frac=0.03)
    r = full_check(M, inp, "mean", True, label="softcap filter trained", cap=30.0)
    assert r["stats"]["tiles_kept"] < r["stats"]["tiles_total"]


@pytest.mark.parametrize("accum", ["deterministic", "atomic"])
def test_softcap_vocab_chunks(M, accum):
    inp = W.custom(530, 200, 1900, "bf16", seed=54, c_std=0.3, ignore_frac=0.05)
    bias = W.bias(1900, "bf16", seed=54)
    full_check(M, inp, "sum", False, accum=accum, vocab_chunk=256, label=f"softcap chunks {accum}", bias=bias,
               want_db=True, cap=5.0)


def test_softcap_saturated(M):
    """Logits of order 300 against a cap of 2: nearly every capped logit is
    +-2 exactly and its gradient factor 1 - (z'/s)^2 exactly 0; only the few
    logits within about 10 of zero carry gradient.  Everything stays finite
    and matches the oracle."""
    inp = W.custom(256, 64, 600, "bf16", seed=55, c_std=0.1)
    inp["e"] = W.round_to_bf16(inp["e"] * 400.0)
    r = full_check(M, inp, "none", True, label="softcap saturated", cap=2.0)
    assert np.isfinite(r["lse"]).all() and np.isfinite(r["dE"]).all() and np.isfinite(r["dC"]).all()


def test_softcap_autograd(M):
    inp = W.custom(260, 64, 900, "bf16", seed=56, c_std=0.3, ignore_frac=0.05)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16").requires_grad_(True)
    t = dev_targets(inp["targets"])
    loss = M.linear_cross_entropy(e, c, t, softcap=3.0, z_loss=1e-3)
    loss.backward()
    kw = dict(softcap=3.0, z_loss=1e-3)
    f = O.forward(inp["e"], inp["c"], inp["targets"], **kw)
    bo = O.backward(inp["e"], inp["c"], inp["targets"], **kw)
    check_loss(loss.detach().float().cpu().numpy(), f.loss, "mean", "autograd softcap", f.n_valid)
    check_grad(c.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL * 2, "autograd softcap dC")
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL * 2, "autograd softcap dE")


def test_softcap_with_smoothing_is_rejected(M):
    inp = W.custom(64, 32, 100, "bf16", seed=57, c_std=0.1)
    with pytest.raises(M.CCEError):
        run(M, inp, "mean", backward=False, ls=0.1, cap=5.0)


# ----------------------------------------------------------------------------- optional gradients
@pytest.mark.parametrize("dt,accum,chunk,ls", [("bf16", "deterministic", 0, 0.0), ("bf16", "deterministic", 512, 0.1),
                                             ("bf16", "atomic", 512, 0.0), ("f32", "deterministic", 0, 0.1)])
def test_optional_gradients(M, dt, accum, chunk, ls):
    """dE alone, dC alone and db alone equal the same gradients of a full
    call (bitwise where the accumulation order is fixed)."""
    import torch
    inp = W.custom(530, 200, 1500, dt, seed=81, c_std=0.05, ignore_frac=0.1)
    print(f"[optional grads] {dt} {accum} chunk={chunk} ls={ls}", flush=True)
    e, c, t = dev(inp["e"], dt), dev(inp["c"], dt), dev_targets(inp["targets"])
    b = dev(W.bias(1500, dt, seed=3), dt)
    loss, lse, nv, ws = M.forward(e, c, t, bias=b, label_smoothing=ls)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    kw = dict(filter=True, accum=accum, vocab_chunk=chunk, bias=b, label_smoothing=ls)
    dE, dC, db = M.backward(e, c, t, lse, g, ws, want_dbias=True, **kw)
    dE1, none1 = M.backward(e, c, t, lse, g, ws, want_dC=False, **kw)
    none2, dC2 = M.backward(e, c, t, lse, g, ws, want_dE=False, **kw)
    none3, none4, db3 = M.backward(e, c, t, lse, g, ws, want_dE=False, want_dC=False, want_dbias=True, **kw)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None and none3 is None and none4 is None
    assert torch.equal(dC2, dC) and torch.equal(db3, db)
    if accum == "deterministic":
        assert torch.equal(dE1, dE)
    else:
        check_grad(dE1.cpu().numpy(), dE.cpu().numpy(), 1e-5, "atomic dE alone")


def test_autograd_frozen_classifier(M):
    """c.requires_grad = False: only e's gradient is formed (dC's contraction
    does not run) and it matches the full gradient."""
    import torch
    inp = W.custom(400, 136, 1100, "bf16", seed=83, c_std=0.1, ignore_frac=0.05)
    e = dev(inp["e"], "bf16").requires_grad_(True)
    c = dev(inp["c"], "bf16")
    t = dev_targets(inp["targets"])
    M.linear_cross_entropy(e, c, t).backward()
    assert c.grad is None and e.grad is not None and e.grad.dtype == torch.bfloat16
    bo = O.backward(inp["e"], inp["c"], inp["targets"])
    check_grad(e.grad.float().cpu().numpy(), bo.dE, GRAD_RTOL_FILTERED, "frozen-classifier dE")
    c2 = dev(inp["c"], "bf16").requires_grad_(True)
    e2 = dev(inp["e"], "bf16")
    M.linear_cross_entropy(e2, c2, t).backward()
    assert e2.grad is None and c2.grad is not None
    check_grad(c2.grad.float().cpu().numpy(), bo.dC, GRAD_RTOL_FILTERED, "frozen-inputs dC")


# ----------------------------------------------------------------------------- HIP graph capture
def test_hip_graph_capture(M):
    """A forward+backward step captured in a HIP graph (torch.cuda.graph) and
    replayed: forward and backward allocate, free, synchronise and memset
    nothing, so the capture holds their kernels alone.  Each replay, with new
    inputs copied in and eager work in between, equals the eager step
    bitwise (deterministic mode), and the first matches the oracle."""
    import torch
    dt = "bf16"
    inps = [W.custom(300, 136, 1100, dt, seed=s, c_std=0.1, ignore_frac=0.05) for s in (91, 92, 93)]
    e, c, t = dev(inps[0]["e"], dt), dev(inps[0]["c"], dt), dev_targets(inps[0]["targets"])
    N, D = e.shape
    V = c.shape[0]
    state = torch.empty(M.state_size(N, D, V, e.dtype), dtype=torch.uint8, device="cuda")
    ws = torch.empty(M.workspace_size(N, D, V, e.dtype), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, dtype=torch.float32, device="cuda")

    def step():
        loss, lse, _, _ = M.forward(e, c, t, state=state)
        dE, dC = M.backward(e, c, t, lse, g, state, filter=True, ws=ws)
        return loss, lse, dE, dC

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    print("[graph] captured", flush=True)
    for k, inp in enumerate(inps * 2):
        e.copy_(dev(inp["e"], dt))
        c.copy_(dev(inp["c"], dt))
        t.copy_(dev_targets(inp["targets"]))
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in out]
        ref = step()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {k} differs from the eager step"
        if k == 0:
            fo = O.forward(inp["e"], inp["c"], inp["targets"])
            check_loss(got[0].cpu().numpy(), fo.loss, "mean", "graph replay", fo.n_valid)
            bo = O.backward(inp["e"], inp["c"], inp["targets"])
            check_grad(got[2].cpu().numpy(), bo.dE, GRAD_RTOL_FILTERED, "graph replay dE")
            check_grad(got[3].cpu().numpy(), bo.dC, GRAD_RTOL_FILTERED, "graph replay dC")


# ----------------------------------------------------------------------------- an empty batch
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_empty_batch(M, dt):
    """N = 0: loss 0 for sum and mean, an empty per-row loss, n_valid 0, dC and
    db exactly 0 (through the C ABI and through autograd)."""
    import torch
    inp = W.custom(8, 64, 1100, dt, seed=111, c_std=0.1)
    c = dev(inp["c"], dt)
    b = dev(W.bias(1100, dt, seed=4), dt)
    tdt = c.dtype
    e = torch.empty((0, 64), dtype=tdt, device="cuda")
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    for red in ("mean", "sum", "none"):
        loss, lse, nv, ws = M.forward(e, c, t, reduction=red, bias=b, label_smoothing=0.1)
        g = torch.ones(1 if red != "none" else 0, dtype=torch.float32, device="cuda")
        dE, dC, db = M.backward(e, c, t, lse, g, ws, reduction=red, bias=b, want_dbias=True, label_smoothing=0.1)
        torch.cuda.synchronize()
        assert int(nv.item()) == 0 and lse.shape == (0,)
        if red == "none":
            assert loss.shape == (0,)
        else:
            assert float(loss) == 0.0
        assert dE.shape == (0, 64) and not dC.any() and not db.any()
        assert M.read_stats(ws, 0, 1100)["tiles_kept"] == 0
    er = torch.empty((0, 64), dtype=tdt, device="cuda", requires_grad=True)
    cr = c.clone().requires_grad_(True)
    loss = M.linear_cross_entropy(er, cr, t)
    loss.backward()
    assert float(loss.detach()) == 0.0 and er.grad.shape == (0, 64) and not cr.grad.any()


# ----------------------------------------------------------------------------- two streams at once
def test_concurrent_streams(M):
    """The library keeps no mutable state of its own: two problems with their
    own workspaces, run at the same time on two streams (default priority),
    give the same results as one after the other."""
    import torch
    cases = [W.custom(600, 136, 1100, "bf16", seed=101, c_std=0.1, ignore_frac=0.05),
             W.custom(300, 200, 2600, "bf16", seed=102, c_std=0.05, ignore_frac=0.1)]
    tens = [(dev(x["e"], "bf16"), dev(x["c"], "bf16"), dev_targets(x["targets"])) for x in cases]
    g = torch.ones(1, dtype=torch.float32, device="cuda")

    def step(e, c, t):
        loss, lse, _, ws = M.forward(e, c, t)
        dE, dC = M.backward(e, c, t, lse, g, ws, filter=True)
        return loss, lse, dE, dC

    serial = [step(*x) for x in tens]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        for s, x in zip(streams, tens):
            with torch.cuda.stream(s):
                outs.append((s, step(*x)))
    torch.cuda.synchronize()
    print("[streams] done", flush=True)
    for k, (s, got) in enumerate(outs):
        want = serial[k % 2]
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"stream run {k} differs"


# ----------------------------------------------------------------------------- a plain C caller
def test_c_caller(M):
    """tests/c_abi/cce_abi_check.c: HIP runtime memory and a non-default
    stream, every entry point from C, checked against the c = 0 closed form."""
    import os
    import subprocess
    from linear_cross_entropy_forward_amd import build as b
    exe = b.C_CHECK_BIN
    assert os.path.exists(exe), "build the C check first (linear_cross_entropy_forward_amd/build.py)"
    print("[c caller]", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "cce C ABI check ok" in r.stdout


# ----------------------------------------------------------------------------- gradients in the operand dtype
# (dtype, N, D, V, filter, accum, vocab_chunk, label smoothing): bf16 dE/dC
# written by the kernels straight from one pass ('direct': one vocab chunk,
# one dE split), or through the fp32 accumulation and a final rounding pass
# (splits, chunks, atomics); fp32 operands keep fp32 gradients.
_GRAD_DTYPE_CASES = {
    "direct": ("bf16", 2048, 8192, 520, False, "deterministic", 0, 0.0),
    "direct_filtered_padded": ("bf16", 2048, 8192, 520, True, "deterministic", 0, 0.1),
    "splits": ("bf16", 600, 136, 1100, True, "deterministic", 0, 0.0),
    "chunks": ("bf16", 530, 200, 1500, False, "deterministic", 512, 0.1),
    "atomic": ("bf16", 530, 200, 1500, True, "atomic", 512, 0.0),
    "fp32": ("f32", 300, 68, 513, True, "deterministic", 0, 0.0),
}


@pytest.mark.parametrize("case", sorted(_GRAD_DTYPE_CASES))
def test_grad_dtype_operand(M, case):
    import torch
    dt, N, D, V, flt, accum, chunk, ls = _GRAD_DTYPE_CASES[case]
    inp = W.custom(N, D, V, dt, seed=71, c_std=0.05, ignore_frac=0.2 if "padded" in case else 0.05)
    print(f"[grad dtype] {case}", flush=True)
    e, c, t = dev(inp["e"], dt), dev(inp["c"], dt), dev_targets(inp["targets"])
    loss, lse, nv, ws = M.forward(e, c, t, label_smoothing=ls)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    kw = dict(filter=flt, accum=accum, vocab_chunk=chunk, label_smoothing=ls)
    dE32, dC32 = M.backward(e, c, t, lse, g, ws, **kw)
    dEo, dCo = M.backward(e, c, t, lse, g, ws, grad_dtype="operand", **kw)
    torch.cuda.synchronize()
    assert dEo.dtype == e.dtype and dCo.dtype == c.dtype
    if accum == "deterministic":
        # the same fp32 sums in the same order, rounded once to nearest-even
        assert torch.equal(dEo, dE32.to(e.dtype)), case
        assert torch.equal(dCo, dC32.to(c.dtype)), case
    f = O.forward(inp["e"], inp["c"], inp["targets"], label_smoothing=ls)
    valid = torch.from_numpy(f.valid).cuda()
    assert (dEo[~valid] == 0).all(), "ignored rows must give exactly 0 gradient"
    keep = O.lse_and_keep(inp["e"], inp["c"], inp["targets"], BLOCK, BLOCK)[1] if flt else None
    b = O.backward(inp["e"], inp["c"], inp["targets"], grad_loss=1.0, keep=keep,
                   tile=(BLOCK, BLOCK) if flt else None, label_smoothing=ls)
    check_grad(dEo.float().cpu().numpy(), b.dE, GRAD_RTOL, case + " dE")
    check_grad(dCo.float().cpu().numpy(), b.dC, GRAD_RTOL, case + " dC")


# ----------------------------------------------------------------------------- full-size, sampled
def _oracle_pass(name, with_bias=False, ls=0.0, zl=0.0, cap=0.0):
    """The oracle's one full pass over a named workload: LSE, keep map and
    per-row loss of every row, and the per-tile margins."""
    inp = W.get(name)
    bias = W.bias(inp["c"].shape[0], inp["workload"].dtype, seed=5) if with_bias else None
    print(f"[full] {name}: oracle full pass", flush=True)
    return O.lse_keep_nll(inp["e"], inp["c"], inp["targets"], BLOCK, BLOCK, bias=bias, label_smoothing=ls,
                          z_loss=zl, softcap=cap, margins=True)


def _sampled_full(M, name, reduction, filter, accum="deterministic", n_rows=48, n_vocab=24, dC_check=True,
                  with_bias=False, ls=0.0, zl=0.0, cap=0.0, grad_dtype="float32", full_pass=True, oracle=None,
                  degenerate=False):
    """A full-size workload in the benchmark's launch configuration.  With
    full_pass (the default), the oracle's whole-vocabulary pass over every row
    (or `oracle`, a pass already made) checks every row's LSE and loss, the
    reduced loss and the keep map tile by tile; dE is checked on sampled rows
    and dC on sampled vocabulary rows (each needs a whole row or column of
    the logits).  degenerate: a softmax saturated on the targets (the literal
    'trained-like' workloads: loss ~ e^-120, so G ~ 0), where relative checks
    mean nothing; per-row losses are held to the LSE bound and the gradients
    to 2e-2 of the one-hot term's norm (scale_i c_{y_i} for dE, the
    scatter of scale_i e_i to the target rows for dC)."""
    import torch
    inp = W.get(name)
    e, c, t = inp["e"], inp["c"], inp["targets"]
    N, V = e.shape[0], c.shape[0]
    bias = W.bias(V, inp["workload"].dtype, seed=5) if with_bias else None
    terms = dict(label_smoothing=ls, z_loss=zl, softcap=cap)
    print(f"[full] {name} N={N} V={V} reduction={reduction} filter={filter} accum={accum} bias={with_bias} "
          f"ls={ls} zl={zl} cap={cap}", flush=True)
    r = run(M, inp, reduction, filter, accum, bias=bias, want_db=with_bias, ls=ls, zl=zl, cap=cap,
            grad_dtype=grad_dtype)
    nll_gpu = r["loss"]
    if reduction != "none":
        # every row's loss, from a forward with per-row output
        dt = inp["workload"].dtype
        ed, cd, td = dev(e, dt), dev(c, dt), dev_targets(t)
        bd = dev(bias, dt) if bias is not None else None
        nll_gpu = M.forward(ed, cd, td, reduction="none", bias=bd, **terms)[0].cpu().numpy()
        del ed, cd, td, bd
    print(f"[full] {name}: GPU done, oracle checks", flush=True)
    rng = np.random.default_rng(99)
    rows = np.sort(rng.choice(N, n_rows, replace=False))
    valid = t != -100
    nv = int(valid.sum())
    assert r["n_valid"] == nv
    Bn, Bv, _ = M.tile_shape()
    tile = (BLOCK, BLOCK)
    keep = None
    if full_pass:
        if oracle is None:
            oracle = _oracle_pass(name, with_bias, ls, zl, cap)
        lse_all, keep, nll, margin, tgt = oracle
        check_lse(r["lse"], lse_all, name + " LSE (all rows)")
        if degenerate:
            err = np.max(np.abs(nll_gpu - nll))
            assert err <= 2e-3, (name, "per-row loss", err)
        else:
            check_loss(nll_gpu, nll, "none", name + " per-row loss (all rows)")
        check_loss(r["loss"], O.reduce_loss(nll, nv, reduction), reduction, name, nv)
        if filter:
            mt, tt = coarsen_keep(margin, tgt, Bn // BLOCK)
            nd = check_keep(r["keep"], mt, tt, O.FILTER_LOG_THRESHOLD, name + " tiles")
            nb = check_keep(r["blocks"], margin, tgt, O.FILTER_LOG_THRESHOLD, name + " blocks")
            kt = (mt >= O.FILTER_LOG_THRESHOLD) | tt
            print(f"[full] {name}: keep map {int(r['keep'].sum())} of {kt.size} tiles kept "
                  f"(oracle {int(kt.sum())}; {nd} near-threshold tiles differ), "
                  f"{int(r['blocks'].sum())} of {keep.size} 32x32 blocks kept (oracle {int(keep.sum())}; "
                  f"{nb} near-threshold blocks differ)", flush=True)
            assert r["stats"]["blocks_kept"] == int(r["blocks"].sum())
        assert r["stats"]["tiles_kept"] == int(r["keep"].sum())
    else:
        fo = O.forward(e, c, t, reduction="none", rows=rows, bias=bias, **terms)
        check_lse(r["lse"][rows], fo.lse, name)
        check_loss(nll_gpu[rows], fo.nll, "none", name)
        assert not filter, "filtered checks need the full pass"
    if not filter:
        want_keep = np.zeros_like(r["keep"])
        want_keep[:-(-nv // Bn)] = True
        assert np.array_equal(r["keep"], want_keep)
    g = r["g"]
    gv = np.broadcast_to(np.asarray(g, dtype=np.float64), (N,)) if reduction == "none" else None
    scale = np.where(valid, gv if reduction == "none" else (float(g) / max(nv, 1) if reduction == "mean"
                                                             else float(g)), 0.0)
    errs = {}

    def grad_check(got, want, rtol, what, onehot_norm):
        if degenerate:
            err = np.linalg.norm(np.asarray(got, np.float64) - want) / onehot_norm
            assert err <= rtol, (name, what, err)
        else:
            err = check_grad(got, want, rtol, name + " " + what)
        errs[what] = err

    dE_x = O.dE_rows(e, c, t, rows, reduction=reduction, grad_loss=g, bias=bias, **terms)
    oh_dE = np.linalg.norm(scale[rows][:, None] * np.asarray(c[np.where(valid[rows], t[rows], 0)], np.float64)
                           * valid[rows][:, None]) if degenerate else None
    if filter:
        dE_f = O.dE_rows(e, c, t, rows, reduction=reduction, grad_loss=g, keep=keep, tile=tile, bias=bias,
                         **terms)
        grad_check(r["dE"][rows], dE_f, GRAD_RTOL, "dE vs filtered", oh_dE)
        errs["filtered oracle dE vs exact"] = rel_fro(dE_f, dE_x)
        grad_check(r["dE"][rows], dE_x, GRAD_RTOL_FILTERED if degenerate else filtered_bound(dE_f, dE_x),
                   "dE vs exact", oh_dE)
    else:
        grad_check(r["dE"][rows], dE_x, GRAD_RTOL, "dE", oh_dE)
    if dC_check:
        assert full_pass, "dC rows need every row's LSE"
        vid = np.unique(np.concatenate([rng.choice(V, n_vocab, replace=False), t[valid][:8]]))
        oh_dC = None
        if degenerate:
            d1 = np.zeros((len(vid), e.shape[1]))
            pos = {int(j): k for k, j in enumerate(vid)}
            for i in np.nonzero(valid & np.isin(t, vid))[0]:
                d1[pos[int(t[i])]] += scale[i] * np.asarray(e[i], np.float64)
            oh_dC = np.linalg.norm(d1)
        dC_x = O.dC_rows(e, c, t, vid, lse_all, reduction=reduction, grad_loss=g, bias=bias, **terms)
        if filter:
            dC_f = O.dC_rows(e, c, t, vid, lse_all, reduction=reduction, grad_loss=g, keep=keep, tile=tile,
                             bias=bias, **terms)
            grad_check(r["dC"][vid], dC_f, GRAD_RTOL, "dC vs filtered", oh_dC)
            errs["filtered oracle dC vs exact"] = rel_fro(dC_f, dC_x)
            grad_check(r["dC"][vid], dC_x, GRAD_RTOL_FILTERED if degenerate else filtered_bound(dC_f, dC_x),
                       "dC vs exact", oh_dC)
        else:
            grad_check(r["dC"][vid], dC_x, GRAD_RTOL, "dC", oh_dC)
        if with_bias:
            db_f = O.db_rows(e, c, t, vid, lse_all, reduction=reduction, grad_loss=g, bias=bias,
                             keep=keep if filter else None, tile=tile if filter else None, **terms)
            check_grad(r["db"][vid], db_f, GRAD_RTOL, name + " db")
    print(f"[errors] {name} reduction={reduction} filter={filter} accum={accum} "
          + " ".join(f"{k}={v:.3g}" for k, v in errs.items()), flush=True)
    torch.cuda.empty_cache()
    r["oracle"] = oracle
    r["errs"] = errs
    return r


@pytest.mark.slow
def test_full_llama8b_none_filtered(M):
    """The benchmark's workload and launch configuration (per-token loss,
    filter on, deterministic, gradients in bf16), and with fp32 gradients."""
    r = _sampled_full(M, "llama8b", "none", True, grad_dtype="operand")
    _sampled_full(M, "llama8b", "none", True, dC_check=False, oracle=r["oracle"])


@pytest.mark.slow
def test_full_llama8b_mean_unfiltered(M):
    _sampled_full(M, "llama8b", "mean", False, dC_check=False)


@pytest.mark.slow
def test_full_llama1b(M):
    r = _sampled_full(M, "llama1b", "mean", True)
    _sampled_full(M, "llama1b", "mean", False, oracle=r["oracle"])


@pytest.mark.slow
def test_full_gemma2b_calibrated(M):
    _sampled_full(M, "gemma2b_cal", "mean", True)


@pytest.mark.slow
def test_full_gemma2b_literal(M):
    """Gemma-2-2B's head with the literal 'trained-like' construction (target
    logits about 138 nats above the rest): the loss is ~e^-120 per row and G
    ~ 0, so the checks are the degenerate ones (every row's LSE and loss to
    2e-3 absolute, gradients to 2e-2 of the one-hot term), as benchmarked
    (mean, filter on, deterministic)."""
    r = _sampled_full(M, "gemma2b", "mean", True, degenerate=True)
    assert r["stats"]["tiles_kept"] < 0.1 * r["stats"]["tiles_total"]


@pytest.mark.slow
def test_full_llama1b_bias(M):
    _sampled_full(M, "llama1b", "mean", True, with_bias=True)


@pytest.mark.slow
def test_full_llama1b_smoothing_zloss(M):
    _sampled_full(M, "llama1b", "mean", True, with_bias=True, ls=0.1, zl=1e-4)


@pytest.mark.slow
def test_full_gemma2b_softcap(M):
    """Gemma 2's own final-logit cap (30) on the calibrated Gemma-2-2B head."""
    _sampled_full(M, "gemma2b_cal", "mean", True, cap=30.0)


@pytest.mark.slow
def test_full_llama8b_padded(M):
    """The 8B head with a quarter of the rows padding: the compacted backward."""
    r = _sampled_full(M, "llama8b_pad25", "mean", True)
    assert r["stats"]["tiles_kept"] <= 12 * 502


@pytest.mark.slow
def test_full_long8b_calibrated(M):
    """The long-context 8B head (N = 16384, sixteen vocabulary chunks) as the
    benchmark runs it: mean, filter on, in the deterministic mode and with
    dE accumulated by fp32 atomics (dC has one mode: each vocabulary row block
    is owned by one work-group); every row's LSE and loss, the keep map tile
    by tile, sampled dE and dC rows, and the two modes against each other
    (dC bitwise equal, dE within 1e-5)."""
    r = _sampled_full(M, "long8b_cal", "mean", True)
    ra = _sampled_full(M, "long8b_cal", "mean", True, accum="atomic", oracle=r["oracle"])
    assert np.array_equal(ra["dC"], r["dC"]) and np.array_equal(ra["keep"], r["keep"])
    d = rel_fro(ra["dE"], r["dE"])
    print(f"[errors] long8b_cal atomic vs deterministic dE {d:.3g}", flush=True)
    assert d < 1e-5


@pytest.mark.slow
def test_full_long8b_calibrated_unfiltered(M):
    """The same head unfiltered, per-token loss: dE added up over sixteen
    vocabulary chunks in both modes."""
    r = _sampled_full(M, "long8b_cal", "none", False, dC_check=False, full_pass=False)
    _sampled_full(M, "long8b_cal", "none", False, accum="atomic", dC_check=False, full_pass=False)


@pytest.mark.slow
def test_full_long8b_literal(M):
    """The long-context 8B head with the literal 'trained-like' construction
    (degenerate checks as for Gemma-2-2B), mean, filter on."""
    r = _sampled_full(M, "long8b", "mean", True, degenerate=True)
    assert r["stats"]["tiles_kept"] < 0.1 * r["stats"]["tiles_total"]


@pytest.mark.slow
def test_full_wide_head(M):
    """D = 8192 with V = 128256: the classifier (2.1 GB of bf16) just under the
    2^31-byte reach of one buffer descriptor, K loops of 128 steps, 32 tiles
    across D; filtered, per-row and reduced checks."""
    _sampled_full(M, "wide8192", "mean", True, n_rows=32, n_vocab=16)


@pytest.mark.slow
def test_full_classifier_beyond_2gib(M):
    """Gemma-2-27B's head (V = 256000, D = 4608: a 2.4 GB bf16 classifier),
    beyond one buffer descriptor's 2^31-byte reach: the backward takes it in
    two vocabulary chunks."""
    assert M.vocab_chunk(1024, 4608, 256000) < 256000
    _sampled_full(M, "gemma27b_1k", "mean", True, n_rows=32, n_vocab=16)


@pytest.mark.slow
def test_full_64k_tokens(M):
    """65536 tokens on the 8B head: sixteen vocabulary chunks of 8192 (1 GiB
    of gradient tiles each), 256 token blocks; per-row checks (the oracle's
    whole-vocabulary pass over 65536 rows would take too long)."""
    assert M.vocab_chunk(65536, 4096, 128256) == 8192
    _sampled_full(M, "long64k", "none", False, dC_check=False, n_rows=32, full_pass=False)


# ----------------------------------------------------------------------------- seeded random configurations
def _random_case(k):
    """Case k of a fixed list: shapes, dtype, reduction, filter, accumulation,
    chunking and loss terms drawn from a seeded generator (combinations the
    library accepts: no softcap with fp32 operands or with label smoothing)."""
    g = np.random.default_rng(1000 + k)
    dt = "f32" if g.random() < 0.2 else "bf16"
    N = int(g.integers(1, 700))
    D = int(g.integers(1, 40)) * (4 if dt == "f32" else 8)
    V = int(g.integers(1, 2100))
    case = dict(dt=dt, N=N, D=D, V=V,
                reduction=str(g.choice(["mean", "sum", "none"])),
                filter=bool(g.random() < 0.5),
                accum=str(g.choice(["deterministic", "atomic"])),
                vocab_chunk=int(g.choice([0, 256, 512])),
                ignore_frac=float(g.choice([0.0, 0.1, 0.5])),
                c_std=float(g.choice([0.05, 0.2, 0.5])),
                bias=bool(g.random() < 0.4),
                ls=float(g.choice([0.0, 0.0, 0.1])),
                zl=float(g.choice([0.0, 1e-3])))
    case["cap"] = float(g.choice([0.0, 5.0])) if dt == "bf16" and case["ls"] == 0.0 else 0.0
    case["grad_dtype"] = str(g.choice(["float32", "operand"]))
    return case


@pytest.mark.parametrize("k", range(40))
def test_random_configuration(M, k):
    cs = _random_case(k)
    print(f"[random {k}] {cs}", flush=True)
    inp = W.custom(cs["N"], cs["D"], cs["V"], cs["dt"], seed=2000 + k, c_std=cs["c_std"],
                   ignore_frac=cs["ignore_frac"])
    bias = W.bias(cs["V"], cs["dt"], seed=2000 + k) if cs["bias"] else None
    full_check(M, inp, cs["reduction"], cs["filter"], accum=cs["accum"], vocab_chunk=cs["vocab_chunk"],
               label=f"random {k}", bias=bias, want_db=cs["bias"], ls=cs["ls"], zl=cs["zl"], cap=cs["cap"],
               grad_dtype=cs["grad_dtype"])
