"""Plain fp64 CPU oracle for Cut Cross-Entropy (linear projection + cross-entropy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product (the HIP library and its
Python binding) never imports, links or calls it, and it shares no code with
the product: it is written from the definitions on the pages, materialises the
logits, and is slow on purpose.

What is computed (all in float64, from operands passed in exactly as the GPU
sees them: bf16 values upcast exactly, or fp32):

  Z = E C^T (+ b)                 logits, materialised here only
                                  (mlx-cross-entropy README, "Usage": the
                                  standard path that forms hidden @ classifier.T;
                                  the optional classifier bias b [V] of the
                                  README "API" table is added to every row)
  LSE_i = m_i + ln sum_j exp(Z_ij - m_i),  m_i = max_j Z_ij
                                  (tirogla "Loss functions", "How it works"
                                  step 1: log-sum-exp with max subtraction)
  loss_i = LSE_i - Z_{i,y_i}      (blog "Cut Cross Entropy from first
                                  principles": the LSE minus the
                                  correct-token logit; Wijmans et al.
                                  abstract: only the correct
                                  token's logit plus the log-sum-exp)
  rows with y_i == ignore_index give loss 0 and gradient 0, and are not counted
                                  (README "API" ignore_index; "Loss functions" "Code":
                                  ignored rows' gradient is zero, mean over
                                  non-ignored rows with the count floored at 1)
  reduction: none -> loss_i; sum -> sum_i loss_i; mean -> sum / max(n_valid, 1)
                                  (README "API" and "Computing related
                                  quantities"; "Loss functions" step 4)
  G = (softmax(Z) - onehot(y)) * scale_i
                                  ("Loss functions" step 2: fused softmax+CE gradient
                                  p - y)
  dE = G C,  dC = G^T E,  db = G^T 1
                                  (chain rule through Z = E C^T + 1 b^T)
  scale_i = g / max(n_valid,1) (mean), g (sum), g_i (none); 0 on ignored rows.

Optional loss terms (both default to 0, which gives the plain loss above):

  label smoothing eps:  the target row becomes the soft target
        T_i = (1 - eps) onehot(y_i) + eps / V   (spread over all V classes,
        the true one included), and loss_i = -sum_j T_ij log softmax_ij
                                  (tirogla "Loss functions", "How it works"
                                  step 3: soft targets; the gradient stays
                                  softmax minus the target)
  z-loss lam:           loss_i += lam * LSE_i^2, whose gradient with respect
                        to Z_ij is 2 lam LSE_i softmax_ij
                                  (tirogla "Implementation notes": z-loss
                                  adds a multiple of the squared log-sum-exp)
  so that G_ij = (softmax_ij (1 + 2 lam LSE_i) - T_ij) * scale_i.

Logit soft-capping s > 0 (NOT defined on the pages; the form used by Gemma 2:
Z'_ij = s tanh(Z_ij / s), applied after the bias): every definition above then
takes Z' in place of Z, and the chain rule multiplies G by
dZ'/dZ = 1 - tanh^2(Z / s) = 1 - (Z' / s)^2.  Soft-capping together with label
smoothing under filtering has no reading here (the smoothing part of G is no
longer uniform) and raises.

Gradient filtering (README "How it works" item 2; Wijmans et al. abstract:
skip gradient entries below numerical precision) is modelled by
`filter_keep`: a tile (row block b, vocab block v) of G is kept iff some valid
row i in b has max_{j in v} softmax_ij >= 2^-12, or some valid row in b has
its target in v.  Row blocks are cut from the non-ignored rows only, in order
(`tile_blocks`): ignored (padding) rows belong to no tile, as the Loss
functions page's "Efficiency" list has padded rows skipped rather than
computed; their G is zero either way.  `backward(..., keep=...)` zeroes G on dropped tiles.  The
target-tile rule and the strict "< 2^-12 everywhere" reading are this
implementation's readings of a criterion the pages state only loosely.  With
label smoothing the filter still decides on the softmax alone and drops only
the softmax term (and the one-hot term, which never lies in a dropped tile);
the uniform -eps/V * scale_i part of G is kept on every entry (a reading: that
part is known exactly, so nothing is gained by dropping it).

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, brute force, finite differences and invariants.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

FILTER_LOG_THRESHOLD = -12.0 * math.log(2.0)   # ln(2^-12)
_ROW_CHUNK = 256


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def valid_rows(targets, V: int, ignore_index: int = -100) -> np.ndarray:
    """Boolean mask of non-ignored rows; any other target outside [0, V) is an error."""
    t = np.asarray(targets, dtype=np.int64)
    valid = t != ignore_index
    bad = valid & ((t < 0) | (t >= V))
    if bad.any():
        raise ValueError(f"{int(bad.sum())} target(s) outside [0, {V}) that are not ignore_index")
    return valid


def logits(e, c, bias=None, softcap: float = 0.0) -> np.ndarray:
    """Z = E C^T (+ b on every row) in float64 (the materialised logit matrix),
    soft-capped to s tanh(Z / s) when softcap = s > 0."""
    z = _f64(e) @ _f64(c).T
    if bias is not None:
        z += _f64(bias)[None, :]
    if softcap:
        z = softcap * np.tanh(z / softcap)
    return z


def row_logsumexp(z: np.ndarray) -> np.ndarray:
    """LSE of each row of z by max subtraction."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


@dataclass
class Forward:
    loss: np.ndarray        # scalar array (mean/sum) or [N] (none)
    nll: np.ndarray         # [N] per-row loss, 0 on ignored rows
    lse: np.ndarray         # [N] LSE of every row (ignored rows included)
    n_valid: int
    valid: np.ndarray       # [N] bool


def reduce_loss(nll: np.ndarray, n_valid: int, reduction: str) -> np.ndarray:
    if reduction == "none":
        return nll.copy()
    s = float(np.sum(nll))
    if reduction == "sum":
        return np.array(s)
    if reduction == "mean":
        return np.array(s / max(n_valid, 1))
    raise ValueError(reduction)


def soft_target_rows(t: np.ndarray, V: int, valid: np.ndarray, label_smoothing: float) -> np.ndarray:
    """T rows: (1 - eps) onehot(t) + eps / V on valid rows, zero rows elsewhere."""
    T = np.zeros((len(t), V))
    r = np.nonzero(valid)[0]
    T[r] = label_smoothing / V
    T[r, t[r]] += 1.0 - label_smoothing
    return T


def forward(e, c, targets, ignore_index: int = -100, reduction: str = "mean",
            rows=None, bias=None, label_smoothing: float = 0.0, z_loss: float = 0.0,
            softcap: float = 0.0) -> Forward:
    """Loss and per-row LSE.  `rows` restricts the work to a subset of rows
    (then `loss` is the reduction over that subset only and n_valid counts it).
    loss_i = -sum_j T_ij (Z_ij - LSE_i) + z_loss * LSE_i^2 on valid rows."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    V = c.shape[0]
    idx = np.arange(e.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    valid = valid_rows(t[idx], V, ignore_index)
    lse = np.empty(len(idx))
    nll = np.zeros(len(idx))
    for s in range(0, len(idx), _ROW_CHUNK):
        sl = slice(s, s + _ROW_CHUNK)
        z = logits(e[idx[sl]], c, bias, softcap)
        lse[sl] = row_logsumexp(z)
        v = valid[sl]
        r = np.nonzero(v)[0]
        T = soft_target_rows(t[idx[sl]], V, v, label_smoothing)
        logp = z - lse[sl][:, None]
        nll[sl][r] = -(T[r] * logp[r]).sum(axis=1) + z_loss * lse[sl][r] ** 2
    n_valid = int(valid.sum())
    return Forward(reduce_loss(nll, n_valid, reduction), nll, lse, n_valid, valid)


def grad_scale(valid: np.ndarray, reduction: str, grad_loss=1.0) -> np.ndarray:
    """Per-row factor multiplying (softmax - onehot): d(loss)/d(nll_i) times the
    upstream gradient; 0 on ignored rows."""
    n_valid = int(valid.sum())
    if reduction == "none":
        g = np.broadcast_to(_f64(grad_loss), valid.shape).astype(np.float64)
    elif reduction == "sum":
        g = np.full(valid.shape, float(grad_loss))
    elif reduction == "mean":
        g = np.full(valid.shape, float(grad_loss) / max(n_valid, 1))
    else:
        raise ValueError(reduction)
    return np.where(valid, g, 0.0)


def tile_row_max(z: np.ndarray, Bv: int) -> np.ndarray:
    """max_{j in vocab block v} Z_ij for each row i and block v = j // Bv."""
    n, V = z.shape
    nvb = -(-V // Bv)
    pad = nvb * Bv - V
    if pad:
        z = np.concatenate([z, np.full((n, pad), -np.inf)], axis=1)
    return z.reshape(n, nvb, Bv).max(axis=2)


def tile_blocks(valid: np.ndarray, Bn: int) -> np.ndarray:
    """Row block of each row in the tiles of G: the non-ignored rows, in
    order, cut into blocks of Bn; ignored rows belong to no block (-1)."""
    v = np.asarray(valid, dtype=bool)
    rank = np.cumsum(v) - 1
    return np.where(v, rank // Bn, -1)


def _mark_keep(keep: np.ndarray, blk: np.ndarray, tm: np.ndarray, t: np.ndarray, Bv: int) -> None:
    """Add rows (block blk >= 0, log tile maxima tm [rows, nvb], targets t) to
    the keep map: a tile is kept by a row whose tile maximum reaches 2^-12,
    and by a row whose target lies in it."""
    r = np.nonzero(blk >= 0)[0]
    if len(r):
        np.logical_or.at(keep, blk[r], tm[r] >= FILTER_LOG_THRESHOLD)
        keep[blk[r], t[r] // Bv] = True


def filter_keep(e, c, targets, Bn: int, Bv: int, ignore_index: int = -100,
                lse=None, bias=None, softcap: float = 0.0) -> np.ndarray:
    """Keep map [ceil(N/Bn), ceil(V/Bv)] of (row block, vocab block) tiles of G
    (row blocks from `tile_blocks`; blocks past the valid rows stay empty).

    Kept iff some valid row i of the block has max_j softmax_ij >= 2^-12 on the
    tile, i.e. max_j Z_ij - LSE_i >= -12 ln 2, or some valid row of the block
    has its target inside the tile's vocab range.
    """
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    N, V = e.shape[0], c.shape[0]
    valid = valid_rows(t, V, ignore_index)
    blk = tile_blocks(valid, Bn)
    keep = np.zeros((-(-N // Bn), -(-V // Bv)), dtype=bool)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        z = logits(e[r0:r1], c, bias, softcap)
        l = row_logsumexp(z) if lse is None else _f64(lse)[r0:r1]
        _mark_keep(keep, blk[r0:r1], tile_row_max(z, Bv) - l[:, None], t[r0:r1], Bv)
    return keep


def softmax_grad_rows(z: np.ndarray, lse: np.ndarray, t: np.ndarray, scale: np.ndarray,
                      valid: np.ndarray, label_smoothing: float = 0.0, z_loss: float = 0.0,
                      colmask=None, softcap: float = 0.0) -> np.ndarray:
    """G rows: (exp(Z - LSE) (1 + 2 z_loss LSE) - T) * scale, zero on ignored
    rows.  colmask [rows, V] (bool), when given, marks the entries the filter
    keeps: elsewhere only the uniform -eps/V part of -T remains.  With
    softcap, z holds the capped logits and G is multiplied by 1 - (z / s)^2."""
    if softcap and label_smoothing and colmask is not None:
        raise NotImplementedError("filtered soft-capping with label smoothing has no reading")
    V = z.shape[1]
    g = np.exp(z - lse[:, None]) * (1.0 + 2.0 * z_loss * lse)[:, None]
    r = np.nonzero(valid)[0]
    g[r, t[r]] -= 1.0 - label_smoothing
    if colmask is not None:
        g[~colmask] = 0.0
    g -= label_smoothing / V
    if softcap:
        g *= 1.0 - (z / softcap) ** 2
    g *= scale[:, None]
    g[~valid] = 0.0
    return g


def _colmask(keep: np.ndarray, blk: np.ndarray, Bv: int, V: int) -> np.ndarray:
    """[rows, V] mask of the entries in kept tiles (rows of no block: none)."""
    m = np.zeros((len(blk), V), dtype=bool)
    r = np.nonzero(blk >= 0)[0]
    m[r] = np.repeat(keep[blk[r]], Bv, axis=1)[:, :V]
    return m


@dataclass
class Backward:
    dE: np.ndarray
    dC: np.ndarray
    db: np.ndarray          # [V] column sums of G (the bias gradient)


def backward(e, c, targets, ignore_index: int = -100, reduction: str = "mean",
             grad_loss=1.0, keep=None, tile=None, bias=None, label_smoothing: float = 0.0,
             z_loss: float = 0.0, softcap: float = 0.0) -> Backward:
    """dE = G C, dC = G^T E and db = G^T 1.  With `keep` (a filter_keep map for
    `tile` = (Bn, Bv)) the softmax part of G is zeroed on the dropped tiles."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    N, V = e.shape[0], c.shape[0]
    valid = valid_rows(t, V, ignore_index)
    scale = grad_scale(valid, reduction, grad_loss)
    dE = np.zeros_like(e)
    dC = np.zeros_like(c)
    db = np.zeros(V)
    blk = tile_blocks(valid, tile[0]) if keep is not None else None
    for s in range(0, N, _ROW_CHUNK):
        sl = slice(s, min(N, s + _ROW_CHUNK))
        z = logits(e[sl], c, bias, softcap)
        lse = row_logsumexp(z)
        cm = None
        if keep is not None:
            cm = _colmask(keep, blk[sl], tile[1], V)
        g = softmax_grad_rows(z, lse, t[sl], scale[sl], valid[sl], label_smoothing, z_loss, cm, softcap)
        dE[sl] = g @ c
        dC += g.T @ e[sl]
        db += g.sum(axis=0)
    return Backward(dE, dC, db)


# ---------------------------------------------------------------------------
# Sampled forms for large shapes: the same definitions evaluated on a subset of
# output rows, so full-size checks stay within seconds to a minute.
# ---------------------------------------------------------------------------

def lse_all(e, c, chunk: int = _ROW_CHUNK, bias=None, softcap: float = 0.0) -> np.ndarray:
    """LSE of every row (the full materialised pass, row chunk by row chunk)."""
    e = _f64(e)
    c = _f64(c)
    out = np.empty(e.shape[0])
    for s in range(0, e.shape[0], chunk):
        out[s:s + chunk] = row_logsumexp(logits(e[s:s + chunk], c, bias, softcap))
    return out


def lse_and_keep(e, c, targets, Bn: int, Bv: int, ignore_index: int = -100, bias=None,
                 softcap: float = 0.0):
    """One pass over all row blocks giving LSE [N] and the filter keep map."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    N, V = e.shape[0], c.shape[0]
    valid = valid_rows(t, V, ignore_index)
    blk = tile_blocks(valid, Bn)
    keep = np.zeros((-(-N // Bn), -(-V // Bv)), dtype=bool)
    lse = np.empty(N)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        z = logits(e[r0:r1], c, bias, softcap)
        l = row_logsumexp(z)
        lse[r0:r1] = l
        _mark_keep(keep, blk[r0:r1], tile_row_max(z, Bv) - l[:, None], t[r0:r1], Bv)
    return lse, keep


def lse_keep_nll(e, c, targets, Bn: int, Bv: int, ignore_index: int = -100, bias=None,
                 label_smoothing: float = 0.0, z_loss: float = 0.0, softcap: float = 0.0,
                 margins: bool = False):
    """One pass over all row blocks giving LSE [N], the filter keep map and
    the per-row loss [N] (0 on ignored rows), the same definitions as
    `forward` and `filter_keep`.  With margins=True it also returns, per tile,
    the largest log-softmax maximum of its valid rows, max_i (max_j Z_ij -
    LSE_i) (-inf for a tile of no valid row), and whether a valid row's target
    lies in it: the two quantities the keep rule compares (kept iff the first
    reaches ln 2^-12 or the second holds), so that a test can tell how close
    each tile's decision is to the threshold."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    N, V = e.shape[0], c.shape[0]
    valid = valid_rows(t, V, ignore_index)
    blk = tile_blocks(valid, Bn)
    keep = np.zeros((-(-N // Bn), -(-V // Bv)), dtype=bool)
    lse = np.empty(N)
    nll = np.zeros(N)
    margin = np.full(keep.shape, -np.inf)
    tgt = np.zeros(keep.shape, dtype=bool)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        z = logits(e[r0:r1], c, bias, softcap)
        l = row_logsumexp(z)
        lse[r0:r1] = l
        tm = tile_row_max(z, Bv) - l[:, None]
        _mark_keep(keep, blk[r0:r1], tm, t[r0:r1], Bv)
        if margins:
            b = blk[r0:r1]
            r = np.nonzero(b >= 0)[0]
            np.maximum.at(margin, b[r], tm[r])
            tgt[b[r], t[r0:r1][r] // Bv] = True
        v = valid[r0:r1]
        if v.any():
            T = soft_target_rows(t[r0:r1], V, v, label_smoothing)
            r = np.nonzero(v)[0]
            nll[r0 + r] = -(T[r] * (z[r] - l[r, None])).sum(axis=1) + z_loss * l[r] ** 2
    if margins:
        return lse, keep, nll, margin, tgt
    return lse, keep, nll


def dE_rows(e, c, targets, rows, ignore_index: int = -100, reduction: str = "mean",
            grad_loss=1.0, n_valid: int | None = None, keep=None, tile=None, bias=None,
            label_smoothing: float = 0.0, z_loss: float = 0.0, softcap: float = 0.0) -> np.ndarray:
    """dE for selected rows: row i of G C needs only row i of Z.  For mean,
    n_valid is the whole batch's count (pass it in); for none, grad_loss is [N]."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    V = c.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    valid_all = valid_rows(t, V, ignore_index)
    if n_valid is None:
        n_valid = int(valid_all.sum())
    if reduction == "mean":
        scale = np.where(valid_all[rows], float(grad_loss) / max(n_valid, 1), 0.0)
    else:
        scale = grad_scale(valid_all, reduction, grad_loss)[rows]
    z = logits(e[rows], c, bias, softcap)
    lse = row_logsumexp(z)
    cm = None
    if keep is not None:
        cm = _colmask(keep, tile_blocks(valid_all, tile[0])[rows], tile[1], V)
    g = softmax_grad_rows(z, lse, t[rows], scale, valid_all[rows], label_smoothing, z_loss, cm, softcap)
    return g @ c


def G_columns(e, c, targets, vocab_ids, lse, ignore_index: int = -100, reduction: str = "mean",
              grad_loss=1.0, keep=None, tile=None, bias=None, label_smoothing: float = 0.0,
              z_loss: float = 0.0, softcap: float = 0.0) -> np.ndarray:
    """Columns j of G for selected vocabulary ids, [N, k]: they need column j of
    Z for all rows and every row's LSE (pass the oracle's own)."""
    e = _f64(e)
    c = _f64(c)
    t = np.asarray(targets, dtype=np.int64)
    V = c.shape[0]
    vocab_ids = np.asarray(vocab_ids, dtype=np.int64)
    valid = valid_rows(t, V, ignore_index)
    scale = grad_scale(valid, reduction, grad_loss)
    zc = e @ c[vocab_ids].T                              # [N, k] = Z[:, vocab_ids]
    if bias is not None:
        zc += _f64(bias)[vocab_ids][None, :]
    if softcap:
        if label_smoothing and keep is not None:
            raise NotImplementedError("filtered soft-capping with label smoothing has no reading")
        zc = softcap * np.tanh(zc / softcap)
    lse = _f64(lse)
    g = np.exp(zc - lse[:, None]) * (1.0 + 2.0 * z_loss * lse)[:, None]
    g -= (1.0 - label_smoothing) * (t[:, None] == vocab_ids[None, :])
    if keep is not None:
        Bn, Bv = tile
        blk = tile_blocks(valid, Bn)
        g *= np.where(blk[:, None] >= 0, keep[np.maximum(blk, 0)][:, vocab_ids // Bv], False)
    g -= label_smoothing / V
    if softcap:
        g *= 1.0 - (zc / softcap) ** 2
    g *= scale[:, None]
    g[~valid] = 0.0
    return g


def db_rows(e, c, targets, vocab_ids, lse, **kw) -> np.ndarray:
    """db for selected vocabulary ids: db_j = sum_i G_ij."""
    return G_columns(e, c, targets, vocab_ids, lse, **kw).sum(axis=0)


def dC_rows(e, c, targets, vocab_ids, lse, ignore_index: int = -100, reduction: str = "mean",
            grad_loss=1.0, keep=None, tile=None, bias=None, label_smoothing: float = 0.0,
            z_loss: float = 0.0, softcap: float = 0.0) -> np.ndarray:
    """dC for selected vocabulary rows j: dC_j = sum_i G_ij e_i, which needs
    column j of Z for all rows and every row's LSE (pass the oracle's own)."""
    g = G_columns(e, c, targets, vocab_ids, lse, ignore_index=ignore_index, reduction=reduction,
                  grad_loss=grad_loss, keep=keep, tile=tile, bias=bias,
                  label_smoothing=label_smoothing, z_loss=z_loss, softcap=softcap)
    return g.T @ _f64(e)
