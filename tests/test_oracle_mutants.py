"""Plant one plausible mistake at a time in the oracle and require that at
least one pin catches it.  This shows the pins constrain every step of the
oracle (scale, mask, normaliser, softmax, value product and each gradient
term), not just its overall shape.  CPU only; the real oracle is restored
after every case by pytest's monkeypatch."""

import numpy as np
import pytest

import oracle
import oracle.attention as A
import oracle.splitkv as SK
import oracle.blocksparse as BS
from tests import oracle_pins


def _bwd_variant(change):
    """A copy of the per-head backward with one term altered by ``change``."""
    def head_backward(q, k, v, dO, scale, vis):
        O, _, P = A._head_forward(q, k, v, scale, vis)
        t = dict(P=P, O=O, q=q, k=k, v=v, dO=dO, scale=scale)
        D = change.get("D", lambda t: (t["dO"] * t["O"]).sum(axis=1))(t)
        t["D"] = D
        dv = change.get("dv", lambda t: t["P"].T @ t["dO"])(t)
        dP = change.get("dP", lambda t: t["dO"] @ t["v"].T)(t)
        t["dP"] = dP
        dS = change.get("dS", lambda t: t["P"] * (t["dP"] - t["D"][:, None]))(t)
        t["dS"] = dS
        dq = change.get("dq", lambda t: t["scale"] * (t["dS"] @ t["k"]))(t)
        dk = change.get("dk", lambda t: t["scale"] * (t["dS"].T @ t["q"]))(t)
        return dq, dk, dv
    return head_backward


FORWARD_MUTANTS = {
    "scale dropped": ("_scores", lambda q, k, s: q @ k.T),
    "scale squared": ("_scores", lambda q, k, s: s * s * (q @ k.T)),
    "mask keeps keys after the query": (
        "visible_mask", lambda Lq, Lk, c: (np.arange(Lk)[None] >= np.arange(Lq)[:, None])
        if c else np.ones((Lq, Lk), bool)),
    "mask hides the diagonal": (
        "visible_mask", lambda Lq, Lk, c: (np.arange(Lk)[None] < np.arange(Lq)[:, None])
        | (np.arange(Lq)[:, None] == 0) & (np.arange(Lk)[None] == 0)
        if c else np.ones((Lq, Lk), bool)),
    "masked scores set to 0 instead of -inf": ("_apply_mask", lambda S, vis: np.where(vis, S, 0.0)),
    "lse in base 2": ("_row_logsumexp", lambda S: np.log2(np.exp(S).sum(axis=1))),
    "lse missing the row max": (
        "_row_logsumexp", lambda S: np.log(np.exp(S - S.max(1, keepdims=True)).sum(axis=1))),
    "lse without max shift": ("_row_logsumexp", lambda S: np.log(np.exp(S).sum(axis=1))),
    "softmax not normalised": ("_probabilities", lambda S, lse: np.exp(S)),
    "softmax over the wrong axis": (
        "_probabilities", lambda S, lse: np.exp(S - np.log(np.exp(S).sum(axis=0, keepdims=True)))),
    "values taken reversed": (
        "_head_forward", lambda q, k, v, s, vis: (lambda O, l, P: (P @ v[::-1], l, P))(
            *_real_head_forward(q, k, v, s, vis))),
}

BACKWARD_MUTANTS = {
    "D term dropped": {"D": lambda t: 0 * t["O"][:, 0]},
    "D from dO only": {"D": lambda t: t["dO"].sum(axis=1)},
    "dV without transpose": {"dv": lambda t: t["P"] @ t["dO"]},
    "dS sign flipped": {"dS": lambda t: t["P"] * (t["D"][:, None] - t["dP"])},
    "dS missing P factor": {"dS": lambda t: t["dP"] - t["D"][:, None]},
    "dQ missing scale": {"dq": lambda t: t["dS"] @ t["k"]},
    "dK missing scale": {"dk": lambda t: t["dS"].T @ t["q"]},
    "dQ uses values instead of keys": {"dq": lambda t: t["scale"] * (t["dS"] @ t["v"])},
    "dK from dS without transpose": {"dk": lambda t: t["scale"] * (t["dS"] @ t["q"])},
    "dP from reversed values": {"dP": lambda t: t["dO"] @ t["v"][::-1].T},
}

_real_head_forward = A._head_forward
_real_keyrange = SK.attn_fwd_keyrange
_real_merge = SK.merge_partials


def _merge_variant(weights):
    def merge(O_parts, lse_parts):
        lse_parts = np.asarray(lse_parts, dtype=np.float64)
        m = lse_parts.max(axis=0)
        lse = m + np.log(np.exp(lse_parts - m).sum(axis=0))
        w = weights(lse_parts, lse, m)
        return (w[..., None] * np.asarray(O_parts)).sum(axis=0), lse
    return merge


_real_block_visible = BS.block_visible


def _vis_variant(change):
    def block_visible(block_mask, Lq, Lk, block, causal):
        bm = np.asarray(block_mask) != 0
        rows, cols = change(np.arange(Lq), np.arange(Lk), block)
        rows = np.clip(rows, 0, bm.shape[0] - 1)
        cols = np.clip(cols, 0, bm.shape[1] - 1)
        return bm[rows[:, None], cols[None, :]] & A.visible_mask(Lq, Lk, causal)
    return block_visible


def _transposed_visible(block_mask, Lq, Lk, block, causal):
    # Entry (i, j) taken from block_mask[j // block, i // block].
    bm = np.asarray(block_mask) != 0
    r = np.clip(np.arange(Lk) // block, 0, bm.shape[0] - 1)
    c = np.clip(np.arange(Lq) // block, 0, bm.shape[1] - 1)
    return bm[r[None, :], c[:, None]] & A.visible_mask(Lq, Lk, causal)


def _bs_bwd_variant(change):
    """A copy of the block-sparse backward with one term altered."""
    real = BS.attn_bwd_blocksparse

    def bwd(q, k, v, dO, scale, causal, block_mask, block=128):
        dq, dk, dv = real(q, k, v, dO, scale, causal, block_mask, block)
        return change(dq, dk, dv, np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(dO))
    return bwd


BLOCKSPARSE_BWD_MUTANTS = {
    "dQ sign flipped": lambda dq, dk, dv, q, k, v, dO: (-dq, dk, dv),
    "dK scaled twice": lambda dq, dk, dv, q, k, v, dO: (dq, 1.3 * dk, dv),
}


BLOCKSPARSE_MUTANTS = {
    "block mask read transposed": ("block_visible", _transposed_visible),
    "block index off by one row": ("block_visible", _vis_variant(lambda i, j, b: ((i + 1) // b, j // b))),
    "block index from the key end": ("block_visible", _vis_variant(lambda i, j, b: (i // b, (j + b - 1) // b))),
    "causal rule ignored": (
        "block_visible", lambda bm, Lq, Lk, b, c: _real_block_visible(bm, Lq, Lk, b, False)),
    "mask ignored": (
        "block_visible", lambda bm, Lq, Lk, b, c: A.visible_mask(Lq, Lk, c)),
}


SPLITKV_MUTANTS = {
    "range drops its last key": (
        "attn_fwd_keyrange", lambda q, k, v, s, c, k0, k1: _real_keyrange(q, k, v, s, c, k0, max(k0, k1 - 1))),
    "causal rule relative to the range start": (
        "attn_fwd_keyrange", lambda q, k, v, s, c, k0, k1: oracle.attn_fwd(
            np.asarray(q), np.asarray(k)[:, :, k0:k1], np.asarray(v)[:, :, k0:k1], s, c)
        if k1 > k0 else _real_keyrange(q, k, v, s, c, k0, k1)),
    "merge weights not normalised": ("merge_partials", _merge_variant(lambda lp, lse, m: np.exp(lp - m))),
    "merge keeps only the largest range": (
        "merge_partials", _merge_variant(lambda lp, lse, m: (lp == m).astype(np.float64))),
    "merge averages ranges equally": (
        "merge_partials", _merge_variant(lambda lp, lse, m: np.ones_like(lp) / lp.shape[0])),
    "merged lse is the largest range's": (
        "merge_partials", lambda O, l: (_real_merge(O, l)[0], np.asarray(l).max(axis=0))),
}


def _failures(pins):
    failed = []
    for pin in pins:
        try:
            pin(oracle)
        except (AssertionError, ValueError, FloatingPointError, IndexError) as e:
            failed.append(f"{pin.__name__}: {e}")
    return failed


@pytest.mark.parametrize("name", sorted(FORWARD_MUTANTS))
def test_forward_mutant_is_caught(name, monkeypatch):
    attr, fn = FORWARD_MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.ALL_PINS)
    assert failed, f"no pin caught the planted mistake: {name}"


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(A, "_head_backward", _bwd_variant(BACKWARD_MUTANTS[name]))
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.BACKWARD_PINS)
    assert failed, f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert _failures(oracle_pins.ALL_PINS) == []


@pytest.mark.parametrize("name", sorted(SPLITKV_MUTANTS))
def test_splitkv_mutant_is_caught(name, monkeypatch):
    attr, fn = SPLITKV_MUTANTS[name]
    monkeypatch.setattr(SK, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.SPLITKV_PINS)
    assert failed, f"no pin caught the planted mistake: {name}"


@pytest.mark.parametrize("name", sorted(BLOCKSPARSE_MUTANTS))
def test_blocksparse_mutant_is_caught(name, monkeypatch):
    attr, fn = BLOCKSPARSE_MUTANTS[name]
    monkeypatch.setattr(BS, attr, fn)
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.BLOCKSPARSE_PINS)
    assert failed, f"no pin caught the planted mistake: {name}"


def test_blocksparse_bwd_ignoring_the_mask_is_caught(monkeypatch):
    dense = lambda q, k, v, dO, scale, causal, block_mask, block=128: oracle.attn_bwd(
        q, k, v, dO, scale, causal)
    monkeypatch.setattr(BS, "attn_bwd_blocksparse", dense)
    monkeypatch.setattr(oracle, "attn_bwd_blocksparse", dense)
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.BLOCKSPARSE_PINS)
    assert failed, "no pin caught the backward ignoring the block mask"


@pytest.mark.parametrize("name", sorted(BLOCKSPARSE_BWD_MUTANTS))
def test_blocksparse_bwd_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(BS, "attn_bwd_blocksparse", _bs_bwd_variant(BLOCKSPARSE_BWD_MUTANTS[name]))
    monkeypatch.setattr(oracle, "attn_bwd_blocksparse", BS.attn_bwd_blocksparse)
    with np.errstate(all="ignore"):
        failed = _failures(oracle_pins.BLOCKSPARSE_PINS)
    assert failed, f"no pin caught the planted mistake: {name}"
