"""Helpers of the GPU parity tests: set up a layer from a workload config, run it
through libmoe's C ABI, and compare with the oracle.

Comparison rules (written out here so every test uses the same bar):
  - expert ids, group offsets, perm, inv_perm: bit-exact;
  - the layer output y: relative L2 <= 5e-3 and max |gpu - oracle| <=
    2e-2 * rms(oracle), in fp64, where "oracle" is the oracle's exact value
    before its final bf16 rounding (so the GPU's own final rounding counts as
    error, and a rounding-boundary straddle cannot fail the bound);
  - intermediates h and expert rows Y (each already rounded to bf16 on both
    sides): relative L2 <= 5e-3 and, per element, |gpu - oracle| <=
    2e-2 * rms(oracle) + 2^-7 * |oracle|, i.e. the same bar plus one bf16
    rounding step: a value whose fp32 (GPU) and fp64 (oracle) pre-rounding
    values straddle a bf16 boundary rounds one unit apart;
  - router weights: |w_gpu - w_oracle| <= 1e-5 (fp32 exp and division);
  - shared gate sigma: |delta| <= 1e-6;
  - router logits (when computed from W_r): |delta| <= 2^-18 * sum_h |x_h W_he|
    (a few fp32 rounding errors per term at most).
When logits are computed on both sides in different summation orders, an id
may legitimately differ where two logits are closer than their rounding
error; such a token is accepted only if (a) the GPU's set is the exact top-k of
the GPU's own logits and (b) every swapped expert lies within the measured
logit error of the oracle's k-th logit.  Its outputs are then excluded from
the downstream comparison and the count is reported.  Grouping (offsets,
perm, inv_perm) is always compared bit for bit with the oracle's grouping of
the GPU's own ids, so a near-tie never skips it."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O

REL_L2 = 5e-3
MAX_ABS_RMS = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, name: str, ulp_slack: bool = False) -> dict:
    """ulp_slack=False: the layer-output bar; True: the intermediate bar."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), name + ": non-finite GPU values"
    diff = gpu - ref
    nref = np.linalg.norm(ref)
    rel = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    assert rel <= REL_L2, "%s: relative L2 %.3e > %.1e" % (name, rel, REL_L2)
    bound = MAX_ABS_RMS * rms + (2.0 ** -7 * np.abs(ref) if ulp_slack else 0.0) + 1e-30
    excess = np.abs(diff) - bound
    assert np.all(excess <= 0), "%s: |d| exceeds the bound by %.3e (max |d| %.3e, rms %.3e)" % (
        name, float(np.max(excess)), mx, rms)
    return dict(rel_l2=rel, max_abs=mx, rms=rms)


def check_ids(gpu_ids: np.ndarray, ora_ids: np.ndarray, gpu_logits=None, ora_logits=None) -> np.ndarray:
    """Returns a bool mask of tokens whose ids match bit-exactly.  Without
    logits (drawn logits, identical inputs) every token must match."""
    same = np.all(gpu_ids == ora_ids, axis=1)
    if gpu_logits is None:
        assert same.all(), "expert ids differ at tokens %s" % np.nonzero(~same)[0][:10]
        return same
    k = gpu_ids.shape[1]
    for t in np.nonzero(~same)[0]:
        gl = gpu_logits[t].astype(np.float64)
        # (a) the GPU's ids are the top-k of its own logits, in order, ties to the lower index
        order = sorted(range(len(gl)), key=lambda e: (-gl[e], e))[:k]
        assert list(gpu_ids[t]) == order, "token %d: GPU ids are not the top-k of its own logits" % t
        # (b) every difference is a near tie in the oracle's logits
        ol = ora_logits[t].astype(np.float64)
        err = float(np.max(np.abs(gl - ol)))
        kth = ol[ora_ids[t, -1]]
        for e in set(gpu_ids[t]) ^ set(ora_ids[t]):
            assert abs(ol[e] - kth) <= 4 * err, "token %d: expert %d is not a near tie (%.3e > 4 x %.3e)" % (
                t, e, abs(ol[e] - kth), err)
        if set(gpu_ids[t]) == set(ora_ids[t]):
            # same set, different slot order: the swapped slots must be near ties too
            for j in np.nonzero(gpu_ids[t] != ora_ids[t])[0]:
                assert abs(ol[gpu_ids[t, j]] - ol[ora_ids[t, j]]) <= 4 * err
    return same


def logit_bound(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    return 2.0 ** -18 * (np.abs(x) @ np.abs(w_router.astype(np.float64)))


def compare_layer(buf, ora: "O.LayerResult", T: int, k: int, E: int, drawn_logits: bool,
                  x64: np.ndarray = None, w_router: np.ndarray = None, check_rows: bool = True) -> dict:
    """Compare one layer's GPU buffers with the oracle's result (ora covers
    ora.tokens for the FFN/combine parts and every token for routing)."""
    stats = {}
    gpu_ids = buf.ids.cpu().numpy()
    if drawn_logits:
        same = check_ids(gpu_ids, ora.ids)
    else:
        gl = buf.logits.cpu().numpy()
        bound = logit_bound(x64, w_router)
        dl = np.abs(gl.astype(np.float64) - ora.logits.astype(np.float64))
        assert np.all(dl <= bound), "router logits: max excess %.3e" % float(np.max(dl - bound))
        stats["logit_max_abs"] = float(dl.max())
        same = check_ids(gpu_ids, ora.ids, gl, ora.logits)
    stats["id_near_ties"] = int((~same).sum())
    w = buf.w.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(w[same] - ora.w[same])) <= 1e-5, "router weights"
    assert np.max(np.abs(buf.sigma.cpu().numpy() - ora.sigma)) <= 1e-6, "shared gate"
    # grouping, bit for bit, always: against the oracle's grouping of the GPU's
    # own ids (the same as ora.groups when every id matched)
    g = ora.groups if same.all() else O.group(gpu_ids, E)
    assert np.array_equal(buf.offsets.cpu().numpy(), g.offsets), "offsets"
    assert np.array_equal(buf.perm.cpu().numpy(), g.perm), "perm"
    assert np.array_equal(buf.inv_perm.cpu().numpy(), g.inv_perm), "inv_perm"
    toks = [int(t) for t in ora.tokens if same[int(t)]]
    if not toks:
        return stats
    if check_rows:
        inv = buf.inv_perm.cpu().numpy()
        rows = [int(inv[t * k + j]) for t in toks for j in range(k)] + [T * k + t for t in toks]
        rows_t = torch.as_tensor(rows, device=buf.h.device)
        h = bf16_to_f64(buf.h.index_select(0, rows_t))
        yr = bf16_to_f64(buf.y_rows.index_select(0, rows_t))
        stats["h"] = assert_close(h, np.stack([ora.h[p] for p in rows]), "h", ulp_slack=True)
        stats["y_rows"] = assert_close(yr, np.stack([ora.y_rows[p] for p in rows]), "expert rows Y", ulp_slack=True)
    sel = [list(ora.tokens).index(t) for t in toks]
    y = bf16_to_f64(buf.y.index_select(0, torch.as_tensor(toks, device=buf.y.device)))
    stats["y"] = assert_close(y, ora.y_pre[sel], "y")
    stats["y_bits_equal_frac"] = float(np.mean(y == ora.y[sel]))
    return stats
