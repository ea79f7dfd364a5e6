"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
call the HIP library through its binding, compare with the CPU oracle.

Tolerances (the method's own, stated with the workloads):
  * indices and every dispatch output are compared bit for bit;
  * a token is EXEMPT from the index comparison when the oracle's margin at a
    decision boundary -- K-th minus (K+1)-th candidate score, or KG-th minus
    (KG+1)-th group score -- is below 1e-6: float32 scores on the GPU may
    order such near-ties differently.  Exempt tokens are counted, not failed;
  * weights agree to 1e-5 relative where the selected sets agree;
  * logits agree to 1e-4 relative (floor 1 on the magnitude).
"""
from __future__ import annotations

import sys

import numpy as np

EXEMPT_MARGIN = 1e-6
WEIGHT_RTOL = 1e-5
LOGIT_RTOL = 1e-4


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev_inputs(gi, device="cuda"):
    import torch
    x = torch.from_numpy(gi.x.view(np.int16)).to(device).view(torch.bfloat16)
    W = torch.from_numpy(gi.W).to(device)
    b = torch.from_numpy(gi.bias).to(device)
    return x, W, b


def compare_gate(w_gpu: np.ndarray, i_gpu: np.ndarray, ref, route_scale: float,
                 rows: np.ndarray | None = None, check_sum: bool = True, *,
                 topk_group: int | None = None, renorm: bool = True,
                 mask_zero: int = 0, denom_eps: float = 0.0):
    """Compare GPU weights/indices (full [T, K] arrays, or ``rows`` of them)
    with an oracle result on the same rows.  Returns a stats dict; raises
    AssertionError on a non-exempt index mismatch, a weight outside
    tolerance, or an exempt token whose GPU selection is not a valid
    resolution of its near-tie (see ``check_near_tie``; that check needs the
    oracle's scores, ``ref.scores``, and ``topk_group`` when there are
    several groups)."""
    if rows is not None:
        w_gpu, i_gpu = w_gpu[rows], i_gpu[rows]
    margin = np.minimum(ref.margins[:, 0], ref.margins[:, 1])
    exempt = margin < EXEMPT_MARGIN
    same = np.all(i_gpu == ref.indices, axis=1)
    bad = ~same & ~exempt
    stats = dict(tokens=int(len(same)), exempt=int(exempt.sum()),
                 exempt_matched=int((exempt & same).sum()),
                 index_mismatch_nonexempt=int(bad.sum()))
    assert not bad.any(), (f"{int(bad.sum())} non-exempt tokens select different experts; "
                           f"first rows {np.nonzero(bad)[0][:5].tolist()}: "
                           f"gpu {i_gpu[bad][:2].tolist()} oracle {ref.indices[bad][:2].tolist()}")
    wr = ref.weights[same]
    wg = w_gpu[same].astype(np.float64)
    rel = np.abs(wg - wr) / np.maximum(np.abs(wr), 1e-30)
    stats["weight_max_rel"] = float(rel.max()) if rel.size else 0.0
    assert stats["weight_max_rel"] <= WEIGHT_RTOL, stats
    # exempt tokens that differ: the GPU's choice must be one of the valid
    # resolutions of the near-tie
    differ = np.nonzero(exempt & ~same)[0]
    stats["exempt_differ_valid"] = 0
    for r in differ:
        assert ref.scores is not None, \
            "an exempt token differs from the oracle; its check needs the oracle's scores"
        G = max(1, ref.scores.group.shape[1])
        assert G == 1 or topk_group is not None, "the near-tie check needs topk_group"
        check_near_tie(i_gpu[r], w_gpu[r], ref.scores.affinity[r], ref.scores.choice[r],
                       ref.scores.group[r] if G > 1 else None, topk_group or 1,
                       route_scale, renorm, mask_zero, denom_eps)
        stats["exempt_differ_valid"] += 1
    # properties that hold for every token, exempt or not
    assert np.all(w_gpu >= 0)
    if check_sum:
        sums = w_gpu.astype(np.float64).sum(1)
        assert np.allclose(sums, route_scale, rtol=1e-5, atol=0), "weights do not sum to route_scale"
    return stats


def _kept_candidates(ids: np.ndarray, gs: np.ndarray, KG: int, S: int):
    """Kept-group sets that a near-tie resolution might have used: the
    groups of the winners filled up with the best other groups, and the
    best KG groups themselves (ties to the lower group index)."""
    G = len(gs)
    rank = sorted(range(G), key=lambda g: (-gs[g], g))
    out = [set(rank[:KG])]
    gw = {int(e) // S for e in ids}
    if len(gw) <= KG:
        fill = [g for g in rank if g not in gw][:KG - len(gw)]
        out.insert(0, gw | set(fill))
    return out


def check_near_tie(ids: np.ndarray, w: np.ndarray, s: np.ndarray, v: np.ndarray,
                   gs: np.ndarray | None, topk_group: int, route_scale: float,
                   renorm: bool = True, mask_zero: int = 0, denom_eps: float = 0.0,
                   tol: float = EXEMPT_MARGIN):
    """One token whose oracle margin is below the exemption threshold and
    whose GPU selection differs from the oracle's.  The selection is valid
    when, against the oracle's float64 scores, some set of topk_group kept
    groups has every kept group scoring at least every dropped group's score
    minus ``tol``, and under it every winner's masked choice score is at
    least every loser's minus ``tol``.  The weights must then equal the
    oracle's weights recomputed on the GPU's set, to the weight tolerance."""
    ids = np.asarray(ids, dtype=np.int64)
    K, E = len(ids), len(v)
    assert len(np.unique(ids)) == K and ids.min() >= 0 and ids.max() < E
    lose = np.ones(E, bool)
    lose[ids] = False
    fill = 0.0 if mask_zero else -np.inf
    ok = False
    if gs is None:
        cands = [None]
    else:
        S = E // len(gs)
        cands = _kept_candidates(ids, gs, topk_group, S)
    for kept in cands:
        if kept is None:
            vm = v
        else:
            drop = [g for g in range(len(gs)) if g not in kept]
            if drop and min(gs[g] for g in kept) < max(gs[g] for g in drop) - tol:
                continue
            inside = np.isin(np.arange(E) // S, list(kept))
            vm = np.where(inside, v, fill)
        if not np.all(np.isfinite(vm[ids])):
            continue
        if not lose.any() or vm[ids].min() >= vm[lose].max() - tol:
            ok = True
            break
    assert ok, (f"exempt token: GPU experts {ids.tolist()} are not a valid resolution of "
                f"the near-tie (choice scores {v[ids].tolist()})")
    ss = s[ids]
    want = route_scale * ss / (ss.sum() + denom_eps) if renorm else route_scale * ss
    rel = np.abs(np.asarray(w, np.float64) - want) / np.maximum(np.abs(want), 1e-30)
    assert rel.max() <= WEIGHT_RTOL, f"exempt token: weights off by {rel.max():.2e} relative"


def check_rows_valid(i_gpu: np.ndarray, E: int, n_group: int, topk_group: int,
                     order: int = 0):
    """Properties every row must have: ids in range, distinct, ascending
    (order 0), and drawn from at most topk_group groups."""
    assert i_gpu.min() >= 0 and i_gpu.max() < E
    s = np.sort(i_gpu, axis=1)
    assert np.all(s[:, 1:] != s[:, :-1]), "a token selected an expert twice"
    if order == 0:
        assert np.array_equal(s, i_gpu), "order 0 rows are not ascending"
    S = E // n_group
    g = s // S
    ngroups = 1 + np.sum(g[:, 1:] != g[:, :-1], axis=1)
    assert np.all(ngroups <= topk_group), "a token uses more groups than topk_group"


def compare_dispatch(out, ref, indices: np.ndarray, x: np.ndarray, K: int,
                     sample_rows: np.ndarray | None = None, oracle=None):
    """Bit-exact comparison of the dispatch outputs with the oracle on the
    same indices.  ``sample_rows`` limits the permuted-row check."""
    tpe = out.tokens_per_expert.cpu().numpy()
    perm = out.perm.cpu().numpy()
    assert np.array_equal(tpe, ref.counts), "tokens_per_expert differs"
    if out.offsets is not None:
        assert np.array_equal(out.offsets.cpu().numpy(), ref.offsets), "offsets differ"
    assert np.array_equal(perm, ref.perm), "perm differs"
    if out.dest is not None:
        dest = out.dest.cpu().numpy()
        inv = np.empty_like(ref.perm)
        inv[ref.perm] = np.arange(len(ref.perm), dtype=ref.perm.dtype)
        assert np.array_equal(dest, inv), "dest is not the inverse of perm"
    n = len(ref.perm)
    if sample_rows is None:
        compare_rows_full(out.permuted_x, x, ref.perm, K, oracle)
        return
    rows = sample_rows
    if len(rows):
        import torch
        got = out.permuted_x[torch.from_numpy(rows).to(out.permuted_x.device)]
        got = got.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.gather_rows(x, ref.perm, K, rows)
        assert np.array_equal(got, want), "permuted_x rows differ"


def compare_rows_full(permuted_x, x: np.ndarray, perm: np.ndarray, K: int, oracle,
                      chunk_bytes: int = 1 << 28):
    """Every row of the GPU's permuted_x against the oracle's row gather on
    the same permutation, copied to the host in chunks of about
    ``chunk_bytes``."""
    import torch
    n = len(perm)
    d = x.shape[1]
    step = max(1, chunk_bytes // (2 * d))
    flat = permuted_x.view(torch.int16)
    for p0 in range(0, n, step):
        p1 = min(n, p0 + step)
        got = flat[p0:p1].cpu().numpy().view(np.uint16)
        want = oracle.gather_rows(x, perm, K, np.arange(p0, p1))
        if not np.array_equal(got, want):
            bad = np.nonzero(np.any(got != want, axis=1))[0]
            raise AssertionError(f"permuted_x rows differ: {len(bad)} rows in [{p0}, {p1}), "
                                 f"first {p0 + int(bad[0])}")


def combine_tolerance(o, outs, w64, dest, y64, K):
    """Bound on |GPU - float64 sum|: one bfloat16 unit of the result (the
    final rounding) plus K float32 roundings of partial sums bounded by the
    sum of absolute terms (computed by the oracle on |out| and |w|)."""
    ya64, _ = o.combine(outs & np.uint16(0x7FFF), np.abs(w64), dest)
    return 2.0 ** -7 * np.abs(y64) + K * 2.0 ** -23 * ya64 + 1e-38


def score_error(lg_gpu: np.ndarray, lg_ref: np.ndarray, bias: np.ndarray,
                margins: np.ndarray, same: np.ndarray) -> dict:
    """Largest |v32 - v64| of the sigmoid choice scores v = sigmoid(L) + b,
    v32 formed in float32 from the GPU's logits and v64 in float64 from the
    oracle's, over every token and expert given; and the tokens whose margin
    lies between the exemption threshold and twice that error (not exempt,
    yet within reach of the score error), with how many differ."""
    one = np.float32(1.0)
    v32 = one / (one + np.exp(-lg_gpu.astype(np.float32))) + bias.astype(np.float32)[None, :]
    v64 = 1.0 / (1.0 + np.exp(-lg_ref)) + bias.astype(np.float64)[None, :]
    err = float(np.abs(v32.astype(np.float64) - v64).max())
    margin = np.minimum(margins[:, 0], margins[:, 1])
    band = (margin >= EXEMPT_MARGIN) & (margin < 2.0 * err)
    return {"score_max_abs_err": err, "near_band_tokens": int(band.sum()),
            "near_band_mismatch": int((band & ~same).sum())}

