"""Pins that tie the CPU oracle to the pages and to the mathematics rather
than to itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when that oracle disagrees with something fixed independently of it:
exact integer arithmetic, enumeration of every candidate subset against the
defining "every winner beats every loser" property, closed forms (x = 0
gives every weight route_scale / K), library routines for the special cases
they cover (numpy sorts and bincount, scipy's expit), invariants the pages
state (weights sum to route_scale, winners lie in kept groups, the bias moves
the selection but not the weights) and metamorphic relations (a constant
added to every bias, permutations of groups and of experts inside a group).

``test_oracle_pins.py`` runs them on the oracle; ``test_oracle_mutants.py``
runs them on copies of the oracle with a planted mistake and expects at least
one to fail.
"""
from __future__ import annotations

import itertools

import numpy as np
from scipy.special import expit

# Small configurations: (E, n_group, topk_group, top_k)
TINY_CFGS = [(8, 4, 2, 3), (12, 3, 2, 4), (16, 4, 2, 4), (16, 1, 1, 4),
             (16, 8, 3, 5), (32, 8, 4, 8), (24, 6, 6, 5), (10, 5, 1, 2)]


def _precedes(va, a, vb, b):
    return va > vb or (va == vb and a < b)


def _is_top_set(members, values, pool):
    """True when every member of ``members`` precedes every other element of
    ``pool`` under (value descending, index ascending)."""
    rest = [e for e in pool if e not in members]
    return all(_precedes(values[m], m, values[r], r) for m in members for r in rest)


def brute_force_gate(v, E, G, KG, K, group_max=False, fill=None):
    """Selected expert set by exhaustive enumeration.  Group score is the
    best pair sum inside the group (= sum of its two largest members), or the
    best single member when ``group_max``; exactly one group subset and one
    expert subset may satisfy the top-set property.  Experts of dropped
    groups are excluded, or -- with ``fill`` -- compete with value ``fill``."""
    S = E // G
    if G > 1:
        if group_max:
            gs = [max(v[g * S + i] for i in range(S)) for g in range(G)]
        else:
            gs = [max(v[g * S + i] + v[g * S + j]
                      for i in range(S) for j in range(i + 1, S)) for g in range(G)]
        kept = [c for c in itertools.combinations(range(G), KG)
                if _is_top_set(set(c), gs, range(G))]
        assert len(kept) == 1, "group top-set not unique"
        kept = kept[0]
    else:
        gs = None
        kept = (0,)
    if fill is None:
        cand = [e for e in range(E) if e // S in kept]
        vals = v
    else:
        cand = list(range(E))
        vals = [v[e] if e // S in kept else fill for e in range(E)]
    sets = [c for c in itertools.combinations(cand, K) if _is_top_set(set(c), vals, cand)]
    assert len(sets) == 1, "expert top-set not unique"
    return sorted(sets[0]), kept, gs, cand


def _discrete_case(rng, E, tie=False):
    """Logits on a coarse lattice (optionally with exact duplicates) and a
    bias on a coarse lattice: distinct choice scores are then far apart."""
    # the offset keeps the lattice asymmetric, so no two pairs of distinct
    # logits can have sigmoid sums that are equal only mathematically
    L = rng.integers(-40, 41, size=E) * 0.0625 + 0.01
    if tie:
        # copy a few experts' logits onto others so scores tie exactly
        for _ in range(max(1, E // 6)):
            a, b = rng.choice(E, size=2, replace=False)
            L[b] = L[a]
    b = (rng.integers(-8, 9, size=E) / 256.0).astype(np.float32)
    if tie:
        b[:] = 0.0
    return L, b


def _v(L, b):
    return expit(L) + b.astype(np.float64)


def pin_exact_integer_logits(o):
    """x small integers (exact in bfloat16), W integers times 2^-8: every
    product and partial sum is exact, so the logits equal integer math."""
    from sigmoid_group_limited_amd.workloads import bf16_bits
    rng = np.random.default_rng(11)
    T, d, E = 5, 37, 7
    xi = rng.integers(-8, 9, size=(T, d))
    wi = rng.integers(-8, 9, size=(E, d))
    x = bf16_bits(xi.astype(np.float32))
    W = (wi / 256.0).astype(np.float32)
    want = (xi.astype(np.int64) @ wi.astype(np.int64).T) / 256.0
    got = o.logits(x, W)
    assert got.shape == (T, E)
    assert np.array_equal(got, want), "logits differ from exact integer arithmetic"


def pin_logits_vs_matmul(o):
    """Random bfloat16 x and float32 W: float64 logits agree with numpy's
    float64 matmul to rounding."""
    from sigmoid_group_limited_amd.workloads import bf16_bits, bf16_to_f32
    rng = np.random.default_rng(12)
    T, d, E = 6, 7168, 10
    x = bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    W = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    want = bf16_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    got = o.logits(x, W)
    assert np.allclose(got, want, rtol=0, atol=1e-12), "logits differ from matmul"


def pin_brute_force_selection(o):
    """Tiny configurations with and without exact ties: the oracle's set is
    the unique enumerated top set, with lower indices winning ties."""
    rng = np.random.default_rng(13)
    for (E, G, KG, K) in TINY_CFGS:
        for trial in range(6):
            L, b = _discrete_case(rng, E, tie=(trial % 2 == 1))
            want, _, _, _ = brute_force_gate(_v(L, b), E, G, KG, K)
            r = o.select(L[None, :], b, G, KG, K, 1.0)
            assert list(r.indices[0]) == want, (
                f"E={E} G={G} KG={KG} K={K}: {list(r.indices[0])} != {want}")


def pin_zero_input_closed_form(o):
    """x = 0 gives L = 0 and s = 1/2 for every expert: each weight is exactly
    route_scale / K and the selection is the group-limited top-K of the bias."""
    rng = np.random.default_rng(14)
    E, G, KG, K, scale, d = 256, 8, 4, 8, 2.5, 64
    x = np.zeros((3, d), dtype=np.uint16)
    W = rng.standard_normal((E, d)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    r = o.gate(x, W, b, G, KG, K, scale)
    assert np.all(r.weights == scale / K), "weights for x=0 are not route_scale/K"
    v = 0.5 + b.astype(np.float64)
    S = E // G
    gs = np.array([np.sort(v[g * S:(g + 1) * S])[-2:].sum() for g in range(G)])
    kept = np.lexsort((np.arange(G), -gs))[:KG]
    cand = np.array([e for e in range(E) if e // S in kept])
    top = cand[np.lexsort((cand, -v[cand]))[:K]]
    for t in range(3):
        assert list(r.indices[t]) == sorted(top.tolist()), "x=0 selection wrong"


def pin_bias_shift_invariance(o):
    """Adding the same constant to every bias shifts every choice score by it
    and every group score by twice it: nothing changes."""
    rng = np.random.default_rng(15)
    E, G, KG, K = 64, 8, 3, 6
    L = rng.standard_normal((40, E))
    b = (rng.integers(-64, 65, size=E) / 1024.0).astype(np.float32)
    r0 = o.select(L, b, G, KG, K, 2.5)
    r1 = o.select(L, (b + np.float32(0.25)).astype(np.float32), G, KG, K, 2.5)
    ok = np.minimum(r0.margins[:, 0], r0.margins[:, 1]) > 1e-9
    assert ok.sum() > 30
    assert np.array_equal(r0.indices[ok], r1.indices[ok]), "bias shift changed selection"
    assert np.array_equal(r0.weights[ok], r1.weights[ok]), "bias shift changed weights"


def pin_weights_follow_unbiased_sigmoid(o):
    """Weights are >= 0, sum to route_scale, and are proportional to the
    UNBIASED sigmoid of the winners' logits (scipy expit); a bias large enough
    to force an expert in changes the set but not this proportionality."""
    rng = np.random.default_rng(16)
    E, G, KG, K, scale = 64, 8, 4, 8, 2.827
    L = rng.standard_normal((50, E)) * 2.0
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    b[5] = 0.75     # forces expert 5 in whenever its group is kept
    b[6] = -0.75    # keeps expert 6 out
    r = o.select(L, b, G, KG, K, scale)
    assert np.all(r.weights >= 0)
    assert np.allclose(r.weights.sum(1), scale, rtol=1e-12, atol=0)
    s = expit(np.take_along_axis(L, r.indices.astype(np.int64), axis=1))
    want = scale * s / s.sum(1, keepdims=True)
    assert np.allclose(r.weights, want, rtol=1e-12, atol=0), "weights not scale*s/sum(s)"
    assert not (r.indices == 6).any(), "a large negative bias did not exclude its expert"
    kept5 = (r.indices == 5).any(1)
    assert kept5.sum() >= 20, "a large positive bias did not pull its expert in"


def pin_winners_in_kept_groups(o):
    """Random DeepSeek-V3-shaped logits: the kept groups are the top
    topk_group by top-2 sum (library sort), every winner lies in them, and the
    winners are the top-K candidates (library lexsort)."""
    rng = np.random.default_rng(17)
    E, G, KG, K = 256, 8, 4, 8
    S = E // G
    L = rng.standard_normal((64, E))
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    # make some biased scores negative so a 0.0 mask would differ from -inf
    b[: S * 2] -= np.float32(0.6)
    # second pass: nearly every choice score negative, where masking the
    # dropped groups with 0.0 instead of -inf would change the winners
    for bb in (b, (b - np.float32(0.9)).astype(np.float32)):
        r = o.select(L, bb, G, KG, K, 2.5)
        v = _v(L, bb)
        for t in range(L.shape[0]):
            gs = np.sort(v[t].reshape(G, S), axis=1)[:, -2:].sum(1)
            kept = np.lexsort((np.arange(G), -gs))[:KG]
            assert set(np.asarray(r.indices[t]) // S) <= set(kept.tolist()), \
                "winner outside kept groups"
            cand = np.array([e for e in range(E) if e // S in kept])
            top = cand[np.lexsort((cand, -v[t][cand]))[:K]]
            assert list(r.indices[t]) == sorted(top.tolist())


def pin_single_group_no_bias_is_topk_of_logits(o):
    """One group and zero bias: the selection is the top-K of the logits
    (sigmoid is increasing), found by a stable library sort."""
    rng = np.random.default_rng(18)
    E, K = 384, 8
    L = rng.standard_normal((32, E))
    r = o.select(L, np.zeros(E, np.float32), 1, 1, K, 2.827)
    top = np.sort(np.argsort(-L, axis=1, kind="stable")[:, :K], axis=1)
    assert np.array_equal(r.indices, top)


def pin_permutation_equivariance(o):
    """Permuting whole groups, and experts inside each group, permutes the
    selected set the same way and leaves each expert's weight unchanged."""
    rng = np.random.default_rng(19)
    E, G, KG, K = 128, 8, 4, 8
    S = E // G
    L = rng.standard_normal((48, E))
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    gperm = rng.permutation(G)
    new_to_old = np.concatenate([gperm[g] * S + rng.permutation(S) for g in range(G)])
    r0 = o.select(L, b, G, KG, K, 2.5)
    r1 = o.select(L[:, new_to_old], b[new_to_old], G, KG, K, 2.5)
    ok = np.minimum(r0.margins[:, 0], r0.margins[:, 1]) > 1e-12
    for t in np.nonzero(ok)[0]:
        mapped = {int(new_to_old[e]): w for e, w in zip(r1.indices[t], r1.weights[t])}
        orig = {int(e): w for e, w in zip(r0.indices[t], r0.weights[t])}
        assert mapped.keys() == orig.keys(), "selection not permutation-equivariant"
        for e in orig:
            assert abs(mapped[e] - orig[e]) <= 1e-12 * abs(orig[e])


def pin_margins(o):
    """Margins: K-th minus (K+1)-th candidate score and KG-th minus
    (KG+1)-th group score, from library sorts."""
    rng = np.random.default_rng(20)
    E, G, KG, K = 64, 8, 3, 5
    S = E // G
    L = rng.standard_normal((30, E))
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    r = o.select(L, b, G, KG, K, 1.0)
    v = _v(L, b)
    for t in range(L.shape[0]):
        gs = np.sort(v[t].reshape(G, S), axis=1)[:, -2:].sum(1)
        gsort = np.sort(gs)[::-1]
        kept = np.lexsort((np.arange(G), -gs))[:KG]
        cand = np.sort(np.concatenate([v[t][g * S:(g + 1) * S] for g in kept]))[::-1]
        assert abs(r.margins[t, 0] - (cand[K - 1] - cand[K])) <= 1e-12
        assert abs(r.margins[t, 1] - (gsort[KG - 1] - gsort[KG])) <= 1e-12
    r1 = o.select(L, b, 1, 1, K, 1.0)
    assert np.all(np.isinf(r1.margins[:, 1])), "single group has no group margin"


def pin_selection_order(o):
    """order=1 lists the same set as order=0, by score descending (index
    ascending on ties)."""
    rng = np.random.default_rng(21)
    E, G, KG, K = 64, 4, 2, 8
    L, b = _discrete_case(rng, E, tie=True)
    L = np.stack([L, rng.standard_normal(E)])
    r0 = o.select(L, b, G, KG, K, 1.0, order=0)
    r1 = o.select(L, b, G, KG, K, 1.0, order=1)
    v = _v(L, b)
    for t in range(2):
        assert sorted(r1.indices[t]) == list(r0.indices[t])
        assert list(r0.indices[t]) == sorted(r0.indices[t])
        seq = [(v[t][e], e) for e in r1.indices[t]]
        for (va, a), (vb, bb) in zip(seq, seq[1:]):
            assert _precedes(va, a, vb, bb), "order=1 is not score-descending"
        w1 = dict(zip(r1.indices[t], r1.weights[t]))
        w0 = dict(zip(r0.indices[t], r0.weights[t]))
        assert all(abs(w1[e] - w0[e]) <= 1e-15 for e in w0)


def pin_dispatch(o):
    """Counts are a bincount, offsets their exclusive prefix sum, the
    permutation a stable argsort of the flat expert ids, and the gathered rows
    are x[perm // K]."""
    from sigmoid_group_limited_amd.workloads import random_indices
    rng = np.random.default_rng(22)
    for (T, K, E) in [(0, 8, 16), (1, 8, 16), (37, 8, 64), (300, 3, 7), (513, 8, 256)]:
        idx = random_indices(T, K, E, seed=T) if T else np.zeros((0, K), np.int32)
        r = o.dispatch(idx, E)
        flat = idx.ravel()
        assert np.array_equal(r.counts, np.bincount(flat, minlength=E))
        assert r.offsets[0] == 0
        assert np.array_equal(r.offsets[1:], np.cumsum(np.bincount(flat, minlength=E)))
        assert np.array_equal(r.perm, np.argsort(flat, kind="stable"))
        if T:
            x = rng.integers(0, 65536, size=(T, 24), dtype=np.uint16)
            rows = o.gather_rows(x, r.perm, K)
            assert np.array_equal(rows, x[r.perm // K])


def pin_softmax_scores(o):
    """Softmax scoring: the affinities are scipy's softmax over all E
    logits; the selection is the enumerated top set of softmax + bias; with
    the default rule the K weights are NOT renormalised (route_scale times
    the gathered probabilities), and forcing renormalisation makes them sum
    to route_scale."""
    from scipy.special import softmax
    rng = np.random.default_rng(23)
    for (E, G, KG, K) in [(16, 4, 2, 4), (12, 3, 2, 3), (16, 1, 1, 5)]:
        for _ in range(4):
            L, b = _discrete_case(rng, E)
            sm = softmax(L)
            want, _, _, _ = brute_force_gate(sm + b.astype(np.float64), E, G, KG, K)
            r = o.select(L[None, :], b, G, KG, K, 1.5, score_func=1)
            assert list(r.indices[0]) == want
            assert np.allclose(r.weights[0], 1.5 * sm[want], rtol=1e-12, atol=0)
            r1 = o.select(L[None, :], b, G, KG, K, 1.5, score_func=1, renorm=1)
            assert np.allclose(r1.weights[0].sum(), 1.5, rtol=1e-12)
            assert np.allclose(r1.weights[0], 1.5 * sm[want] / sm[want].sum(), rtol=1e-12)


def pin_no_bias_group_max(o):
    """No bias: the choice score is the affinity and a group scores by its
    largest member (enumerated); sigmoid weights still renormalise."""
    rng = np.random.default_rng(24)
    for (E, G, KG, K) in [(8, 4, 2, 3), (16, 4, 2, 4), (16, 8, 3, 5), (24, 6, 2, 4)]:
        for trial in range(4):
            L, _ = _discrete_case(rng, E, tie=(trial % 2 == 1))
            s = expit(L)
            want, _, _, _ = brute_force_gate(s, E, G, KG, K, group_max=True)
            r = o.select(L[None, :], None, G, KG, K, 2.0)
            assert list(r.indices[0]) == want
            assert np.allclose(r.weights[0], 2.0 * s[want] / s[want].sum(), rtol=1e-12)


def pin_renorm_off(o):
    """renorm=2 (off) with sigmoid: each weight is route_scale * sigmoid of
    its logit (scipy expit)."""
    rng = np.random.default_rng(25)
    L = rng.standard_normal((20, 64))
    b = rng.uniform(-0.05, 0.05, size=64).astype(np.float32)
    r = o.select(L, b, 8, 4, 8, 2.5, renorm=2)
    s = expit(np.take_along_axis(L, r.indices.astype(np.int64), axis=1))
    assert np.allclose(r.weights, 2.5 * s, rtol=1e-12, atol=0)


def pin_mask_zero(o):
    """mask_zero: experts of dropped groups compete with value 0.0 (the
    Kimi K2 page's masked_fill), so with negative choice scores in the kept
    groups the zero-filled experts win, lowest ids first (enumeration)."""
    rng = np.random.default_rng(26)
    for (E, G, KG, K) in [(16, 4, 2, 4), (12, 3, 2, 5), (16, 8, 3, 6)]:
        for shift in (0.0, -0.9):
            L, b = _discrete_case(rng, E)
            b = (b + np.float32(shift)).astype(np.float32)
            v = expit(L) + b.astype(np.float64)
            want, kept, _, _ = brute_force_gate(v, E, G, KG, K, fill=0.0)
            r = o.select(L[None, :], b, G, KG, K, 1.0, mask_zero=1)
            assert list(r.indices[0]) == want
            if shift < 0:
                S = E // G
                assert any(e // S not in kept for e in want), "case does not exercise the fill"


def pin_denominator_epsilon(o):
    """An epsilon in the denominator is invisible at ordinary scores but
    dominates when every affinity underflows towards zero: logits near -700
    give s ~ 1e-304, so with epsilon 1e-20 the weights collapse to ~0 while
    without it they still sum to route_scale."""
    L = np.full((1, 16), -700.0) + np.arange(16)[None, :] * 0.01
    b = np.zeros(16, np.float32)
    r0 = o.select(L, b, 1, 1, 4, 2.827)
    r1 = o.select(L, b, 1, 1, 4, 2.827, denom_eps=1e-20)
    assert np.isclose(r0.weights.sum(), 2.827, rtol=1e-12)
    assert r1.weights.max() < 1e-250
    Ln = np.random.default_rng(27).standard_normal((5, 16))
    a = o.select(Ln, b, 1, 1, 4, 2.827)
    c = o.select(Ln, b, 1, 1, 4, 2.827, denom_eps=1e-20)
    assert np.array_equal(a.indices, c.indices)
    assert np.allclose(a.weights, c.weights, rtol=1e-15, atol=0)


def pin_combine(o):
    """Combine: equals numpy's float64 einsum over the un-permuted rows; with
    identity experts (outputs = dispatched rows) it returns
    (sum of the token's weights) * x, i.e. route_scale * x for gate weights."""
    from sigmoid_group_limited_amd.workloads import bf16_bits, bf16_to_f32, random_indices
    rng = np.random.default_rng(28)
    T, K, E, d = 37, 8, 32, 24
    idx = random_indices(T, K, E, seed=5)
    disp = o.dispatch(idx, E)
    dest = np.empty(T * K, np.int32)
    dest[disp.perm] = np.arange(T * K, dtype=np.int32)
    outs = bf16_bits(rng.standard_normal((T * K, d), dtype=np.float32))
    w = rng.uniform(0, 1, size=(T, K))
    y64, y16 = o.combine(outs, w, dest)
    rows = bf16_to_f32(outs).astype(np.float64)[dest.reshape(T, K)]
    want = np.einsum("tk,tkd->td", w, rows)
    assert np.allclose(y64, want, rtol=0, atol=1e-12)
    assert np.array_equal(y16, bf16_bits(y64.astype(np.float32)))
    x = bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    gw = o.select(rng.standard_normal((T, E)), np.zeros(E, np.float32), 1, 1, K, 2.827).weights
    ident = o.gather_rows(x, disp.perm, K)
    y64, _ = o.combine(ident, gw, dest)
    assert np.allclose(y64, 2.827 * bf16_to_f32(x).astype(np.float64), rtol=1e-12, atol=1e-300)


def _ep_case(rng, T, K, E):
    from sigmoid_group_limited_amd.workloads import random_indices
    return random_indices(T, K, E, seed=int(rng.integers(1 << 30)))


def pin_ep_send_splits(o):
    """Per-rank send splits are numpy's segment sums of tokens_per_expert."""
    rng = np.random.default_rng(29)
    for (E, R) in [(256, 8), (384, 8), (384, 3), (16, 16), (16, 1)]:
        tpe = rng.integers(0, 1000, size=E).astype(np.int32)
        c, off = o.ep_send_splits(tpe, R)
        assert np.array_equal(c, tpe.reshape(R, -1).sum(1))
        assert np.array_equal(off, np.r_[0, np.cumsum(c)])


def pin_ep_regroup(o):
    """Receive-side regroup is a stable library argsort of the received
    rows' local-expert labels; and end to end, simulating the exchange with
    numpy between R ranks that each dispatch their own tokens, every rank
    ends up with, per local expert, the rows all sources sent for it, source
    rank by source rank in the sources' dispatch order."""
    rng = np.random.default_rng(30)
    for (R, per) in [(8, 32), (4, 3), (1, 5), (3, 1)]:
        counts = rng.integers(0, 6, size=(R, per)).astype(np.int32)
        lc, rg = o.ep_regroup(counts)
        labels = np.repeat(np.tile(np.arange(per), R), counts.ravel())
        assert np.array_equal(rg, np.argsort(labels, kind="stable"))
        assert np.array_equal(lc, counts.sum(0))
    R, T, K, E, d = 4, 50, 4, 32, 3
    per = E // R
    xs = [rng.integers(0, 65536, size=(T, d), dtype=np.uint16) for _ in range(R)]
    idxs = [_ep_case(rng, T, K, E) for _ in range(R)]
    sent = []            # sent[src][dst] = rows in src's dispatch order
    sent_counts = []     # sent_counts[src][dst, j]
    for src in range(R):
        disp = o.dispatch(idxs[src], E)
        rows = o.gather_rows(xs[src], disp.perm, K)
        c, off = o.ep_send_splits(disp.counts, R)
        sent.append([rows[off[r]:off[r + 1]] for r in range(R)])
        sent_counts.append(disp.counts.reshape(R, per))
    for dst in range(R):
        received = np.concatenate([sent[src][dst] for src in range(R)])
        counts = np.stack([sent_counts[src][dst] for src in range(R)])
        lc, rg = o.ep_regroup(counts)
        grouped = received[rg]
        pos = 0
        for j in range(per):
            want = []
            for src in range(R):
                flat = idxs[src].ravel()
                ps = np.nonzero(flat == dst * per + j)[0]      # ascending pair ids
                want.append(xs[src][ps // K])
            want = np.concatenate(want)
            assert lc[j] == len(want)
            assert np.array_equal(grouped[pos:pos + len(want)], want)
            pos += len(want)


def pin_ep_dedup(o):
    """De-duplicated send list: rank r receives exactly the tokens with at
    least one top-K expert on r, once each, ascending (numpy unique); every
    pair's slot holds its own token inside its rank's segment."""
    rng = np.random.default_rng(31)
    for (T, K, E, R) in [(60, 8, 64, 8), (33, 4, 16, 4), (10, 3, 12, 1), (40, 8, 384, 48)]:
        idx = _ep_case(rng, T, K, E)
        per = E // R
        rcnt, roff, send, slot = o.ep_dedup(idx, E, R)
        for r in range(R):
            want = np.unique(np.nonzero((idx // per == r).any(axis=1))[0])
            assert rcnt[r] == len(want)
            assert np.array_equal(send[roff[r]:roff[r + 1]], want)
        tok = np.repeat(np.arange(T), K)
        assert np.array_equal(send[slot], tok)
        rank_of_slot = np.searchsorted(roff, slot, side="right") - 1
        assert np.array_equal(rank_of_slot, idx.ravel() // per)


def pin_scores(o):
    """The scores the oracle ranks (its ``scores`` entry point, the code its
    selection runs): affinities are scipy's expit (or softmax) of the
    logits, choice scores add the bias (nothing without one), and a group
    scores the sum of its two largest choice scores (numpy sort), or its
    largest without a bias."""
    from scipy.special import softmax
    rng = np.random.default_rng(32)
    for (E, G) in [(256, 8), (384, 1), (16, 4), (128, 64)]:
        T = 9
        L = rng.standard_normal((T, E)) * 2.0
        b = rng.uniform(-0.3, 0.3, size=E).astype(np.float32)
        S = E // G
        sc = o.scores(L, b, G)
        assert np.allclose(sc.affinity, expit(L), rtol=1e-14, atol=0)
        assert np.allclose(sc.choice, expit(L) + b.astype(np.float64), rtol=1e-14, atol=1e-16)
        if G > 1:
            top2 = np.sort(sc.choice.reshape(T, G, S), axis=2)[:, :, -2:].sum(axis=2)
            assert np.array_equal(sc.group, top2)
        else:
            assert sc.group.shape == (T, 0)
        sm = o.scores(L, None, G, score_func=1)
        assert np.allclose(sm.affinity, softmax(L, axis=1), rtol=1e-12, atol=0)
        assert np.array_equal(sm.choice, sm.affinity)
        if G > 1:
            assert np.array_equal(sm.group, sm.choice.reshape(T, G, S).max(axis=2))
    # the selection ranks exactly these scores: its winners are the top set
    # of the choice scores inside the best groups
    E, G, KG, K = 64, 8, 3, 6
    L = rng.standard_normal((50, E))
    b = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    r = o.select(L, b, G, KG, K, 2.5, with_scores=True)
    for t in range(50):
        gs = r.scores.group[t]
        kept = sorted(range(G), key=lambda g: (-gs[g], g))[:KG]
        pool = [e for e in range(E) if e // (E // G) in kept]
        assert _is_top_set(set(r.indices[t].tolist()), r.scores.choice[t], pool)


ALL_PINS = [pin_exact_integer_logits, pin_logits_vs_matmul, pin_brute_force_selection,
            pin_zero_input_closed_form, pin_bias_shift_invariance,
            pin_weights_follow_unbiased_sigmoid, pin_winners_in_kept_groups,
            pin_single_group_no_bias_is_topk_of_logits, pin_permutation_equivariance,
            pin_margins, pin_selection_order, pin_dispatch, pin_softmax_scores,
            pin_no_bias_group_max, pin_renorm_off, pin_mask_zero, pin_denominator_epsilon,
            pin_combine, pin_ep_send_splits, pin_ep_regroup, pin_ep_dedup, pin_scores]
