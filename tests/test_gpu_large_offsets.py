"""A batch whose tensors reach past 2^32 bytes, so every offset the kernels
form must be 64-bit.  Needs an MI355X and about 50 GB of its memory.

T = 320000 tokens at d = 7168:
  * x is 4.59 GB, and its rows from 299594 on start past 2^31 elements;
  * the permuted rows are 36.7 GB, with most of them past 2^32 bytes;
  * the combined output is 4.59 GB.

x repeats a seeded block of R rows (row t is block row t mod R), so only the
block is drawn on the host.  A 32-bit wrap of an element or byte offset
shifts it by 2^31 or 2^32 units.  That is not a whole number of 7168-element
rows, so a wrapped access would read parts of two rows and change the logits
or the copied bytes, which the comparisons below catch.

Checks:
  * the gate on both logits routes, sampled rows against the oracle (rows
    past the boundary among them), and the row properties on every token;
  * every repeat of a block row gets bit-equal weights and indices;
  * the dispatch in full: counts, offsets, perm and dest;
  * the permuted rows and the combined output at sampled positions past
    2^32 bytes, against the oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import workloads as wl
from parity import check_rows_valid, combine_tolerance, compare_dispatch, compare_gate, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

T_BIG = 320_000
D = 7168
R = 4093


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_offsets_past_32_bits(o):
    gc = wl.DSV3
    T, d, K, E = T_BIG, D, gc.top_k, gc.n_experts
    first_far = -(-(2 ** 31) // d)          # first row starting at element >= 2^31
    assert T * d * 2 > 2 ** 32 and first_far < T
    say(f"[large] T={T} d={d} E={E}: x {T * d * 2 / 1e9:.2f} GB, "
        f"permuted rows {T * K * d * 2 / 1e9:.1f} GB")
    gi = wl.make_gate_inputs(R, d, gc, seed=77)
    block = torch.from_numpy(gi.x.view(np.int16)).cuda()
    x = block.repeat(-(-T // R), 1)[:T].view(torch.bfloat16)
    del block
    W = torch.from_numpy(gi.W).cuda()
    b = torch.from_numpy(gi.bias).cuda()
    rng = np.random.default_rng(13)
    rows = np.unique(np.r_[0, first_far - 1, first_far, T - 1,
                           rng.integers(first_far, T, 384), rng.integers(0, T, 128)])
    ref = o.gate(gi.x[rows % R], gi.W, gi.bias, gc.n_group, gc.topk_group, K, gc.route_scale,
                 with_scores=True)

    base = sg.Cfg(T, d, E, gc.n_group, gc.topk_group, K, gc.route_scale)
    wg = ig = None
    for lp in (0, 1):
        cfg = dataclasses.replace(base, logits_path=lp)
        w, i = sg.siggate_forward(x, W, b, cfg)
        torch.cuda.synchronize()
        w_np, i_np = w.cpu().numpy(), i.cpu().numpy()
        check_rows_valid(i_np, E, gc.n_group, gc.topk_group)
        # equal rows of x give bit-equal results wherever they sit in the
        # batch (every row's sums run in the same order)
        same_row = np.arange(T) % R
        assert np.array_equal(i_np, i_np[same_row]) and np.array_equal(w_np, w_np[same_row]), \
            "repeated rows of x were routed differently"
        stats = compare_gate(w_np, i_np, ref, gc.route_scale, rows, topk_group=gc.topk_group)
        say(f"    gate logits_path={lp}: {stats}")
        if lp == 0:
            wg, ig, idx = w, i, i_np
        del w, i

    out = sg.siggate_dispatch(x, ig, base)
    torch.cuda.synchronize()
    dref = o.dispatch(idx, E)
    # counts, offsets, perm and dest in full; rows separately (x repeats)
    compare_dispatch(out, dref, idx, gi.x, K, np.zeros(0, np.int64), o)
    n = T * K
    first_far_pos = -(-(2 ** 32) // (2 * d))
    pos = np.unique(np.r_[first_far_pos, n - 1, rng.integers(first_far_pos, n, 2048),
                          rng.integers(0, n, 256)])
    got = out.permuted_x[torch.from_numpy(pos).cuda()].view(torch.int16).cpu().numpy()
    # a pair p = t*K + k of token t reads block row t mod R
    p_block = (dref.perm // K) % R * K + dref.perm % K
    want = o.gather_rows(gi.x, p_block, K, pos)
    assert np.array_equal(got.view(np.uint16), want), "permuted rows past 2^32 bytes differ"
    say(f"    dispatch ok: {len(pos)} sampled rows, {int((pos >= first_far_pos).sum())} past 2^32 bytes")

    y = sg.siggate_combine(out.permuted_x, wg, out.dest, base)
    torch.cuda.synchronize()
    tok = np.unique(np.r_[T - 1, first_far, rng.integers(first_far, T, 96), rng.integers(0, T, 32)])
    dest = out.dest.cpu().numpy().reshape(T, K)[tok]
    sub_out = out.permuted_x[torch.from_numpy(dest.ravel().astype(np.int64)).cuda()]
    sub_out = sub_out.view(torch.int16).cpu().numpy().view(np.uint16)
    local = np.arange(len(tok) * K, dtype=np.int32)
    w64 = wg.cpu().numpy()[tok].astype(np.float64)
    y64, want16 = o.combine(sub_out, w64, local)
    got16 = y[torch.from_numpy(tok).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    gotf = wl.bf16_to_f32(got16).astype(np.float64)
    # Every row combined here is route_scale * x[t] up to rounding, and for
    # bfloat16 x that product often lies exactly halfway between two
    # bfloat16 values: the final rounding then goes either way with the
    # float32 weight sum, so only the error bound is checked, not bit
    # equality with the oracle's rounding.
    assert np.all(np.abs(gotf - y64) <= combine_tolerance(o, sub_out, w64, local, y64, K))
    say(f"    combine ok: {len(tok)} sampled tokens, "
        f"{float((got16 != want16).mean()):.3f} of elements rounded the other way")
    del x, out, y, wg, ig
