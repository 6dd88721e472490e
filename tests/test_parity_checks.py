"""The near-tie-aware comparison helpers of the GPU parity tests, checked on the CPU:
the oracle's own results pass as decided, and a result with a planted mistake at a
decided position fails."""
import numpy as np
import pytest

from oracle import select as osel
from oracle import tree as otree
from oracle import verify as over
from parity_checks import (Tally, accept_bounds, cdf_margin, check_draw, check_rejection, check_tree, check_walk,
                           draw_bound)


def _tree_outputs(z, B, anchor):
    L, V = z.shape
    q = osel.softmax(z, 1.0)
    ids = np.stack([osel.topk(z[j], min(B, V)) for j in range(L)])
    tok, par, dep, _ = otree.build_tree(np.take_along_axis(q, ids, axis=1), ids, B)
    tok = tok.copy()
    tok[0] = anchor
    return tok, par, dep


def test_tree_check_accepts_oracle_and_rejects_swaps():
    z = np.random.default_rng(1).standard_normal((6, 300)) * 2.5
    tok, par, dep = _tree_outputs(z, 40, anchor=7)
    bits = otree.mask_bits(otree.ancestor_mask(par))
    tn, ts = Tally("nodes"), Tally("sets")
    assert check_tree(tn, ts, tok, par, dep, bits, z, 40, 7)
    assert tn.ties == 0 and ts.ties == 0
    # planted mistake: swap the tokens of two first-level siblings (a decided order)
    kids = [i for i in range(1, len(par)) if par[i] == 0]
    bad = tok.copy()
    bad[kids[0]], bad[kids[1]] = bad[kids[1]], bad[kids[0]]
    with pytest.raises(AssertionError):
        check_tree(Tally("n"), Tally("s"), bad, par, dep, bits, z, 40, 7)
    # planted mistake: a wrong mask bit
    bits2 = bits.copy()
    bits2[3, 0] ^= np.uint64(1 << 2)
    with pytest.raises(AssertionError):
        check_tree(Tally("n"), Tally("s"), tok, par, dep, bits2, z, 40, 7)


def test_tree_check_tolerates_a_swap_inside_a_near_tie():
    z = np.random.default_rng(2).standard_normal((3, 50)) * 2.0
    z[0, 5] = z[0, 9] = z[0].max() + 0.5                    # exact tie at the top of position 1
    tok, par, dep = _tree_outputs(z, 12, anchor=0)
    assert tok[1] == 5 and tok[2] == 9
    bad = tok.copy()
    bad[1], bad[2] = 9, 5                                    # the other order of the tie
    # children of node 1 / node 2 follow their parents: swap the parents of their subtrees too
    par2 = par.copy()
    for i in range(3, len(par)):
        if par[i] in (1, 2):
            par2[i] = 3 - par[i]
    bits = otree.mask_bits(otree.ancestor_mask(par2))
    tn = Tally("nodes")
    check_tree(tn, Tally("sets"), bad, par2, dep, bits, z, 12, 0)
    assert tn.ties >= 2


def test_draw_check():
    w = np.array([0.1, 0.2, 0.3, 0.4])
    t = Tally("draws")
    check_draw(t, 2, w, 0.45, 1e-6)                          # cum 0.1 0.3 0.6 1.0 -> id 2
    with pytest.raises(AssertionError):
        check_draw(t, 1, w, 0.45, 1e-6)
    check_draw(t, 1, w, 0.3 - 1e-9, 1e-6)                   # near-tie at the 0.3 boundary: 1 or 2 valid
    check_draw(t, 2, w, 0.3 - 1e-9, 1e-6)
    with pytest.raises(AssertionError):
        check_draw(t, 3, w, 0.3 - 1e-9, 1e-6)
    assert t.decided == 2 and t.ties == 3        # the failing calls were counted too


def test_rejection_and_walk_checks_accept_the_oracle():
    rng = np.random.default_rng(3)
    K, V, T = 5, 200, 1.0
    z = rng.standard_normal((K, V)) * 2.0
    t = np.concatenate([z, np.zeros((1, V))], axis=0) + rng.standard_normal((K + 1, V))
    tal = Tally("rejection")
    for step in range(20):
        d = osel.select_block(z, T, 0, 5, 1, step)["draft_ids"]
        ref = over.verify_rejection(d, z, t, T, 5, 1, step)
        check_rejection(tal, ref["out_tokens"], ref["out_len"], d, ref, accept_bounds(d, z, t, T),
                        draw_bound(ref, z, t, T))
        # planted mistake at a decided draw: another token
        if all(m > b for (m, _), b in zip(ref["tests"], accept_bounds(d, z, t, T))) and \
                ref["draw_margin"] > draw_bound(ref, z, t, T):
            bad = ref["out_tokens"].copy()
            bad[-1] = (bad[-1] + 1) % V
            with pytest.raises(AssertionError):
                check_rejection(Tally("x"), bad, ref["out_len"], d, ref, accept_bounds(d, z, t, T),
                                draw_bound(ref, z, t, T))
    tal.assert_floor(0.9)
    # walk on a chain tree
    tok = np.array([0, 3, 4, 5])
    par = np.array([-1, 0, 1, 2])
    tr = rng.standard_normal((4, V)) * 3.0
    tr[0, 3] += 9.0
    tr[1, 4] += 9.0
    tw = Tally("walk")
    for step in range(10):
        ref = over.verify_tree_walk(tok, par, tr, 1.0, seed=2, slot=0, step=step)
        check_walk(tw, ref["out_tokens"], ref["out_len"], ref["path"], tok, par, ref, tr, 1.0)
    assert tw.total == 10
    assert cdf_margin(tr[2], 1.0) < 1e-5
