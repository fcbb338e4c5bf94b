"""Checks of a step's decisions against the oracle run on the logits the GPU
stored (host-side helpers of the GPU step tests).

Both sides then read identical inputs, so the only differences left are the
GPU's float32 arithmetic against the oracle's float64:
* per-row entropy H within 1e-4 + 1e-5 |H| (float32 sums over V <= 152064);
* argmax exact (lowest id among equal maxima on both sides);
* top-1 probability within its float32 error bound, 1e-5 relative plus
  2^-23 |m| log2(e), m the row's largest logit: the GPU takes exponents as
  fma(x, log2 e, -m log2 e), whose rounded constant m log2 e shifts every
  exponent of a segment by up to half an ulp of m log2 e.  The shift cancels
  in H but scales p1 = 1/z (at logits of a few hundred, 2^-23 |m| log2 e is
  5e-5);
* the unmask set exact, except where the candidates swapped between the two
  sets have top-1 probabilities within the sum of their float32 error bounds
  (1e-6 relative plus the shift term above): the GPU ranks its float32
  values, which cannot order such candidates, and equal values go to the
  lower position (the tie zone of the stated reading: a decision whose margin
  is below the GPU's error bound is reported, not counted as a mismatch);
* E within 1e-4 + 1e-5 |E|, and the flag exact unless |E - tau| <= 1e-4 nats.
EntropyCache, Chinese summary page §2.2 (E_{t+1} and the threshold rule).
"""
import math
import sys

import numpy as np

import oracle as O

FLAG_TIE_NATS = 1e-4
LOG2E = 1.4426950408889634


def p1_shift_rel(z):
    """Per row: 2^-23 |m| log2(e), the relative change of p1 that the float32
    rounding of m log2(e) can cause (m = the row's largest finite logit)."""
    z = np.asarray(z, dtype=np.float64)
    m = np.where(np.isfinite(z), np.abs(z), 0.0).max(axis=1)
    return 2.0 ** -23 * m * LOG2E


def h_close(got, want):
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    both_nan = np.isnan(got) & np.isnan(want)
    ok = both_nan | (np.abs(got - want) <= 1e-4 + 1e-5 * np.abs(want))
    return bool(ok.all())


def decisions_on_stored_logits(g, cand, n_unmask, tau, where):
    """Check a step's H / argmax / p1 / chosen / E / flag against the oracle
    applied to the GPU's stored logits g["logits"] ([len(cand), V]).

    Returns the number of unmask-set differences accepted as float32 p1 ties.
    """
    cand = np.asarray(cand)
    m = len(cand)
    z = np.asarray(g["logits"][:m], dtype=np.float64)
    H, A, P = O.row_stats(z)
    assert h_close(g["H"][:m], H), (where, "H", np.abs(g["H"][:m] - H).max())
    np.testing.assert_array_equal(g["argmax"][:m], A, err_msg=f"{where} argmax")
    shift = p1_shift_rel(z)
    rel = np.abs(g["p1"][:m] - P) / P
    assert np.all(rel <= 1e-5 + shift), (where, "p1", float(rel.max()), float(shift.max()))
    chosen = np.asarray(g["chosen"])
    want = O.choose(cand, P, n_unmask)
    ties = 0
    if not np.array_equal(chosen, want):
        assert len(chosen) == len(want), (where, chosen, want)
        swapped = np.searchsorted(cand, sorted(set(chosen.tolist()) ^ set(want.tolist())))
        pv = P[swapped]
        bound = ((1e-6 + shift[swapped]) * pv).sum()
        assert pv.max() - pv.min() <= bound, (where, "unmask set", cand[swapped], pv)
        ties = 1
        print(f"{where}: float32 p1 tie, unmask set {chosen} vs {want}", file=sys.stderr)
    # E over the set the GPU chose (a tie above changes which rows count)
    pick = np.searchsorted(cand, chosen)
    E = O.max_entropy(H, pick)
    gE = g["E"]
    if math.isinf(E) or math.isnan(E):
        assert gE == E or (math.isnan(E) and math.isnan(gE)), (where, gE, E)
    else:
        assert abs(gE - E) <= 1e-4 + 1e-5 * abs(E), (where, "E", gE, E)
    want_flag = O.decide(E, tau)
    if g["flag"] != want_flag:
        assert abs(E - tau) <= FLAG_TIE_NATS, (where, "flag", g["flag"], E, tau)
        ties += 1
        print(f"{where}: flag tie, E = {E} tau = {tau}", file=sys.stderr)
    return ties
