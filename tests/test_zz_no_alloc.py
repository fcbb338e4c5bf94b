"""ec_entropy_max_noalloc (partial statistics in a static device array, no
workspace) against ec_entropy_max (caller workspace) through the C ABI.

Both run the same kernels on the same logits, so every output must be
identical bit for bit: per-row H, argmax and p1, E and the flag.  Three calls
in a row on one stream, each smaller than the one before, so a later call
runs on an array that still holds the earlier call's larger contents: the
4096 x 126464 bf16 workload (every row decoded), 300 x 126464 bf16 with a
decoded subset, and 7 x 1000 fp32 with a decoded subset.  A call whose
partial statistics would not fit in the array is refused on the host.
EntropyCache, Chinese summary page §2.2 (the entropy pass and threshold rule).
"""
import numpy as np
import pytest
import torch

from entropy_gated_kv_amd import lib as L
from synth import configs as C
from synth import generators as G

pytestmark = pytest.mark.gpu


def outputs(n):
    return (torch.full((n,), float("nan"), device="cuda"),
            torch.full((n,), -1, dtype=torch.int32, device="cuda"),
            torch.full((n,), float("nan"), device="cuda"),
            torch.full((1,), float("nan"), device="cuda"),
            torch.full((1,), -1, dtype=torch.int32, device="cuda"))


def both(x, tau, decoded):
    n = x.shape[0]
    D = None if decoded is None else torch.tensor(decoded, dtype=torch.int32, device="cuda")
    nD = None if decoded is None else torch.tensor([len(decoded)], dtype=torch.int32, device="cuda")
    maxD = 0 if decoded is None else len(decoded)
    a = outputs(n)
    ws = torch.empty(L.ec_entropy_workspace_bytes(n, x.shape[1]), dtype=torch.uint8, device="cuda")
    L.ec_entropy_max(x, tau, a[0], a[3], a[4], ws, decoded_rows=D, n_decoded=nD,
                     max_decoded=maxD, row_argmax=a[1], row_top1=a[2])
    b = outputs(n)
    L.ec_entropy_max_noalloc(x, tau, b[0], b[3], b[4], decoded_rows=D, n_decoded=nD,
                             max_decoded=maxD, row_argmax=b[1], row_top1=b[2])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in b]


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls():
    cfg = C.ENTROPY_ONLY
    big = torch.from_numpy(G.entropy_logits(cfg)).to(torch.bfloat16).cuda()
    cases = [
        (big, cfg.tau, None),
        (big[:300].contiguous(), 2.0, [0, 5, 17, 299]),
        (torch.from_numpy(G.random_logits(3, 7, 1000, "f32")).cuda(), 6.0, [1, 6]),
    ]
    for i, (x, tau, decoded) in enumerate(cases):
        a, b = both(x, tau, decoded)
        for what, u, v in zip(("H", "argmax", "p1", "E", "flag"), a, b):
            assert np.array_equal(u.view(np.uint32) if u.dtype != np.int32 else u,
                                  v.view(np.uint32) if v.dtype != np.int32 else v), (i, what)
        assert np.isfinite(a[0]).all() and a[4][0] in (0, 1), i


def test_noalloc_refuses_a_call_beyond_the_array():
    x = torch.zeros((1, 16), dtype=torch.bfloat16, device="cuda")
    H, A, P, E, F = outputs(1)
    rows = L.EC_NOALLOC_SCRATCH_BYTES // 16 + 1        # one segment per row, one row too many
    st = L.load().ec_entropy_max_noalloc(x.data_ptr(), L.EC_BF16, rows, 16, 16, None, None, 0,
                                         1.0, H.data_ptr(), None, None, E.data_ptr(),
                                         F.data_ptr(), None)
    assert st == -4
