"""libec.so used from plain C++ (tests/c_abi_driver.cpp: include/ec.h and the HIP
runtime, no Python binding): the entropy pass with its decision and the row
selection, on inputs this test writes, checked against the oracle.

Tolerances are those of the binding-level tests: H within 1e-4 + 1e-5 H
(float32 sums over V terms), p1 within 1e-5 relative, argmax and rows exact,
the flag exact unless the oracle's E lies within the H tolerance of tau.  The
driver also reports the status of two calls the host checks refuse (a NULL
logits pointer, a workspace one byte short).
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from synth import generators as G

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")
H_ATOL, H_RTOL = 1e-4, 1e-5


def stored_bytes(z: np.ndarray, dtype: str) -> bytes:
    t = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().tobytes()
    return t.numpy().tobytes()


def run_driver(tmp_path, z, dtype, decoded, tau, L, bs, bl, bc, cap, hist, k, flag, masked):
    n, V = z.shape
    ring = np.zeros(cap, dtype=np.int32)
    for i, p in enumerate(hist):                       # entry i at i % cap: the last cap survive
        ring[i % cap] = p
    blob = (np.array([0x45430001, n, V, 1 if dtype == "bf16" else 0, len(decoded)], np.int32).tobytes()
            + np.array([tau], np.float32).tobytes() + stored_bytes(z, dtype)
            + np.asarray(decoded, np.int32).tobytes()
            + np.array([L, bs, bl, bc, cap, len(hist), k, flag], np.int32).tobytes()
            + np.asarray(masked, np.uint8).tobytes() + ring.tobytes())
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(blob)
    print(f"c_abi_driver: n={n} V={V} {dtype} L={L} k={k}", flush=True)
    r = subprocess.run([DRIVER, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    b = fout.read_bytes()
    off = 0

    def take(dt, cnt):
        nonlocal off
        a = np.frombuffer(b, dtype=dt, count=cnt, offset=off)
        off += a.nbytes
        return a

    st = take(np.int32, 4)
    H, A, P = take(np.float32, n), take(np.int32, n), take(np.float32, n)
    E, F = float(take(np.float32, 1)[0]), int(take(np.int32, 1)[0])
    ns = int(take(np.int32, 1)[0])
    rows = take(np.int32, ns)
    assert off == len(b)
    return st, H, A, P, E, F, rows


@pytest.fixture(scope="module", autouse=True)
def driver_built():
    if not os.path.exists(DRIVER):
        pytest.fail("tests/c_abi_driver is not built; run __graft_entry__.build() first")


@pytest.mark.parametrize("case", ["bf16_partial", "fp32_full", "bf16_none_decoded"])
def test_driver_results_match_the_oracle(tmp_path, case):
    rng = np.random.default_rng({"bf16_partial": 1, "fp32_full": 2, "bf16_none_decoded": 3}[case])
    dtype = "fp32" if case == "fp32_full" else "bf16"
    n, V = (37, 50001) if dtype == "bf16" else (5, 1000)       # odd V: rows padded to 16 bytes
    z = G.random_logits(40 + len(case), n, V, "bf16" if dtype == "bf16" else "f32")
    decoded = [] if case == "bf16_none_decoded" else sorted(rng.choice(n, size=min(9, n), replace=False))
    Ho, Ao, Po = O.row_stats(np.asarray(z, np.float64))
    tau = float(np.median(Ho)) if decoded else 1.0
    # selection state: a block with masked positions and a history ring that wrapped
    L, bs, bl, cap, k = 300, 128, 32, 24, 16
    masked = np.zeros(L, bool)
    masked[bs + rng.choice(bl, size=11, replace=False)] = True
    masked[bs + bl:] = True
    hist = list(rng.permutation(np.flatnonzero(~masked[:bs + bl]))[:40])
    flag = 1 if case == "fp32_full" else 0
    st, H, A, P, E, F, rows = run_driver(tmp_path, z, dtype, decoded, tau, L, bs, bl, 0, cap, hist, k,
                                         flag, masked)
    assert list(st) == [0, 0, -1, -4], st                      # ok, ok, EC_E_NULL, EC_E_WORKSPACE
    err = np.abs(H - Ho)
    assert np.all(err <= H_ATOL + H_RTOL * np.abs(Ho)), err.max()
    np.testing.assert_array_equal(A, Ao)
    np.testing.assert_allclose(P, Po, rtol=1e-5, atol=0)
    Eo = O.max_entropy(Ho, decoded)
    if decoded:
        assert E == max(H[d] for d in decoded)                 # the maximum of the GPU's own H
        assert abs(E - Eo) <= H_ATOL + H_RTOL * abs(Eo)
        if abs(Eo - tau) > H_ATOL + H_RTOL * abs(Eo):
            assert F == O.decide(Eo, tau)
    else:
        assert E == -np.inf and F == 0
    want = O.select_rows(flag, masked, bs, bl, hist, k)
    np.testing.assert_array_equal(rows, want)
