"""Shared helpers of the GPU parity tests (host-side data movement only)."""
import numpy as np
import torch

TOL = {"f32": 2e-3, "bf16": 2e-2}       # abs and rel, per the stated parity bar


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def assert_close(got, want, dtype, what):
    tol = TOL[dtype]
    err = np.abs(got - want)
    bad = err > tol + tol * np.abs(want)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside {tol} "
                           f"(max abs err {err.max():.3g})")
    return float(err.max()) if err.size else 0.0
