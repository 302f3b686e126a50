"""Shared helpers of the GPU parity tests: upload of the seeded words, the
tolerance gates, and sampled-row selection.

Gates (tolerances: O max-abs 1e-2 for bf16, 2e-3 for fp16 and fp32; LSE
max-abs 1e-3):

* G1 -- a launch that writes O in fp32 (no final 16-bit rounding) must be
  within the tolerance of the float64 oracle, element by element.
* G2 -- the normal launch, O in the input type, must satisfy
  max(|O - O_ref| - half_ulp(O_ref)) <= tolerance: a 16-bit output cannot be
  closer to the exact value than half a unit in its last place, which for
  |O| >= 4 in bf16 (0.0156) already exceeds 1e-2.
* LSE (always fp32) is compared directly.
"""

import numpy as np
import torch

import fa_workloads as W

TOL_O = {"bf16": 1e-2, "f16": 2e-3, "f32": 2e-3}
TOL_LSE = 1e-3
MANT = {"bf16": 7, "f16": 10, "f32": 23}
MIN_EXP = {"bf16": -126, "f16": -14, "f32": -126}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_dev(words, dtype, device="cuda"):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(words))
    return t.to(device)


def out_to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp(x, dtype):
    """Half a unit in the last place of the 16-bit type at |x| (subnormal
    spacing below the normal range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** MIN_EXP[dtype])))
    e = np.maximum(e, MIN_EXP[dtype])
    return 0.5 * 2.0 ** (e - MANT[dtype])


def gate_errors(o_f32, o_dt, lse, o_ref, lse_ref, dtype):
    """Returns dict of the gate quantities (floats)."""
    out = {}
    if o_f32 is not None:
        out["g1"] = float(np.max(np.abs(o_f32 - o_ref))) if o_ref.size else 0.0
    if o_dt is not None:
        err = np.abs(o_dt - o_ref)
        out["literal"] = float(err.max()) if err.size else 0.0
        out["g2"] = float(np.max(err - half_ulp(o_ref, dtype))) if err.size else 0.0
    out["lse"] = float(np.max(np.abs(lse - lse_ref))) if lse_ref.size else 0.0
    return out


def assert_gates(errs, dtype, what=""):
    tol = TOL_O[dtype]
    msg = f"{what} {dtype} errors {errs}"
    if "g1" in errs:
        assert errs["g1"] <= tol, msg
    if "g2" in errs:
        assert errs["g2"] <= tol, msg
    assert errs["lse"] <= TOL_LSE, msg


def sample_rows(N, tile, rng, n_random=24, cap=None):
    """Rows 0, 1, N-1, N-2, both sides of every multiple of `tile` (of `cap`
    randomly chosen ones when a cap is given), and random rows."""
    rows = {0, 1, N - 1, N - 2}
    bounds = list(range(tile, N, tile))
    if cap is not None and len(bounds) > cap:
        bounds = list(rng.choice(bounds, cap, replace=False))
    for b in bounds:
        rows.update({b - 1, b})
    rows.update(rng.choice(N, min(N, n_random), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


def head_values(words, dtype, b, h):
    return W.decode64(words[b, h], dtype)
