"""Power of the full-size regression guard (CPU only).

The GPU tests hold every full-size f16 / bf16 workload to a normalised error
of at most FULL_SIZE_GUARD besides the mandated 1e-3 bar.  These tests show,
on the very seeded inputs and sampled entries those tests use, that the
guard rejects the mistakes the bar lets through at full size:

  * one K-step (64 products) missing from every entry of 8192^3 (the first
    or the last step);
  * a 256 x 256 output tile of the bf16 4096^3 accumulate workload left
    unwritten, so that it keeps its initial value C_in.

The size of each mistake is computed with the oracle from the stored inputs
(the difference such a result would show against the oracle), so nothing here
depends on the GPU path."""
import numpy as np
import pytest

import synthetic as S
from gpu_util import FULL_SIZE_GUARD, TOL, value_range

pytestmark = pytest.mark.slow


def _denominator(p, g):
    d = p.K * value_range(g["A"], p.dtype) * value_range(g["B"], p.dtype)
    if g["bias"] is not None:
        d += float(np.max(np.abs(g["bias"])))
    if p.accum:
        d += value_range(g["C_in"], S.C_TYPE_CODE.get(p.c_type, S.F32))
    return d


@pytest.mark.parametrize("name", ["f16_8192", "bf16_8192"])
@pytest.mark.parametrize("step", ["first", "last"])
def test_guard_rejects_a_dropped_k_step_at_8192(oracle_lib, name, step):
    p = S.workload(name)
    assert p.b_col and not p.a_col
    g = S.generate(p)
    ii, jj = S.sample_entries(p)
    k0 = 0 if step == "first" else p.K - 64
    # the 64 products of one K-step at each sampled entry: the same product
    # restricted to columns k0 .. k0+63 of A and of (column-major) B
    A = np.ascontiguousarray(g["A"][:, k0:k0 + 64])
    B = np.ascontiguousarray(g["B"][:, k0:k0 + 64])
    part = oracle_lib.gemm_entries(p.M, p.N, 64, A, 64, False, B, 64, True, p.dtype, ii, jj)
    err = float(np.max(np.abs(part))) / _denominator(p, g)
    print(f"{name}: a dropped {step} K-step gives normalised error {err:.3e}; bar {TOL[p.dtype]:.0e}, "
          f"guard {FULL_SIZE_GUARD:.0e}")
    assert err > 20 * FULL_SIZE_GUARD
    assert err < TOL[p.dtype]  # the reason for the guard: the bar alone would pass it


def test_guard_rejects_an_unwritten_tile_of_the_accumulate_workload(oracle_lib):
    p = S.workload("bf16_4096_accum")
    g = S.generate(p)
    ii, jj = S.sample_entries(p)
    ref = oracle_lib.gemm_entries(p.M, p.N, p.K, g["A"], p.LDA, p.a_col, g["B"], p.LDB, p.b_col, p.dtype, ii, jj,
                                  bias=g["bias"], relu=p.relu, c_in=g["C_in"].reshape(-1),
                                  c_in_type=S.C_TYPE_CODE[p.c_type], ldcin=p.LDC)
    import torch
    cin = torch.from_numpy(g["C_in"].reshape(p.M, p.LDC).view(np.int16).copy()).view(torch.bfloat16)
    kept = cin.to(torch.float64).numpy()[ii, jj]
    u = 2.0 ** -8  # the bf16 output rounding the check allows
    excess = np.abs(kept - ref) - u * np.abs(ref)
    denom = _denominator(p, g)
    # every 256 x 256 tile of the planned data-parallel kernel, by its sampled entries
    tile = (ii // 256) * (p.N // 256) + jj // 256
    worst = np.full(tile.max() + 1, -np.inf)
    np.maximum.at(worst, tile, excess / denom)
    assert np.all(np.isfinite(worst)), "some tile holds no sampled entry"
    print(f"bf16_4096_accum: an unwritten tile gives normalised error >= {worst.min():.3e}; guard {FULL_SIZE_GUARD:.0e}")
    assert worst.min() > 20 * FULL_SIZE_GUARD
