"""Shared test helpers: tolerances and host copies.  No method arithmetic here."""
import numpy as np

# bf16 outputs: |g - o| <= 1e-2 + 2e-2 |o| elementwise, and ||g - o|| / ||o|| <= 1e-2.
BF16_ATOL, BF16_RTOL, BF16_NRM = 1e-2, 2e-2, 1e-2
# float32 outputs: 1e-5 absolute + 1e-5 relative.
F32_ATOL, F32_RTOL = 1e-5, 1e-5


def host64(t) -> np.ndarray:
    """Exact float64 image of a (GPU or CPU) torch tensor."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, want, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    if dtype == "bf16":
        bound = BF16_ATOL + BF16_RTOL * np.abs(want)
        nrm = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (f"{what}: max excess {np.max(err - bound):.3e} at {worst} "
                                      f"(got {got[worst]:.6f} want {want[worst]:.6f})")
        assert nrm <= BF16_NRM, f"{what}: normalised error {nrm:.3e} > {BF16_NRM}"
    else:
        bound = F32_ATOL + F32_RTOL * np.abs(want)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (f"{what}: max excess {np.max(err - bound):.3e} at {worst} "
                                      f"(got {got[worst]:.8f} want {want[worst]:.8f})")


def assert_bf16_rounding(got, want, what: str = ""):
    """got is want rounded once to bf16 (half an ulp: 2^-9 relative, plus slack)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 1e-5
    assert np.all(err <= bound), f"{what}: max excess {np.max(err - bound):.3e}"
