"""Helpers shared by the GPU parity tests: host <-> device copies of raw
bf16 / fp32 / int64 buffers, and the error measures the parity bar uses."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from megatron_tensor_layer_tp_amd import inputs as I  # noqa: E402

DEV = "cuda:0"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a: np.ndarray):
    """Copy a host array to the GPU bit for bit (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def empty_like_dt(shape, dt_bf16: bool):
    return torch.empty(shape, dtype=torch.int16 if dt_bf16 else torch.float32, device=DEV)


def fill_garbage(t):
    """Outputs start as NaN-ish garbage so that a skipped store shows."""
    if t.dtype == torch.int16:
        t.fill_(0x7fc1)  # a bf16 NaN pattern
    else:
        t.fill_(float("nan"))
    return t


def host(t) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def host_f64(t) -> np.ndarray:
    a = host(t)
    if a.dtype == np.uint16:
        return I.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def rel_fro(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def workspace(nbytes: int):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=DEV), nbytes


# Element-wise bound for bf16 outputs, next to the relative Frobenius bar:
#   |got - want| <= 2^-7 |want| + 2^-5 rms(want)   (rms over the compared entries)
# The first term covers the output's own round-to-nearest-even (at most 2^-8
# relative) with a factor 2 to spare; the second covers the bf16 roundings of
# the intermediates a product consumes (Z, H, A, dZ, dG, P): each is at most
# 2^-8 relative, so the error they carry into an output has a standard
# deviation near 0.6 * 2^-8 rms per rounded operand -- the bound sits at more
# than 6 of those standard deviations for two chained roundings.  A wrong or
# skipped element is off by the order of rms(want) and fails it.
BF16_REL = 2.0 ** -7
BF16_RMS = 2.0 ** -5


def elem_bound(got: np.ndarray, want: np.ndarray, name: str, rel: float = BF16_REL, rms_frac: float = BF16_RMS,
               atol: float = 0.0):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if want.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU result"
    rms = float(np.sqrt(np.mean(want * want)))
    err = np.abs(got - want)
    lim = rel * np.abs(want) + rms_frac * rms + atol
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{name}: {bad.shape[0]} of {want.size} entries outside |err| <= {rel:.3g}|want| + "
                           f"{rms_frac:.3g} rms; first at {tuple(bad[0])}: got {got[tuple(bad[0])]!r}, "
                           f"want {want[tuple(bad[0])]!r}, rms {rms:.3g}")


def check_bf16(got: np.ndarray, want: np.ndarray, name: str, tol: float = 5e-3, rel: float = BF16_REL,
               rms_frac: float = BF16_RMS, atol: float = 0.0) -> float:
    """The parity bar for a bf16 output (or a sample of one): relative
    Frobenius error <= tol over the whole tensor and the element-wise bound
    (``atol``: an absolute floor for outputs that are exactly zero)."""
    err = rel_fro(got, want)
    assert err <= tol, f"{name}: relative Frobenius error {err:.3e} > {tol}"
    elem_bound(got, want, name, rel, rms_frac, atol)
    return err
