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
