"""Helpers shared by the GPU parity tests (host-side conversions and error metrics)."""
import numpy as np
import torch

from oracle.model import bf16_bits_to_f64


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor (f32 / bf16 / int) -> float64 numpy, exact."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def rel_err(a, b) -> float:
    """||a - b|| / ||b|| over the whole array (b is the oracle)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def row_rel_err(a, b) -> float:
    """max over rows of ||a_i - b_i|| / ||b_i||."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b, axis=-1)
    nb[nb == 0] = 1.0
    return float((np.linalg.norm(a - b, axis=-1) / nb).max())


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f64_to_bf16_tensor(x: np.ndarray, device="cuda") -> torch.Tensor:
    """float64 values that are exactly bf16 (e.g. the oracle's mirrored cache) -> bf16 tensor."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(device)


MARGIN_GATE = 1e-2


def margin_gate(top1, margin):
    """Rows whose top-1/top-2 logit margin exceeds 1e-2 of max(1, |top-1|).

    An absolute 1e-2 is below one bf16 step for |logit| >= 2 (the step there is
    1/64), so the gate is taken relative to the logit's magnitude; for
    |logit| <= 1 it is the absolute 1e-2.
    """
    top1 = np.asarray(top1, dtype=np.float64)
    return np.asarray(margin) > MARGIN_GATE * np.maximum(1.0, np.abs(top1))
