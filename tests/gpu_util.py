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


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits): 2^(e - 8) for |x| in [2^(e-1), 2^e)."""
    _, e = np.frexp(np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def id_gate_threshold(top1, dtype):
    """Smallest top-1/top-2 margin (or confidence gap at the selection cut, in log space)
    above which decoded ids / positions must agree.

    fp32 models: the absolute 1e-2. bf16 models store their logits in bf16, so two
    implementations that agree to within one bf16 step on every stored logit can still
    close a margin of two steps (top-1 down one step, top-2 up one); the gate is then
    max(1e-2, 2 bf16 ulps of |top-1|), which is the absolute 1e-2 for |top-1| < 1 and two
    steps of the format above it.
    """
    if dtype != "bf16":
        return np.full(np.shape(top1), MARGIN_GATE)
    return np.maximum(MARGIN_GATE, 2.0 * bf16_ulp(top1))


def margin_gate(top1, margin, dtype="bf16"):
    """Rows whose top-1/top-2 logit margin clears id_gate_threshold."""
    return np.asarray(margin, dtype=np.float64) > id_gate_threshold(top1, dtype)


def cut_gate_threshold(c_a, top_a, c_b, top_b, dtype):
    """Smallest confidence gap (|ln c_a - ln c_b|) at the selection cut above which the
    unmask order must agree.

    ln c = x_top - logsumexp(x), so a change of every stored logit by at most delta moves
    ln c by at most (1 - c)(|delta_top| + max |delta_other|) <= 2 (1 - c) delta. For bf16
    models delta is one bf16 step of the row's top-1 logit (the stored values of two
    implementations within one step of each other), so the two rows at the cut can close a
    gap of 2 (1 - c_a) ulp(top_a) + 2 (1 - c_b) ulp(top_b); fp32 models use 1e-2.
    """
    if dtype != "bf16":
        return MARGIN_GATE
    return max(1e-6, 2.0 * (1.0 - float(c_a)) * float(bf16_ulp(top_a))
               + 2.0 * (1.0 - float(c_b)) * float(bf16_ulp(top_b)))
