"""Shared helpers of the GPU parity tests: oracle-side inputs and error metrics."""
import os
import sys

import numpy as np
import torch

from oracle import nf4 as onf4

TOL = 2e-2   # max|gpu - oracle| / max|oracle| per output tensor


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a (CPU or GPU) bf16/fp32 tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(gpu, ref: np.ndarray) -> float:
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(g - ref)) / (den if den > 0 else 1.0))


def quantize_dense(w_bf16: torch.Tensor):
    """Oracle quantization of a bf16 CPU tensor -> (codes, absmax) CPU tensors."""
    bits = w_bf16.view(torch.int16).numpy().view(np.uint16)
    packed, absmax = onf4.quantize(bits)
    return torch.from_numpy(packed), torch.from_numpy(absmax)


def dequant_oracle(codes: torch.Tensor, absmax: torch.Tensor) -> np.ndarray:
    return onf4.dequant_f64(codes.numpy(), absmax.numpy())


def say(msg: str) -> None:
    """Progress line that names the case before a GPU step (flushed)."""
    print(msg, file=sys.stderr, flush=True)


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        raise RuntimeError("HIP library not built; run python -m qlora_fine_tuning_amd.build")
