"""Helpers for the GPU parity tests: device buffers from seeded host arrays."""
import ctypes as C
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from layer_streamed_qlora_nf4_amd import lib


def dev_bits(bits, device="cuda"):
    """uint16 bf16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def dev(x, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host_bits(t):
    return t.cpu().numpy().view(np.uint16)


def bits_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def stream():
    return lib.stream_handle(torch.cuda.current_stream())


def empty_bytes(n, device="cuda"):
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def rel_err(got, ref):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def print_case(**kw):
    print("CASE " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def row_blocks(fn, *arrays, threads=16):
    """fn applied to row blocks of the arrays on a thread pool, results stacked
    by rows.  Quantizing and dequantizing are row-local (a 64-block never
    crosses a row), so this is the same result as one call on the whole
    arrays; it only spreads the oracle's work over the host's cores."""
    n = arrays[0].shape[0]
    step = max(1, -(-n // (4 * threads)))
    starts = list(range(0, n, step))
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r0: fn(*(a[r0:r0 + step] for a in arrays)), starts))
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))
    return np.concatenate(parts)
