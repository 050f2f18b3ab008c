"""Seeded synthetic inputs shared by the HIP path and the oracle.

This module draws numbers and nothing else: it holds none of the method's
arithmetic (no quantisation, no layer maths).  Every tensor comes from its own
NumPy PCG64 stream keyed by (base seed, workload id, layer, tensor id, chunk),
so any tensor can be regenerated alone, in any order, on any host.  Weights
are drawn in float32 and rounded once to bfloat16 (round to nearest even);
they are returned as uint16 bit patterns.

Distributions (the pages run real checkpoints on real text; these stand in):
projection weights, q/k/v biases, embedding and head ~ N(0, 0.02); RMSNorm
weights ~ N(1, 0.1); LoRA A and B ~ N(0, 0.01); activations and upstream
gradients ~ N(0, 1); token ids uniform over the vocabulary.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 0
_CHUNK_ROWS_ELEMS = 1 << 22      # elements per independently seeded chunk

TENSOR_IDS = {
    "q": 1, "k": 2, "v": 3, "o": 4, "gate": 5, "up": 6, "down": 7,
    "norm1": 8, "norm2": 9, "bq": 10, "bk": 11, "bv": 12,
    "embed": 20, "head": 21, "final_norm": 22, "ids": 23,
    "x": 30, "dy": 31, "dx_out": 32,
    "lora_A": 40, "lora_B": 41,
}


def _to_bf16_bits(x32):
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _threads():
    n = os.environ.get("LSQ_SYNTH_THREADS")
    if n:
        return max(1, int(n))
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 4


def normal_bf16(shape, mean, std, key):
    """bf16 bits of N(mean, std^2) draws, seeded by ``key`` (a tuple of ints)."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.uint16)
    chunks = [(c, min(_CHUNK_ROWS_ELEMS, total - c)) for c in range(0, total, _CHUNK_ROWS_ELEMS)]

    def fill(ci):
        start, n = chunks[ci]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence((BASE_SEED,) + tuple(key) + (ci,))))
        x = g.standard_normal(n, dtype=np.float32)
        x *= np.float32(std)
        if mean:
            x += np.float32(mean)
        out[start:start + n] = _to_bf16_bits(x)

    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(chunks))))
    elif chunks:
        fill(0)
    return out.reshape(shape)


def token_ids(batch, seq, vocab, key):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence((BASE_SEED,) + tuple(key))))
    return g.integers(0, vocab, size=(batch, seq), dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------- workload tensors
def layer_weights(cfg, wid, layer):
    """bf16 bits of one decoder layer's frozen tensors for workload ``wid``."""
    out = {}
    for name in ("q", "k", "v", "o", "gate", "up", "down"):
        out[name] = normal_bf16(cfg.proj_shape(name), 0.0, 0.02, (wid, layer, TENSOR_IDS[name]))
    out["norm1"] = normal_bf16((cfg.hidden,), 1.0, 0.1, (wid, layer, TENSOR_IDS["norm1"]))
    out["norm2"] = normal_bf16((cfg.hidden,), 1.0, 0.1, (wid, layer, TENSOR_IDS["norm2"]))
    if cfg.qkv_bias:
        for name in ("q", "k", "v"):
            out["b" + name] = normal_bf16((cfg.proj_shape(name)[0],), 0.0, 0.02,
                                          (wid, layer, TENSOR_IDS["b" + name]))
    return out


def layer_lora(cfg, wid, layer):
    """bf16 bits of one layer's adapters: name -> (A [r, in], B [out, r])."""
    out = {}
    r = cfg.lora_r
    for name in ("q", "k", "v", "o", "gate", "up", "down"):
        n_out, n_in = cfg.proj_shape(name)
        A = normal_bf16((r, n_in), 0.0, 0.01, (wid, layer, TENSOR_IDS[name], TENSOR_IDS["lora_A"]))
        B = normal_bf16((n_out, r), 0.0, 0.01, (wid, layer, TENSOR_IDS[name], TENSOR_IDS["lora_B"]))
        out[name] = (A, B)
    return out


def resident_weights(cfg, wid):
    """Embedding, final norm and (untied) head bf16 bits."""
    out = {"embed": normal_bf16((cfg.vocab, cfg.hidden), 0.0, 0.02, (wid, 0, TENSOR_IDS["embed"])),
           "final_norm": normal_bf16((cfg.hidden,), 1.0, 0.1, (wid, 0, TENSOR_IDS["final_norm"]))}
    if not cfg.tied:
        out["head"] = normal_bf16((cfg.vocab, cfg.hidden), 0.0, 0.02, (wid, 0, TENSOR_IDS["head"]))
    return out
