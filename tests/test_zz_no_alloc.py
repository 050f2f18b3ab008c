"""The no-allocation entry point, nf4_lora_linear_bwd_noalloc (for callers
that cannot allocate: its scratch is a static per-GPU array), against
nf4_lora_linear_bwd with a caller workspace on the same inputs: dX, dA and dB
bit for bit, over two calls in a row on one GPU, the second smaller than the
first (the shared array still holds the first call's partials and counters
state).  The shapes split every reduction over workgroups, so the arrival
counters and the split-K partials in the array are all exercised.  (Its
refusal of a shape beyond the array needs no GPU and is in test_host.py.)"""
import ctypes as C

import pytest
import torch

from layer_streamed_qlora_nf4_amd import lib, synth
from oracle import nf4 as onf4
from tests.gpu_util import dev, dev_bits, empty_bytes, print_case, ptr, rel_err, stream

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, r, wid):
    X = synth.normal_bf16((M, K), 0.0, 1.0, (wid, 0, synth.TENSOR_IDS["x"]))
    Wb = synth.normal_bf16((N, K), 0.0, 0.02, (wid, 0, synth.TENSOR_IDS["q"]))
    A = synth.normal_bf16((r, K), 0.0, 0.01, (wid, 0, synth.TENSOR_IDS["lora_A"]))
    B = synth.normal_bf16((N, r), 0.0, 0.01, (wid, 0, synth.TENSOR_IDS["lora_B"]))
    dY = synth.normal_bf16((M, N), 0.0, 1.0, (wid, 0, synth.TENSOR_IDS["dy"]))
    return X, Wb, A, B, dY


def _bwd(noalloc, weight, tX, tA, tB, tdY, M, K, N, r, s):
    dX = torch.empty((M, K), dtype=torch.int16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    if noalloc:
        lib.call("nf4_lora_linear_bwd_noalloc", C.byref(weight), ptr(tX), None, M, ptr(tA), ptr(tB), r, s,
                 lib.LSQ_BF16, ptr(tdY), ptr(dX), ptr(dA), ptr(dB), 0, stream())
    else:
        nws = lib.raw("nf4_lora_linear_workspace_size")(M, N, K, r, lib.LSQ_BF16)
        ws = empty_bytes(nws)
        lib.call("nf4_lora_linear_bwd", C.byref(weight), ptr(tX), None, M, ptr(tA), ptr(tB), r, s, lib.LSQ_BF16,
                 ptr(tdY), ptr(dX), ptr(dA), ptr(dB), 0, ptr(ws), nws, stream())
    torch.cuda.synchronize()
    return dX, dA, dB


def test_noalloc_backward_equals_workspace_backward_on_two_calls(gpu):
    K, N, r, s = 4096, 1024, 16, 2.0
    Wb = synth.normal_bf16((N, K), 0.0, 0.02, (61, 0, synth.TENSOR_IDS["q"]))
    packed, absmax = onf4.quantize(Wb)
    wp, wa = dev(packed), dev(absmax)
    weight = lib.Weight(lib.LSQ_W_NF4, 0, wp.data_ptr(), wa.data_ptr(), N, K)
    for M in (300, 100):   # the second call smaller
        print_case(test="noalloc_bwd", M=M, K=K, N=N, r=r)
        assert lib.raw("nf4_lora_linear_workspace_size")(M, N, K, r, lib.LSQ_BF16) <= lib.LSQ_NOALLOC_SCRATCH_BYTES
        X, _, A, B, dY = _inputs(M, K, N, r, 60 + M)
        tX, tA, tB, tdY = dev_bits(X), dev_bits(A), dev_bits(B), dev_bits(dY)
        ref = _bwd(False, weight, tX, tA, tB, tdY, M, K, N, r, s)
        got = _bwd(True, weight, tX, tA, tB, tdY, M, K, N, r, s)
        for name, a, b in zip(("dX", "dA", "dB"), got, ref):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), (M, name)
            assert rel_err(a.float().cpu().numpy() if a.dtype == torch.float32 else a.cpu().numpy(),
                           b.float().cpu().numpy() if b.dtype == torch.float32 else b.cpu().numpy()) == 0.0
