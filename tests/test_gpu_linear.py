"""GPU parity of NF4 quantize / dequantize (bit-exact) and the NF4-LoRA linear
(bf16 tier 1e-2, float32 tier 1e-5) against the oracle, through the C ABI."""
import ctypes as C

import numpy as np
import pytest
import torch

from layer_streamed_qlora_nf4_amd import configs, lib, synth
from oracle import lora as olora
from oracle import nf4 as onf4
from tests.gpu_util import (bits_f64, dev, dev_bits, empty_bytes, host_bits, print_case, ptr, rel_err, row_blocks,
                            stream)

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
F32_TOL = 1e-5


def _quantize_gpu(w_bits, f32=None):
    """bf16 bits (or, with f32, that float32 array) through nf4_quantize with a device flag."""
    n, k = w_bits.shape if f32 is None else f32.shape
    w = dev_bits(w_bits) if f32 is None else dev(f32)
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    absmax = torch.empty((n, k // 64), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.call("nf4_quantize", ptr(w), lib.LSQ_BF16 if f32 is None else lib.LSQ_F32, n, k, 64, ptr(packed),
             ptr(absmax), ptr(flag), stream())
    torch.cuda.synchronize()
    return packed, absmax, flag


@pytest.mark.parametrize("shape", [(1024, 512), (37, 192), (1, 64), (4096, 4096)])
def test_nf4_quantize_bit_exact(gpu, shape):
    print_case(test="nf4_quantize", shape=shape)
    w = synth.normal_bf16(shape, 0.0, 0.02, (77, shape[0], shape[1]))
    w[0, :64] = 0                                   # all-zero block
    if shape[0] > 2:
        w[1, :64] = synth.normal_bf16((64,), 0.0, 1e-30, (78,))   # tiny magnitudes
        w[2, 3] = 0x3F80                                          # an outlier 1.0
    packed, absmax, flag = _quantize_gpu(w)
    rp, ra = row_blocks(onf4.quantize, w)   # every row, the oracle spread over the host's cores
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert flag.item() == 0


def test_nf4_quantize_flags_nonfinite(gpu):
    w = synth.normal_bf16((4, 128), 0.0, 0.02, (79,))
    w[2, 70] = 0x7F80   # +inf
    _, _, flag = _quantize_gpu(w)
    assert flag.item() == 1


def test_nf4_quantize_f32_input_bit_exact(gpu):
    """float32 weights (values no bf16 holds, tiny blocks, an all-zero block and
    exact level midpoints, which only a float32 input can reach)."""
    print_case(test="nf4_quantize_f32", shape=(96, 320))
    x = (synth.normal_bf16((96, 320), 0.0, 0.02, (91,)).astype(np.uint32) << 16).view(np.float32)
    x = x * np.float32(1.0 + 2.0 ** -12)               # off the bf16 grid
    x[0, :64] = 0
    x[1, :64] *= np.float32(1e-30)
    c = onf4.codebook().astype(np.float64)
    mids = [np.float32((c[j] + c[j + 1]) / 2) for j in range(15)
            if float(np.float32((c[j] + c[j + 1]) / 2)) == (c[j] + c[j + 1]) / 2]
    x[2, :64] = 0
    x[2, 0] = 1.0
    x[2, 1:1 + len(mids)] = mids
    packed, absmax, flag = _quantize_gpu(None, f32=x)
    rp, ra = onf4.quantize_f32(x)
    assert np.array_equal(packed.cpu().numpy(), rp)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    assert flag.item() == 0


def test_nf4_quantize_without_flag_returns_nonfinite(gpu):
    """Called without a device flag, the call waits and returns the status itself,
    and a finite input after a refused one still succeeds."""
    w = synth.normal_bf16((4, 128), 0.0, 0.02, (92,))
    bad = w.copy()
    bad[1, 5] = 0x7FC0   # NaN
    out_p = torch.empty((4, 64), dtype=torch.uint8, device="cuda")
    out_a = torch.empty((4, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.LsqError) as e:
        lib.call("nf4_quantize", ptr(dev_bits(bad)), lib.LSQ_BF16, 4, 128, 64, ptr(out_p), ptr(out_a), None,
                 stream())
    assert e.value.status == "LSQ_ERR_NONFINITE"
    lib.call("nf4_quantize", ptr(dev_bits(w)), lib.LSQ_BF16, 4, 128, 64, ptr(out_p), ptr(out_a), None, stream())
    rp, ra = onf4.quantize(w)
    assert np.array_equal(out_p.cpu().numpy(), rp) and np.array_equal(out_a.cpu().numpy(), ra)


# whole and partial 2048-weight wave segments, down to a single 64-block
@pytest.mark.parametrize("shape", [(1024, 512), (40, 320), (1, 64), (7, 4416)])
def test_nf4_dequantize_bit_exact(gpu, shape):
    print_case(test="nf4_dequantize", shape=shape)
    w = synth.normal_bf16(shape, 0.0, 0.02, (80, shape[0]))
    rp, ra = onf4.quantize(w)
    packed, absmax = dev(rp), dev(ra)
    n = shape[0] * shape[1]
    # 8192 guard elements after the output must keep their fill
    out_b = torch.full((n + 8192,), 0x5A5A, dtype=torch.int16, device="cuda")
    out_f = torch.full((n + 8192,), 7.0, dtype=torch.float32, device="cuda")
    lib.call("nf4_dequantize", ptr(packed), ptr(absmax), shape[0], shape[1], lib.LSQ_BF16, ptr(out_b), stream())
    lib.call("nf4_dequantize", ptr(packed), ptr(absmax), shape[0], shape[1], lib.LSQ_F32, ptr(out_f), stream())
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out_b[:n].view(shape)), onf4.dequantize_bf16_bits(rp, ra))
    assert np.array_equal(out_f[:n].view(shape).cpu().numpy().view(np.uint32),
                          onf4.dequantize_f32(rp, ra).view(np.uint32))
    assert bool((out_b[n:] == 0x5A5A).all()) and bool((out_f[n:] == 7.0).all())


# ------------------------------------------------------------------ linear
def _linear_inputs(M, K, N, r, wid):
    X = synth.normal_bf16((M, K), 0.0, 1.0, (wid, 0, synth.TENSOR_IDS["x"]))
    W = synth.normal_bf16((N, K), 0.0, 0.02, (wid, 0, synth.TENSOR_IDS["q"]))
    A = synth.normal_bf16((r, K), 0.0, 0.01, (wid, 0, synth.TENSOR_IDS["lora_A"]))
    B = synth.normal_bf16((N, r), 0.0, 0.01, (wid, 0, synth.TENSOR_IDS["lora_B"]))
    dY = synth.normal_bf16((M, N), 0.0, 1.0, (wid, 0, synth.TENSOR_IDS["dy"]))
    return X, W, A, B, dY


def _run_linear(X, packed, absmax, A, B, dY, M, K, N, r, s, dtype, kind=lib.LSQ_W_NF4, wbf16=None):
    if kind == lib.LSQ_W_NF4:
        wp, wa = dev(packed), dev(absmax)
        weight = lib.Weight(kind, 0, wp.data_ptr(), wa.data_ptr(), N, K)
    else:
        wp = dev_bits(wbf16)
        weight = lib.Weight(kind, 0, wp.data_ptr(), None, N, K)
    if dtype == lib.LSQ_BF16:
        tX, tA, tB, tdY = dev_bits(X), dev_bits(A), dev_bits(B), dev_bits(dY)
        Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        U = torch.empty((M, r), dtype=torch.int16, device="cuda")
        dX = torch.empty((M, K), dtype=torch.int16, device="cuda")
    else:
        tX, tA, tB, tdY = (dev(bits_f64(a).astype(np.float32)) for a in (X, A, B, dY))
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        U = torch.empty((M, r), dtype=torch.float32, device="cuda")
        dX = torch.empty((M, K), dtype=torch.float32, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    wsb = lib.raw("nf4_lora_linear_workspace_size")(M, N, K, r, dtype)
    ws = empty_bytes(wsb)
    lib.call("nf4_lora_linear_fwd", C.byref(weight), None, ptr(tX), M, ptr(tA), ptr(tB), r, s, dtype, ptr(Y),
             ptr(U), ptr(ws), wsb, stream())
    lib.call("nf4_lora_linear_bwd", C.byref(weight), ptr(tX), ptr(U), M, ptr(tA), ptr(tB), r, s, dtype, ptr(tdY),
             ptr(dX), ptr(dA), ptr(dB), 0, ptr(ws), wsb, stream())
    torch.cuda.synchronize()
    conv = (lambda t: bits_f64(host_bits(t))) if dtype == lib.LSQ_BF16 else (lambda t: t.cpu().numpy().astype(np.float64))
    return conv(Y), conv(U), conv(dX), dA.cpu().numpy().astype(np.float64), dB.cpu().numpy().astype(np.float64)


LINEAR_CASES = [
    # (M, K, N, r): the single-linear workload, then ragged M / N, a larger rank,
    # several tiles in every direction.
    (128, 512, 1024, 8),
    (77, 320, 200, 16),
    (300, 1024, 656, 32),
    (1, 64, 16, 8),
    # an odd number of 64-deep reduction steps split several ways (the last
    # split shorter or empty), and a one-row M tail with an odd step count
    (64, 1600, 520, 16),
    (64, 1344, 264, 8),
    (513, 192, 264, 8),
    # ragged last column tiles of many-tile launches: 192-wide tiles split
    # four ways, 256-wide unsplit
    (200, 1024, 7600, 16),
    (300, 256, 28680, 8),
    # 224-wide tiles (two row tiles of 112 wide ones would leave 32 CUs idle),
    # the last column tile ragged
    (512, 256, 28632, 8),
]


@pytest.mark.parametrize("M,K,N,r", LINEAR_CASES)
@pytest.mark.parametrize("dtype", [lib.LSQ_BF16, lib.LSQ_F32])
def test_nf4_lora_linear_matches_oracle(gpu, M, K, N, r, dtype):
    print_case(test="linear", M=M, K=K, N=N, r=r, dtype=dtype)
    alpha = 2.0 * r
    s = alpha / r
    X, W, A, B, dY = _linear_inputs(M, K, N, r, 101 + M)
    packed, absmax = onf4.quantize(W)
    Y, U, dX, dA, dB = _run_linear(X, packed, absmax, A, B, dY, M, K, N, r, s, dtype)
    Wd = onf4.dequantize_bf16_f64(packed, absmax) if dtype == lib.LSQ_BF16 else \
        onf4.dequantize_f32(packed, absmax).astype(np.float64)
    Xf, Af, Bf, dYf = (bits_f64(a) for a in (X, A, B, dY))
    rY, rU = olora.linear_fwd(Xf, Wd, Af, Bf, s)
    rdX, rdA, rdB = olora.linear_bwd(Xf, Wd, Af, Bf, s, dYf)
    tol = BF16_TOL if dtype == lib.LSQ_BF16 else F32_TOL
    for name, got, ref in (("Y", Y, rY), ("U", U, s * rU), ("dX", dX, rdX), ("dA", dA, rdA), ("dB", dB, rdB)):
        e = rel_err(got, ref)
        assert e <= tol, f"{name}: {e:.3e} > {tol}"


def test_linear_bwd_with_no_tokens_clears_or_keeps_the_adapter_grads(gpu):
    """M = 0: dA and dB are zero (accumulate = 0) or left as they were (accumulate = 1)."""
    K, N, r = 256, 320, 8
    print_case(test="linear_bwd_empty", K=K, N=N, r=r)
    w = synth.normal_bf16((N, K), 0.0, 0.02, (130, 0))
    packed, absmax = (dev(a) for a in onf4.quantize(w))
    weight = lib.Weight(lib.LSQ_W_NF4, 0, packed.data_ptr(), absmax.data_ptr(), N, K)
    A = torch.zeros((r, K), dtype=torch.int16, device="cuda")
    B = torch.zeros((N, r), dtype=torch.int16, device="cuda")
    dummy = torch.zeros(64, dtype=torch.int16, device="cuda")
    wsb = lib.raw("nf4_lora_linear_workspace_size")(0, N, K, r, lib.LSQ_BF16)
    ws = empty_bytes(max(wsb, 256))
    for dtype in (lib.LSQ_BF16, lib.LSQ_F32):
        lib.call("nf4_lora_linear_fwd", C.byref(weight), None, ptr(dummy), 0, ptr(A), ptr(B), r, 2.0, dtype,
                 ptr(dummy), ptr(dummy), ptr(ws), wsb, stream())
        for accumulate in (1, 0):
            dA = torch.full((r, K), 7.0, dtype=torch.float32, device="cuda")
            dB = torch.full((N, r), 7.0, dtype=torch.float32, device="cuda")
            lib.call("nf4_lora_linear_bwd", C.byref(weight), ptr(dummy), ptr(dummy), 0, ptr(A), ptr(B), r, 2.0,
                     dtype, ptr(dummy), ptr(dummy), ptr(dA), ptr(dB), accumulate, ptr(ws), wsb, stream())
            torch.cuda.synchronize()
            want = 7.0 if accumulate else 0.0
            assert bool((dA == want).all()) and bool((dB == want).all()), (dtype, accumulate)


IDENTITY_CASES = [
    # (M, K, N): 256-wide tiles with several row tiles; a ragged N with an odd
    # number of k-steps; the 192-wide forward tile (N = 6144 at 512 rows); a
    # forward split four or more ways over its k-steps; the 224-wide tile
    (1024, 512, 1024),
    (600, 320, 600),
    (512, 512, 6144),
    (2048, 2048, 256),
    (1024, 1024, 14336),   # 224-wide forward tiles: 256 of them against 224 of 256
]


@pytest.mark.parametrize("M,K,N", IDENTITY_CASES)
@pytest.mark.parametrize("dtype", [lib.LSQ_BF16, lib.LSQ_F32])
def test_in_gemm_decode_is_the_dequantized_weight(gpu, M, K, N, dtype):
    """With X = I the forward's output is W^T, and with dY = I (and B = 0) the
    backward's dX is W: each output is one product with 1.0 accumulated in
    float32, so it must equal the oracle's dequantized weight exactly (bf16
    bits, or the float32 product, compared as values so that +0 and -0 of an
    all-zero block agree).  Random codes cover all 16 levels; the absmax values
    span 1e-30 to 1e30 and include zero blocks."""
    print_case(test="in_gemm_decode", M=M, K=K, N=N, dtype=dtype)
    rng = np.random.default_rng(7000 + M + K + N)
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    mag = 10.0 ** rng.choice([-30, -12, -3, -1, 0, 2, 12, 30], size=(N, K // 64))
    absmax = (mag * rng.uniform(0.5, 1.0, size=mag.shape)).astype(np.float32)
    absmax[rng.random(absmax.shape) < 0.02] = 0.0
    one = np.uint16(0x3F80)
    X = np.zeros((M, K), dtype=np.uint16)
    X[np.arange(min(M, K)), np.arange(min(M, K))] = one
    dY = np.zeros((M, N), dtype=np.uint16)
    dY[np.arange(min(M, N)), np.arange(min(M, N))] = one
    r = 8
    A = synth.normal_bf16((r, K), 0.0, 0.01, (140, 0))
    B = np.zeros((N, r), dtype=np.uint16)
    Y, _, dX, _, _ = _run_linear(X, packed, absmax, A, B, dY, M, K, N, r, 2.0, dtype)
    Wd = onf4.dequantize_bf16_f64(packed, absmax) if dtype == lib.LSQ_BF16 else \
        onf4.dequantize_f32(packed, absmax).astype(np.float64)
    kk, nn = min(M, K), min(M, N)
    assert np.array_equal(Y[:kk], Wd.T[:kk]) and not Y[kk:].any()
    assert np.array_equal(dX[:nn], Wd[:nn]) and not dX[nn:].any()


@pytest.mark.parametrize("M,K,N", [
    # one tile; ragged rows and columns over several tiles; a reduction split
    # several ways with an odd step count; a one-row M tail
    (96, 256, 320), (300, 1024, 656), (64, 1600, 520), (513, 192, 264)])
def test_bf16_base_linear_matches_oracle(gpu, M, K, N):
    print_case(test="bf16_linear", M=M, K=K, N=N)
    r, s = 16, 2.0
    X, W, A, B, dY = _linear_inputs(M, K, N, r, 120 + M)
    Y, U, dX, dA, dB = _run_linear(X, None, None, A, B, dY, M, K, N, r, s, lib.LSQ_BF16, kind=lib.LSQ_W_BF16, wbf16=W)
    Wf, Xf, Af, Bf, dYf = (bits_f64(a) for a in (W, X, A, B, dY))
    rY, _ = olora.linear_fwd(Xf, Wf, Af, Bf, s)
    rdX, rdA, rdB = olora.linear_bwd(Xf, Wf, Af, Bf, s, dYf)
    for name, got, ref in (("Y", Y, rY), ("dX", dX, rdX), ("dA", dA, rdA), ("dB", dB, rdB)):
        assert rel_err(got, ref) <= BF16_TOL, name


def test_linear_is_deterministic(gpu):
    M, K, N, r = 300, 1024, 656, 16
    X, W, A, B, dY = _linear_inputs(M, K, N, r, 130)
    packed, absmax = onf4.quantize(W)
    a = _run_linear(X, packed, absmax, A, B, dY, M, K, N, r, 2.0, lib.LSQ_BF16)
    b = _run_linear(X, packed, absmax, A, B, dY, M, K, N, r, 2.0, lib.LSQ_BF16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
