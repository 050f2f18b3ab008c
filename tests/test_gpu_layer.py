"""GPU parity of decoder_layer_fwd / decoder_layer_bwd against the oracle."""
import ctypes as C

import numpy as np
import pytest
import torch

from layer_streamed_qlora_nf4_amd import configs, lib, model, synth
from oracle import layer as olayer
from oracle import nf4 as onf4
from tests.gpu_util import bits_f64, dev, empty_bytes, print_case, ptr, rel_err, row_blocks, stream

pytestmark = pytest.mark.gpu
TOL = 1e-2


def oracle_cfg(cfg):
    return olayer.LayerCfg(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.eps,
                           cfg.theta, cfg.qkv_bias)


def oracle_layer_params(cfg, layer, rows=None):
    """Oracle weights (float64) from the same seeded bits the store was written from."""
    w = synth.layer_weights(cfg, cfg.wid, layer)
    W = {}
    for name in model.PROJ:
        if cfg.quant == "nf4":
            packed, absmax = row_blocks(onf4.quantize, w[name])
            W[name] = row_blocks(onf4.dequantize_bf16_f64, packed, absmax)
        else:
            W[name] = bits_f64(w[name])
    for k in ("norm1", "norm2", "bq", "bk", "bv"):
        if k in w:
            W[k] = bits_f64(w[k])
    ad = {n: (bits_f64(a), bits_f64(b)) for n, (a, b) in synth.layer_lora(cfg, cfg.wid, layer).items()}
    return W, ad


def run_layer(cfg, x_bits, dout_f32, want_bwd=True):
    cfg1 = cfg.with_(n_layers=1)
    store = model.Store(cfg1)
    blob = dev(store.host_blob(0).copy())
    lora = dev(model.lora_arena_host(cfg1)[0].view(np.int16))
    ccfg = lib.model_cfg(cfg1)
    B, S, H = cfg.batch, cfg.seq, cfg.hidden
    wsb = lib.raw("decoder_layer_workspace_size")(C.byref(ccfg), B, S)
    ws = empty_bytes(wsb)
    x = dev(bits_f64(x_bits).astype(np.float32))
    xo = torch.empty_like(x)
    lib.call("decoder_layer_fwd", C.byref(ccfg), ptr(blob), ptr(lora), ptr(x), B, S, ptr(xo), ptr(ws), wsb, stream())
    out = {"x_out": xo}
    if want_bwd:
        dxo = dev(dout_f32)
        dxi = torch.empty_like(x)
        grad = torch.zeros(lora.numel(), dtype=torch.float32, device="cuda")
        lib.call("decoder_layer_bwd", C.byref(ccfg), ptr(blob), ptr(lora), ptr(x), ptr(dxo), B, S, ptr(dxi), ptr(grad),
                 0, ptr(ws), wsb, stream())
        out["dx_in"] = dxi
        out["grad"] = grad
    torch.cuda.synchronize()
    store.close()
    return {k: v.cpu().numpy() for k, v in out.items()}


def inputs(cfg, seq=None):
    S = seq or cfg.seq
    x = synth.normal_bf16((cfg.batch, S, cfg.hidden), 0.0, 1.0, (cfg.wid, 99, synth.TENSOR_IDS["x"]))
    d = synth.normal_bf16((cfg.batch, S, cfg.hidden), 0.0, 1.0, (cfg.wid, 99, synth.TENSOR_IDS["dx_out"]))
    return x, bits_f64(d).astype(np.float32)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_QWEN,
                                 configs.TINY.with_(name="tiny-b1-s200", batch=1, seq=200, wid=11),
                                 # one-token sequences; head_dim 128 with one kv head per two query
                                 # heads and a sequence one past a whole query block
                                 configs.TINY.with_(name="tiny-s1", batch=3, seq=1, wid=13),
                                 configs.TINY.with_(name="tiny-hd128", n_heads=2, n_kv_heads=1, head_dim=128,
                                                    batch=2, seq=129, wid=14),
                                 # 1000 tokens: the adapter-gradient token reduction split 7 ways, the last range short
                                 configs.TINY.with_(name="tiny-t1000", batch=2, seq=500, wid=15)])
def test_decoder_layer_matches_oracle(gpu, cfg):
    print_case(test="decoder_layer", cfg=cfg.name, B=cfg.batch, S=cfg.seq)
    x_bits, dout = inputs(cfg)
    got = run_layer(cfg, x_bits, dout)
    W, ad = oracle_layer_params(cfg, 0)
    oc = oracle_cfg(cfg)
    x = bits_f64(x_bits)
    ref_out = olayer.layer_fwd(oc, x, W, ad, cfg.lora_scale)
    ref_dx, ref_g = olayer.layer_bwd(oc, x, W, ad, cfg.lora_scale, dout.astype(np.float64))
    assert rel_err(got["x_out"].reshape(ref_out.shape), ref_out) <= TOL
    assert rel_err(got["dx_in"].reshape(ref_dx.shape), ref_dx) <= TOL
    g = model.split_lora_grads(cfg, got["grad"])
    # With one-token sequences the softmax has a single key, so q and k get no
    # gradient at all: their references are exactly zero and the GPU's rounding
    # noise is measured against the layer's largest adapter gradient instead.
    scale = max(float(np.abs(ref_g[n][w]).max()) for n in model.PROJ for w in (0, 1))
    for name in model.PROJ:
        for which in (0, 1):
            ref = ref_g[name][which]
            if np.abs(ref).max() == 0.0:
                e = float(np.abs(g[name][which]).max()) / scale
            else:
                e = rel_err(g[name][which], ref)
            assert e <= TOL, f"{name} d{'AB'[which]}: {e:.3e}"


def layer_errors(cfg, got, x_bits, dout):
    """Every output of one layer's forward and backward against the oracle:
    the layer output and dx over all rows, and each of the 14 adapter
    gradients, as max|diff| / max|ref|.  Printed before any assertion so a
    run's log carries the margin of every tensor."""
    W, ad = oracle_layer_params(cfg, 0)
    oc = oracle_cfg(cfg)
    x = bits_f64(x_bits)
    ref_out = olayer.layer_fwd(oc, x, W, ad, cfg.lora_scale)
    ref_dx, ref_g = olayer.layer_bwd(oc, x, W, ad, cfg.lora_scale, dout.astype(np.float64))
    errs = {"out": rel_err(got["x_out"].reshape(ref_out.shape), ref_out),
            "dx": rel_err(got["dx_in"].reshape(ref_dx.shape), ref_dx)}
    g = model.split_lora_grads(cfg, got["grad"])
    for name in model.PROJ:
        for which in (0, 1):
            errs[f"{name}.d{'AB'[which]}"] = rel_err(g[name][which], ref_g[name][which])
    worst = max(errs, key=errs.get)
    print(f"ERRORS {cfg.name} B={cfg.batch} S={cfg.seq}: worst {worst} {errs[worst]:.3e}; " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    return errs


# Each workload's layer at its own widths.  The 8B layer runs at a short ragged
# sequence and at its full 1 x 2048 tokens (32 query blocks of causal
# attention, every row compared); the Qwen2.5-3B-shaped layer has a bf16 base,
# q/k/v biases and eight query heads per KV head, with two sequences; the
# 72B-shaped layer has hidden 8192 (the widest row the RMSNorm kernels hold),
# 64 query and 8 KV heads and intermediate 29568.
WORKLOAD_LAYERS = [
    configs.LAYER_8B.with_(name="llama8b-layer-s100", seq=100, wid=12),
    configs.LAYER_8B,
    # ragged length (not a multiple of 64 or 128) in the 128-query attention blocks
    configs.LAYER_8B.with_(name="llama8b-layer-s1000", seq=1000, wid=14),
    configs.STACK_3B_BF16.with_(name="qwen3b-bf16-layer", n_layers=1, batch=2, seq=200, wid=42),
    configs.STACK_72B.with_(name="qwen72b-layer", n_layers=1, batch=1, seq=100, wid=43),
]


@pytest.mark.parametrize("cfg", WORKLOAD_LAYERS, ids=lambda c: c.name)
def test_workload_layer_matches_oracle(gpu, cfg):
    print_case(test="workload_layer", cfg=cfg.name, B=cfg.batch, S=cfg.seq, H=cfg.hidden, I=cfg.intermediate,
               heads=f"{cfg.n_heads}/{cfg.n_kv_heads}", quant=cfg.quant)
    x_bits, dout = inputs(cfg)
    got = run_layer(cfg, x_bits, dout)
    errs = layer_errors(cfg, got, x_bits, dout)
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, bad
