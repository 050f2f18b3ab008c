"""Host-side checks that need no GPU: the library loads and exports every
symbol the header declares, its constants and layouts agree with the oracle's
closed forms, the pre-flight refuses what does not fit, the store's page-lock
fallback behaves as documented, and bad arguments fail before any launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from layer_streamed_qlora_nf4_amd import configs, lib
from oracle import nf4 as onf4
from oracle import sizes as osizes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lsq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_library_exports_every_declared_symbol():
    lib.load()
    cdll = C.CDLL(lib.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 30
    missing = [n for n in names if not hasattr(cdll, n)]
    assert missing == [], missing
    assert lib.load().missing_symbols == []
    assert set(lib.exported_symbols()) <= set(names)


def test_codebook_is_the_oracle_codebook_bitwise():
    got = np.array(lib.codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), onf4.codebook().view(np.uint32))


SHAPES = {"llama8b": (configs.STACK_8B, (4096, 32, 8, 128, 14336, False)),
          "qwen72b": (configs.STACK_72B, (8192, 64, 8, 128, 29568, True))}


@pytest.mark.parametrize("name", list(SHAPES))
def test_blob_layout_matches_closed_form(name):
    cfg, shape = SHAPES[name]
    L = lib.blob_layout(cfg)
    algo = osizes.layer_bytes_fp32_absmax(shape)
    # 4 KiB header and 4 KiB alignment of each of the 8 weight sections + small tensors
    assert algo <= L.total_bytes <= algo + 4096 * 12
    assert L.total_bytes % 4096 == 0
    for off in list(L.w_off) + list(L.absmax_off):
        assert off % 4096 == 0
    nq, nkv, H, I = shape[1] * shape[3], shape[2] * shape[3], shape[0], shape[4]
    assert L.absmax_off[0] - L.w_off[0] >= (nq + 2 * nkv) * H // 2
    if name == "llama8b":
        assert L.total_bytes == 122703872       # 117.02 MiB: the blob every step moves twice


def test_bf16_blob_and_lora_layout():
    cfg = configs.STACK_3B_BF16
    L = lib.blob_layout(cfg)
    lin = osizes.layer_linear_params(2048, 16, 2, 128, 11008)
    assert 2 * lin <= L.total_bytes <= 2 * lin + 4096 * 12
    assert list(L.absmax_off) == [0, 0, 0, 0] and L.bias_off > 0
    ll = lib.lora_layout(configs.STACK_8B)
    r, H, I = 16, 4096, 14336
    params = r * (3 * H + 4096 + 2 * H + I) + r * (6144 + H + 2 * I + H)
    assert params <= ll.layer_elems <= params + 8 * 128


def _cfg_struct(cfg):
    return C.byref(lib.model_cfg(cfg))


def test_vram_prediction_terms_and_refusal():
    cfg = configs.STACK_8B
    b = lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(cfg), 1, 512, 2, 0, C.byref(b))
    blob = lib.blob_layout(cfg).total_bytes
    assert b.slots == 2 * blob
    assert b.resident == 2 * 2 * cfg.vocab * cfg.hidden + 2 * cfg.hidden
    assert b.checkpoints == 4 * 512 * cfg.hidden * (cfg.n_layers + 1)
    # the prediction errs high: the caller's ids and loss, per-buffer allocator
    # rounding, and a margin of 1% (at least 1 MiB) on top of the buffers
    parts = b.slots + b.resident + b.adapters + b.checkpoints + b.saved_activations + b.step_workspace
    assert b.caller >= 4 * 512 + 4 + 8 * 511
    assert b.margin == max((parts + b.caller) // 100, 1 << 20)
    assert b.total == parts + b.caller + b.margin
    # the logits term scales with batch x seq x vocab: that is what streaming does not bound
    b2 = lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(cfg), 4, 512, 2, 0, C.byref(b2))
    assert b2.step_workspace - b.step_workspace >= 3 * 512 * cfg.vocab * 6
    # refused before any GPU work when the (overridden) free memory is too small
    with pytest.raises(lib.LsqError) as e:
        lib.call("lsq_preflight", _cfg_struct(cfg), 1, 512, 2, 0, int(b.total) - 1, None)
    assert e.value.status == "LSQ_ERR_REFUSED"
    assert "predicted to need" in str(e.value)
    lib.call("lsq_preflight", _cfg_struct(cfg), 1, 512, 2, 0, int(b.total), None)
    # kept activations are a term of their own, proportional to layers x tokens
    k = lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(cfg), 1, 512, 2, lib.LSQ_STEP_KEEP_ACTIVATIONS, C.byref(k))
    rc = lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(cfg), 1, 512, 2, lib.LSQ_STEP_RECOMPUTE_ALL, C.byref(rc))
    # the default keeps the three layers whose backward runs with the link idle (L-1, 1, 0)
    assert rc.saved_activations == 0 and k.saved_activations > 0
    assert b.saved_activations * cfg.n_layers == 3 * k.saved_activations
    assert (b.total - b.margin) - (rc.total - rc.margin) == b.saved_activations
    per_token_layer = k.saved_activations / (512 * cfg.n_layers)
    H, I, r = cfg.hidden, cfg.intermediate, cfg.lora_r
    # the bf16/f32 tensors the backward reads, 256-byte aligned each: the normed
    # input as a bf16 hi/lo pair, q/k/v in float32, the attention output (bf16,
    # f32), the log-sum-exp, the mid residual, its norm, gate/up, the SwiGLU
    # product, and every U in bf16 and f32
    approx = 4 * H + 4 * 6144 + 2 * 4096 + 4 * 4096 + 4 * 32 + 4 * H + 2 * H + 4 * I + 2 * I + 2 * 7 * r + 4 * 7 * r
    assert approx <= per_token_layer <= approx * 1.01
    assert k.total - k.saved_activations < rc.total   # the layer scratch no longer holds them


def test_store_pageable_fallback_and_refusal(capfd):
    cfg = configs.TINY
    h = C.c_void_p()
    with pytest.raises(lib.LsqError) as e:
        lib.call("shard_store_create", _cfg_struct(cfg), lib.LSQ_STORE_FAIL_PIN, C.byref(h))
    assert e.value.status == "LSQ_ERR_OOM" and "page-lock" in str(e.value)
    lib.call("shard_store_create", _cfg_struct(cfg), lib.LSQ_STORE_FAIL_PIN | lib.LSQ_STORE_ALLOW_PAGEABLE, C.byref(h))
    assert lib.raw("shard_store_is_pinned")(h) == 0
    assert "PAGEABLE" in capfd.readouterr().err
    assert lib.raw("shard_store_layer_bytes")(h) == lib.blob_layout(cfg).total_bytes
    base = lib.raw("shard_store_layer_host")(h, 0)
    assert lib.raw("shard_store_layer_host")(h, 1) == base + lib.blob_layout(cfg).total_bytes
    assert lib.raw("shard_store_layer_host")(h, cfg.n_layers) is None
    lib.raw("shard_store_destroy")(h)
    lib.call("shard_store_create", _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h))
    assert lib.raw("shard_store_is_pinned")(h) == 0
    lib.raw("shard_store_destroy")(h)


def test_arguments_are_refused_before_any_launch():
    cfg = configs.TINY
    bad = cfg.with_(lora_r=12)
    with pytest.raises(lib.LsqError) as e:
        lib.blob_layout(bad)
    assert e.value.status == "LSQ_ERR_SHAPE"
    w = lib.Weight(lib.LSQ_W_NF4, 0, 4096, 8192, 64, 96)
    with pytest.raises(lib.LsqError) as e:
        lib.call("nf4_lora_linear_fwd", C.byref(w), None, C.c_void_p(4096), 8, C.c_void_p(4096), C.c_void_p(4096), 8,
                 2.0, lib.LSQ_BF16, C.c_void_p(4096), None, None, 0, None)
    assert e.value.status == "LSQ_ERR_SHAPE"
    w = lib.Weight(lib.LSQ_W_NF4, 0, 4096 + 8, 8192, 64, 128)
    with pytest.raises(lib.LsqError) as e:
        lib.call("nf4_lora_linear_fwd", C.byref(w), None, C.c_void_p(4096), 8, C.c_void_p(4096), C.c_void_p(4096), 8,
                 2.0, lib.LSQ_BF16, C.c_void_p(4096), None, None, 0, None)
    assert e.value.status == "LSQ_ERR_ALIGN"
    # stream_buffers outside [2, 8] is a refusal, not a clamp
    h = C.c_void_p()
    lib.call("shard_store_create", _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h))
    p = C.c_void_p()
    for n in (1, 9):
        with pytest.raises(lib.LsqError) as e:
            lib.call("layer_pool_create", h, n, C.c_void_p(1 << 20), 1 << 20, C.c_void_p(1), C.c_void_p(2), 0,
                     C.byref(p))
        assert e.value.status == "LSQ_ERR_INVALID" and "[2, 8]" in str(e.value)
    lib.raw("shard_store_destroy")(h)
    with pytest.raises(lib.LsqError) as e:
        lib.call("decoder_layer_fwd", _cfg_struct(cfg.with_(n_layers=1)), C.c_void_p(4096), C.c_void_p(4096),
                 C.c_void_p(4096), 1, 8, C.c_void_p(8192), C.c_void_p(16384), 16, None)
    assert e.value.status == "LSQ_ERR_WORKSPACE"


def test_workspace_queries_are_consistent():
    for cfg in (configs.TINY, configs.STACK_8B, configs.STACK_3B_BF16):
        c = _cfg_struct(cfg)
        lw = lib.raw("decoder_layer_workspace_size")(c, cfg.batch, cfg.seq)
        sw = lib.raw("lsq_step_workspace_size")(c, cfg.batch, cfg.seq, 0)
        sr = lib.raw("lsq_step_workspace_size")(c, cfg.batch, cfg.seq, lib.LSQ_STEP_RECOMPUTE_ALL)
        assert 0 < lw < sr < sw
        assert lib.raw("lsq_step_workspace_size")(c, cfg.batch, cfg.seq, lib.LSQ_STEP_KEEP_ACTIVATIONS) > sr
        assert lib.raw("decoder_layer_workspace_size")(c, cfg.batch, 2 * cfg.seq) > lw


def _fill_store_with_blobs(h, cfg, seed):
    """Random blob bytes with a valid per-layer header (magic + layer index)."""
    rng = np.random.default_rng(seed)
    nbytes = lib.raw("shard_store_layer_bytes")(h)
    blobs = []
    for layer in range(cfg.n_layers):
        p = lib.raw("shard_store_layer_host")(h, layer)
        arr = np.ctypeslib.as_array((C.c_uint8 * nbytes).from_address(p))
        arr[:] = rng.integers(0, 256, nbytes, dtype=np.uint8)
        arr[:8] = np.frombuffer(b"LSQBLOB1", dtype=np.uint8)
        arr[8:12] = np.frombuffer(np.int32(layer).tobytes(), dtype=np.uint8)
        blobs.append(arr.copy())
    return blobs


def _store_bytes(h, cfg):
    nbytes = lib.raw("shard_store_layer_bytes")(h)
    return [np.ctypeslib.as_array((C.c_uint8 * nbytes).from_address(lib.raw("shard_store_layer_host")(h, l))).copy()
            for l in range(cfg.n_layers)]


def test_shard_store_save_load_roundtrip_and_refusals(tmp_path):
    cfg = configs.TINY
    h = C.c_void_p()
    lib.call("shard_store_create", _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h))
    blobs = _fill_store_with_blobs(h, cfg, 3)
    path = str(tmp_path / "tiny.lsqstore")
    lib.call("shard_store_save", h, path.encode())
    lib.raw("shard_store_destroy")(h)
    assert not os.path.exists(path + ".tmp")
    size = os.path.getsize(path)
    assert size == 4096 + 4096 + cfg.n_layers * lib.blob_layout(cfg).total_bytes

    h2 = C.c_void_p()
    lib.call("shard_store_load", path.encode(), _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h2))
    got = _store_bytes(h2, cfg)
    lib.raw("shard_store_destroy")(h2)
    assert all(np.array_equal(a, b) for a, b in zip(blobs, got))

    # a run asking for another shape is told which field differs (re-shard, not stream)
    with pytest.raises(lib.LsqError) as e:
        lib.call("shard_store_load", path.encode(), _cfg_struct(cfg.with_(intermediate=cfg.intermediate + 64)),
                 lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h2))
    assert e.value.status == "LSQ_ERR_STATE" and "intermediate" in str(e.value)
    with pytest.raises(lib.LsqError) as e:
        lib.call("shard_store_load", path.encode(), _cfg_struct(cfg.with_(quant="bf16")),
                 lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h2))
    assert e.value.status == "LSQ_ERR_STATE" and "weight_kind" in str(e.value)

    raw = bytearray(open(path, "rb").read())
    # one flipped byte inside layer 1's blob fails its checksum
    bad = bytearray(raw)
    bad[8192 + lib.blob_layout(cfg).total_bytes + 777] ^= 0x40
    p_bad = str(tmp_path / "bad.lsqstore")
    open(p_bad, "wb").write(bytes(bad))
    with pytest.raises(lib.LsqError) as e:
        lib.call("shard_store_load", p_bad.encode(), _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h2))
    assert e.value.status == "LSQ_ERR_IO" and "checksum" in str(e.value) and "layer 1" in str(e.value)
    # truncated, trailing bytes, not a store
    for name, data, word in (("short", bytes(raw[:-100]), "truncated"), ("long", bytes(raw) + b"x", "trailing"),
                             ("magic", b"NOTSTORE" + bytes(raw[8:]), "not a version")):
        p = str(tmp_path / f"{name}.lsqstore")
        open(p, "wb").write(data)
        with pytest.raises(lib.LsqError) as e:
            lib.call("shard_store_load", p.encode(), _cfg_struct(cfg), lib.LSQ_STORE_FORCE_PAGEABLE, C.byref(h2))
        assert e.value.status == "LSQ_ERR_IO" and word in str(e.value), (name, str(e.value))
    with pytest.raises(lib.LsqError) as e:
        lib.call("shard_store_load", str(tmp_path / "missing").encode(), None, 0, C.byref(h2))
    assert e.value.status == "LSQ_ERR_IO"


def test_large_layer_streaming_and_loss_chunk_terms():
    cfg = configs.STACK_8B
    V, H, T = cfg.vocab, cfg.hidden, 512
    base, large = lib.VramBreakdown(), lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(cfg), 1, T, 2, 0, C.byref(base))
    lib.call("vram_predict_peak", _cfg_struct(cfg), 1, T, 2, lib.LSQ_STEP_STREAM_LARGE, C.byref(large))
    # embedding and head leave the resident term; one head-sized buffer joins the workspace
    assert large.resident == 2 * H
    assert large.step_workspace - base.step_workspace == 2 * V * H
    assert (base.total - base.margin) - (large.total - large.margin) == 2 * V * H
    # stream_loss_chunk bounds the logits buffers at chunk x vocab (fp32 logits + bf16 dlogits)
    c1 = cfg.with_(loss_chunk=128)
    ch = lib.VramBreakdown()
    lib.call("vram_predict_peak", _cfg_struct(c1), 1, T, 2, 0, C.byref(ch))
    saved = base.step_workspace - ch.step_workspace
    assert saved >= (T - 128) * V * 6 - (16 << 20)   # less any larger split-K partials of the shorter head GEMMs
    with pytest.raises(lib.LsqError) as e:
        lib.call("vram_predict_peak", _cfg_struct(cfg.with_(loss_chunk=-1)), 1, T, 2, 0, C.byref(ch))
    assert e.value.status == "LSQ_ERR_INVALID"


# Refusals of the compute calls.  They hand the library addresses that are not
# memory at all: every check runs before the first HIP call, so nothing is
# ever dereferenced or launched, and they run without a GPU.
def test_nf4_shape_errors_enqueue_nothing():
    fake = C.c_void_p(16)
    for args, status in (((lib.LSQ_BF16, 4, 96, 64), "LSQ_ERR_SHAPE"),      # n_in % 64 != 0
                         ((lib.LSQ_BF16, 4, 128, 32), "LSQ_ERR_SHAPE"),     # the store format's block is 64
                         ((7, 4, 128, 64), "LSQ_ERR_INVALID")):             # not bf16 or float32 input
        with pytest.raises(lib.LsqError) as e:
            lib.call("nf4_quantize", fake, *args, fake, fake, None, None)
        assert e.value.status == status, args


def test_bf16_linear_rejects_n_out_not_a_multiple_of_8():
    """The bf16 kernels read rows of dY and B in 8-element chunks: n_out % 8 != 0
    is refused before anything is enqueued (the float32 tier takes any n_out)."""
    fake = C.c_void_p(256)
    w = lib.Weight(lib.LSQ_W_NF4, 0, 256, 256, 12, 64)
    for name, args in (("nf4_lora_linear_fwd", (None, fake, 4, fake, fake, 8, 2.0, lib.LSQ_BF16, fake, None,
                                                  fake, 1 << 20, None)),
                       ("nf4_lora_linear_bwd", (fake, None, 4, fake, fake, 8, 2.0, lib.LSQ_BF16, fake, fake, fake,
                                                  fake, 0, fake, 1 << 20, None))):
        with pytest.raises(lib.LsqError) as e:
            lib.call(name, C.byref(w), *args)
        assert e.value.status == "LSQ_ERR_SHAPE", name


def test_noalloc_backward_refuses_a_shape_beyond_its_scratch():
    """nf4_lora_linear_bwd_noalloc checks the shape's scratch need against its
    static array before it looks up the array's device address."""
    M, N, K, r = 3072, 4096, 14336, 16   # its split-K partials alone pass the array
    need = lib.raw("nf4_lora_linear_workspace_size")(M, N, K, r, lib.LSQ_BF16)
    assert need > lib.LSQ_NOALLOC_SCRATCH_BYTES
    weight = lib.Weight(lib.LSQ_W_NF4, 0, 4096, 8192, N, K)
    fake = C.c_void_p(4096)
    with pytest.raises(lib.LsqError) as e:
        lib.call("nf4_lora_linear_bwd_noalloc", C.byref(weight), fake, None, M, fake, fake, r, 2.0, lib.LSQ_BF16,
                 fake, fake, fake, fake, 0, None)
    assert e.value.status == "LSQ_ERR_WORKSPACE"


def test_layer_rejects_bad_arguments():
    cfg = configs.TINY.with_(n_layers=1)
    ccfg = lib.model_cfg(cfg)
    with pytest.raises(lib.LsqError) as e:
        lib.call("decoder_layer_fwd", C.byref(ccfg), C.c_void_p(256), C.c_void_p(256), C.c_void_p(256), 1, 8,
                 C.c_void_p(512), C.c_void_p(1024), 16, None)
    assert e.value.status == "LSQ_ERR_WORKSPACE"


def test_bench_kernel_family_mapping_and_profile_records():
    """bench.py's attribution of rocprofv3 kernel names to the library's
    families (exact identifiers: "ce_kernel" must not catch
    splitk_reduce_kernel, and the first template argument splits the
    register-path GEMMs by weight kind), and the committed per-family traffic
    records are current for the sources they name."""
    import bench
    cases = {
        "void lsq::(anonymous namespace)::gemm_fwd_nf4_dma_kernel<0, 256>(lsq::FwdParams)": "gemm_fwd_nf4_lora",
        "void lsq::(anonymous namespace)::gemm_fwd_pp_kernel<1, 2>(lsq::FwdParams)": "gemm_bf16_weights",
        "void lsq::(anonymous namespace)::gemm_fwd_pp_kernel<0, 2>(lsq::FwdParams)": "gemm_fwd_nf4_lora",
        "void lsq::(anonymous namespace)::splitk_reduce_kernel<1>(float const*, int, int, int)": "other",
        "lsq::(anonymous namespace)::ce_kernel(float const*, int const*, int, int)": "elementwise",
        "void lsq::(anonymous namespace)::attn_prep_bwd_kernel<128>(float const*, long)": "attention",
        "lsq::(anonymous namespace)::lora_grads_kernel(lsq::(anonymous namespace)::GradsArgs)": "lora_skinny",
        "Cijk_Ailk_Bljk_BBS_BH_Bias_HA_S_SAV_UserArgs_MT256x256x64_MI16x16x1_SN": None,
        "__amd_rocclr_copyBuffer": None,
    }
    for name, fam in cases.items():
        assert bench.family_of(name) == fam, name
    # the dominant family's committed counters were taken on the current source
    rec = bench.profile_record("gemm_fwd_nf4_lora", "llama8b-stack")
    assert rec is not None and rec["source"].endswith("gemm.hip")
    assert rec["traffic_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"] > 0
