"""ctypes binding of liblsq.so (declared in include/lsq.h).

Argument marshalling only: every function forwards to the C ABI of the same
name and raises LsqError on a non-zero status.  There is no fallback: if the
library is missing, ``load()`` raises.
"""
import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsq.so")

LSQ_BF16, LSQ_F32 = 0, 1
LSQ_W_NF4, LSQ_W_BF16 = 0, 1
LSQ_STORE_ALLOW_PAGEABLE, LSQ_STORE_FORCE_PAGEABLE, LSQ_STORE_FAIL_PIN = 1, 2, 4
LSQ_POOL_RESIDENT, LSQ_POOL_POISON = 1, 2
LSQ_STEP_FORWARD_ONLY, LSQ_STEP_DEBUG_EARLY_RELEASE, LSQ_STEP_KEEP_ACTIVATIONS, LSQ_STEP_REFERENCE_FORWARD = 1, 2, 4, 8
LSQ_STEP_STREAM_LARGE, LSQ_STEP_RECOMPUTE_ALL = 16, 32
LSQ_TL_COPY, LSQ_TL_FWD, LSQ_TL_BWD, LSQ_TL_HEAD, LSQ_TL_LARGE_COPY = 0, 1, 2, 3, 4
LSQ_NOALLOC_SCRATCH_BYTES = 128 << 20

STATUS = {0: "LSQ_OK", -1: "LSQ_ERR_INVALID", -2: "LSQ_ERR_SHAPE", -3: "LSQ_ERR_ALIGN", -4: "LSQ_ERR_NONFINITE",
          -5: "LSQ_ERR_OOM", -6: "LSQ_ERR_HIP", -7: "LSQ_ERR_STATE", -8: "LSQ_ERR_REFUSED", -9: "LSQ_ERR_WORKSPACE",
          -10: "LSQ_ERR_IO"}


class LsqError(RuntimeError):
    def __init__(self, code, fn, msg):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class Weight(C.Structure):
    _fields_ = [("kind", C.c_int32), ("reserved", C.c_int32), ("data", C.c_void_p),
                ("absmax", C.c_void_p), ("n_out", C.c_int64), ("n_in", C.c_int64)]


class ModelCfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("vocab", C.c_int32),
                ("n_layers", C.c_int32), ("qkv_bias", C.c_int32), ("tied", C.c_int32),
                ("weight_kind", C.c_int32), ("lora_r", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("lora_scale", C.c_float), ("loss_chunk", C.c_int32)]


class BlobLayout(C.Structure):
    _fields_ = [("total_bytes", C.c_uint64), ("w_off", C.c_uint64 * 4), ("absmax_off", C.c_uint64 * 4),
                ("norm1_off", C.c_uint64), ("norm2_off", C.c_uint64), ("bias_off", C.c_uint64)]


class LoraLayout(C.Structure):
    _fields_ = [("a_off", C.c_uint64 * 4), ("b_off", C.c_uint64 * 4), ("layer_elems", C.c_uint64)]


class LayerSrc(C.Structure):
    _fields_ = [("w", C.c_void_p * 7), ("norm1", C.c_void_p), ("norm2", C.c_void_p), ("bias", C.c_void_p * 3)]


class PoolStats(C.Structure):
    _fields_ = [("copies", C.c_uint64), ("copy_bytes", C.c_uint64), ("hits", C.c_uint64), ("copy_ms", C.c_double),
                ("large_copies", C.c_uint64), ("large_bytes", C.c_uint64),
                ("timed_copies", C.c_uint64), ("timed_bytes", C.c_uint64)]


class TimelineEntry(C.Structure):
    _fields_ = [("kind", C.c_int32), ("layer", C.c_int32), ("start_ms", C.c_double), ("end_ms", C.c_double)]


class Resident(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("head", C.c_void_p), ("final_norm", C.c_void_p),
                ("lora", C.c_void_p), ("lora_grad", C.c_void_p)]


class StepExtra(C.Structure):
    _fields_ = [("x_trace", C.c_void_p), ("dx_trace", C.c_void_p), ("ref_nll_rows", C.c_void_p),
                ("ref_loss", C.c_void_p)]


class VramBreakdown(C.Structure):
    _fields_ = [("slots", C.c_uint64), ("resident", C.c_uint64), ("adapters", C.c_uint64),
                ("checkpoints", C.c_uint64), ("saved_activations", C.c_uint64), ("step_workspace", C.c_uint64),
                ("caller", C.c_uint64), ("margin", C.c_uint64), ("total", C.c_uint64)]


class ProfEntry(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_uint64), ("ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double)]


_P = C.c_void_p
_I32, _I64, _U64, _F, _SZ = C.c_int32, C.c_int64, C.c_uint64, C.c_float, C.c_size_t
_SIGS = {
    "lsq_last_error": (C.c_char_p, []),
    "lsq_version": (_I32, []),
    "lsq_nf4_codebook": (None, [_P]),
    "nf4_quantize": (C.c_int, [_P, _I32, _I64, _I64, _I32, _P, _P, _P, _P]),
    "nf4_dequantize": (C.c_int, [_P, _P, _I64, _I64, _I32, _P, _P]),
    "nf4_lora_linear_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32]),
    "nf4_lora_linear_fwd": (C.c_int, [C.POINTER(Weight), _P, _P, _I64, _P, _P, _I32, _F, _I32, _P, _P, _P, _SZ, _P]),
    "nf4_lora_linear_bwd": (C.c_int, [C.POINTER(Weight), _P, _P, _I64, _P, _P, _I32, _F, _I32, _P, _P, _P, _P, _I32,
                                      _P, _SZ, _P]),
    "nf4_lora_linear_bwd_noalloc": (C.c_int, [C.POINTER(Weight), _P, _P, _I64, _P, _P, _I32, _F, _I32, _P, _P, _P,
                                              _P, _I32, _P]),
    "lsq_blob_layout_get": (C.c_int, [C.POINTER(ModelCfg), C.POINTER(BlobLayout)]),
    "lsq_lora_layout_get": (C.c_int, [C.POINTER(ModelCfg), C.POINTER(LoraLayout)]),
    "decoder_layer_workspace_size": (_SZ, [C.POINTER(ModelCfg), _I32, _I32]),
    "decoder_layer_fwd": (C.c_int, [C.POINTER(ModelCfg), _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "decoder_layer_bwd": (C.c_int, [C.POINTER(ModelCfg), _P, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
    "shard_store_create": (C.c_int, [C.POINTER(ModelCfg), _I32, C.POINTER(_P)]),
    "shard_store_destroy": (None, [_P]),
    "shard_store_is_pinned": (_I32, [_P]),
    "shard_store_layer_bytes": (_U64, [_P]),
    "shard_store_layer_host": (_P, [_P, _I32]),
    "shard_store_write_layer": (C.c_int, [_P, _I32, C.POINTER(LayerSrc), _P, _SZ, _P]),
    "shard_store_save": (C.c_int, [_P, C.c_char_p]),
    "shard_store_load": (C.c_int, [C.c_char_p, C.POINTER(ModelCfg), _I32, C.POINTER(_P)]),
    "layer_pool_create": (C.c_int, [_P, _I32, _P, _U64, _P, _P, _I32, C.POINTER(_P)]),
    "layer_pool_destroy": (None, [_P]),
    "layer_pool_copy_stream": (C.c_int, [_P, C.POINTER(_P)]),
    "stream_layer_prefetch": (C.c_int, [_P, _I32]),
    "layer_pool_acquire": (C.c_int, [_P, _I32, C.POINTER(_P)]),
    "layer_pool_release": (C.c_int, [_P, _I32]),
    "layer_pool_stats": (C.c_int, [_P, _I32, C.POINTER(PoolStats)]),
    "lsq_timeline_enable": (C.c_int, [_P, _I32]),
    "lsq_timeline_read": (C.c_int, [_P, C.POINTER(TimelineEntry), _I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "lsq_step_workspace_size": (_SZ, [C.POINTER(ModelCfg), _I32, _I32, _I32]),
    "lsq_train_step": (C.c_int, [C.POINTER(ModelCfg), _P, C.POINTER(Resident), _P, _I32, _I32, _P, _P, _I32, _P,
                                 _SZ]),
    "lsq_train_step_ex": (C.c_int, [C.POINTER(ModelCfg), _P, C.POINTER(Resident), _P, _I32, _I32, _P, _P, _I32, _P,
                                    _SZ, C.POINTER(StepExtra)]),
    "lsq_train_step_traced": (C.c_int, [C.POINTER(ModelCfg), _P, C.POINTER(Resident), _P, _I32, _I32, _P, _P, _I32,
                                        _P, _SZ, _P, _P]),
    "vram_predict_peak": (C.c_int, [C.POINTER(ModelCfg), _I32, _I32, _I32, _I32, C.POINTER(VramBreakdown)]),
    "lsq_preflight": (C.c_int, [C.POINTER(ModelCfg), _I32, _I32, _I32, _I32, _U64, C.POINTER(VramBreakdown)]),
    "lsq_prof_enable": (C.c_int, [_I32]),
    "lsq_prof_read": (C.c_int, [C.POINTER(ProfEntry), _I32, C.POINTER(_I32)]),
}

_lib = None


def load():
    """Load liblsq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m layer_streamed_qlora_nf4_amd.build`")
    lib = C.CDLL(LIB_PATH)
    missing = []
    for name, (res, args) in _SIGS.items():
        try:
            f = getattr(lib, name)
        except AttributeError:
            missing.append(name)
            continue
        f.restype = res
        f.argtypes = args
    lib.missing_symbols = missing
    _lib = lib
    return lib


def exported_symbols():
    return list(_SIGS)


def _call(name, *args):
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise LsqError(rc, name, lib.lsq_last_error().decode(errors="replace"))
    return rc


def call(name, *args):
    """Call a status-returning entry point; raise LsqError on failure."""
    return _call(name, *args)


def raw(name):
    """The bare ctypes function (for size queries and getters)."""
    return getattr(load(), name)


# ------------------------------------------------------------------ small helpers
def model_cfg(cfg):
    """configs.ModelCfg -> ctypes ModelCfg."""
    return ModelCfg(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.vocab,
                    cfg.n_layers, int(cfg.qkv_bias), int(cfg.tied),
                    LSQ_W_NF4 if cfg.quant == "nf4" else LSQ_W_BF16, cfg.lora_r, cfg.eps, cfg.theta,
                    cfg.lora_scale, cfg.loss_chunk)


def codebook():
    buf = (C.c_float * 16)()
    load().lsq_nf4_codebook(buf)
    return list(buf)


def blob_layout(cfg):
    out = BlobLayout()
    call("lsq_blob_layout_get", C.byref(model_cfg(cfg)), C.byref(out))
    return out


def lora_layout(cfg):
    out = LoraLayout()
    call("lsq_lora_layout_get", C.byref(model_cfg(cfg)), C.byref(out))
    return out


def stream_handle(stream):
    """torch.cuda.Stream -> void* for the C ABI."""
    return C.c_void_p(stream.cuda_stream)
