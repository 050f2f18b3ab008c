"""Thin driver over liblsq: device memory and streams from PyTorch, every
computation in the library.

Store      the per-layer shard store (pinned host arena), written once from
           seeded synthetic bf16 weights through nf4_quantize on the GPU.
Resident   embedding, final norm, head, adapters and adapter gradients.
Runner     a layer pool (streamed N slots, or resident) with its compute and
           copy streams and the step workspace; ``step`` is one lsq_train_step.
"""
import ctypes as C

import numpy as np
import torch

from . import lib, synth

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def _bits_to_dev(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def _ptr(t):
    return C.c_void_p(t.data_ptr())


class Store:
    """One layer blob per decoder layer in a host arena (pinned unless refused)."""

    def __init__(self, cfg, device="cuda", flags=0, layer_source=None, distinct_layers=None):
        """distinct_layers: when set, layer i takes the weights drawn for layer
        i mod distinct_layers (each blob is still quantized and written on its
        own), so a deep stack is built without drawing every layer on the host."""
        self.cfg = cfg
        self.ccfg = lib.model_cfg(cfg)
        h = C.c_void_p()
        lib.call("shard_store_create", C.byref(self.ccfg), flags, C.byref(h))
        self.handle = h
        self.layer_bytes = int(lib.raw("shard_store_layer_bytes")(h))
        self.pinned = bool(lib.raw("shard_store_is_pinned")(h))
        src = layer_source or (lambda i: synth.layer_weights(cfg, cfg.wid, i))
        stream = torch.cuda.current_stream(device)
        staging = torch.empty(self.layer_bytes + 256, dtype=torch.uint8, device=device)
        nd = min(distinct_layers, cfg.n_layers) if distinct_layers else cfg.n_layers
        drawn = {}
        for i in range(cfg.n_layers):
            d = i % nd
            w = drawn.get(d)
            if w is None:
                w = src(d)
                if nd < cfg.n_layers:
                    drawn[d] = w   # kept on the host: the device holds one layer's weights at a time
            dev = {k: _bits_to_dev(v, device) for k, v in w.items()}
            ls = lib.LayerSrc()
            for j, name in enumerate(PROJ):
                ls.w[j] = dev[name].data_ptr()
            ls.norm1 = dev["norm1"].data_ptr()
            ls.norm2 = dev["norm2"].data_ptr()
            if cfg.qkv_bias:
                for j, name in enumerate(("bq", "bk", "bv")):
                    ls.bias[j] = dev[name].data_ptr()
            lib.call("shard_store_write_layer", h, i, C.byref(ls), _ptr(staging), staging.numel(),
                     lib.stream_handle(stream))
            del dev
        del staging, drawn

    @classmethod
    def load(cls, cfg, path, flags=0):
        """A store read back from shard_store_save's file (refused if its shape differs from cfg)."""
        self = cls.__new__(cls)
        self.cfg = cfg
        self.ccfg = lib.model_cfg(cfg)
        h = C.c_void_p()
        lib.call("shard_store_load", str(path).encode(), C.byref(self.ccfg), flags, C.byref(h))
        self.handle = h
        self.layer_bytes = int(lib.raw("shard_store_layer_bytes")(h))
        self.pinned = bool(lib.raw("shard_store_is_pinned")(h))
        return self

    @classmethod
    def blank(cls, cfg, flags=0):
        """A store of the right shape whose blobs are all zero bytes (weights of
        zero): a step over it allocates and launches exactly what a step over
        real weights does, without the cost of drawing and quantizing them."""
        self = cls.__new__(cls)
        self.cfg = cfg
        self.ccfg = lib.model_cfg(cfg)
        h = C.c_void_p()
        lib.call("shard_store_create", C.byref(self.ccfg), flags, C.byref(h))
        self.handle = h
        self.layer_bytes = int(lib.raw("shard_store_layer_bytes")(h))
        self.pinned = bool(lib.raw("shard_store_is_pinned")(h))
        for i in range(cfg.n_layers):
            C.memset(lib.raw("shard_store_layer_host")(h, i), 0, self.layer_bytes)
        return self

    @classmethod
    def copy_of(cls, other, flags):
        """Another arena (e.g. pageable) holding the same blobs, byte for byte."""
        self = cls.__new__(cls)
        self.cfg = other.cfg
        self.ccfg = lib.model_cfg(other.cfg)
        h = C.c_void_p()
        lib.call("shard_store_create", C.byref(self.ccfg), flags, C.byref(h))
        self.handle = h
        self.layer_bytes = int(lib.raw("shard_store_layer_bytes")(h))
        self.pinned = bool(lib.raw("shard_store_is_pinned")(h))
        for i in range(self.cfg.n_layers):
            C.memmove(lib.raw("shard_store_layer_host")(h, i), lib.raw("shard_store_layer_host")(other.handle, i),
                      self.layer_bytes)
        return self

    def save(self, path):
        lib.call("shard_store_save", self.handle, str(path).encode())

    def host_blob(self, i):
        p = lib.raw("shard_store_layer_host")(self.handle, i)
        return np.ctypeslib.as_array((C.c_uint8 * self.layer_bytes).from_address(p))

    def close(self):
        if self.handle:
            lib.raw("shard_store_destroy")(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lora_arena_host(cfg, layers=None):
    """Host bf16 bits of every layer's adapters in the library's stacked layout."""
    L = lib.lora_layout(cfg)
    n = cfg.n_layers if layers is None else layers
    arena = np.zeros((n, L.layer_elems), dtype=np.uint16)
    for i in range(n):
        ad = synth.layer_lora(cfg, cfg.wid, i)
        groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
        for g, names in enumerate(groups):
            A = np.concatenate([ad[nm][0] for nm in names], axis=0)
            B = np.concatenate([ad[nm][1] for nm in names], axis=0)
            arena[i, L.a_off[g]:L.a_off[g] + A.size] = A.ravel()
            arena[i, L.b_off[g]:L.b_off[g] + B.size] = B.ravel()
    return arena


def split_lora_grads(cfg, grad_layer):
    """float32 gradient block of one layer -> name -> (dA [r, in], dB [out, r])."""
    L = lib.lora_layout(cfg)
    r = cfg.lora_r
    out = {}
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    for g, names in enumerate(groups):
        ao, bo = L.a_off[g], L.b_off[g]
        for nm in names:
            n_out, n_in = cfg.proj_shape(nm)
            dA = grad_layer[ao:ao + r * n_in].reshape(r, n_in)
            dB = grad_layer[bo:bo + n_out * r].reshape(n_out, r)
            out[nm] = (dA, dB)
            ao += r * n_in
            bo += n_out * r
    return out


class Resident:
    """Embedding, final norm, head, adapters.  large_in_host: the untied
    embedding and head stay in page-locked host memory instead (large-layer
    streaming: the step reads the batch's embedding rows in place and copies
    the head in once per step)."""

    def __init__(self, cfg, device="cuda", large_in_host=False, blank=False):
        self.cfg = cfg
        self.large_in_host = large_in_host
        if blank:   # zeros of the same shapes (memory and launch tests)
            z = (lambda *shape: torch.zeros(shape, dtype=torch.int16, device=device))
            self.embed = z(cfg.vocab, cfg.hidden)
            self.head = self.embed if cfg.tied else z(cfg.vocab, cfg.hidden)
            self.final_norm = z(cfg.hidden)
            self.lora = z(cfg.n_layers, lib.lora_layout(cfg).layer_elems)
            self.layer_elems = self.lora.shape[1]
            return
        rw = synth.resident_weights(cfg, cfg.wid)
        if large_in_host:
            assert not cfg.tied, "a tied embedding stays resident"
            host = (lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).pin_memory())
            self.embed = host(rw["embed"])
            self.head = host(rw["head"])
        else:
            self.embed = _bits_to_dev(rw["embed"], device)
            self.head = self.embed if cfg.tied else _bits_to_dev(rw["head"], device)
        self.final_norm = _bits_to_dev(rw["final_norm"], device)
        self.lora = _bits_to_dev(lora_arena_host(cfg), device)
        self.layer_elems = self.lora.shape[1]

    def new_grads(self):
        return torch.zeros(self.lora.shape, dtype=torch.float32, device=self.lora.device)

    def struct(self, grads):
        return lib.Resident(self.embed.data_ptr(), self.head.data_ptr(), self.final_norm.data_ptr(),
                            self.lora.data_ptr(), grads.data_ptr() if grads is not None else None)


class Runner:
    """A pool over a store plus the step workspace.  mode: 'streamed' or 'resident'."""

    def __init__(self, cfg, store, resident, mode="streamed", n_buffers=None, pool_flags=0, device="cuda",
                 keep_activations=False, reference=False, recompute_all=False, copy_on_compute=False):
        """copy_on_compute: hand the pool the compute stream as its copy stream
        (the pool must then copy on a stream of its own)."""
        self.cfg, self.store, self.res = cfg, store, resident
        self.step_flags = (lib.LSQ_STEP_KEEP_ACTIVATIONS if keep_activations else 0) | \
                          (lib.LSQ_STEP_RECOMPUTE_ALL if recompute_all else 0) | \
                          (lib.LSQ_STEP_STREAM_LARGE if resident.large_in_host else 0)
        # the workspace is sized for the reference forward when it may be asked for
        ws_flags = self.step_flags | (lib.LSQ_STEP_REFERENCE_FORWARD if reference else 0)
        self.ccfg = lib.model_cfg(cfg)
        self.compute = torch.cuda.Stream(device)
        self.copy = torch.cuda.Stream(device)
        stride = (store.layer_bytes + 4095) // 4096 * 4096
        n = cfg.n_layers if mode == "resident" else (n_buffers or cfg.n_buffers)
        flags = pool_flags | (lib.LSQ_POOL_RESIDENT if mode == "resident" else 0)
        self.slots = torch.empty(n * stride, dtype=torch.uint8, device=device)
        h = C.c_void_p()
        lib.call("layer_pool_create", store.handle, n, _ptr(self.slots), stride, lib.stream_handle(self.compute),
                 lib.stream_handle(self.compute if copy_on_compute else self.copy), flags, C.byref(h))
        self.pool = h
        self.n_buffers = n
        self.ws_bytes = int(lib.raw("lsq_step_workspace_size")(C.byref(self.ccfg), cfg.batch, cfg.seq, ws_flags))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.grads = resident.new_grads()

    def step(self, ids, forward_only=False, early_release=False, logits=None, x_trace=None, dx_trace=None,
             ref_nll_rows=None, ref_loss=None):
        """One lsq_train_step.  ref_nll_rows / ref_loss (float32 device tensors)
        ask for the adapters-off reference forward as well."""
        reference = ref_nll_rows is not None or ref_loss is not None
        flags = (lib.LSQ_STEP_FORWARD_ONLY if forward_only else 0) | \
                (lib.LSQ_STEP_DEBUG_EARLY_RELEASE if early_release else 0) | self.step_flags | \
                (lib.LSQ_STEP_REFERENCE_FORWARD if reference else 0)
        self.compute.wait_stream(torch.cuda.current_stream())
        rs = self.res.struct(self.grads)
        opt = (lambda t: _ptr(t) if t is not None else None)
        if reference:
            ex = lib.StepExtra(opt(x_trace), opt(dx_trace), opt(ref_nll_rows), opt(ref_loss))
            lib.call("lsq_train_step_ex", C.byref(self.ccfg), self.pool, C.byref(rs), _ptr(ids), self.cfg.batch,
                     self.cfg.seq, _ptr(self.loss), opt(logits), flags, _ptr(self.ws), self.ws_bytes, C.byref(ex))
        elif x_trace is None and dx_trace is None:
            lib.call("lsq_train_step", C.byref(self.ccfg), self.pool, C.byref(rs), _ptr(ids), self.cfg.batch,
                     self.cfg.seq, _ptr(self.loss), opt(logits), flags, _ptr(self.ws), self.ws_bytes)
        else:
            lib.call("lsq_train_step_traced", C.byref(self.ccfg), self.pool, C.byref(rs), _ptr(ids), self.cfg.batch,
                     self.cfg.seq, _ptr(self.loss), opt(logits), flags, _ptr(self.ws), self.ws_bytes,
                     opt(x_trace), opt(dx_trace))
        torch.cuda.current_stream().wait_stream(self.compute)
        return self.loss

    def copy_stream_handle(self):
        """The stream the pool copies layers on (an int handle)."""
        sp = C.c_void_p()
        lib.call("layer_pool_copy_stream", self.pool, C.byref(sp))
        return sp.value or 0

    def stats(self, reset=False):
        st = lib.PoolStats()
        lib.call("layer_pool_stats", self.pool, int(reset), C.byref(st))
        return st

    def timeline(self, capacity):
        """Start recording copy/compute intervals (capacity records; 0 stops)."""
        lib.call("lsq_timeline_enable", self.pool, int(capacity))
        self._tl_cap = int(capacity)

    def read_timeline(self):
        """[(kind, layer, start_ms, end_ms)] since the last read, and the dropped count."""
        cap = getattr(self, "_tl_cap", 0)
        buf = (lib.TimelineEntry * max(1, cap))()
        n, dropped = C.c_int32(), C.c_int32()
        lib.call("lsq_timeline_read", self.pool, buf, cap, C.byref(n), C.byref(dropped))
        return [(e.kind, e.layer, e.start_ms, e.end_ms) for e in buf[:n.value]], dropped.value

    def close(self):
        if self.pool:
            torch.cuda.synchronize()
            lib.raw("layer_pool_destroy")(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
