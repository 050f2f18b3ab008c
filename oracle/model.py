"""Decoder stack with a resident embedding and head, mean next-token CE (oracle; test infrastructure).

What the pages fix: the embedding, the final norm, an untied head and the
adapters are the only tensors that get device storage; the decoder layers are
streamed (LS-docs "How it works").  Nothing but the adapters trains: no grad
for the embedding, norms or head (LS-docs "Honest scope": a LoRA target on a
streamed head or embedding is refused).  The non-quantised tensors stay in the
store dtype (LS-docs "How it works", scope of the NF4 comparison).

Readings (the pages leave these open): the loss is the mean cross-entropy over the
B*(S-1) next-token positions of each sequence; a tied model uses the
embedding matrix as its head.

``layer_source(i)`` returns (W, ad) for decoder layer i as float64 arrays, so
that a store far larger than memory can be dequantized one layer at a time.
"""
import numpy as np

from . import layer as L


def embed(ids, table):
    return table[ids]


def ce_loss_and_grad(logits, ids):
    """logits [B,S,V] float64, ids [B,S] -> (mean loss, dlogits [B,S,V])."""
    Bsz, S, V = logits.shape
    z = logits[:, :-1]
    tgt = ids[:, 1:]
    zmax = z.max(axis=-1, keepdims=True)
    lse = zmax[..., 0] + np.log(np.sum(np.exp(z - zmax), axis=-1))
    picked = np.take_along_axis(z, tgt[..., None], axis=-1)[..., 0]
    count = Bsz * (S - 1)
    loss = float(np.sum(lse - picked) / count)
    p = np.exp(z - lse[..., None])
    np.put_along_axis(p, tgt[..., None], np.take_along_axis(p, tgt[..., None], axis=-1) - 1.0, axis=-1)
    dlogits = np.zeros_like(logits)
    dlogits[:, :-1] = p / count
    return loss, dlogits


def stack_fwd(cfg, ids, embed_table, layer_source, n_layers, final_norm, head, s,
              keep_inputs=False):
    """Forward to logits [B,S,V]; optionally return every layer's input."""
    x = embed(ids, embed_table)
    inputs = []
    for i in range(n_layers):
        if keep_inputs:
            inputs.append(x)
        W, ad = layer_source(i)
        x = L.layer_fwd(cfg, x, W, ad, s)
    xf = L.rmsnorm(x, final_norm, cfg.eps)
    logits = xf @ head.T
    return (logits, x, inputs) if keep_inputs else logits


def stack_fwd_bwd(cfg, ids, embed_table, layer_source, n_layers, final_norm, head, s):
    """One training step's maths: (loss, logits, grads[i][name] = (dA, dB))."""
    logits, x_last, inputs = stack_fwd(cfg, ids, embed_table, layer_source, n_layers,
                                       final_norm, head, s, keep_inputs=True)
    loss, dlogits = ce_loss_and_grad(logits, ids)
    dxf = dlogits @ head
    dx = L.rmsnorm_bwd(x_last, final_norm, cfg.eps, dxf)
    grads = [None] * n_layers
    for i in reversed(range(n_layers)):
        W, ad = layer_source(i)
        dx, grads[i] = L.layer_bwd(cfg, inputs[i], W, ad, s, dx)
    return loss, logits, grads
