"""Closed-form shard and store sizes (oracle; test infrastructure).

The pages print store and buffer sizes but not the layout that produces them:
a 3.60 GB pinned store over 32 layers and two 113 MB layer buffers for the 8B
(LS-docs intro, the pre-flight panel), 1.43 GB NF4 and 5.55 GB bf16 stores for
Qwen2.5-3B (LS-docs "Why NF4 also made the 3B row faster"), a 33.74 GB store
for 72B (LS-docs "Honest scope"), 2.10 GB for the untied 8B embedding and head,
and a 5.70 GB store once those moved into it (LS-docs "Why NF4 also made the
3B row faster"; "Disk space and the second cache").

Reading: those figures are reproduced exactly by a
layout with 4-bit codes, an 8-bit absmax per 64-element block and one float32
second-level scale per 256 blocks, bf16 norms and biases, in decimal GB (the
72B figure is in GiB).  This build stores a plain float32 absmax per block
instead, so its shards are about 9% larger; ``layer_bytes_fp32_absmax`` gives
that size before alignment padding.
"""


def layer_linear_params(hidden, n_heads, n_kv_heads, head_dim, intermediate):
    nq, nkv = n_heads * head_dim, n_kv_heads * head_dim
    return 2 * nq * hidden + 2 * nkv * hidden + 3 * intermediate * hidden


def layer_extra_params(hidden, n_heads, n_kv_heads, head_dim, qkv_bias):
    """Two RMSNorm weights and, for Qwen2, the q/k/v biases; all bf16 in the store."""
    bias = (n_heads + 2 * n_kv_heads) * head_dim if qkv_bias else 0
    return 2 * hidden + bias


def nf4_bytes_double_quant(n_params):
    """Pages' layout: 0.5 B code + 1 B absmax per 64 + 4 B per 256 blocks."""
    return n_params * 0.5 + n_params / 64 + 4 * n_params / (64 * 256)


def nf4_bytes_fp32_absmax(n_params):
    """This build's layout: 0.5 B code + one float32 absmax per 64 elements."""
    return n_params // 2 + 4 * (n_params // 64)


def layer_bytes_pages(shape, quant):
    lin = layer_linear_params(*shape[:5])
    extra = 2 * layer_extra_params(shape[0], shape[1], shape[2], shape[3], shape[5])
    body = nf4_bytes_double_quant(lin) if quant == "nf4" else 2 * lin
    return body + extra


def layer_bytes_fp32_absmax(shape):
    lin = layer_linear_params(*shape[:5])
    extra = 2 * layer_extra_params(shape[0], shape[1], shape[2], shape[3], shape[5])
    return nf4_bytes_fp32_absmax(lin) + extra


def embed_bytes(vocab, hidden):
    return 2 * vocab * hidden
