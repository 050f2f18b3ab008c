"""Pre-norm decoder layer, forward and hand-derived backward (oracle; test infrastructure).

What the pages fix: the streamed layer is the unmodified decoder layer of the
model family running over substituted weight bytes, and the model classes are
transformers' own (LS-docs "How it works").  Each layer is read twice per step
because the backward recomputes it (LS-docs "How it works"); recomputation
does not change the mathematics, so this oracle simply computes the forward
again inside the backward.

Readings of transformers' Llama / Qwen2 decoder layer (the pages print none of it):

* RMSNorm: y = w * x / sqrt(mean(x^2) + eps).
* Rotary embedding, rotate-half form, on head_dim d: for i < d/2 the pair
  (x[i], x[i + d/2]) is rotated by angle pos * theta^(-2i/d); positions are
  0 .. S-1 within each sequence; no frequency rescaling.
* Causal softmax(Q K^T / sqrt(d)) V with grouped-query attention: query head
  h reads key/value head h // (n_heads / n_kv_heads).
* SwiGLU MLP: down(silu(gate(x)) * up(x)), silu(g) = g * sigmoid(g).
* Two pre-norm residual blocks; Qwen2 adds a frozen bias to q, k and v.
* Every projection is a LoRA linear (``oracle.lora``) with scale s.

All arrays are float64.  x has shape [B, S, H].
"""
import numpy as np

from . import lora

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


class LayerCfg:
    def __init__(self, hidden, n_heads, n_kv_heads, head_dim, intermediate,
                 eps, theta, qkv_bias=False):
        self.hidden = hidden
        self.n_heads = n_heads
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.intermediate = intermediate
        self.eps = eps
        self.theta = theta
        self.qkv_bias = qkv_bias

    def proj_shape(self, name):
        """(out, in) of each projection."""
        H, I = self.hidden, self.intermediate
        nq, nkv = self.n_heads * self.head_dim, self.n_kv_heads * self.head_dim
        return {"q": (nq, H), "k": (nkv, H), "v": (nkv, H), "o": (H, nq),
                "gate": (I, H), "up": (I, H), "down": (H, I)}[name]


# ---------------------------------------------------------------- RMSNorm
def rmsnorm(x, w, eps):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return w * x * r


def rmsnorm_bwd(x, w, eps, dy):
    n = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    wdy = w * dy
    return r * wdy - x * (r ** 3) * np.sum(wdy * x, axis=-1, keepdims=True) / n


# ---------------------------------------------------------------- rotary
def rope_tables(seq, head_dim, theta):
    inv = theta ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)                     # [S, d/2]


def rope(x, cos, sin):
    """x [B, S, heads, d] -> rotated, rotate-half pairing (i, i + d/2)."""
    h = x.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation."""
    h = dy.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    d1, d2 = dy[..., :h], dy[..., h:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


# ---------------------------------------------------------------- attention
def _probs(qh, kh, scale):
    S = qh.shape[0]
    sc = (qh @ kh.T) * scale
    sc = np.where(np.tril(np.ones((S, S), dtype=bool)), sc, -np.inf)
    sc = sc - sc.max(axis=-1, keepdims=True)
    p = np.exp(sc)
    return p / p.sum(axis=-1, keepdims=True)


def attention(q, k, v):
    """q [B,S,nh,d], k/v [B,S,nkv,d] -> o [B,S,nh,d]; causal, GQA."""
    B, S, nh, d = q.shape
    group = nh // k.shape[2]
    scale = 1.0 / np.sqrt(d)
    o = np.empty_like(q)
    for b in range(B):
        for h in range(nh):
            g = h // group
            o[b, :, h] = _probs(q[b, :, h], k[b, :, g], scale) @ v[b, :, g]
    return o


def attention_bwd(q, k, v, do):
    B, S, nh, d = q.shape
    group = nh // k.shape[2]
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(nh):
            g = h // group
            p = _probs(q[b, :, h], k[b, :, g], scale)
            dv[b, :, g] += p.T @ do[b, :, h]
            dp = do[b, :, h] @ v[b, :, g].T
            ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
            dq[b, :, h] = (ds @ k[b, :, g]) * scale
            dk[b, :, g] += (ds.T @ q[b, :, h]) * scale
    return dq, dk, dv


# ---------------------------------------------------------------- SwiGLU
def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def swiglu(g, u):
    return g * _sigmoid(g) * u


def swiglu_bwd(g, u, dm):
    sg = _sigmoid(g)
    dg = dm * u * sg * (1.0 + g * (1.0 - sg))
    du = dm * g * sg
    return dg, du


# ---------------------------------------------------------------- layer
def _lin(x2, W, ad, s, bias=None):
    A, B = ad
    return lora.linear_fwd(x2, W, A, B, s, bias)[0]


def layer_fwd(cfg, x, W, ad, s, cache=False):
    """x [B,S,H]; W: dict of base weights [out,in] plus 'norm1', 'norm2' (and
    'bq','bk','bv' when cfg.qkv_bias); ad: dict name -> (A [r,in], B [out,r])."""
    Bsz, S, H = x.shape
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    x2 = x.reshape(-1, H)
    xn1 = rmsnorm(x2, W["norm1"], cfg.eps)
    bias = (lambda n: W["b" + n]) if cfg.qkv_bias else (lambda n: None)
    q = _lin(xn1, W["q"], ad["q"], s, bias("q")).reshape(Bsz, S, nh, d)
    k = _lin(xn1, W["k"], ad["k"], s, bias("k")).reshape(Bsz, S, nkv, d)
    v = _lin(xn1, W["v"], ad["v"], s, bias("v")).reshape(Bsz, S, nkv, d)
    cos, sin = rope_tables(S, d, cfg.theta)
    qr, kr = rope(q, cos, sin), rope(k, cos, sin)
    a = attention(qr, kr, v).reshape(-1, nh * d)
    h = x2 + _lin(a, W["o"], ad["o"], s)
    xn2 = rmsnorm(h, W["norm2"], cfg.eps)
    g = _lin(xn2, W["gate"], ad["gate"], s)
    u = _lin(xn2, W["up"], ad["up"], s)
    m = swiglu(g, u)
    out = h + _lin(m, W["down"], ad["down"], s)
    out = out.reshape(Bsz, S, H)
    if not cache:
        return out
    return out, dict(x2=x2, xn1=xn1, qr=qr, kr=kr, v=v, a=a, h=h, xn2=xn2,
                     g=g, u=u, m=m, cos=cos, sin=sin)


def layer_bwd(cfg, x, W, ad, s, dout):
    """Recompute the forward from the saved input x, then backprop dout [B,S,H].

    Returns (dx [B,S,H], grads dict name -> (dA [r,in], dB [out,r]))."""
    Bsz, S, H = x.shape
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    _, c = layer_fwd(cfg, x, W, ad, s, cache=True)
    grads = {}
    dout2 = dout.reshape(-1, H)

    def lin_bwd(name, xin, dy):
        A, B = ad[name]
        dxin, dA, dB = lora.linear_bwd(xin, W[name], A, B, s, dy)
        grads[name] = (dA, dB)
        return dxin

    # MLP block: out = h + down(swiglu(gate(xn2), up(xn2)))
    dm = lin_bwd("down", c["m"], dout2)
    dg, du = swiglu_bwd(c["g"], c["u"], dm)
    dxn2 = lin_bwd("gate", c["xn2"], dg) + lin_bwd("up", c["xn2"], du)
    dh = dout2 + rmsnorm_bwd(c["h"], W["norm2"], cfg.eps, dxn2)
    # attention block: h = x + o(attn(rope(q), rope(k), v))
    da = lin_bwd("o", c["a"], dh).reshape(Bsz, S, nh, d)
    dqr, dkr, dv = attention_bwd(c["qr"], c["kr"], c["v"], da)
    dq = rope_bwd(dqr, c["cos"], c["sin"]).reshape(-1, nh * d)
    dk = rope_bwd(dkr, c["cos"], c["sin"]).reshape(-1, nkv * d)
    dxn1 = (lin_bwd("q", c["xn1"], dq) + lin_bwd("k", c["xn1"], dk)
            + lin_bwd("v", c["xn1"], dv.reshape(-1, nkv * d)))
    dx = dh + rmsnorm_bwd(c["x2"], W["norm1"], cfg.eps, dxn1)
    return dx.reshape(Bsz, S, H), grads
