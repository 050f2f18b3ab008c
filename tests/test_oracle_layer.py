"""Pins of the oracle's LoRA linear, decoder layer and stack.

Each pin is independent of the formula it checks: central finite differences
of the forward, an autograd run over a separately written torch float64
forward, torch's own attention routine, closed forms and invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as L
from oracle import lora, model

CFG = L.LayerCfg(hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, intermediate=48,
                 eps=1e-5, theta=1e4, qkv_bias=False)
CFG_B = L.LayerCfg(hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, intermediate=48,
                   eps=1e-6, theta=1e6, qkv_bias=True)
R, S_SCALE = 3, 1.7


def _layer_params(cfg, seed, r=R):
    g = np.random.default_rng(seed)
    W, ad = {}, {}
    for n in L.PROJ:
        o, i = cfg.proj_shape(n)
        W[n] = g.standard_normal((o, i)) * 0.2
        ad[n] = (g.standard_normal((r, i)) * 0.3, g.standard_normal((o, r)) * 0.3)
    W["norm1"] = 1 + 0.1 * g.standard_normal(cfg.hidden)
    W["norm2"] = 1 + 0.1 * g.standard_normal(cfg.hidden)
    if cfg.qkv_bias:
        for n in ("q", "k", "v"):
            W["b" + n] = 0.1 * g.standard_normal(cfg.proj_shape(n)[0])
    return W, ad


# ------------------------------------------------------------------ LoRA linear
def test_lora_linear_finite_differences():
    g = np.random.default_rng(0)
    X, W = g.standard_normal((4, 128)), g.standard_normal((64, 128)) * 0.1
    A, B = g.standard_normal((2, 128)) * 0.1, g.standard_normal((64, 2)) * 0.1
    dY = g.standard_normal((4, 64))
    dX, dA, dB = lora.linear_bwd(X, W, A, B, 2.0, dY)

    def f(X_, A_, B_):
        return float(np.sum(lora.linear_fwd(X_, W, A_, B_, 2.0)[0] * dY))

    eps = 1e-6
    for arr, grad, name in ((X, dX, "X"), (A, dA, "A"), (B, dB, "B")):
        it = np.random.default_rng(1).choice(arr.size, 12, replace=False)
        for flat in it:
            idx = np.unravel_index(flat, arr.shape)
            p, m = [a.copy() for a in (X, A, B)], [a.copy() for a in (X, A, B)]
            k = {"X": 0, "A": 1, "B": 2}[name]
            p[k][idx] += eps
            m[k][idx] -= eps
            num = (f(*p) - f(*m)) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(num))


def test_lora_linear_special_cases_and_merged_weight():
    g = np.random.default_rng(2)
    X, W = g.standard_normal((5, 64)), g.standard_normal((48, 64))
    A, B = g.standard_normal((4, 64)), g.standard_normal((48, 4))
    dY = g.standard_normal((5, 48))
    # s = 0: plain linear
    assert np.allclose(lora.linear_fwd(X, W, A, B, 0.0)[0], X @ W.T)
    # A = 0 -> dB = 0 ; B = 0 -> dA = 0
    assert np.all(lora.linear_bwd(X, W, np.zeros_like(A), B, 2.0, dY)[2] == 0)
    assert np.all(lora.linear_bwd(X, W, A, np.zeros_like(B), 2.0, dY)[1] == 0)
    # LoRA == a plain linear over the merged weight W + s B A, forward and dX
    Wm = W + 1.5 * B @ A
    assert np.allclose(lora.linear_fwd(X, W, A, B, 1.5)[0], X @ Wm.T)
    assert np.allclose(lora.linear_bwd(X, W, A, B, 1.5, dY)[0], dY @ Wm)


# ------------------------------------------------------------------ pieces
def test_rmsnorm_unit_rms_and_bwd_fd():
    g = np.random.default_rng(3)
    x = g.standard_normal((6, 32)) * 3
    y = L.rmsnorm(x, np.ones(32), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), 1.0)
    w, dy = 1 + g.standard_normal(32) * 0.1, g.standard_normal((6, 32))
    dx = L.rmsnorm_bwd(x, w, 1e-5, dy)
    eps = 1e-6
    for idx in [(0, 0), (3, 17), (5, 31)]:
        p, m = x.copy(), x.copy()
        p[idx] += eps
        m[idx] -= eps
        num = (np.sum(L.rmsnorm(p, w, 1e-5) * dy) - np.sum(L.rmsnorm(m, w, 1e-5) * dy)) / (2 * eps)
        assert abs(num - dx[idx]) < 1e-7


def test_rope_identity_at_zero_norm_preserving_and_relative():
    g = np.random.default_rng(4)
    d, S = 16, 12
    cos, sin = L.rope_tables(S, d, 1e4)
    x = g.standard_normal((1, S, 2, d))
    y = L.rope(x, cos, sin)
    assert np.allclose(y[:, 0], x[:, 0])
    # each (i, i + d/2) pair keeps its length
    assert np.allclose(y[..., :8] ** 2 + y[..., 8:] ** 2, x[..., :8] ** 2 + x[..., 8:] ** 2)
    # the score of a rotated query at m with a rotated key at n depends on m - n only
    q, k = g.standard_normal(d), g.standard_normal(d)
    Q = L.rope(np.broadcast_to(q, (1, S, 1, d)).copy(), cos, sin)[0, :, 0]
    K = L.rope(np.broadcast_to(k, (1, S, 1, d)).copy(), cos, sin)[0, :, 0]
    assert np.isclose(Q[7] @ K[3], Q[5] @ K[1]) and np.isclose(Q[9] @ K[9], q @ k)
    # the backward is the transpose of the (linear) rotation
    dy = g.standard_normal(y.shape)
    assert np.isclose(np.sum(y * dy), np.sum(x * L.rope_bwd(dy, cos, sin)))


def test_attention_matches_torch_sdpa_with_gqa():
    g = np.random.default_rng(5)
    B, S, nh, nkv, d = 2, 9, 4, 2, 8
    q, k, v = g.standard_normal((B, S, nh, d)), g.standard_normal((B, S, nkv, d)), g.standard_normal((B, S, nkv, d))
    o = L.attention(q, k, v)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(nh // nkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(nh // nkv, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_causality():
    g = np.random.default_rng(6)
    q, k, v = (g.standard_normal((1, 10, 2, 4)) for _ in range(3))
    o = L.attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, 6:] += 5.0
    v2[:, 6:] -= 3.0
    o2 = L.attention(q, k2, v2)
    assert np.allclose(o[:, :6], o2[:, :6]) and not np.allclose(o[:, 6:], o2[:, 6:])


def test_swiglu_bwd_fd():
    g = np.random.default_rng(7)
    gg, u, dm = g.standard_normal(20), g.standard_normal(20), g.standard_normal(20)
    dg, du = L.swiglu_bwd(gg, u, dm)
    eps = 1e-6
    assert np.allclose((L.swiglu(gg + eps, u) - L.swiglu(gg - eps, u)) / (2 * eps) * dm, dg, atol=1e-8)
    assert np.allclose((L.swiglu(gg, u + eps) - L.swiglu(gg, u - eps)) / (2 * eps) * dm, du, atol=1e-8)


# ------------------------------------------------------------------ layer
def _torch_layer(cfg, x, W, ad, s):
    """An independent float64 torch forward, differentiated by autograd."""
    Bsz, S, H = x.shape
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim

    def rms(t, w):
        return w * t * torch.rsqrt(t.pow(2).mean(-1, keepdim=True) + cfg.eps)

    def lin(t, n, bias=None):
        A, Bm = ad[n]
        y = t @ W[n].T + s * (t @ A.T) @ Bm.T
        return y if bias is None else y + bias

    def rot(t):
        inv = 1.0 / (cfg.theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
        ang = torch.outer(torch.arange(S, dtype=torch.float64), inv)
        emb = torch.cat([ang, ang], -1)
        c, sn = emb.cos()[None, :, None], emb.sin()[None, :, None]
        t1, t2 = t[..., : d // 2], t[..., d // 2:]
        return t * c + torch.cat([-t2, t1], -1) * sn

    b = (lambda n: W["b" + n]) if cfg.qkv_bias else (lambda n: None)
    xn = rms(x, W["norm1"])
    q = rot(lin(xn, "q", b("q")).view(Bsz, S, nh, d)).transpose(1, 2)
    k = rot(lin(xn, "k", b("k")).view(Bsz, S, nkv, d)).transpose(1, 2)
    v = lin(xn, "v", b("v")).view(Bsz, S, nkv, d).transpose(1, 2)
    k = k.repeat_interleave(nh // nkv, 1)
    v = v.repeat_interleave(nh // nkv, 1)
    a = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(1, 2).reshape(Bsz, S, nh * d)
    h = x + lin(a, "o")
    xn2 = rms(h, W["norm2"])
    m = F.silu(lin(xn2, "gate")) * lin(xn2, "up")
    return h + lin(m, "down")


@pytest.mark.parametrize("cfg", [CFG, CFG_B])
def test_layer_backward_matches_autograd(cfg):
    Wn, adn = _layer_params(cfg, 10)
    g = np.random.default_rng(11)
    x = g.standard_normal((2, 7, cfg.hidden))
    dout = g.standard_normal((2, 7, cfg.hidden))
    out = L.layer_fwd(cfg, x, Wn, adn, S_SCALE)
    dx, grads = L.layer_bwd(cfg, x, Wn, adn, S_SCALE, dout)

    W = {k: torch.from_numpy(v) for k, v in Wn.items()}
    ad = {k: (torch.from_numpy(a).requires_grad_(), torch.from_numpy(b).requires_grad_())
          for k, (a, b) in adn.items()}
    tx = torch.from_numpy(x).requires_grad_()
    tout = _torch_layer(cfg, tx, W, ad, S_SCALE)
    assert np.allclose(out, tout.detach().numpy(), atol=1e-10)
    (tout * torch.from_numpy(dout)).sum().backward()
    assert np.allclose(dx, tx.grad.numpy(), atol=1e-10)
    for n in L.PROJ:
        assert np.allclose(grads[n][0], ad[n][0].grad.numpy(), atol=1e-10), n
        assert np.allclose(grads[n][1], ad[n][1].grad.numpy(), atol=1e-10), n


def test_layer_backward_finite_differences():
    Wn, adn = _layer_params(CFG, 12)
    g = np.random.default_rng(13)
    x = g.standard_normal((1, 6, CFG.hidden))
    dout = g.standard_normal((1, 6, CFG.hidden))
    dx, grads = L.layer_bwd(CFG, x, Wn, adn, S_SCALE, dout)

    def f(x_, ad_):
        return float(np.sum(L.layer_fwd(CFG, x_, Wn, ad_, S_SCALE) * dout))

    eps = 1e-6
    for idx in [(0, 0, 0), (0, 3, 17), (0, 5, 31)]:
        p, m = x.copy(), x.copy()
        p[idx] += eps
        m[idx] -= eps
        num = (f(p, adn) - f(m, adn)) / (2 * eps)
        assert abs(num - dx[idx]) < 1e-6 * max(1, abs(num))
    for n in L.PROJ:
        for which in (0, 1):
            arr = adn[n][which]
            idx = tuple(int(i) for i in np.unravel_index(7 % arr.size, arr.shape))
            pa = {k: (a.copy(), b.copy()) for k, (a, b) in adn.items()}
            ma = {k: (a.copy(), b.copy()) for k, (a, b) in adn.items()}
            pa[n][which][idx] += eps
            ma[n][which][idx] -= eps
            num = (f(x, pa) - f(x, ma)) / (2 * eps)
            assert abs(num - grads[n][which][idx]) < 1e-6 * max(1, abs(num)), (n, which)


def test_layer_merged_lora_and_identity_special_cases():
    Wn, adn = _layer_params(CFG, 14)
    x = np.random.default_rng(15).standard_normal((1, 5, CFG.hidden))
    merged = dict(Wn)
    zero = {}
    for n in L.PROJ:
        A, B = adn[n]
        merged[n] = Wn[n] + S_SCALE * B @ A
        zero[n] = (np.zeros_like(A), np.zeros_like(B))
    assert np.allclose(L.layer_fwd(CFG, x, Wn, adn, S_SCALE), L.layer_fwd(CFG, x, merged, zero, S_SCALE))
    # with o and down zeroed and no adapters the layer is the identity
    ident = dict(Wn)
    ident["o"], ident["down"] = np.zeros_like(Wn["o"]), np.zeros_like(Wn["down"])
    assert np.allclose(L.layer_fwd(CFG, x, ident, zero, S_SCALE), x)


def test_single_token_sequences_give_q_and_k_no_gradient():
    """With one key the attention output is that key's value whatever the
    scores, so the loss does not depend on q or k: their adapter gradients are
    zero, while v, o and the MLP adapters still receive gradient (checked by
    finite differences on v)."""
    Wn, adn = _layer_params(CFG, 18)
    g = np.random.default_rng(19)
    x = g.standard_normal((3, 1, CFG.hidden))
    dout = g.standard_normal((3, 1, CFG.hidden))
    _, grads = L.layer_bwd(CFG, x, Wn, adn, S_SCALE, dout)
    for n in ("q", "k"):
        assert np.abs(grads[n][0]).max() <= 1e-12 and np.abs(grads[n][1]).max() <= 1e-12, n
    for n in ("v", "o", "gate", "up", "down"):
        assert np.abs(grads[n][0]).max() > 1e-3 and np.abs(grads[n][1]).max() > 1e-3, n

    def f(ad_):
        return float(np.sum(L.layer_fwd(CFG, x, Wn, ad_, S_SCALE) * dout))

    eps = 1e-6
    pa = {k: (a.copy(), b.copy()) for k, (a, b) in adn.items()}
    ma = {k: (a.copy(), b.copy()) for k, (a, b) in adn.items()}
    pa["v"][1][2, 1] += eps
    ma["v"][1][2, 1] -= eps
    num = (f(pa) - f(ma)) / (2 * eps)
    assert abs(num - grads["v"][1][2, 1]) < 1e-6 * max(1, abs(num))


def test_gqa_equals_repeated_kv_heads():
    Wn, adn = _layer_params(CFG, 16)
    x = np.random.default_rng(17).standard_normal((1, 6, CFG.hidden))
    zero = {n: (np.zeros_like(a), np.zeros_like(b)) for n, (a, b) in adn.items()}
    full = L.LayerCfg(hidden=32, n_heads=4, n_kv_heads=4, head_dim=8, intermediate=48, eps=1e-5, theta=1e4)
    Wf = dict(Wn)
    for n in ("k", "v"):
        Wf[n] = np.repeat(Wn[n].reshape(2, 8, 32), 2, axis=0).reshape(32, 32)
    zf = dict(zero)
    for n in ("k", "v"):
        zf[n] = (np.zeros((R, 32)), np.zeros((32, R)))
    assert np.allclose(L.layer_fwd(CFG, x, Wn, zero, S_SCALE), L.layer_fwd(full, x, Wf, zf, S_SCALE))


# ------------------------------------------------------------------ stack + CE
def test_ce_uniform_logits_is_log_vocab_and_grad_sums_to_zero():
    ids = np.array([[1, 2, 3, 4]])
    loss, d = model.ce_loss_and_grad(np.zeros((1, 4, 50)), ids)
    assert np.isclose(loss, np.log(50))
    assert np.allclose(d.sum(-1), 0) and np.all(d[:, -1] == 0)


def test_ce_matches_torch_cross_entropy():
    g = np.random.default_rng(18)
    logits, ids = g.standard_normal((2, 6, 30)) * 3, g.integers(0, 30, (2, 6))
    loss, d = model.ce_loss_and_grad(logits, ids)
    tl = torch.from_numpy(logits).requires_grad_()
    ref = F.cross_entropy(tl[:, :-1].reshape(-1, 30), torch.from_numpy(ids[:, 1:]).reshape(-1))
    ref.backward()
    assert np.isclose(loss, ref.item()) and np.allclose(d, tl.grad.numpy())


def _stack(cfg, n_layers, V, seed):
    g = np.random.default_rng(seed)
    layers = [_layer_params(cfg, seed + 1 + i) for i in range(n_layers)]
    emb = g.standard_normal((V, cfg.hidden)) * 0.5
    head = g.standard_normal((V, cfg.hidden)) * 0.3
    fn = 1 + 0.1 * g.standard_normal(cfg.hidden)
    return layers, emb, head, fn


def test_stack_grads_finite_differences_and_prefix_causality():
    V, n_layers = 40, 2
    layers, emb, head, fn = _stack(CFG, n_layers, V, 20)
    ids = np.random.default_rng(21).integers(0, V, (2, 6))
    loss, logits, grads = model.stack_fwd_bwd(CFG, ids, emb, lambda i: layers[i], n_layers, fn, head, S_SCALE)

    def f():
        lg = model.stack_fwd(CFG, ids, emb, lambda i: layers[i], n_layers, fn, head, S_SCALE)
        return model.ce_loss_and_grad(lg, ids)[0]

    assert np.isclose(f(), loss)
    eps = 1e-6
    for li in range(n_layers):
        for n in ("q", "v", "down", "gate"):
            for which in (0, 1):
                arr = layers[li][1][n][which]
                idx = tuple(int(i) for i in np.unravel_index(5 % arr.size, arr.shape))
                arr[idx] += eps
                lp = f()
                arr[idx] -= 2 * eps
                lm = f()
                arr[idx] += eps
                num = (lp - lm) / (2 * eps)
                assert abs(num - grads[li][n][which][idx]) < 1e-6 * max(1, abs(num)), (li, n, which)
    # logits of the first P positions depend on the first P tokens only
    ids2 = ids.copy()
    ids2[:, 4:] = (ids2[:, 4:] + 7) % V
    lg2 = model.stack_fwd(CFG, ids2, emb, lambda i: layers[i], n_layers, fn, head, S_SCALE)
    assert np.allclose(lg2[:, :4], logits[:, :4])
