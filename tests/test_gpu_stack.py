"""The streamed training step: oracle parity on small stacks, streamed ==
resident bit for bit (logits and every adapter gradient, counted n of n), and
the aliasing control that must break the gradients."""
import numpy as np
import pytest
import torch

from layer_streamed_qlora_nf4_amd import configs, lib, model, synth
from oracle import layer as olayer
from oracle import model as omodel
from tests.gpu_util import bits_f64, print_case, rel_err
from tests.test_gpu_layer import oracle_cfg, oracle_layer_params

pytestmark = pytest.mark.gpu
TOL = 1e-2


def ids_for(cfg):
    return synth.token_ids(cfg.batch, cfg.seq, cfg.vocab, (cfg.wid, 500, synth.TENSOR_IDS["ids"]))


def run(cfg, mode, store, res, ids, early=False, n_buffers=None):
    r = model.Runner(cfg, store, res, mode=mode, n_buffers=n_buffers)
    logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
    loss = r.step(ids, logits=logits, early_release=early).clone()
    torch.cuda.synchronize()
    out = dict(loss=loss.item(), logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy(), stats=r.stats())
    r.close()
    return out


def oracle_step(cfg, ids_np):
    rw = synth.resident_weights(cfg, cfg.wid)
    emb = bits_f64(rw["embed"])
    head = emb if cfg.tied else bits_f64(rw["head"])
    params = [oracle_layer_params(cfg, i) for i in range(cfg.n_layers)]
    return omodel.stack_fwd_bwd(oracle_cfg(cfg), ids_np.astype(np.int64), emb, lambda i: params[i], cfg.n_layers,
                                bits_f64(rw["final_norm"]), head, cfg.lora_scale)


def traced_step(cfg, store, res, ids, mode="streamed"):
    r = model.Runner(cfg, store, res, mode=mode)
    T, H, L = cfg.tokens, cfg.hidden, cfg.n_layers
    logits = torch.empty((T, cfg.vocab), dtype=torch.float32, device="cuda")
    xt = torch.empty((L + 1, T, H), dtype=torch.float32, device="cuda")
    dxt = torch.empty((L + 1, T, H), dtype=torch.float32, device="cuda")
    loss = r.step(ids, logits=logits, x_trace=xt, dx_trace=dxt).item()
    torch.cuda.synchronize()
    out = dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy(), x=xt.cpu().numpy(),
               dx=dxt.cpu().numpy())
    r.close()
    return out


def check_layers_against_oracle(cfg, got, layers, tol=TOL):
    """Each sampled layer recomputed by the oracle from the exact input and upstream
    gradient this run used (bf16 rounding does not compound across layers here)."""
    oc = oracle_cfg(cfg)
    B, S, H = cfg.batch, cfg.seq, cfg.hidden
    for i in layers:
        W, ad = oracle_layer_params(cfg, i)
        x = got["x"][i].astype(np.float64).reshape(B, S, H)
        out = olayer.layer_fwd(oc, x, W, ad, cfg.lora_scale)
        e = rel_err(got["x"][i + 1].reshape(B, S, H), out)
        assert e <= tol, f"layer {i} forward: {e:.3e}"
        dx, g_ref = olayer.layer_bwd(oc, x, W, ad, cfg.lora_scale, got["dx"][i + 1].astype(np.float64).reshape(B, S, H))
        e = rel_err(got["dx"][i].reshape(B, S, H), dx)
        assert e <= tol, f"layer {i} dx: {e:.3e}"
        g = model.split_lora_grads(cfg, got["grads"][i])
        for name in model.PROJ:
            for which in (0, 1):
                e = rel_err(g[name][which], g_ref[name][which])
                assert e <= tol, f"layer {i} {name} d{'AB'[which]}: {e:.3e}"


def check_head_against_oracle(cfg, got, ids_np, tol=TOL):
    rw = synth.resident_weights(cfg, cfg.wid)
    head = bits_f64(rw["embed"] if cfg.tied else rw["head"])
    fn = bits_f64(rw["final_norm"])
    B, S, H = cfg.batch, cfg.seq, cfg.hidden
    xL = got["x"][cfg.n_layers].astype(np.float64).reshape(B, S, H)
    logits = olayer.rmsnorm(xL, fn, cfg.eps) @ head.T
    assert rel_err(got["logits"].reshape(logits.shape), logits) <= tol
    loss, dlogits = omodel.ce_loss_and_grad(logits, ids_np.astype(np.int64))
    assert abs(got["loss"] - loss) <= tol * abs(loss)
    dxL = olayer.rmsnorm_bwd(xL, fn, cfg.eps, dlogits @ head)
    assert rel_err(got["dx"][cfg.n_layers].reshape(B, S, H), dxL) <= tol


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_QWEN])
def test_streamed_step_matches_oracle(gpu, cfg):
    print_case(test="stack_oracle", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids_np = ids_for(cfg)
    ids = torch.from_numpy(ids_np).cuda()
    got = traced_step(cfg, store, res, ids)
    # end to end: loss and logits against the oracle's own forward of the whole stack
    loss, logits, _ = oracle_step(cfg, ids_np)
    assert abs(got["loss"] - loss) <= TOL * abs(loss)
    assert rel_err(got["logits"].reshape(logits.shape), logits) <= TOL
    # the head and every layer, each from the exact inputs this step used
    check_head_against_oracle(cfg, got, ids_np)
    check_layers_against_oracle(cfg, got, range(cfg.n_layers))


def _compare_bitwise(cfg, a, b):
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32)), "logits differ"
    exact = total = 0
    for i in range(cfg.n_layers):
        ga = model.split_lora_grads(cfg, a["grads"][i])
        gb = model.split_lora_grads(cfg, b["grads"][i])
        for name in model.PROJ:
            for which in (0, 1):
                total += 1
                exact += int(np.array_equal(ga[name][which].view(np.uint32), gb[name][which].view(np.uint32)))
    return exact, total


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_QWEN, configs.TINY.with_(name="tiny-5L", n_layers=5,
                                                                                     n_buffers=3, wid=13)])
def test_streamed_equals_resident_and_control_breaks_it(gpu, cfg):
    print_case(test="streamed_vs_resident", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    streamed = run(cfg, "streamed", store, res, ids)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    print(f"streamed == resident: {exact} of {total} gradient tensors bit-identical, max|dlogit| = 0.0")
    assert exact == total == cfg.n_layers * 14
    # slot reuse: the last layers at the turn and the first at the next step are not re-copied
    assert streamed["stats"].copies == 2 * cfg.n_layers - min(cfg.n_buffers, cfg.n_layers)
    # the control: a slot refilled before its backward GEMMs must change the gradients
    bad = run(cfg, "streamed", store, res, ids, early=True)
    assert np.array_equal(bad["logits"].view(np.uint32), resident["logits"].view(np.uint32))
    exact_bad, _ = _compare_bitwise(cfg, resident, {**bad, "logits": resident["logits"], "loss": resident["loss"]})
    print(f"early-release control: {exact_bad} of {total} gradient tensors bit-identical")
    assert exact_bad < total


@pytest.mark.parametrize("n_layers", [1, 2])
def test_short_stacks_match_oracle_and_resident(gpu, n_layers):
    """Stacks no longer than the pool: every layer stays in a slot across the
    turn, one copy per layer on the first step, and the results still match
    the oracle and the resident run."""
    cfg = configs.TINY.with_(name=f"tiny-{n_layers}L", n_layers=n_layers, wid=20 + n_layers)
    print_case(test="short_stack", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids_np = ids_for(cfg)
    ids = torch.from_numpy(ids_np).cuda()
    got = traced_step(cfg, store, res, ids)
    loss, logits, _ = oracle_step(cfg, ids_np)
    assert abs(got["loss"] - loss) <= TOL * abs(loss)
    assert rel_err(got["logits"].reshape(logits.shape), logits) <= TOL
    check_head_against_oracle(cfg, got, ids_np)
    check_layers_against_oracle(cfg, got, range(cfg.n_layers))
    resident = run(cfg, "resident", store, res, ids)
    streamed = run(cfg, "streamed", store, res, ids)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    assert exact == total == cfg.n_layers * 14
    assert streamed["stats"].copies == 2 * cfg.n_layers - min(cfg.n_buffers, cfg.n_layers) == n_layers


def test_step_is_deterministic_and_repeats(gpu):
    cfg = configs.TINY
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    r = model.Runner(cfg, store, res)
    losses, grads = [], []
    for _ in range(3):
        losses.append(r.step(ids).item())
        grads.append(r.grads.cpu().numpy().copy())
    assert losses[0] == losses[1] == losses[2]
    assert np.array_equal(grads[0], grads[2])
    st = r.stats()
    # first step copies 2L - N, every later step 2L - 2N (layer 0.. N-1 stay in their slots)
    assert st.copies == (2 * cfg.n_layers - cfg.n_buffers) + 2 * (2 * cfg.n_layers - 2 * cfg.n_buffers)
    r.close()


def test_saved_store_reloads_and_streams_identically(gpu, tmp_path):
    """A store written to disk and read back streams the same bytes: same loss,
    logits and every adapter gradient, bit for bit."""
    cfg = configs.TINY.with_(name="tiny-saved", wid=17)
    print_case(test="store_save_load", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    path = tmp_path / "tiny.lsqstore"
    store.save(path)
    loaded = model.Store.load(cfg, path)
    assert loaded.pinned
    for i in range(cfg.n_layers):
        assert np.array_equal(store.host_blob(i), loaded.host_blob(i))
    a = run(cfg, "streamed", store, res, ids)
    b = run(cfg, "streamed", loaded, res, ids)
    exact, total = _compare_bitwise(cfg, a, b)
    assert exact == total
    loaded.close()
    store.close()


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY_QWEN])
def test_kept_activations_equal_recompute_bit_for_bit(gpu, cfg):
    """stream_recompute off: the backward reads the forward's kept activations
    instead of recomputing them.  Recompute is deterministic, so every policy
    (recompute all, the default that keeps layers L-1, 1 and 0, keep all) must
    give the same loss, logits and adapter gradients bit for bit, and all still
    re-read every layer's weights (same copy count)."""
    print_case(test="keep_vs_recompute", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    out = {}
    for mode in ("recompute_all", "default", "keep_all"):
        r = model.Runner(cfg, store, res, keep_activations=mode == "keep_all", recompute_all=mode == "recompute_all")
        logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
        loss = r.step(ids, logits=logits).item()
        torch.cuda.synchronize()
        out[mode] = dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy(), stats=r.stats())
        r.close()
    for mode in ("default", "keep_all"):
        exact, total = _compare_bitwise(cfg, out["recompute_all"], out[mode])
        assert exact == total == cfg.n_layers * 14, mode
        assert out[mode]["stats"].copies == out["recompute_all"]["stats"].copies == 2 * cfg.n_layers - cfg.n_buffers


def test_pageable_store_streams_the_same_bytes(gpu):
    """The pageable fallback only changes how the copies run (synchronously),
    never what they carry: gradients equal the pinned store's bit for bit."""
    cfg = configs.TINY.with_(name="tiny-pageable", wid=19)
    print_case(test="pageable_store", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    pstore = model.Store.copy_of(store, lib.LSQ_STORE_FORCE_PAGEABLE)
    assert store.pinned and not pstore.pinned
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    a = run(cfg, "streamed", store, res, ids)
    b = run(cfg, "streamed", pstore, res, ids)
    exact, total = _compare_bitwise(cfg, a, b)
    assert exact == total
    pstore.close()
    store.close()


def test_reference_forward_rides_the_same_stream(gpu):
    """The adapters-off reference forward (preference losses) runs on each layer
    while it is in its slot: the policy step is unchanged bit for bit, no extra
    layer copies are made, the reference loss equals a step whose adapters
    contribute nothing (B = 0), and its per-token NLL matches the oracle's
    adapters-off stack."""
    cfg = configs.TINY.with_(name="tiny-ref", wid=23)
    print_case(test="reference_forward", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids_np = ids_for(cfg)
    ids = torch.from_numpy(ids_np).cuda()
    base = run(cfg, "streamed", store, res, ids)
    r = model.Runner(cfg, store, res, reference=True)
    logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
    rows = torch.empty(cfg.tokens, dtype=torch.float32, device="cuda")
    rloss = torch.empty(1, dtype=torch.float32, device="cuda")
    loss = r.step(ids, logits=logits, ref_nll_rows=rows, ref_loss=rloss).item()
    torch.cuda.synchronize()
    withref = dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy(), stats=r.stats())
    r.close()
    exact, total = _compare_bitwise(cfg, base, withref)
    assert exact == total
    assert withref["stats"].copies == base["stats"].copies == 2 * cfg.n_layers - cfg.n_buffers
    # adapters contributing nothing: zero every B block
    zres = model.Resident(cfg)
    L = lib.lora_layout(cfg)
    for g in range(4):
        nb = sum(cfg.proj_shape(n)[0] for n in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))[g]) * cfg.lora_r
        zres.lora[:, L.b_off[g]:L.b_off[g] + nb] = 0
    zero = run(cfg, "streamed", store, zres, ids)
    assert rloss.item() == zero["loss"]
    # oracle: the stack with s = 0, per-row NLL
    rw = synth.resident_weights(cfg, cfg.wid)
    params = [oracle_layer_params(cfg, i) for i in range(cfg.n_layers)]
    ref_logits = omodel.stack_fwd(oracle_cfg(cfg), ids_np.astype(np.int64), bits_f64(rw["embed"]),
                                  lambda i: params[i], cfg.n_layers, bits_f64(rw["final_norm"]),
                                  bits_f64(rw["head"]), 0.0)
    B, S, V = cfg.batch, cfg.seq, cfg.vocab
    lg = ref_logits.reshape(B, S, V)
    lse = np.log(np.exp(lg - lg.max(-1, keepdims=True)).sum(-1)) + lg.max(-1)
    nll = np.zeros((B, S))
    tgt = ids_np.reshape(B, S)
    for b in range(B):
        for t in range(S - 1):
            nll[b, t] = lse[b, t] - lg[b, t, tgt[b, t + 1]]
    got = rows.cpu().numpy().reshape(B, S)
    assert rel_err(got, nll) <= TOL
    assert np.all(got[:, S - 1] == 0)
    assert abs(rloss.item() - nll[:, :S - 1].mean()) <= TOL * nll[:, :S - 1].mean()
    store.close()


def test_loss_chunk_matches_oracle_and_whole_batch(gpu):
    """stream_loss_chunk: the head and cross-entropy run chunk by chunk of tokens
    (48 + 48 + 48 + 16 here); rows are independent, so the loss, logits and
    every layer still match the oracle, and the whole-batch step to float32
    rounding of the head GEMM."""
    cfg = configs.TINY.with_(name="tiny-chunk", wid=29, loss_chunk=48)
    print_case(test="loss_chunk", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids_np = ids_for(cfg)
    ids = torch.from_numpy(ids_np).cuda()
    got = traced_step(cfg, store, res, ids)
    loss, logits, _ = oracle_step(cfg, ids_np)
    assert abs(got["loss"] - loss) <= TOL * abs(loss)
    assert rel_err(got["logits"].reshape(logits.shape), logits) <= TOL
    check_head_against_oracle(cfg, got, ids_np)
    check_layers_against_oracle(cfg, got, range(cfg.n_layers))
    whole = traced_step(cfg.with_(loss_chunk=0), store, res, ids)
    assert abs(got["loss"] - whole["loss"]) <= 1e-5 * abs(whole["loss"])
    assert rel_err(got["logits"], whole["logits"].astype(np.float64)) <= 1e-5
    store.close()


def test_large_layer_streaming_is_bit_identical(gpu):
    """Untied embedding and head in page-locked host memory: the gather reads the
    batch's rows over the link and the head is copied in once per step; the
    step is bit for bit the resident one, and the head copy is counted."""
    cfg = configs.TINY.with_(name="tiny-large", wid=31)
    print_case(test="stream_large", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    hres = model.Resident(cfg, large_in_host=True)
    assert not hres.embed.is_cuda and hres.embed.is_pinned()
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    a = run(cfg, "streamed", store, res, ids)
    r = model.Runner(cfg, store, hres)
    logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(2):
        loss = r.step(ids, logits=logits).item()
        torch.cuda.synchronize()
        outs.append(dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy()))
    st = r.stats()
    r.close()
    for b in outs:
        exact, total = _compare_bitwise(cfg, a, b)
        assert exact == total
    assert st.large_copies == 2 and st.large_bytes == 2 * 2 * cfg.vocab * cfg.hidden
    store.close()


def test_timeline_orders_copies_before_their_layer_passes(gpu):
    """The copy/compute timeline of a 5-layer stack over 2 slots: every layer
    copy and layer pass is recorded once per step, each interval is well formed,
    and no layer pass starts before the copy that filled its slot has finished
    (the pool's ready-event handoff seen from the clock)."""
    cfg = configs.TINY.with_(name="tiny-5L", n_layers=5, wid=41)
    print_case(test="timeline", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    r = model.Runner(cfg, store, res)
    r.step(ids)
    torch.cuda.synchronize()
    r.stats(reset=True)
    steps = 3
    r.timeline(steps * (3 * cfg.n_layers + 8))
    for _ in range(steps):
        r.step(ids)
    torch.cuda.synchronize()
    ent, dropped = r.read_timeline()
    st = r.stats()
    r.timeline(0)
    r.close()
    store.close()
    assert dropped == 0
    kinds = [e[0] for e in ent]
    assert kinds.count(lib.LSQ_TL_COPY) == st.copies
    assert st.timed_copies == st.copies and st.timed_bytes == st.copy_bytes
    assert kinds.count(lib.LSQ_TL_FWD) == steps * cfg.n_layers
    assert kinds.count(lib.LSQ_TL_BWD) == steps * cfg.n_layers
    assert kinds.count(lib.LSQ_TL_HEAD) == steps
    assert all(0.0 <= a <= b for _, _, a, b in ent)
    last_copy_end = {}
    eps = 1e-3
    for k, l, a, b in ent:   # recording order: a layer's copy is queued before the pass that acquires it
        if k == lib.LSQ_TL_COPY:
            last_copy_end[l] = b
        elif k in (lib.LSQ_TL_FWD, lib.LSQ_TL_BWD) and l in last_copy_end:
            assert a >= last_copy_end[l] - eps, (k, l, a, last_copy_end[l])


@pytest.mark.parametrize("cfg", [configs.TINY, configs.TINY.with_(name="tiny-5L-3buf", n_layers=5, n_buffers=3,
                                                                   wid=13)])
def test_poisoned_slots_stream_identically(gpu, cfg):
    """LSQ_POOL_POISON fills a slot with 0xFF bytes (NaN absmax, NaN bf16)
    before each refill: any read of a slot before its copy lands would turn
    into NaNs.  Two steps over poisoned slots equal the resident run bit for
    bit, and every refill was poisoned (the copy count)."""
    print_case(test="poisoned_slots", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    r = model.Runner(cfg, store, res, pool_flags=lib.LSQ_POOL_POISON)
    logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
    for _ in range(2):
        loss = r.step(ids, logits=logits).item()
        torch.cuda.synchronize()
        got = dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy())
        exact, total = _compare_bitwise(cfg, resident, got)
        assert exact == total == cfg.n_layers * 14
    assert r.stats().copies == (2 * cfg.n_layers - cfg.n_buffers) + (2 * cfg.n_layers - 2 * cfg.n_buffers)
    r.close()
    store.close()


def test_pool_copies_on_a_stream_that_runs_beside_compute(gpu):
    """HIP maps streams onto a few hardware queues, and two streams on one
    queue run in order, which would serialize the layer copies with compute.
    Handed the compute stream itself as its copy stream, the pool must find a
    stream of its own that runs beside it, and the step must still equal the
    resident run bit for bit; a normal runner's copy stream is never the
    compute stream either."""
    cfg = configs.TINY
    print_case(test="copy_stream_beside_compute", cfg=cfg.name)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    for on_compute in (True, False):
        r = model.Runner(cfg, store, res, copy_on_compute=on_compute)
        used = r.copy_stream_handle()
        assert used not in (0, r.compute.cuda_stream)
        logits = torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda")
        loss = r.step(ids, logits=logits).item()
        torch.cuda.synchronize()
        got = dict(loss=loss, logits=logits.cpu().numpy(), grads=r.grads.cpu().numpy())
        exact, total = _compare_bitwise(cfg, resident, got)
        assert exact == total == cfg.n_layers * 14
        r.close()
    store.close()


def test_store_with_repeated_layer_weights(gpu):
    """A store whose layers reuse the weights of the first few (the deep
    stack's build shortcut) holds, past each blob's header, the same bytes as
    the full store's blob of layer i mod n, and every header names its own
    layer."""
    cfg = configs.TINY.with_(name="tiny-5L-rep", n_layers=5, wid=43)
    print_case(test="store_repeated_layers", layers=cfg.n_layers)
    full = model.Store(cfg)
    rep = model.Store(cfg, distinct_layers=2)
    hdr = 4096
    for i in range(cfg.n_layers):
        a, b = rep.host_blob(i), full.host_blob(i % 2)
        assert np.array_equal(a[hdr:], b[hdr:]), f"layer {i}"
        assert np.array_equal(a[:hdr], full.host_blob(i)[:hdr]), f"header of layer {i}"
    assert not np.array_equal(full.host_blob(2)[hdr:], full.host_blob(0)[hdr:])
    rep.close()
    full.close()
