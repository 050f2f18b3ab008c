"""The pages' workloads at their full sizes, in the launch configuration the
bench times: streamed == resident bit for bit (logits and every adapter
gradient, counted n of n), the aliasing control, slot reuse, and oracle parity
on sampled layers recomputed from the exact inputs of the run."""
import numpy as np
import pytest
import torch

from layer_streamed_qlora_nf4_amd import configs, lib, model, synth
from tests.gpu_util import print_case
from tests.test_gpu_stack import (_compare_bitwise, check_head_against_oracle, check_layers_against_oracle, ids_for,
                                  run, traced_step)

pytestmark = pytest.mark.gpu


def test_8b_stack_streamed_equals_resident_and_sampled_layers_match_oracle(gpu):
    cfg = configs.STACK_8B
    print_case(test="fullsize_8b_stack", layers=cfg.n_layers, T=cfg.tokens)
    store = model.Store(cfg)
    assert store.pinned
    res = model.Resident(cfg)
    ids_np = ids_for(cfg)
    ids = torch.from_numpy(ids_np).cuda()
    streamed = traced_step(cfg, store, res, ids)
    resident = run(cfg, "resident", store, res, ids)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    print(f"8B stack: {exact} of {total} gradient tensors bit-identical; logits identical", flush=True)
    assert exact == total == 32 * 14
    assert np.isfinite(streamed["loss"])
    check_head_against_oracle(cfg, streamed, ids_np)
    check_layers_against_oracle(cfg, streamed, [0, cfg.n_layers // 2, cfg.n_layers - 1])


def test_72b_subset_streamed_equals_resident_above_165_mib(gpu):
    """72B-shaped layers (~471 MiB each, above the size where the pages' NF4
    backward read a refilled slot), six layers through two slots."""
    cfg = configs.STACK_72B.with_(n_layers=6)
    print_case(test="fullsize_72b_subset", layers=cfg.n_layers, T=cfg.tokens)
    store = model.Store(cfg)
    assert store.layer_bytes > 165 * 2 ** 20
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    streamed = run(cfg, "streamed", store, res, ids)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    print(f"72B subset: {exact} of {total} gradient tensors bit-identical", flush=True)
    assert exact == total == 6 * 14
    assert streamed["stats"].copies == 2 * cfg.n_layers - cfg.n_buffers
    bad = run(cfg, "streamed", store, res, ids, early=True)
    exact_bad, _ = _compare_bitwise(cfg, resident, {**bad, "logits": resident["logits"], "loss": resident["loss"]})
    print(f"72B early-release control: {exact_bad} of {total} bit-identical", flush=True)
    assert exact_bad < total


def test_3b_bf16_stack_streamed_equals_resident(gpu):
    cfg = configs.STACK_3B_BF16
    print_case(test="fullsize_3b_bf16", layers=cfg.n_layers, T=cfg.tokens)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    streamed = run(cfg, "streamed", store, res, ids)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    print(f"3B bf16 stack: {exact} of {total} gradient tensors bit-identical", flush=True)
    assert exact == total == 36 * 14


def test_8b_layer_2048_streamed_equals_resident(gpu):
    cfg = configs.LAYER_8B
    print_case(test="fullsize_8b_layer", T=cfg.tokens)
    store = model.Store(cfg)
    res = model.Resident(cfg.with_(vocab=cfg.vocab))
    ids = torch.from_numpy(ids_for(cfg)).cuda()
    resident = run(cfg, "resident", store, res, ids)
    streamed = run(cfg, "streamed", store, res, ids, n_buffers=2)
    exact, total = _compare_bitwise(cfg, resident, streamed)
    assert exact == total == 14


def _same_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_8b_stack_soak_streamed_equals_resident_every_step_then_control(gpu):
    """The pages' acceptance for the slot-aliasing repair (LS-docs "If you
    streamed a 32B or larger model in NF4"): many consecutive backward passes
    with streamed == resident on every one, then a control run in the same
    process that must break it.  50 steps of the 8B-shaped stack over two
    slots, a fresh batch of token ids each step; every step compares the loss,
    the logits and the whole adapter-gradient block (all 448 tensors) bit for
    bit, and a third runner whose slots are filled with 0xFF bytes before each
    refill (LSQ_POOL_POISON) must match too.  Stops at the first mismatch."""
    cfg = configs.STACK_8B
    steps = 50
    print_case(test="soak_8b_stack", layers=cfg.n_layers, T=cfg.tokens, steps=steps)
    store = model.Store(cfg)
    res = model.Resident(cfg)
    runners = {"resident": model.Runner(cfg, store, res, mode="resident"),
               "streamed": model.Runner(cfg, store, res),
               "poisoned": model.Runner(cfg, store, res, pool_flags=lib.LSQ_POOL_POISON)}
    logits = {k: torch.empty((cfg.tokens, cfg.vocab), dtype=torch.float32, device="cuda") for k in runners}
    for k in range(steps):
        ids = torch.from_numpy(synth.token_ids(cfg.batch, cfg.seq, cfg.vocab,
                                               (cfg.wid, 600 + k, synth.TENSOR_IDS["ids"]))).cuda()
        loss = {name: r.step(ids, logits=logits[name]).clone() for name, r in runners.items()}
        torch.cuda.synchronize()
        ref = runners["resident"]
        for name in ("streamed", "poisoned"):
            r = runners[name]
            assert _same_bits(loss[name], loss["resident"]), (k, name, "loss")
            assert _same_bits(logits[name], logits["resident"]), (k, name, "logits")
            if not _same_bits(r.grads, ref.grads):
                exact, total = _compare_bitwise(cfg, dict(loss=0, logits=np.zeros(1, np.float32),
                                                          grads=ref.grads.cpu().numpy()),
                                                dict(loss=0, logits=np.zeros(1, np.float32),
                                                     grads=r.grads.cpu().numpy()))
                pytest.fail(f"step {k}: {name} differs from resident in {total - exact} of {total} gradient tensors")
        assert np.isfinite(loss["resident"].item())
    print(f"soak: {steps} steps, streamed == poisoned == resident bit for bit on every step", flush=True)
    # the control, same process: a slot refilled before its backward GEMMs read it
    bad = runners["streamed"]
    bad.step(ids, early_release=True)
    torch.cuda.synchronize()
    assert not _same_bits(bad.grads, runners["resident"].grads), "the early-release control did not change anything"
    copies = runners["poisoned"].stats().copies
    assert copies == (2 * cfg.n_layers - cfg.n_buffers) + (steps - 1) * (2 * cfg.n_layers - 2 * cfg.n_buffers)
    for r in runners.values():
        r.close()
    store.close()
