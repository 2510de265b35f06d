"""Seeded random configurations against the oracle: head size, k-heads, v-heads
per k-head, conv width, page padding, ragged lengths (empty and one-token
sequences included), warm/cold rows, a padding row (slot out of range), conv
bias and q scale are drawn per case, for the varlen prefill and the decode
step.  Each case is small; together they cover combinations the fixed cases
do not.  GDN_RANDOM_SEEDS sets the number of seeds (default 40; a wider sweep,
e.g. 5440, takes a couple of minutes), and a tenth as many window-first
layouts run, at least 6.  The long-sequence cases (GDN_LONG_SEEDS, default 4)
draw ragged sequences of up to 3000 tokens, so that rounding has many chunks
to build up over.  The grouped decode cases (GDN_GROUPED_SEEDS, default 8)
draw small heads with 2-16 k-heads, the shapes whose decode runs several
k-heads per workgroup.  The chained cases (GDN_CHAIN_SEEDS, default 8) run a
prefill and then several decode steps on the same slots, so that each kernel
reads the state and window the other wrote."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import (DevicePool, check_outputs, check_pages, log, run_decode, run_prefill,
                      to_dev, u16)

pytestmark = pytest.mark.gpu

N_SEEDS = int(os.environ.get("GDN_RANDOM_SEEDS", "40"))
N_LONG = int(os.environ.get("GDN_LONG_SEEDS", "4"))
N_GROUPED = int(os.environ.get("GDN_GROUPED_SEEDS", "8"))
N_CHAIN = int(os.environ.get("GDN_CHAIN_SEEDS", "8"))


def draw_case(seed: int, decode: bool):
    r = np.random.default_rng(seed)
    d = int(r.choice([16, 32, 64, 128]))
    Hk = int(r.integers(1, 4))
    G = int(r.integers(1, 5))
    W = int(r.integers(2, 5))
    pad = int(r.choice([0, 128, 4096]))
    g = wl.make_geometry(24, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128, extra_pad=pad)
    n = int(r.integers(1, 7))
    lengths = [1] * n if decode else [int(x) for x in r.choice([0, 1, 2, 5, 16, 17, 31, 48, 95],
                                                              size=n)]
    slots = r.permutation(g.num_slots)[:n].astype(np.int32)
    if n > 1 and r.random() < 0.5:
        slots[int(r.integers(0, n))] = int(r.choice([-1, g.num_slots]))  # a padding row
    warm = (r.random(n) < 0.6).astype(np.uint8)
    rng = wl.rng_for(10_000 + seed)
    valid = (slots >= 0) & (slots < g.num_slots)
    img = wl.make_pool_image(g, rng, warm_slots=slots[valid & (warm == 1)],
                             nan_slots=slots[valid & (warm == 0)], sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lengths, slots, warm, bias=bool(r.random() < 0.5),
                         long_memory=bool(r.random() < 0.3))
    inp.scale = float(r.uniform(0.5, 1.5))
    what = (f"seed {seed}: {'decode' if decode else 'prefill'} d={d} Hk={Hk} G={G} W={W} "
            f"pad={pad} lengths={lengths} slots={slots.tolist()} warm={warm.tolist()}")
    return g, inp, img, what


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_configuration_matches_oracle(seed, decode):
    g, inp, img, what = draw_case(seed, decode)
    log(what)
    dp = DevicePool(g, [img])
    t = (run_decode if decode else run_prefill)(dp, 0, inp)
    torch.cuda.synchronize()
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    if inp.total_tokens:
        check_outputs(u16(t["out"]), o64, what)
    valid = [int(s) for s in inp.state_indices if 0 <= s < g.num_slots]
    check_pages(g, dp.host(), ref, slots=valid, what=what)


def window_first_geometry(r, num_slots=20):
    """A page with the window region first, then the state region, with gaps
    (multiples of 16 bytes) before, between and after them."""
    d = int(r.choice([32, 64, 128]))
    Hk = int(r.integers(1, 3))
    Hv = Hk * int(r.integers(1, 4))
    W = int(r.integers(2, 5))
    C = 2 * Hk * d + Hv * d
    conv_off = 16 * int(r.integers(0, 9))
    ssm_off = wl.round_up(conv_off + (W - 1) * C * 2, 16) + 16 * int(r.integers(0, 9))
    stride = wl.round_up(ssm_off + Hv * d * d * 4, 16) + 16 * int(r.integers(0, 17))
    return wl.Geometry(num_slots=num_slots, C=C, W=W, Hk=Hk, Hv=Hv, dk=d, dv=d,
                       page_stride=stride, ssm_off=ssm_off, conv_off=conv_off)


@pytest.mark.parametrize("seed", range(max(6, N_SEEDS // 10)))
def test_window_first_layout_matches_oracle(seed):
    """Decode, prefill, restore, gather and scatter on pages whose window region
    comes first and whose regions are separated by gaps: every kernel takes the
    region offsets from the pool descriptor."""
    r = np.random.default_rng(500 + seed)
    g = window_first_geometry(r)
    rng = wl.rng_for(20_000 + seed)
    slots = r.permutation(g.num_slots).astype(np.int32)
    live, ckpt = slots[:6], slots[6:10]
    warm = np.array([1, 0, 1, 1, 0, 1], np.uint8)
    img = wl.make_pool_image(g, rng, warm_slots=np.concatenate([live[warm == 1], ckpt]),
                             nan_slots=live[warm == 0], sigma_s=0.5)
    what = (f"seed {seed}: window-first page d={g.dk} Hk={g.Hk} Hv={g.Hv} W={g.W} "
            f"conv_off={g.conv_off} ssm_off={g.ssm_off} stride={g.page_stride}")
    log(what)
    dp = DevicePool(g, [img])
    ref = img.copy()
    # restore two checkpoints into the first two rows (their pages become warm)
    ops = np.array([[int(live[0]), int(ckpt[0]), 1], [int(live[1]), int(ckpt[1]), 1]], np.int32)
    hs = torch.zeros(2, dtype=torch.uint8, device="cuda")
    assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs) == gdn.GDN_OK
    hs_ref = np.zeros(2, np.uint8)
    oracle.restore([ref], g, ops, hs_ref)
    warm = warm.copy()
    warm[:2] = hs_ref
    dinp = wl.step_inputs(g, rng, [1] * 6, live, warm, bias=True)
    td = run_decode(dp, 0, dinp)
    pinp = wl.step_inputs(g, rng, [19, 1, 40, 16, 3, 0], live, np.ones(6, np.uint8),
                          conv=(dinp.conv_w, dinp.conv_b))
    tp = run_prefill(dp, 0, pinp)
    # gather the live pages, scatter them onto the checkpoint slots shifted by one
    gidx = live[:4].copy()
    sidx = np.roll(ckpt, 1).astype(np.int32)
    ssm = torch.empty((4, g.ssm_region_bytes), dtype=torch.uint8, device="cuda")
    conv = torch.empty((4, g.conv_region_bytes), dtype=torch.uint8, device="cuda")
    gdn.gdn_gather_states(dp.pool, 0, to_dev(gidx), 4, conv, ssm)
    gdn.gdn_scatter_states(dp.pool, 0, to_dev(sidx), 4, conv, ssm)
    torch.cuda.synchronize()
    assert np.array_equal(hs.cpu().numpy(), hs_ref)
    od, _ = oracle.gdn_layer(ref, g, dinp.cu_seqlens, live, warm, dinp.x, dinp.conv_w,
                             dinp.conv_b, dinp.alpha, dinp.beta, dinp.scale, dinp.eps)
    op, _ = oracle.gdn_layer(ref, g, pinp.cu_seqlens, live, pinp.has_initial_state, pinp.x,
                             pinp.conv_w, pinp.conv_b, pinp.alpha, pinp.beta, pinp.scale,
                             pinp.eps)
    check_outputs(u16(td["out"]), od, what + " decode")
    check_outputs(u16(tp["out"]), op, what + " prefill")
    got = dp.host()
    # the gathered rows are the GPU's own live pages: the dense copies must be
    # exactly their payloads, and the scatter must put exactly those bytes
    gs, gc = oracle.gather(got, g, gidx)
    assert np.array_equal(ssm.cpu().numpy(), gs) and np.array_equal(conv.cpu().numpy(), gc)
    oracle.scatter(ref, g, sidx, gs, gc)
    # pages the steps touched: within tolerance of the oracle; the rest bit-exact
    check_pages(g, got, ref, slots=np.concatenate([live, ckpt]), what=what)
    for s in ckpt:  # scattered pages hold the GPU's gathered bytes exactly
        pay = np.ones(g.page_stride, bool)
        pay[:g.conv_off] = False
        pay[g.conv_off + g.conv_region_bytes:g.ssm_off] = False
        pay[g.ssm_off + g.ssm_region_bytes:] = False
        assert np.array_equal(got[s][~pay], img[s][~pay]), what + ": gap or padding bytes changed"


@pytest.mark.parametrize("seed", range(N_LONG))
def test_random_long_sequences_match_oracle(seed):
    r = np.random.default_rng(50_000 + seed)
    d = int(r.choice([32, 64, 128, 128]))
    Hk = int(r.integers(1, 3))
    G = int(r.integers(1, 3))
    W = int(r.integers(2, 5))
    g = wl.make_geometry(16, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128)
    n = int(r.integers(1, 5))
    lengths = [int(x) for x in r.integers(1, 3000, size=n)]
    slots = r.permutation(g.num_slots)[:n].astype(np.int32)
    warm = (r.random(n) < 0.6).astype(np.uint8)
    rng = wl.rng_for(60_000 + seed)
    img = wl.make_pool_image(g, rng, warm_slots=slots[warm == 1], nan_slots=slots[warm == 0],
                             sigma_s=0.5)
    long_memory = bool(r.random() < 0.5)
    inp = wl.step_inputs(g, rng, lengths, slots, warm, bias=bool(r.random() < 0.5),
                         long_memory=long_memory)
    inp.scale = float(r.uniform(0.5, 1.5))
    what = (f"long seed {seed}: d={d} Hk={Hk} G={G} W={W} lengths={lengths} "
            f"warm={warm.tolist()} long_memory={long_memory}")
    log(what)
    dp = DevicePool(g, [img])
    t = run_prefill(dp, 0, inp)
    torch.cuda.synchronize()
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    check_outputs(u16(t["out"]), o64, what)
    check_pages(g, dp.host(), ref, slots=[int(x) for x in slots], what=what)


@pytest.mark.parametrize("seed", range(N_GROUPED))
def test_random_grouped_decode_matches_oracle(seed):
    r = np.random.default_rng(123_000 + seed)
    d = int(r.choice([16, 32, 64]))
    Hk = int(r.choice([2, 4, 8, 16]))
    G = int(r.integers(1, 5))
    W = int(r.integers(2, 5))
    g = wl.make_geometry(48, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128,
                         extra_pad=int(r.choice([0, 128])))
    n = int(r.integers(1, 12))
    slots = r.permutation(g.num_slots)[:n].astype(np.int32)
    if n > 1 and r.random() < 0.5:
        slots[int(r.integers(0, n))] = int(r.choice([-1, g.num_slots]))  # a padding row
    warm = (r.random(n) < 0.7).astype(np.uint8)
    rng = wl.rng_for(124_000 + seed)
    valid = (slots >= 0) & (slots < g.num_slots)
    img = wl.make_pool_image(g, rng, warm_slots=slots[valid & (warm == 1)],
                             nan_slots=slots[valid & (warm == 0)], sigma_s=0.5)
    inp = wl.step_inputs(g, rng, [1] * n, slots, warm, bias=bool(r.random() < 0.5),
                         long_memory=bool(r.random() < 0.3))
    inp.scale = float(r.uniform(0.5, 1.5))
    what = f"grouped seed {seed}: d={d} Hk={Hk} G={G} W={W} slots={slots.tolist()}"
    log(what)
    dp = DevicePool(g, [img])
    t = run_decode(dp, 0, inp)
    torch.cuda.synchronize()
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    check_outputs(u16(t["out"]), o64, what)
    check_pages(g, dp.host(), ref, slots=[int(x) for x in slots[valid]], what=what)


@pytest.mark.parametrize("seed", range(N_CHAIN))
def test_random_prefill_then_decode_steps_match_oracle(seed):
    r = np.random.default_rng(140_000 + seed)
    d = int(r.choice([16, 32, 64, 128]))
    Hk = int(r.choice([1, 2, 4, 8]))
    G = int(r.integers(1, 4))
    W = int(r.integers(2, 5))
    g = wl.make_geometry(24, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128,
                         extra_pad=int(r.choice([0, 128])))
    n = int(r.integers(1, 6))
    slots = r.permutation(g.num_slots)[:n].astype(np.int32)
    warm = (r.random(n) < 0.5).astype(np.uint8)
    lens = [int(x) for x in r.integers(0, 80, size=n)]
    rng = wl.rng_for(141_000 + seed)
    img = wl.make_pool_image(g, rng, warm_slots=slots[warm == 1], nan_slots=slots[warm == 0],
                             sigma_s=0.5)
    long_memory = bool(r.random() < 0.5)
    pre = wl.step_inputs(g, rng, lens, slots, warm, bias=bool(r.random() < 0.5),
                         long_memory=long_memory)
    pre.scale = float(r.uniform(0.5, 1.5))
    what = (f"chain seed {seed}: d={d} Hk={Hk} G={G} W={W} lens={lens} warm={warm.tolist()}")
    log(what)
    dp = DevicePool(g, [img])
    ref = img.copy()
    if pre.total_tokens:
        t = run_prefill(dp, 0, pre)
        torch.cuda.synchronize()
        o64, _ = oracle.gdn_layer(ref, g, pre.cu_seqlens, pre.state_indices,
                                  pre.has_initial_state, pre.x, pre.conv_w, pre.conv_b,
                                  pre.alpha, pre.beta, pre.scale, pre.eps)
        check_outputs(u16(t["out"]), o64, f"{what}: prefill")
    # a row whose prefill was empty keeps its own start state for the decode steps
    hs = np.where(np.asarray(lens) > 0, 1, warm).astype(np.uint8)
    for k in range(int(r.integers(1, 6))):
        x = wl.draw_x(rng, n, g.C)
        alpha, beta = wl.draw_gates(rng, n, g.Hv, long_memory)
        step = dataclasses.replace(pre, x=x, alpha=alpha, beta=beta,
                                   cu_seqlens=np.arange(n + 1, dtype=np.int32),
                                   has_initial_state=hs.copy())
        t = run_decode(dp, 0, step)
        torch.cuda.synchronize()
        o64, _ = oracle.gdn_layer(ref, g, step.cu_seqlens, step.state_indices,
                                  step.has_initial_state, step.x, step.conv_w, step.conv_b,
                                  step.alpha, step.beta, step.scale, step.eps)
        check_outputs(u16(t["out"]), o64, f"{what}: decode step {k}")
        hs[:] = 1
    check_pages(g, dp.host(), ref, slots=[int(x) for x in slots], what=what)
