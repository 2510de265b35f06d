"""Invariants of the oracle that the pages fix (CPU only).

- cold start equals a zero state (the page is not even read);
- restore at a block-aligned checkpoint, then continue, equals the
  uninterrupted run (the 1000-token / 800-checkpoint example of the Kapitsa
  page, and the tiny 64 / 32 case);
- a decode step is a one-token prefill: stepping token by token equals one
  varlen call;
- rows are independent: permuting rows with their slots permutes the result;
- padding, unselected slots and padding rows are never touched;
- the restore truth table (not requested / miss / hit), attention-only layers
  skipped, and the soft failure when no layer is copied.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def run(img, inp):
    return oracle.gdn_layer(img, inp.geom, inp.cu_seqlens, inp.state_indices,
                            inp.has_initial_state, inp.x, inp.conv_w, inp.conv_b, inp.alpha,
                            inp.beta, inp.scale, inp.eps)


def sub_inputs(inp, t_from, t_to, state_indices=None, hs=None):
    """Tokens [cu[n]+t_from, cu[n]+t_to) of every sequence (equal-length rows)."""
    n = inp.num_seqs
    lens = np.diff(inp.cu_seqlens)
    assert (lens == lens[0]).all()
    L = int(lens[0])
    sel = np.concatenate([np.arange(i * L + t_from, i * L + t_to) for i in range(n)])
    cu = np.arange(n + 1, dtype=np.int32) * (t_to - t_from)
    return wl.StepInputs(
        geom=inp.geom, x=inp.x[sel], conv_w=inp.conv_w, conv_b=inp.conv_b,
        alpha=inp.alpha[sel], beta=inp.beta[sel],
        state_indices=inp.state_indices if state_indices is None else np.asarray(
            state_indices, np.int32),
        has_initial_state=inp.has_initial_state if hs is None else np.asarray(hs, np.uint8),
        cu_seqlens=cu, scale=inp.scale, eps=inp.eps)


def tiny_case(seed=0, long_memory=False, extra_pad=128, L=64, n=4, bias=True):
    g = wl.tiny_geometry(extra_pad=extra_pad)
    rng = wl.rng_for(seed)
    idx = rng.permutation(g.num_slots)[:n].astype(np.int32)
    img = wl.make_pool_image(g, rng, warm_slots=[], nan_slots=idx)
    inp = wl.step_inputs(g, rng, [L] * n, idx, np.zeros(n, np.uint8), bias=bias,
                         long_memory=long_memory)
    return g, img, inp


def payload(g, page):
    return (page[g.ssm_off:g.ssm_off + g.ssm_region_bytes],
            page[g.conv_off:g.conv_off + g.conv_region_bytes])


# ---------------------------------------------------------------------------
def test_cold_equals_zero_state_bit_exact():
    g, img, inp = tiny_case(seed=1)
    o_cold, _ = run(img, inp)          # NaN pages, has_initial_state = 0
    zero = img.copy()
    for s in inp.state_indices:
        zero[s, g.ssm_off:g.ssm_off + g.ssm_region_bytes] = 0
        zero[s, g.conv_off:g.conv_off + g.conv_region_bytes] = 0
    inp_warm = sub_inputs(inp, 0, 64, hs=np.ones(inp.num_seqs))
    o_zero, _ = run(zero, inp_warm)
    assert np.isfinite(o_cold).all()
    assert np.array_equal(o_cold, o_zero)
    assert np.array_equal(img, zero)


@pytest.mark.parametrize("long_memory", [False, True])
def test_restore_at_checkpoint_continues_exactly(long_memory):
    """64 tokens straight vs 32 on slots A, restore A -> B, 32 more on B."""
    g, img, inp = tiny_case(seed=2, long_memory=long_memory)
    A = inp.state_indices
    B = np.array([s for s in range(g.num_slots) if s not in set(A)], np.int32)
    straight = img.copy()
    o_straight, _ = run(straight, inp)

    split = img.copy()
    o_first, _ = run(split, sub_inputs(inp, 0, 32))
    ckpt = split.copy()
    hs = np.ones(4, np.uint8)  # prefilled: the rows reused cached tokens
    ops = np.stack([B, A, np.ones(4, np.int32)], axis=1)
    assert oracle.restore([split], g, ops, hs) == 0
    assert hs.tolist() == [1, 1, 1, 1]
    o_second, _ = run(split, sub_inputs(inp, 32, 64, state_indices=B, hs=hs))

    o_s = o_straight.reshape(4, 64, g.Hv, g.dv)
    assert np.array_equal(o_first.reshape(4, 32, g.Hv, g.dv), o_s[:, :32])
    assert np.array_equal(o_second.reshape(4, 32, g.Hv, g.dv), o_s[:, 32:])
    for a, b in zip(A, B):
        assert all(np.array_equal(x, y) for x, y in zip(payload(g, split[b]), payload(g, straight[a])))
        # the checkpoint itself is not modified by the continuation
        assert np.array_equal(split[a], ckpt[a])
        # page padding is not modified by anything
        pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
        assert (split[b][pad] == wl.PAD_BYTE).all()


def test_thousand_tokens_checkpoint_at_800_block_16():
    """The Kapitsa example: identical 1000-token prefix, state saved at 800
    (a multiple of block 16); restoring there and recomputing 200 tokens gives
    the same outputs and final state as running all 1000."""
    block, ckpt_at, total = 16, 800, 1000
    assert ckpt_at % block == 0
    g = wl.make_geometry(4, Hk=1, Hv=2, dk=16, dv=16, W=4, page_align=128)
    rng = wl.rng_for(3)
    img = wl.make_pool_image(g, rng, warm_slots=[0], nan_slots=[])
    inp = wl.step_inputs(g, rng, [total], [0], [1], long_memory=True)
    straight = img.copy()
    o_all, _ = run(straight, inp)
    part = img.copy()
    run(part, sub_inputs(inp, 0, ckpt_at))
    hs = np.zeros(1, np.uint8)
    oracle.restore([part], g, np.array([[2, 0, 1]]), hs)
    assert hs[0] == 1
    o_rest, _ = run(part, sub_inputs(inp, ckpt_at, total, state_indices=[2], hs=hs))
    assert np.array_equal(o_rest, o_all[ckpt_at:])
    assert all(np.array_equal(x, y) for x, y in zip(payload(g, part[2]), payload(g, straight[0])))
    # the check has power: a checkpoint one block early does not continue exactly
    early = img.copy()
    run(early, sub_inputs(inp, 0, ckpt_at - block))
    o_wrong, _ = run(early, sub_inputs(inp, ckpt_at, total))
    assert not np.allclose(o_wrong[:10], o_all[ckpt_at:ckpt_at + 10], rtol=1e-3, atol=1e-6)


def test_decode_steps_equal_one_prefill():
    g, img, inp = tiny_case(seed=4, L=24)
    pre = img.copy()
    o_pre, _ = run(pre, inp)
    dec = img.copy()
    outs = []
    hs = inp.has_initial_state.copy()
    for t in range(24):
        step = sub_inputs(inp, t, t + 1, hs=hs)
        o, _ = oracle.decode(dec, g, step.state_indices, step.has_initial_state, step.x,
                             step.conv_w, step.conv_b, step.alpha, step.beta)
        outs.append(o)
        hs = np.ones_like(hs)
    o_dec = np.stack(outs, axis=1).reshape(o_pre.shape)
    assert np.array_equal(o_dec, o_pre)
    assert np.array_equal(dec, pre)


def test_row_permutation_permutes_result():
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(5)
    idx = rng.permutation(8)[:5].astype(np.int32)
    hs = np.array([1, 0, 1, 1, 0], np.uint8)
    img = wl.make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0])
    lens = [5, 9, 1, 3, 7]
    inp = wl.step_inputs(g, rng, lens, idx, hs, bias=True)
    a = img.copy()
    o_a, _ = run(a, inp)
    perm = np.array([3, 0, 4, 2, 1])
    cu = inp.cu_seqlens
    tok = np.concatenate([np.arange(cu[p], cu[p + 1]) for p in perm])
    cu2 = np.zeros(6, np.int32)
    cu2[1:] = np.cumsum([lens[p] for p in perm])
    inp2 = wl.StepInputs(geom=g, x=inp.x[tok], conv_w=inp.conv_w, conv_b=inp.conv_b,
                         alpha=inp.alpha[tok], beta=inp.beta[tok], state_indices=idx[perm],
                         has_initial_state=hs[perm], cu_seqlens=cu2)
    b = img.copy()
    o_b, _ = run(b, inp2)
    assert np.array_equal(o_b, o_a[tok])
    assert np.array_equal(a, b)


def test_padding_rows_zero_length_and_untouched_pages():
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(6)
    img = wl.make_pool_image(g, rng, warm_slots=[1, 2], nan_slots=[])
    before = img.copy()
    # row 0: slot -1 (padding row), row 1: slot 8 (out of range), row 2: empty, row 3: live
    inp = wl.step_inputs(g, rng, [3, 2, 0, 4], [-1, 8, 1, 2], [1, 1, 1, 1])
    o64, o16 = run(img, inp)
    assert (o64[:5] == 0).all() and (o16[:5] == 0).all()
    assert np.abs(o64[5:]).max() > 0
    for s in range(g.num_slots):
        if s != 2:
            assert np.array_equal(img[s], before[s])
        else:
            pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
            assert np.array_equal(img[s][pad], before[s][pad])


# ---------------------------------------------------------------------------
# Restore truth table
# ---------------------------------------------------------------------------
def test_restore_truth_table_and_attention_layers():
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(9)
    pools = [wl.make_pool_image(g, rng, range(8), []), None,
             wl.make_pool_image(g, rng, range(8), []), None]
    before = [None if p is None else p.copy() for p in pools]
    # row 0: not requested; row 1: miss; rows 2, 3: hits sharing source 5
    ops = np.array([[0, 3, 0], [4, -1, 1], [1, 5, 1], [2, 5, 1]], np.int32)
    hs = np.array([1, 1, 0, 0], np.uint8)
    assert oracle.restore(pools, g, ops, hs) == 0
    assert hs.tolist() == [1, 0, 1, 1]
    for p, b in zip(pools, before):
        if p is None:
            continue
        for s in range(8):
            if s in (1, 2):
                for region in (slice(g.ssm_off, g.ssm_off + g.ssm_region_bytes),
                               slice(g.conv_off, g.conv_off + g.conv_region_bytes)):
                    assert np.array_equal(p[s][region], b[5][region])
                pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
                assert np.array_equal(p[s][pad], b[s][pad])
            else:
                assert np.array_equal(p[s], b[s])


def test_restore_soft_failure_without_linear_layers():
    g = wl.tiny_geometry()
    ops = np.array([[0, 3, 1], [1, -1, 1], [2, 4, 0]], np.int32)
    hs = np.array([1, 1, 1], np.uint8)
    assert oracle.restore([None, None], g, ops, hs) == 1
    assert hs.tolist() == [0, 0, 1]


def test_gather_scatter_round_trip_and_bounds():
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(10)
    img = wl.make_pool_image(g, rng, range(8), [])
    before = img.copy()
    idx = np.array([3, -1, 7, 8], np.int32)
    sd, cd = oracle.gather(img, g, idx)
    assert (sd[1] == 0).all() and (cd[1] == 0).all() and (sd[3] == 0).all()
    assert np.array_equal(sd[0], before[3, g.ssm_off:g.ssm_off + g.ssm_region_bytes])
    assert np.array_equal(cd[2], before[7, g.conv_off:g.conv_off + g.conv_region_bytes])
    oracle.scatter(img, g, idx, sd, cd)
    assert np.array_equal(img, before)
    sd2 = rng.integers(0, 256, sd.shape, dtype=np.uint8)
    cd2 = rng.integers(0, 256, cd.shape, dtype=np.uint8)
    oracle.scatter(img, g, idx, sd2, cd2)
    for s in range(8):
        if s in (3, 7):
            r = 0 if s == 3 else 2
            assert np.array_equal(img[s, g.ssm_off:g.ssm_off + g.ssm_region_bytes], sd2[r])
            assert np.array_equal(img[s, g.conv_off:g.conv_off + g.conv_region_bytes], cd2[r])
            pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
            assert np.array_equal(img[s][pad], before[s][pad])
        else:
            assert np.array_equal(img[s], before[s])
