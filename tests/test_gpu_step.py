"""GPU parity of the decode step and the varlen prefill against the oracle
(through the C-ABI).  Tolerances are those stated in gpu_util."""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import (DevicePool, check_outputs, check_pages, log, run_decode, run_prefill,
                      step_tensors, u16)

pytestmark = pytest.mark.gpu


def oracle_layer(img, inp):
    return oracle.gdn_layer(img, inp.geom, inp.cu_seqlens, inp.state_indices,
                            inp.has_initial_state, inp.x, inp.conv_w, inp.conv_b, inp.alpha,
                            inp.beta, inp.scale, inp.eps)


def case(g, seed, lengths, warm, slots=None, bias=False, scale=1.0, long_memory=False,
         sigma_s=0.5):
    rng = wl.rng_for(seed)
    n = len(lengths)
    idx = rng.permutation(g.num_slots)[:n].astype(np.int32) if slots is None else \
        np.asarray(slots, np.int32)
    hs = np.asarray(warm, np.uint8)
    valid = (idx >= 0) & (idx < g.num_slots)
    img = wl.make_pool_image(g, rng, warm_slots=idx[valid & (hs == 1)],
                             nan_slots=idx[valid & (hs == 0)], sigma_s=sigma_s)
    inp = wl.step_inputs(g, rng, lengths, idx, hs, bias=bias, long_memory=long_memory)
    inp.scale = scale
    return inp, img


def run_and_check(g, inp, img, mode, what):
    dp = DevicePool(g, [img])
    log(f"{what}: {mode} T={inp.total_tokens} N={inp.num_seqs}")
    t = (run_decode if mode == "decode" else run_prefill)(dp, 0, inp)
    torch.cuda.synchronize()
    ref = img.copy()
    o64, _ = oracle_layer(ref, inp)
    e_out = check_outputs(u16(t["out"]), o64, what)
    e_st = check_pages(g, dp.host(), ref, slots=inp.state_indices, what=what)
    log(f"{what}: worst rel err out {e_out:.2e} state {e_st:.2e}")
    return dp, t, ref


DIMS = [(1, 2, 16), (2, 4, 32), (2, 2, 64), (4, 8, 128)]


@pytest.mark.parametrize("Hk,Hv,d", DIMS)
@pytest.mark.parametrize("W", [2, 3, 4])
def test_decode_matches_oracle(Hk, Hv, d, W):
    g = wl.make_geometry(12, Hk=Hk, Hv=Hv, dk=d, dv=d, W=W, page_align=128, extra_pad=128)
    inp, img = case(g, 100 + d + W, [1] * 7, [1, 0, 1, 1, 0, 1, 1], bias=(W == 4), scale=0.7)
    run_and_check(g, inp, img, "decode", f"decode d={d} W={W}")


@pytest.mark.parametrize("Hk,Hv,d", DIMS)
@pytest.mark.parametrize("W", [2, 3, 4])
def test_prefill_matches_oracle(Hk, Hv, d, W):
    g = wl.make_geometry(12, Hk=Hk, Hv=Hv, dk=d, dv=d, W=W, page_align=128, extra_pad=128)
    # ragged lengths: several chunks, a ragged tail, shorter than the window, empty
    lens = [70, 1, 33, 2, 0, 97, 32]
    inp, img = case(g, 200 + d + W, lens, [1, 0, 1, 1, 0, 0, 1], bias=(W == 3), scale=0.7)
    run_and_check(g, inp, img, "prefill", f"prefill d={d} W={W}")


@pytest.mark.parametrize("Hk,Hv,d", [(1, 3, 32), (2, 8, 64), (1, 4, 128), (2, 6, 128)])
def test_wider_gqa_groups_match_oracle(Hk, Hv, d):
    """Three or four v-heads per k-head: the decode's head pairs then include
    a second pair or a single head."""
    g = wl.make_geometry(10, Hk=Hk, Hv=Hv, dk=d, dv=d, W=4, page_align=128, extra_pad=128)
    inp, img = case(g, 400 + Hv + d, [1] * 6, [1, 0, 1, 1, 0, 1], bias=True)
    run_and_check(g, inp, img, "decode", f"decode G={Hv // Hk} d={d}")
    inp, img = case(g, 500 + Hv + d, [37, 16, 1, 50], [1, 0, 1, 0], bias=True)
    run_and_check(g, inp, img, "prefill", f"prefill G={Hv // Hk} d={d}")


@pytest.mark.parametrize("Hk,Hv,d", [(2, 4, 64), (4, 4, 64), (8, 16, 32), (16, 16, 32),
                                     (24, 48, 32), (8, 24, 16), (16, 32, 16)])
def test_decode_grouped_workgroups_match_oracle(Hk, Hv, d):
    """Small heads run several k-heads per workgroup (2 at head size 64, 8 at
    32 and 16) when the k-head count allows: each group of waves has its own
    window channels, tiles and partial sums, and a padding row zeroes the
    outputs of all the workgroup's k-heads."""
    g = wl.make_geometry(40, Hk=Hk, Hv=Hv, dk=d, dv=d, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(800 + Hk + d)
    slots = rng.permutation(g.num_slots)[:9].astype(np.int32)
    slots[3], slots[7] = -1, g.num_slots  # padding rows
    inp, img = case(g, 801 + Hk + d, [1] * 9, [1, 0, 1, 1, 1, 0, 1, 1, 0], slots=slots,
                    bias=True, scale=0.9)
    run_and_check(g, inp, img, "decode", f"decode grouped Hk={Hk} G={Hv // Hk} d={d}")


def extreme_decays(rng, T, Hv):
    """Decays that drive the running product of a chunk below 2^-40: runs of
    0.02 (below it after 8 tokens), exact zeros, 1e-30 and a subnormal, exact
    ones, mixed with the ordinary draw."""
    a = np.exp(-np.logaddexp(0.0, rng.standard_normal((T, Hv)))).astype(np.float32)
    kind = rng.integers(0, 6, size=(T, Hv))
    a[kind == 1] = 0.02
    a[(kind == 2) & (rng.random((T, Hv)) < 0.1)] = 0.0
    a[(kind == 3) & (rng.random((T, Hv)) < 0.1)] = 1e-30
    a[(kind == 3) & (rng.random((T, Hv)) < 0.05)] = np.float32(1e-40)
    a[kind == 4] = 1.0
    a[:, 0] = 0.02  # one head decays at 0.02 throughout
    return a


@pytest.mark.parametrize("d", [32, 128])
def test_prefill_extreme_decays_match_oracle(d):
    """The prefill keeps the state as a scale times a matrix and folds the
    scale in when it gets small; decays of 0, 1e-30, subnormals and long runs
    of 0.02 must still give the oracle's results, and a split at token 32
    (a chunk boundary) the straight run's bits."""
    g = wl.make_geometry(16, Hk=2, Hv=4, dk=d, dv=d, W=4, page_align=128, extra_pad=128)
    lens = [64, 64, 41, 17]
    inp, img = case(g, 900 + d, lens, [1, 0, 1, 0], bias=True)
    rng = wl.rng_for(901 + d)
    inp.alpha = extreme_decays(rng, inp.total_tokens, g.Hv)
    run_and_check(g, inp, img, "prefill", f"extreme decays d={d}")
    # straight 64 tokens vs 32 + 32 on the first two sequences
    two = dataclasses.replace(inp, x=inp.x[:128], alpha=inp.alpha[:128], beta=inp.beta[:128],
                              cu_seqlens=np.array([0, 64, 128], np.int32),
                              state_indices=inp.state_indices[:2],
                              has_initial_state=inp.has_initial_state[:2])
    sel = [np.r_[0:32, 64:96], np.r_[32:64, 96:128]]
    halves = [dataclasses.replace(two, x=two.x[s], alpha=two.alpha[s], beta=two.beta[s],
                                  cu_seqlens=np.array([0, 32, 64], np.int32),
                                  has_initial_state=two.has_initial_state if i == 0 else
                                  np.ones(2, np.uint8))
              for i, s in enumerate(sel)]
    a = DevicePool(g, [img])
    t_s = run_prefill(a, 0, two)
    b = DevicePool(g, [img])
    run_prefill(b, 0, halves[0])
    t_2 = run_prefill(b, 0, halves[1])
    torch.cuda.synchronize()
    o_s = u16(t_s["out"]).reshape(2, 64, g.Hv, g.dv)
    o_2 = u16(t_2["out"]).reshape(2, 32, g.Hv, g.dv)
    assert np.array_equal(o_2, o_s[:, 32:]), "split run differs from the straight run"
    assert np.array_equal(a.host(), b.host()), "split run's pages differ"


@pytest.mark.parametrize("d", [32, 128])
def test_decode_extreme_decays_match_oracle(d):
    """Decode rows stepped 12 times with decays of 0, 1e-30, a subnormal, runs
    of 0.02 and exact ones: a = 0 must leave only the rank-one write, a = 1 no
    decay, and the state must stay finite and within tolerance every step."""
    g = wl.make_geometry(16, Hk=2, Hv=4, dk=d, dv=d, W=4, page_align=128, extra_pad=128)
    rows, steps = 6, 12
    inp, img = case(g, 700 + d, [1] * rows, [1, 0, 1, 1, 0, 1], bias=True)
    rng = wl.rng_for(701 + d)
    alphas = extreme_decays(rng, rows * steps, g.Hv).reshape(steps, rows, g.Hv)
    alphas[0, 0] = 0.0                 # one row forgets everything at its first step
    alphas[:, 1] = np.float32(1e-40)   # one row decays by a subnormal every step
    alphas[:, 2] = 1.0                 # one row never decays
    dp = DevicePool(g, [img])
    ref = img.copy()
    log(f"decode extreme decays d={d}: {steps} steps x {rows} rows")
    for k in range(steps):
        step = dataclasses.replace(inp, x=wl.draw_x(rng, rows, g.C), alpha=alphas[k].copy(),
                                   beta=wl.draw_gates(rng, rows, g.Hv)[1],
                                   has_initial_state=inp.has_initial_state if k == 0 else
                                   np.ones(rows, np.uint8))
        t = run_decode(dp, 0, step)
        torch.cuda.synchronize()
        o64, _ = oracle_layer(ref, step)
        check_outputs(u16(t["out"]), o64, f"extreme decays d={d} step {k}")
    e_st = check_pages(g, dp.host(), ref, slots=inp.state_indices, what=f"extreme decays d={d}")
    log(f"decode extreme decays d={d}: worst state rel err {e_st:.2e}")


@pytest.mark.parametrize("W,Hk,Hv", [(2, 4, 8), (3, 4, 8), (4, 4, 8), (4, 4, 4), (3, 2, 6)])
def test_prefill_workgroup_shapes_agree_bit_for_bit(W, Hk, Hv):
    """Head size 128 runs in 64-column workgroups when a batch's workgroups all
    fit on the GPU at once and in whole-head workgroups otherwise.  The same
    sequences alone (the first shape) and followed by empty sequences that
    push the batch past the GPU's compute units (the second) must give the
    same bits: every value is computed the same way in both; and both
    match the oracle.  Every conv width, and 1, 2 or 3 v-heads per k-head."""
    g = wl.make_geometry(80, Hk=Hk, Hv=Hv, dk=128, dv=128, W=W, page_align=128, extra_pad=128)
    lens = [70, 33, 1, 48]
    inp, img = case(g, 321, lens, [1, 0, 1, 0], bias=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_pad = cus // (2 * g.Hv) + 1 - len(lens)
    assert len(lens) * g.Hv * 2 <= cus < (len(lens) + n_pad) * g.Hv * 2
    padded = dataclasses.replace(
        inp, cu_seqlens=np.concatenate([inp.cu_seqlens,
                                        np.full(n_pad, inp.cu_seqlens[-1], np.int32)]),
        state_indices=np.concatenate([inp.state_indices, np.arange(n_pad, dtype=np.int32) % 4 +
                                      g.num_slots - 4]),
        has_initial_state=np.concatenate([inp.has_initial_state, np.zeros(n_pad, np.uint8)]))
    a = DevicePool(g, [img])
    log(f"prefill d=128 W={W} G={Hv // Hk} in 64-column workgroups ({len(lens)} sequences)")
    t_a = run_prefill(a, 0, inp)
    b = DevicePool(g, [img])
    log(f"prefill d=128 W={W} G={Hv // Hk} in whole-head workgroups ({len(lens) + n_pad} sequences, "
        f"{n_pad} empty)")
    t_b = run_prefill(b, 0, padded)
    torch.cuda.synchronize()
    assert np.array_equal(u16(t_a["out"]), u16(t_b["out"])), "outputs differ between shapes"
    assert np.array_equal(a.host(), b.host()), "pages differ between shapes"
    ref = img.copy()
    o64, _ = oracle_layer(ref, inp)
    check_outputs(u16(t_b["out"]), o64, "whole-head workgroups")
    check_pages(g, b.host(), ref, slots=inp.state_indices, what="whole-head workgroups")


def test_prefill_word_aligned_inputs():
    """x only 4-byte and out only 8-byte aligned (views into larger buffers),
    with the last sequence's rows ending exactly at the end of x's buffer and
    short last chunks, so that some producer waves of a last chunk have no
    token inside the sequence: every input row read must still lie inside it."""
    g = wl.make_geometry(8, Hk=2, Hv=4, dk=128, dv=128, W=4, page_align=128, extra_pad=128)
    inp, img = case(g, 990, [37, 19, 3], [1, 0, 1], bias=True)
    t = step_tensors(inp)
    xb = torch.empty(t["x"].numel() + 2, dtype=t["x"].dtype, device="cuda")
    xb[2:].copy_(t["x"].reshape(-1))
    t["x"] = xb[2:].view(t["x"].shape)
    ob = torch.full((t["out"].numel() + 4,), 0x7FC0, dtype=torch.int16, device="cuda")
    t["out"] = ob[4:].view(t["out"].shape)
    assert t["x"].data_ptr() % 16 == 4 and t["out"].data_ptr() % 16 == 8
    dp = DevicePool(g, [img])
    log(f"word-aligned prefill T={inp.total_tokens}")
    run_prefill(dp, 0, inp, t)
    torch.cuda.synchronize()
    ref = img.copy()
    o64, _ = oracle_layer(ref, inp)
    check_outputs(u16(t["out"]), o64, "word-aligned prefill")
    check_pages(g, dp.host(), ref, slots=inp.state_indices, what="word-aligned prefill")
    assert (ob[:4] == 0x7FC0).all(), "write before out"


def test_prefill_skips_sequences_outside_total_tokens():
    """cu_seqlens is not checkable on the host: a sequence whose range is empty
    or runs past total_tokens is skipped (its slot and output rows untouched);
    the well-formed ones are computed as usual."""
    g = wl.make_geometry(8, Hk=1, Hv=2, dk=32, dv=32, W=4, page_align=128, extra_pad=128)
    inp, img = case(g, 950, [20, 12, 8], [1, 1, 0], bias=True)
    bad = dataclasses.replace(inp, cu_seqlens=np.array([0, 20, 48, 40], np.int32))
    dp = DevicePool(g, [img])
    log("prefill with cu = [0, 20, 48, 40], total_tokens = 40")
    t = run_prefill(dp, 0, bad)
    torch.cuda.synchronize()
    got = dp.host()
    out = u16(t["out"])
    assert (out[20:] == 0x7FC0).all(), "skipped sequences' output rows were written"
    ref = img.copy()
    first = dataclasses.replace(inp, x=inp.x[:20], alpha=inp.alpha[:20], beta=inp.beta[:20],
                                cu_seqlens=np.array([0, 20], np.int32),
                                state_indices=inp.state_indices[:1],
                                has_initial_state=inp.has_initial_state[:1])
    o64, _ = oracle_layer(ref, first)
    check_outputs(out[:20], o64, "well-formed sequence")
    check_pages(g, got, ref, slots=inp.state_indices[:1], what="skipped sequences")


def test_prefill_long_sequence():
    """One sequence of 65,536 tokens (4,096 chunks) beside a short one: long
    token loop, within the tolerance all the way."""
    g = wl.make_geometry(4, Hk=1, Hv=2, dk=32, dv=32, W=4, page_align=128, extra_pad=128)
    inp, img = case(g, 990, [65536, 3], [1, 0], bias=True)
    run_and_check(g, inp, img, "prefill", "65536-token sequence")


def test_prefill_many_short_sequences():
    """More sequences than one wave can rank (the placement by length then
    keeps the natural order), lengths 0..20 including many shorter than the
    conv window."""
    g = wl.make_geometry(96, Hk=2, Hv=4, dk=32, dv=32, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(77)
    lens = rng.integers(0, 21, size=80)
    warm = (rng.random(80) < 0.5).astype(np.uint8)
    inp, img = case(g, 78, lens, warm, bias=True)
    run_and_check(g, inp, img, "prefill", "prefill 80 short sequences")


def test_padding_rows_and_out_of_range_slots():
    g = wl.tiny_geometry(extra_pad=128)
    inp, img = case(g, 7, [1, 1, 1, 1], [1, 1, 0, 1], slots=[2, -1, 5, 8])
    _, t, _ = run_and_check(g, inp, img, "decode", "decode padding rows")
    out = u16(t["out"])
    assert (out[1] == 0).all() and (out[3] == 0).all()
    inp, img = case(g, 8, [5, 3, 4], [1, 0, 1], slots=[-1, 4, 9])
    _, t, _ = run_and_check(g, inp, img, "prefill", "prefill padding rows")
    out = u16(t["out"])
    assert (out[:5] == 0).all() and (out[8:] == 0).all()


@pytest.mark.parametrize("long_memory", [False, True])
def test_tiny_config_continuation_on_gpu(long_memory):
    """4 seqs x 64 tokens from a cold start: 64 straight vs 32, restore into the
    other four slots, 32 more -- as a prefill and as decode steps, each
    bit-exact against its own straight run on the GPU and within tolerance of
    the oracle.  With the long-memory gate alpha = exp(-0.01 softplus(z)) the
    state after the restore point still carries the first 32 tokens, so a
    continuation from a cold slot must differ (the check is sensitive)."""
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(0)
    perm = rng.permutation(g.num_slots).astype(np.int32)
    A, B = perm[:4], perm[4:]
    img = wl.make_pool_image(g, rng, warm_slots=[], nan_slots=A)
    full = wl.step_inputs(g, rng, [64] * 4, A, np.zeros(4, np.uint8), bias=True,
                          long_memory=long_memory)
    what = "tiny long-memory" if long_memory else "tiny"

    def part(t0, t1, slots, hs):
        sel = np.concatenate([np.arange(i * 64 + t0, i * 64 + t1) for i in range(4)])
        return dataclasses.replace(full, x=full.x[sel], alpha=full.alpha[sel],
                                   beta=full.beta[sel], state_indices=np.asarray(slots, np.int32),
                                   has_initial_state=np.asarray(hs, np.uint8),
                                   cu_seqlens=np.arange(5, dtype=np.int32) * (t1 - t0))

    def restore(dp, hs_val=1):
        hs = torch.full((4,), hs_val, dtype=torch.uint8, device="cuda")
        assert gdn.gdn_restore_slots(dp.pool, [(int(b), int(a), 1) for a, b in zip(A, B)],
                                     hs) == gdn.GDN_OK
        return hs

    def decode_steps(dp, t0, t1, slots, hs0):
        outs = []
        for t in range(t0, t1):
            hs = hs0 if t == t0 else [1] * 4
            outs.append(u16(run_decode(dp, 0, part(t, t + 1, slots, hs))["out"]))
        return np.stack(outs, axis=1)  # [4, steps, Hv, dv]

    def payload(host, s_):
        return host[s_][:g.conv_off + g.conv_region_bytes]

    log(f"{what}: prefill straight vs 32 + restore + 32")
    straight = DevicePool(g, [img])
    t_s = run_prefill(straight, 0, full)
    split = DevicePool(g, [img])
    run_prefill(split, 0, part(0, 32, A, [0] * 4))
    restore(split)
    t_2 = run_prefill(split, 0, part(32, 64, B, [1] * 4))
    # the same continuation as 32 decode steps after the restore
    dec = DevicePool(g, [img])
    run_prefill(dec, 0, part(0, 32, A, [0] * 4))
    restore(dec)
    d_cont = decode_steps(dec, 32, 64, B, [1] * 4)
    # decode all the way: 64 steps straight vs 32 + restore + 32
    log(f"{what}: decode straight vs 32 + restore + 32")
    d_straight_pool = DevicePool(g, [img])
    d_straight = decode_steps(d_straight_pool, 0, 64, A, [0] * 4)
    d_split_pool = DevicePool(g, [img])
    decode_steps(d_split_pool, 0, 32, A, [0] * 4)
    restore(d_split_pool)
    d_split = decode_steps(d_split_pool, 32, 64, B, [1] * 4)
    torch.cuda.synchronize()
    o_s = u16(t_s["out"]).reshape(4, 64, g.Hv, g.dv)
    o_2 = u16(t_2["out"]).reshape(4, 32, g.Hv, g.dv)
    assert np.array_equal(o_2, o_s[:, 32:]), "restored prefill differs from the straight run"
    assert np.array_equal(d_split, d_straight[:, 32:]), "restored decode differs from straight"
    host_s, host_2 = straight.host(), split.host()
    host_ds, host_d2 = d_straight_pool.host(), d_split_pool.host()
    for a, b in zip(A, B):
        assert np.array_equal(payload(host_2, b), payload(host_s, a))
        assert np.array_equal(payload(host_d2, b), payload(host_ds, a))
    # against the oracle
    ref = img.copy()
    o64, _ = oracle_layer(ref, full)
    check_outputs(u16(t_s["out"]), o64, f"{what} straight prefill")
    check_pages(g, host_s, ref, slots=A, what=f"{what} straight prefill")
    check_pages(g, host_ds, ref, slots=A, what=f"{what} straight decode")
    o64 = o64.reshape(4, 64, g.Hv, g.dv)
    check_outputs(d_straight.reshape(-1, g.Hv, g.dv), o64.reshape(-1, g.Hv, g.dv),
                  f"{what} straight decode")
    check_outputs(d_cont.reshape(-1, g.Hv, g.dv), o64[:, 32:].reshape(-1, g.Hv, g.dv),
                  f"{what} decode continuation")
    if long_memory:
        # a continuation that starts cold (a lost restore) is outside the tolerance
        cold = DevicePool(g, [img])
        run_prefill(cold, 0, part(0, 32, A, [0] * 4))
        t_c = run_prefill(cold, 0, part(32, 64, B, [0] * 4))
        torch.cuda.synchronize()
        with pytest.raises(AssertionError):
            check_outputs(u16(t_c["out"]), o64[:, 32:].reshape(-1, g.Hv, g.dv), "cold")
        oc = wl.bf16_bits_to_f32(u16(t_c["out"]).reshape(4, 32, g.Hv, g.dv)).astype(np.float64)
        ref_last = o64[:, -1]
        rel = np.abs(oc[:, -1] - ref_last).max(-1) / np.abs(ref_last).max(-1)
        assert (rel > 0.05).all(), "the long-memory state forgot the restored part"


@pytest.mark.parametrize("extra_pad", [0, 4096])
def test_decode_full_shape_matches_oracle(extra_pad):
    """256 rows x 32 heads x 128x128 fp32, 1024-slot pool with 4 KiB pages,
    90 % warm rows (the decode workload), all rows against the oracle; also
    with 4 KiB of padding after each payload (a page stride that is no longer
    the payload rounded up)."""
    inp, pages = wl.decode_workload(seed=0, extra_pad=extra_pad)
    g = inp.geom
    log(f"decode workload (+{extra_pad} B padding): filling 1024-slot pool")
    gen = torch.Generator(device="cuda").manual_seed(1)
    pool = torch.randint(0, 256, (g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda",
                         generator=gen)
    idx_t = torch.from_numpy(inp.state_indices.astype(np.int64)).cuda()
    pool[idx_t] = torch.from_numpy(pages).cuda()
    others_before = pool[:64].clone()
    dp = DevicePool.__new__(DevicePool)
    dp.g, dp.bufs = g, [pool]
    dp.pool = gdn.gdn_pool_create([pool], g.num_slots, g.page_stride, g.conv_off, g.ssm_off,
                                  g.C, g.W, g.Hk, g.Hv, g.dk, g.dv)
    t = run_decode(dp, 0, inp)
    torch.cuda.synchronize()
    got = pool[idx_t].cpu().numpy()
    sub = dataclasses.replace(g, num_slots=inp.num_seqs)
    ref = pages.copy()
    loc = dataclasses.replace(inp, state_indices=np.arange(inp.num_seqs, dtype=np.int32),
                              geom=sub)
    o64, _ = oracle_layer(ref, loc)
    e_out = check_outputs(u16(t["out"]), o64, "decode full")
    e_st = check_pages(sub, got, ref, what="decode full")
    log(f"decode full: worst rel err out {e_out:.2e} state {e_st:.2e}")
    untouched = [s for s in range(64) if s not in set(inp.state_indices.tolist())]
    assert torch.equal(pool[untouched], others_before[untouched])


def test_prefill_varlen_full_shape_matches_oracle():
    """8 sequences, lengths U{512..4096}, 16 heads x 128x128, half warm half cold."""
    inp, img = wl.prefill_workload(seed=0)
    g = inp.geom
    log(f"prefill workload: lengths {np.diff(inp.cu_seqlens).tolist()}")
    run_and_check(g, inp, img, "prefill", "prefill full")
