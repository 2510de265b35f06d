"""Block-boundary checkpoint emission inside a varlen prefill
(gdn_prefill_varlen_checkpoint), through the C-ABI.

For each sequence with a checkpoint request the page ckpt_slot must hold,
after the call, the window and state the sequence had after its first
ckpt_len tokens -- that is, what a prefill of just those tokens leaves in the
sequence's own page.  Checked against the oracle's prefix runs (small shapes,
every head size, ragged lengths, requests at token 1, at chunk edges, at the
end, and ignored ones) and, at the 8-sequence workload's full size, bit for
bit against a separate GPU prefill of the prefixes.  The call's ordinary
results must be those of gdn_prefill_varlen.  Seeded random cases (head size,
GQA ratio, conv width, lengths, request positions, ignored requests; the
number of seeds from GDN_CKPT_SEEDS, default 8) cover the combinations the
fixed ones do not, and so do random cycles of checkpoint, restore into a fresh
slot and continuation, checked against the oracle's straight run.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import (DevicePool, check_outputs, check_pages, log, step_tensors, to_dev, u16,
                      args_of)

pytestmark = pytest.mark.gpu

DIMS = [(1, 2, 16), (2, 4, 32), (2, 2, 64), (4, 8, 128)]


def oracle_prefix_page(img, inp, n, length):
    """Page of sequence n after its first `length` tokens (oracle)."""
    g = inp.geom
    t0 = int(inp.cu_seqlens[n])
    sub = dataclasses.replace(g, num_slots=1)
    page = img[int(inp.state_indices[n])][None].copy()
    sl = slice(t0, t0 + length)
    oracle.gdn_layer(page, sub, np.array([0, length], np.int32), np.zeros(1, np.int32),
                     inp.has_initial_state[n:n + 1], inp.x[sl], inp.conv_w, inp.conv_b,
                     inp.alpha[sl], inp.beta[sl], inp.scale, inp.eps)
    return page


@pytest.mark.parametrize("Hk,Hv,d", DIMS)
def test_checkpoint_emission_matches_oracle_prefix(Hk, Hv, d):
    g = wl.make_geometry(16, Hk=Hk, Hv=Hv, dk=d, dv=d, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(300 + d)
    lens = [70, 1, 33, 40, 0, 97, 32]
    warm = [1, 0, 1, 1, 0, 0, 1]
    perm = rng.permutation(g.num_slots).astype(np.int32)
    idx, spare = perm[:7], perm[7:]
    # requests: mid-chunk, first token, at the end, at a chunk edge, on an empty
    # sequence (ignored), past the end (ignored), none
    ck_len = np.array([23, 1, 33, 16, 1, 98, 0], np.int32)
    ck_slot = np.array([spare[0], spare[1], spare[2], spare[3], spare[4], spare[5], -1], np.int32)
    valid = [0, 1, 2, 3]
    hs = np.asarray(warm, np.uint8)
    img = wl.make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0], sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lens, idx, hs, bias=True)
    inp.scale = 0.8
    dp = DevicePool(g, [img])
    t = step_tensors(inp)
    log(f"checkpoint emission d={d}")
    rc = gdn.gdn_prefill_varlen_checkpoint(dp.pool, 0, inp.num_seqs, t["cu"], inp.max_seqlen,
                                           inp.total_tokens, args_of(t, inp), to_dev(ck_slot),
                                           to_dev(ck_len))
    assert rc == gdn.GDN_OK
    torch.cuda.synchronize()
    got = dp.host()
    # the ordinary results, and every page that is neither a sequence's nor a
    # valid checkpoint's, as the oracle says
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    check_outputs(u16(t["out"]), o64, f"d={d} outputs")
    ck_valid = set(int(ck_slot[n]) for n in valid)
    for n in valid:
        ref[ck_slot[n]] = got[ck_slot[n]]  # compared below against the prefix runs
    check_pages(g, got, ref, slots=list(idx), what=f"d={d} pages")
    sub = dataclasses.replace(g, num_slots=1)
    for n in valid:
        want = oracle_prefix_page(img, inp, n, int(ck_len[n]))
        page = got[ck_slot[n]][None].copy()
        # the checkpoint page's padding must be the original bytes
        pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
        assert np.array_equal(page[0, pad], img[ck_slot[n], pad])
        want[0, pad] = page[0, pad]
        check_pages(sub, page, want, what=f"d={d} checkpoint of sequence {n}")
    assert len(ck_valid) == len(valid)


def test_checkpoint_emission_full_size_equals_prefix_prefill():
    """8 sequences, 16 heads x 128x128: each sequence emits its state at its
    last 256-token block boundary; the checkpoint pages equal the pages a
    separate prefill of those prefixes leaves, bit for bit, and the call's
    outputs equal those of the plain prefill."""
    inp, img = wl.prefill_workload(seed=0)
    g = inp.geom
    lens = np.diff(inp.cu_seqlens)
    ck_len = (lens // 256 * 256).astype(np.int32)
    spare = np.array([s for s in range(g.num_slots) if s not in set(inp.state_indices.tolist())],
                     np.int32)
    ck_slot = spare[:inp.num_seqs].copy()
    log(f"full size: lengths {lens.tolist()}, checkpoints at {ck_len.tolist()}")
    a = DevicePool(g, [img])
    ta = step_tensors(inp)
    assert gdn.gdn_prefill_varlen_checkpoint(a.pool, 0, inp.num_seqs, ta["cu"], inp.max_seqlen,
                                             inp.total_tokens, args_of(ta, inp), to_dev(ck_slot),
                                             to_dev(ck_len)) == gdn.GDN_OK
    # the same call without checkpoints
    b = DevicePool(g, [img])
    tb = step_tensors(inp)
    assert gdn.gdn_prefill_varlen(b.pool, 0, inp.num_seqs, tb["cu"], inp.max_seqlen,
                                  inp.total_tokens, args_of(tb, inp)) == gdn.GDN_OK
    # the prefixes alone, into the sequences' own slots of a third pool
    sel = np.concatenate([np.arange(inp.cu_seqlens[n], inp.cu_seqlens[n] + ck_len[n])
                          for n in range(inp.num_seqs)])
    pre = dataclasses.replace(inp, x=inp.x[sel], alpha=inp.alpha[sel], beta=inp.beta[sel],
                              cu_seqlens=np.concatenate([[0], np.cumsum(ck_len)]).astype(np.int32))
    c = DevicePool(g, [img])
    tc = step_tensors(pre)
    assert gdn.gdn_prefill_varlen(c.pool, 0, pre.num_seqs, tc["cu"], pre.max_seqlen,
                                  pre.total_tokens, args_of(tc, pre)) == gdn.GDN_OK
    torch.cuda.synchronize()
    assert torch.equal(ta["out"], tb["out"])
    idx_t = torch.from_numpy(inp.state_indices.astype(np.int64)).cuda()
    ck_t = torch.from_numpy(ck_slot.astype(np.int64)).cuda()
    assert torch.equal(a.bufs[0][idx_t], b.bufs[0][idx_t])
    pay = g.conv_off + g.conv_region_bytes
    assert torch.equal(a.bufs[0][ck_t][:, :pay], c.bufs[0][idx_t][:, :pay])
    assert torch.equal(a.bufs[0][ck_t][:, pay:], b.bufs[0][ck_t][:, pay:])  # padding as it was


def test_checkpoint_emission_in_whole_head_workgroups():
    """Head size 128 in whole-head workgroups (the batch padded with empty
    sequences past the GPU's compute units) emits the same checkpoint pages,
    bit for bit, as in 64-column workgroups, and they match the oracle's
    prefix runs."""
    g = wl.make_geometry(96, Hk=4, Hv=8, dk=128, dv=128, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(777)
    lens = [70, 33, 48, 17]
    warm = np.array([1, 0, 1, 0], np.uint8)
    perm = rng.permutation(g.num_slots - 8).astype(np.int32)
    idx, spare = perm[:4], perm[4:8]
    ck_len = np.array([23, 16, 48, 1], np.int32)  # mid-chunk, chunk edge, at the end, first token
    img = wl.make_pool_image(g, rng, warm_slots=idx[warm == 1], nan_slots=idx[warm == 0], sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lens, idx, warm, bias=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_pad = cus // (2 * g.Hv) + 1 - len(lens)
    assert len(lens) * g.Hv * 2 <= cus < (len(lens) + n_pad) * g.Hv * 2
    padded = dataclasses.replace(
        inp, cu_seqlens=np.concatenate([inp.cu_seqlens, np.full(n_pad, inp.cu_seqlens[-1], np.int32)]),
        state_indices=np.concatenate([inp.state_indices,
                                      np.arange(n_pad, dtype=np.int32) % 8 + g.num_slots - 8]),
        has_initial_state=np.concatenate([inp.has_initial_state, np.zeros(n_pad, np.uint8)]))
    pages = []
    for what, run_inp, cks, ckl in (
            ("64-column", inp, spare, ck_len),
            ("whole-head", padded, np.concatenate([spare, np.full(n_pad, -1, np.int32)]),
             np.concatenate([ck_len, np.zeros(n_pad, np.int32)]))):
        dp = DevicePool(g, [img])
        t = step_tensors(run_inp)
        log(f"checkpoints in {what} workgroups ({run_inp.num_seqs} sequences)")
        assert gdn.gdn_prefill_varlen_checkpoint(dp.pool, 0, run_inp.num_seqs, t["cu"],
                                                 run_inp.max_seqlen, run_inp.total_tokens,
                                                 args_of(t, run_inp), to_dev(cks.astype(np.int32)),
                                                 to_dev(ckl.astype(np.int32))) == gdn.GDN_OK
        torch.cuda.synchronize()
        pages.append((dp.host(), u16(t["out"])))
    (pa, oa), (pb, ob) = pages
    assert np.array_equal(oa, ob), "outputs differ between shapes"
    assert np.array_equal(pa, pb), "pages (sequences' and checkpoints') differ between shapes"
    sub = dataclasses.replace(g, num_slots=1)
    pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
    for n in range(len(lens)):
        want = oracle_prefix_page(img, inp, n, int(ck_len[n]))
        page = pb[spare[n]][None].copy()
        assert np.array_equal(page[0, pad], img[spare[n], pad])
        want[0, pad] = page[0, pad]
        check_pages(sub, page, want, what=f"whole-head checkpoint of sequence {n}")


@pytest.mark.parametrize("seed", range(int(os.environ.get("GDN_CKPT_SEEDS", "8"))))
def test_random_checkpoint_requests_match_oracle_prefix(seed):
    r = np.random.default_rng(70_000 + seed)
    d = int(r.choice([16, 32, 64, 128]))
    Hk = int(r.integers(1, 3))
    G = int(r.integers(1, 4))
    W = int(r.integers(2, 5))
    g = wl.make_geometry(24, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128, extra_pad=128)
    n = int(r.integers(1, 6))
    lens = [int(x) for x in r.integers(0, 200, size=n)]
    perm = r.permutation(g.num_slots).astype(np.int32)
    idx, spare = perm[:n], perm[n:2 * n]
    hs = (r.random(n) < 0.6).astype(np.uint8)
    ck_len = np.zeros(n, np.int32)
    ck_slot = np.full(n, -1, np.int32)
    valid = []
    for i in range(n):
        kind = r.random()
        if kind < 0.7 and lens[i] > 0:  # a request inside the sequence
            ck_len[i] = int(r.integers(1, lens[i] + 1))
            ck_slot[i] = spare[i]
            valid.append(i)
        elif kind < 0.85:  # ignored: zero tokens, or past the end
            ck_len[i] = int(r.choice([0, lens[i] + 1 + int(r.integers(0, 20))]))
            ck_slot[i] = spare[i]
        # otherwise no request (slot -1)
    rng = wl.rng_for(80_000 + seed)
    img = wl.make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0],
                             sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lens, idx, hs, bias=bool(r.random() < 0.5),
                         long_memory=bool(r.random() < 0.3))
    inp.scale = float(r.uniform(0.5, 1.5))
    what = (f"checkpoint seed {seed}: d={d} Hk={Hk} G={G} W={W} lens={lens} "
            f"ck_len={ck_len.tolist()} ck_slot={ck_slot.tolist()} warm={hs.tolist()}")
    log(what)
    dp = DevicePool(g, [img])
    t = step_tensors(inp)
    rc = gdn.gdn_prefill_varlen_checkpoint(dp.pool, 0, inp.num_seqs, t["cu"], inp.max_seqlen,
                                           inp.total_tokens, args_of(t, inp), to_dev(ck_slot),
                                           to_dev(ck_len))
    assert rc == gdn.GDN_OK
    torch.cuda.synchronize()
    got = dp.host()
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    if inp.total_tokens:
        check_outputs(u16(t["out"]), o64, what)
    for i in valid:
        ref[ck_slot[i]] = got[ck_slot[i]]  # compared below against the prefix runs
    check_pages(g, got, ref, slots=[int(x) for x in idx], what=what)
    sub = dataclasses.replace(g, num_slots=1)
    pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
    for i in valid:
        want = oracle_prefix_page(img, inp, i, int(ck_len[i]))
        page = got[ck_slot[i]][None].copy()
        assert np.array_equal(page[0, pad], img[ck_slot[i], pad]), what
        want[0, pad] = page[0, pad]
        check_pages(sub, page, want, what=f"{what}: checkpoint of sequence {i}")


@pytest.mark.parametrize("seed", range(int(os.environ.get("GDN_CKPT_SEEDS", "8"))))
def test_random_checkpoint_restore_continue_matches_oracle(seed):
    """The prefix-cache cycle on random shapes: a prefill emits each sequence's
    state after its first c tokens into a checkpoint page, the restore copies
    the checkpoint into a fresh slot, and a second prefill continues the last
    L - c tokens there.  The continuation's outputs and final pages must be
    those of the oracle's straight run over all L tokens."""
    r = np.random.default_rng(150_000 + seed)
    d = int(r.choice([16, 32, 64, 128]))
    Hk = int(r.integers(1, 3))
    G = int(r.integers(1, 3))
    W = int(r.integers(2, 5))
    g = wl.make_geometry(32, Hk=Hk, Hv=Hk * G, dk=d, dv=d, W=W, page_align=128, extra_pad=128)
    n = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(2, 160, size=n)]
    cks = [int(r.integers(1, L)) for L in lens]  # 1 <= c < L
    perm = r.permutation(g.num_slots).astype(np.int32)
    idx, ck_slots, fresh = perm[:n], perm[n:2 * n], perm[2 * n:3 * n]
    hs = (r.random(n) < 0.5).astype(np.uint8)
    rng = wl.rng_for(151_000 + seed)
    img = wl.make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0],
                             sigma_s=0.5)
    inp = wl.step_inputs(g, rng, lens, idx, hs, bias=bool(r.random() < 0.5),
                         long_memory=bool(r.random() < 0.5))
    inp.scale = float(r.uniform(0.5, 1.5))
    what = f"cycle seed {seed}: d={d} Hk={Hk} G={G} W={W} lens={lens} cks={cks} warm={hs.tolist()}"
    log(what)
    # the oracle's straight run over all L tokens of every sequence
    ref = img.copy()
    o64, _ = oracle.gdn_layer(ref, g, inp.cu_seqlens, inp.state_indices, inp.has_initial_state,
                              inp.x, inp.conv_w, inp.conv_b, inp.alpha, inp.beta, inp.scale,
                              inp.eps)
    # 1. prefill of every sequence with its checkpoint after c tokens
    dp = DevicePool(g, [img])
    t = step_tensors(inp)
    assert gdn.gdn_prefill_varlen_checkpoint(
        dp.pool, 0, inp.num_seqs, t["cu"], inp.max_seqlen, inp.total_tokens, args_of(t, inp),
        to_dev(ck_slots), to_dev(np.array(cks, np.int32))) == gdn.GDN_OK
    # 2. restore each checkpoint into a fresh slot
    ops = np.stack([fresh, ck_slots, np.ones(n, np.int32)], axis=1).astype(np.int32)
    hs2 = to_dev(np.zeros(n, np.uint8))
    assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs2) == gdn.GDN_OK
    torch.cuda.synchronize()
    assert hs2.cpu().numpy().tolist() == [1] * n
    # 3. the last L - c tokens of each sequence, continued on the fresh slot
    cu = inp.cu_seqlens
    rows = np.concatenate([np.arange(cu[i] + cks[i], cu[i + 1]) for i in range(n)])
    rest = [L - c for L, c in zip(lens, cks)]
    cont = dataclasses.replace(inp, x=inp.x[rows], alpha=inp.alpha[rows], beta=inp.beta[rows],
                               state_indices=fresh.copy(), has_initial_state=np.ones(n, np.uint8),
                               cu_seqlens=np.concatenate([[0], np.cumsum(rest)]).astype(np.int32))
    t2 = step_tensors(cont)
    rc = gdn.gdn_prefill_varlen(dp.pool, 0, cont.num_seqs, t2["cu"], cont.max_seqlen,
                                cont.total_tokens, args_of(t2, cont))
    assert rc == gdn.GDN_OK
    torch.cuda.synchronize()
    check_outputs(u16(t2["out"]), o64[rows], f"{what}: continued outputs")
    got = dp.host()
    # the fresh slots now hold what the straight run left in the sequences' own slots
    sub = dataclasses.replace(g, num_slots=1)
    pad = slice(g.conv_off + g.conv_region_bytes, g.page_stride)
    for i in range(n):
        page = got[fresh[i]][None].copy()
        want = ref[idx[i]][None].copy()
        want[0, pad] = page[0, pad]
        assert np.array_equal(page[0, pad], img[fresh[i], pad]), what
        check_pages(sub, page, want, what=f"{what}: continued page of sequence {i}")
