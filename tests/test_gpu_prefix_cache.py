"""The prefix-cache round trip on the GPU, driven by the host slot manager
(include/gdn_slots.h) and the C-ABI kernels.

The Kapitsa page's example ("相同前缀不一定能全部复用"): a 1000-token prefix is
cached only up to token 800; a later request restores the state saved at 800
and recomputes the remaining 200.  Here, with block size 16 (800 = 50 blocks),
on a stack of [GDN, attention-only, GDN] layers:
  A: 800 tokens with a save request -> resolve reserves the promotion, the
     prefill runs, commit turns A's live slot into the checkpoint of the
     prefix and hands A a cold replacement ("Linear-State Prefix Cache 内部机制"
     §3.1-§3.2);
  B: same prefix, 800 cached KV tokens, cold slot -> resolve matches the
     checkpoint, the worker copies it across the GDN layers (§4), prefill of
     tokens 800..999 starts warm;
  C: the 1000 tokens straight.
B's outputs and final pages equal C's bit for bit; the checkpoint page is
left as it was; C matches the oracle.  Then A, cold again after its
promotion, restores its own checkpoint and takes one decode step (§5).
"""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import check_outputs, check_pages, log, to_dev, u16

pytestmark = pytest.mark.gpu

BLOCK = 16
TOTAL, CACHED = 1000, 800
H800 = 0x5EED_0800


def test_prefix_cache_round_trip_1000_tokens_checkpoint_at_800():
    g = wl.make_geometry(8, Hk=4, Hv=8, dk=128, dv=128, W=4, page_align=4096, extra_pad=4096)
    rng = wl.rng_for(11)
    layers = [0, None, 1]  # GDN, attention-only, GDN
    imgs = [None if l is None else wl.make_pool_image(g, rng, warm_slots=[], nan_slots=[])
            for l in layers]
    bufs = [None if im is None else to_dev(im) for im in imgs]
    pool = gdn.gdn_pool_create(bufs, g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                               g.W, g.Hk, g.Hv, g.dk, g.dv)
    conv = [wl.draw_conv_params(rng, g.C, g.W, bias=True) for _ in range(2)]
    xs = [wl.draw_x(rng, TOTAL, g.C) for _ in range(2)]
    gates = [wl.draw_gates(rng, TOTAL, g.Hv) for _ in range(2)]
    gdn_layers = [0, 2]

    def forward(slot, hs, t0, t1):
        """Prefill tokens [t0, t1) of the request on every GDN layer."""
        outs = []
        for j, l in enumerate(gdn_layers):
            out = torch.empty((t1 - t0, g.Hv, g.dv), dtype=torch.int16, device="cuda")
            args = gdn.make_step_args(to_dev(xs[j][t0:t1]), to_dev(conv[j][0]), to_dev(conv[j][1]),
                                      to_dev(gates[j][0][t0:t1]), to_dev(gates[j][1][t0:t1]),
                                      to_dev(np.array([slot], np.int32)), hs, out, 1.0, 1e-6)
            cu = to_dev(np.array([0, t1 - t0], np.int32))
            assert gdn.gdn_prefill_varlen(pool, l, 1, cu, t1 - t0, t1 - t0, args) == gdn.GDN_OK
            outs.append(out)
        return outs

    def worker(ops):
        """The worker side of a step: default warm bits, then the restore copies."""
        hs = to_dev(np.array([o["has_initial_state"] for o in ops], np.uint8))
        rc = gdn.gdn_restore_slots(pool, gdn.gdn_slots_restore_ops(ops), hs)
        assert rc == gdn.GDN_OK
        return hs

    m = gdn.gdn_slots_create(g.num_slots, BLOCK)
    a0 = gdn.gdn_slots_add_sequence(m, 1)
    # A: 800 tokens, save the prefix
    log("A: prefill 800 tokens with a save request")
    ops = gdn.gdn_slots_resolve(m, [(1, 0, CACHED, 0, H800)])
    assert ops[0]["save_dst_slot_id"] == a0 and ops[0]["has_initial_state"] == 0
    forward(a0, worker(ops), 0, CACHED)
    gdn.gdn_slots_commit(m)
    assert gdn.gdn_slots_lookup(m, H800) == a0
    a1, a1_init = gdn.gdn_slots_sequence_info(m, 1)
    assert a1 != a0 and a1_init == 0
    torch.cuda.synchronize()
    ckpt_pages = [bufs[l][a0].clone() for l in gdn_layers]
    # B: same prefix, restores it, computes 200 more
    b = gdn.gdn_slots_add_sequence(m, 2)
    log("B: restore the 800-token checkpoint, prefill 200 tokens")
    ops = gdn.gdn_slots_resolve(m, [(2, CACHED, TOTAL, H800, 0)])
    assert ops[0]["restore_src_slot_id"] == a0 and ops[0]["linear_state_id"] == b
    hs_b = worker(ops)
    out_b = forward(b, hs_b, CACHED, TOTAL)
    gdn.gdn_slots_commit(m)
    assert hs_b.cpu().numpy().tolist() == [1]
    # C: straight
    c = gdn.gdn_slots_add_sequence(m, 3)
    log("C: prefill 1000 tokens straight")
    ops = gdn.gdn_slots_resolve(m, [(3, 0, TOTAL, 0, 0)])
    out_c = forward(c, worker(ops), 0, TOTAL)
    gdn.gdn_slots_commit(m)
    torch.cuda.synchronize()
    for j, l in enumerate(gdn_layers):
        assert torch.equal(out_b[j], out_c[j][CACHED:]), f"layer {l}: restored outputs differ"
        assert torch.equal(bufs[l][b], bufs[l][c]), f"layer {l}: final pages differ"
        assert torch.equal(bufs[l][a0], ckpt_pages[j]), f"layer {l}: checkpoint page changed"
    # C against the oracle, first GDN layer
    log("oracle: 1000 tokens")
    sub = dataclasses.replace(g, num_slots=1)
    ref = np.full((1, g.page_stride), wl.PAD_BYTE, np.uint8)
    o64, _ = oracle.gdn_layer(ref, sub, np.array([0, TOTAL], np.int32), np.zeros(1, np.int32),
                              np.zeros(1, np.uint8), xs[0], conv[0][0], conv[0][1], gates[0][0],
                              gates[0][1])
    e = check_outputs(u16(out_c[0]), o64, "straight run")
    check_pages(sub, bufs[0][c:c + 1].cpu().numpy(), ref, what="straight run")
    log(f"straight run vs oracle: worst rel err {e:.2e}")
    # A is cold after its promotion: it restores its own checkpoint, one decode step
    log("A: restore its own checkpoint, decode token 800")
    ops = gdn.gdn_slots_resolve(m, [(1, CACHED, CACHED + 1, H800, 0)])
    assert ops[0]["linear_state_id"] == a1 and ops[0]["restore_src_slot_id"] == a0
    hs_a = worker(ops)
    for j, l in enumerate(gdn_layers):
        out = torch.empty((1, g.Hv, g.dv), dtype=torch.int16, device="cuda")
        t = slice(CACHED, CACHED + 1)
        args = gdn.make_step_args(to_dev(xs[j][t]), to_dev(conv[j][0]), to_dev(conv[j][1]),
                                  to_dev(gates[j][0][t]), to_dev(gates[j][1][t]),
                                  to_dev(np.array([a1], np.int32)), hs_a, out, 1.0, 1e-6)
        assert gdn.gdn_decode_step(pool, l, 1, args) == gdn.GDN_OK
        torch.cuda.synchronize()
        check_outputs(u16(out), wl.bf16_bits_to_f32(u16(out_c[j][CACHED:CACHED + 1]))
                      .astype(np.float64), f"layer {l}: decode after restore")
    gdn.gdn_slots_commit(m)
    assert gdn.gdn_slots_sequence_info(m, 1) == (a1, 1)
    gdn.gdn_slots_destroy(m)
