"""Restore on a separate prepare stream, the forward on another stream that
waits on an event recorded after it, with no host synchronisation between
them ("Linear-State Prefix Cache 内部机制" §4.2: the worker enqueues the copy on
its prepare stream before the forward).  The decode reads the
has_initial_state bytes the restore wrote on the other stream; a prefill
continues the same sequences.  Results against the oracle's restore followed
by the same steps."""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import (DevicePool, check_outputs, check_pages, log, run_decode, run_prefill,
                      step_tensors, u16)

pytestmark = pytest.mark.gpu


def test_restore_on_prepare_stream_then_forward_on_another():
    g = wl.make_geometry(16, Hk=2, Hv=4, dk=64, dv=64, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(4242)
    live = np.arange(6, dtype=np.int32)      # the rows' live slots (NaN until restored)
    ckpt = np.arange(8, 14, dtype=np.int32)  # checkpoints
    img = wl.make_pool_image(g, rng, warm_slots=ckpt, nan_slots=live, sigma_s=0.5)
    # rows 0-3 hit, row 4 misses, row 5 asks for nothing (its hs stays 0)
    ops = np.array([[0, 8, 1], [1, 9, 1], [2, 10, 1], [3, 11, 1], [4, -1, 1], [5, 12, 0]],
                   np.int32)
    dinp = wl.step_inputs(g, rng, [1] * 6, live, np.zeros(6, np.uint8))
    pinp = wl.step_inputs(g, rng, [20, 3, 17, 1, 32, 9], live, np.ones(6, np.uint8),
                          conv=(dinp.conv_w, dinp.conv_b))

    dp = DevicePool(g, [img])
    hs = torch.zeros(6, dtype=torch.uint8, device="cuda")
    filler = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    prep, fwd = torch.cuda.Stream(), torch.cuda.Stream()
    log("restore on the prepare stream (behind a 256 MB fill), decode + prefill on another")
    with torch.cuda.stream(prep):
        filler.fill_(7)  # keeps the prepare stream busy when the forward is enqueued
        assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs, stream=prep) == gdn.GDN_OK
        done = torch.cuda.Event()
        done.record(prep)
    with torch.cuda.stream(fwd):
        fwd.wait_event(done)
        td = run_decode(dp, 0, dinp, t=_tensors(dinp, hs))
        tp = run_prefill(dp, 0, pinp)
    torch.cuda.synchronize()

    ref = img.copy()
    hs_ref = np.zeros(6, np.uint8)
    oracle.restore([ref], g, ops, hs_ref)
    assert np.array_equal(hs.cpu().numpy(), hs_ref)
    assert hs_ref.tolist() == [1, 1, 1, 1, 0, 0]
    od, _ = oracle.gdn_layer(ref, g, dinp.cu_seqlens, live, hs_ref, dinp.x, dinp.conv_w,
                             dinp.conv_b, dinp.alpha, dinp.beta, dinp.scale, dinp.eps)
    op, _ = oracle.gdn_layer(ref, g, pinp.cu_seqlens, live, pinp.has_initial_state, pinp.x,
                             pinp.conv_w, pinp.conv_b, pinp.alpha, pinp.beta, pinp.scale,
                             pinp.eps)
    check_outputs(u16(td["out"]), od, "decode after a restore on another stream")
    check_outputs(u16(tp["out"]), op, "prefill after it")
    check_pages(g, dp.host(), ref, slots=np.concatenate([live, ckpt]),
                what="pages after restore, decode and prefill on two streams")


def _tensors(inp, hs):
    """Device inputs of a decode step whose has_initial_state is `hs` (device)."""
    t = step_tensors(inp)
    t["has_initial_state"] = hs
    return t
