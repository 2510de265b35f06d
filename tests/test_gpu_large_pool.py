"""Pages past 4 GiB of one layer buffer: a 2048-slot pool of the decode
geometry (2,146,304-byte pages, 4.4 GB), whose slots from 2002 up start beyond
2^32 bytes.  Decode, varlen prefill, restore and gather/scatter through pages
on both sides of that mark must match the oracle (bit-exact for the copies),
and every other page must stay untouched."""
import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import (DevicePool, check_outputs, check_pages, log, run_decode, run_prefill,
                      to_dev, u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    g = wl.decode_geometry(num_slots=2048)
    assert 1990 * g.page_stride < 2**32 < 2002 * g.page_stride
    rng = wl.rng_for(4096)
    high = rng.permutation(np.arange(1990, 2048)).astype(np.int32)  # both sides of the mark
    warm = high[::2]
    # pages not named keep the sentinel bytes (filling 4 GB with random bytes
    # would only slow the test down)
    img = wl.make_pool_image(g, rng, warm_slots=warm, nan_slots=high[1::2], other="sentinel")
    return g, rng, high, img


def oracle_layer(img, inp):
    return oracle.gdn_layer(img, inp.geom, inp.cu_seqlens, inp.state_indices,
                            inp.has_initial_state, inp.x, inp.conv_w, inp.conv_b, inp.alpha,
                            inp.beta, inp.scale, inp.eps)


def test_decode_and_prefill_beyond_4gib(big):
    g, rng, high, img = big
    hs_of = lambda s: np.array([1 if (high[::2] == x).any() else 0 for x in s], np.uint8)  # noqa: E731
    dslots = high[:24]
    dinp = wl.step_inputs(g, rng, [1] * len(dslots), dslots, hs_of(dslots))
    pslots = high[24:28]
    pinp = wl.step_inputs(g, rng, [37, 16, 3, 50], pslots, hs_of(pslots))
    dp = DevicePool(g, [img])
    log(f"decode {len(dslots)} rows and prefill {pinp.total_tokens} tokens in slots "
        f"{int(high.min())}..{int(high.max())} of a {g.num_slots}-slot pool")
    td = run_decode(dp, 0, dinp)
    tp = run_prefill(dp, 0, pinp)
    torch.cuda.synchronize()
    ref = img.copy()
    od, _ = oracle_layer(ref, dinp)
    op, _ = oracle_layer(ref, pinp)
    check_outputs(u16(td["out"]), od, "decode beyond 4 GiB")
    check_outputs(u16(tp["out"]), op, "prefill beyond 4 GiB")
    got = dp.host()
    del dp
    torch.cuda.empty_cache()
    check_pages(g, got, ref, slots=np.concatenate([dslots, pslots]), what="beyond 4 GiB")


def test_restore_gather_scatter_beyond_4gib(big):
    g, rng, high, img = big
    # restore: high -> low, low -> high, high -> high; a miss
    ops = np.array([[100, int(high[0]), 1], [int(high[1]), 7, 1], [int(high[2]), int(high[3]), 1],
                    [int(high[4]), -1, 1]], np.int32)
    hs0 = np.array([0, 0, 0, 1], np.uint8)
    dp = DevicePool(g, [img])
    hs = to_dev(hs0)
    log("restore across the 4 GiB mark")
    assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs) == gdn.GDN_OK
    # gather four high pages, scatter them back shifted by one
    gidx = high[5:9].astype(np.int32)
    ssm = torch.empty((4, g.ssm_region_bytes), dtype=torch.uint8, device="cuda")
    conv = torch.empty((4, g.conv_region_bytes), dtype=torch.uint8, device="cuda")
    gdn.gdn_gather_states(dp.pool, 0, to_dev(gidx), 4, conv, ssm)
    sidx = np.roll(gidx, 1).astype(np.int32)
    gdn.gdn_scatter_states(dp.pool, 0, to_dev(sidx), 4, conv, ssm)
    torch.cuda.synchronize()
    ref = img.copy()
    h_ref = hs0.copy()
    oracle.restore([ref], g, ops, h_ref)
    gs, gc = oracle.gather(ref, g, gidx)
    assert np.array_equal(ssm.cpu().numpy(), gs) and np.array_equal(conv.cpu().numpy(), gc)
    oracle.scatter(ref, g, sidx, gs, gc)
    assert np.array_equal(hs.cpu().numpy(), h_ref)
    got = dp.host()
    del dp
    torch.cuda.empty_cache()
    assert np.array_equal(got, ref), "pool differs from the oracle after restore/gather/scatter"
