"""State snapshots through the C-ABI on the GPU ("Kapitsa 源码拆解 05": a disk
copy of a slot's state outlives the slot; written through a temporary file
with header and payload CRC-32C; checked when read; damaged files dropped;
loading it back and continuing the prefill is the same as never leaving).

A slot of a [GDN, attention-only, GDN] pool is saved, read back by the
oracle's parser (the payload is exactly the slot's window and state bytes of
the two GDN layers), loaded into another slot (payload equal, padding and
other pages untouched), and a prefill continued from the loaded slot gives
the same bits as one continued from the original.  A damaged file is
refused without touching the device and dropped on request; a pool with
another layout or another key is refused.
"""
import os

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import workloads as wl
from gpu_util import log, to_dev
from oracle.snapshot import parse_file

pytestmark = pytest.mark.gpu


def test_snapshot_round_trip_and_continuation(tmp_path):
    g = wl.make_geometry(8, Hk=2, Hv=4, dk=64, dv=64, W=4, page_align=4096, extra_pad=4096)
    rng = wl.rng_for(21)
    imgs = [wl.make_pool_image(g, rng, warm_slots=[3], nan_slots=[]), None,
            wl.make_pool_image(g, rng, warm_slots=[3], nan_slots=[])]
    bufs = [None if im is None else to_dev(im) for im in imgs]
    pool = gdn.gdn_pool_create(bufs, g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                               g.W, g.Hk, g.Hv, g.dk, g.dv)
    path = str(tmp_path / "st" / "slot3.snap")
    os.makedirs(os.path.dirname(path))
    log("snapshot: save slot 3")
    gdn.gdn_snapshot_save(pool, 3, key=0xC0FFEE, position=512, path=path)
    assert not os.path.exists(path + ".tmp")
    fields, payload = parse_file(open(path, "rb").read())
    assert (fields["key"], fields["position"], fields["num_linear_layers"]) == (0xC0FFEE, 512, 2)
    pay = g.conv_off + g.conv_region_bytes
    for i, l in enumerate((0, 2)):
        page = imgs[l][3]
        per = g.conv_region_bytes + g.ssm_region_bytes
        part = np.frombuffer(payload[i * per:(i + 1) * per], np.uint8)
        assert np.array_equal(part[:g.conv_region_bytes],
                              page[g.conv_off:g.conv_off + g.conv_region_bytes])
        assert np.array_equal(part[g.conv_region_bytes:],
                              page[g.ssm_off:g.ssm_off + g.ssm_region_bytes])
    log("snapshot: load into slot 6")
    before = [b.clone() for b in bufs if b is not None]
    assert gdn.gdn_snapshot_load(pool, 6, path, key=0xC0FFEE) == 512
    for j, l in enumerate((0, 2)):
        b = bufs[l]
        assert torch.equal(b[6, :pay], b[3, :pay])
        assert torch.equal(b[6, pay:], before[j][6, pay:])            # padding untouched
        others = [s for s in range(g.num_slots) if s != 6]
        assert torch.equal(b[others], before[j][others])
    # continuing the prefill from the loaded slot == from the original slot
    inp = wl.step_inputs(g, rng, [40, 40], np.array([3, 6], np.int32), np.ones(2, np.uint8))
    inp.x[40:] = inp.x[:40]
    inp.alpha[40:], inp.beta[40:] = inp.alpha[:40], inp.beta[:40]
    out = torch.empty((80, g.Hv, g.dv), dtype=torch.int16, device="cuda")
    args = gdn.make_step_args(to_dev(inp.x), to_dev(inp.conv_w), None, to_dev(inp.alpha),
                              to_dev(inp.beta), to_dev(inp.state_indices),
                              to_dev(inp.has_initial_state), out, 1.0, 1e-6)
    assert gdn.gdn_prefill_varlen(pool, 0, 2, to_dev(inp.cu_seqlens), 40, 80, args) == gdn.GDN_OK
    torch.cuda.synchronize()
    assert torch.equal(out[:40], out[40:])
    assert torch.equal(bufs[0][3, :pay], bufs[0][6, :pay])


def test_snapshot_refuses_damaged_foreign_and_other_key(tmp_path):
    g = wl.make_geometry(6, Hk=1, Hv=2, dk=16, dv=16, W=4, page_align=128, extra_pad=128)
    rng = wl.rng_for(22)
    img = wl.make_pool_image(g, rng, warm_slots=[1], nan_slots=[])
    buf = to_dev(img)
    pool = gdn.gdn_pool_create([buf], g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                               g.W, g.Hk, g.Hv, g.dk, g.dv)
    path = str(tmp_path / "s.snap")
    gdn.gdn_snapshot_save(pool, 1, key=5, position=16, path=path)
    # another key: refused, file kept
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_load(pool, 2, path, key=6)
    assert e.value.code == gdn.GDN_EINVAL and os.path.exists(path)
    # another layout (dk = 32): refused, file kept
    g2 = wl.make_geometry(6, Hk=1, Hv=2, dk=32, dv=32, W=4, page_align=128)
    buf2 = torch.zeros((g2.num_slots, g2.page_stride), dtype=torch.uint8, device="cuda")
    pool2 = gdn.gdn_pool_create([buf2], g2.num_slots, g2.page_stride, g2.conv_off, g2.ssm_off,
                                g2.C, g2.W, g2.Hk, g2.Hv, g2.dk, g2.dv)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_load(pool2, 0, path, key=5)
    assert e.value.code == gdn.GDN_EINVAL
    # one flipped payload byte: refused, device untouched; dropped on request
    blob = bytearray(open(path, "rb").read())
    blob[-3] ^= 0x40
    open(path, "wb").write(bytes(blob))
    before = buf.clone()
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_load(pool, 2, path, key=5)
    assert e.value.code == gdn.GDN_ECORRUPT and os.path.exists(path)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_snapshot_load(pool, 2, path, key=5, drop_damaged=True)
    assert e.value.code == gdn.GDN_ECORRUPT and not os.path.exists(path)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
