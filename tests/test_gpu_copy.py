"""GPU parity of restore / gather / scatter against the oracle: bit-exact,
padding and unselected pages included (via the C-ABI).  Seeded random cases
(GDN_COPY_SEEDS, default 8) draw the page layout, the layer stack, the ops and
the dense rows' alignment."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import DevicePool, log, to_dev

pytestmark = pytest.mark.gpu


def test_block_stride_example_on_gpu():
    """The page's worked example: 48 bf16 per block in 128-byte pages; every
    call touches elements [64 s, 64 s + 48) of the slots it names only."""
    g = wl.Geometry(num_slots=6, C=16, W=4, Hk=0, Hv=0, dk=0, dv=0, page_stride=128, ssm_off=0,
                    conv_off=0)
    img = np.arange(6 * 64, dtype=np.uint16).view(np.uint8).reshape(6, 128).copy()
    dp = DevicePool(g, [img])
    idx = to_dev(np.arange(6, dtype=np.int32))
    dense = torch.zeros((6, 96), dtype=torch.uint8, device="cuda")
    log("gather 48-element blocks")
    gdn.gdn_gather_states(dp.pool, 0, idx, 6, dense, None)
    torch.cuda.synchronize()
    got = dense.cpu().numpy().view(np.uint16)
    for s in range(6):
        assert np.array_equal(got[s], np.arange(64 * s, 64 * s + 48))
    # scatter into slots 1 and 4, restore 5 -> 2
    src = torch.full((2, 96), 0xFF, dtype=torch.uint8, device="cuda")
    gdn.gdn_scatter_states(dp.pool, 0, to_dev(np.array([1, 4], np.int32)), 2, src, None)
    hs = torch.zeros(1, dtype=torch.uint8, device="cuda")
    assert gdn.gdn_restore_slots(dp.pool, [(2, 5, 1)], hs) == gdn.GDN_OK
    torch.cuda.synchronize()
    ref = img.copy()
    oracle.scatter(ref, g, np.array([1, 4]), np.zeros((2, 0), np.uint8),
                   np.full((2, 96), 0xFF, np.uint8))
    h_ref = np.zeros(1, np.uint8)
    oracle.restore([ref], g, np.array([[2, 5, 1]]), h_ref)
    assert np.array_equal(dp.host(), ref)
    assert hs.cpu().numpy()[0] == h_ref[0] == 1


def tiny_layers(seed, n_layers, attention):
    g = wl.tiny_geometry(extra_pad=128)
    rng = wl.rng_for(seed)
    imgs = [None if l in attention else wl.make_pool_image(g, rng, range(8), [])
            for l in range(n_layers)]
    return g, imgs


def test_restore_truth_table_matches_oracle():
    g, imgs = tiny_layers(40, 4, attention=(1, 3))
    dp = DevicePool(g, imgs)
    ops = np.array([[0, 3, 0], [4, -1, 1], [1, 5, 1], [2, 5, 1], [6, 7, 1]], np.int32)
    hs0 = np.array([1, 1, 0, 0, 0], np.uint8)
    hs = to_dev(hs0)
    log("restore truth table")
    assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs) == gdn.GDN_OK
    torch.cuda.synchronize()
    ref = [None if im is None else im.copy() for im in imgs]
    h_ref = hs0.copy()
    assert oracle.restore(ref, g, ops, h_ref) == 0
    assert np.array_equal(hs.cpu().numpy(), h_ref)
    for l in (0, 2):
        assert np.array_equal(dp.host(l), ref[l])


def test_restore_soft_failure_all_attention():
    g = wl.tiny_geometry()
    dp = DevicePool(g, [None, None])
    hs = to_dev(np.array([1, 1, 1], np.uint8))
    rc = gdn.gdn_restore_slots(dp.pool, [(0, 3, 1), (1, -1, 1), (2, 4, 0)], hs)
    torch.cuda.synchronize()
    assert rc == gdn.GDN_WARN_COLD_FALLBACK
    assert hs.cpu().numpy().tolist() == [0, 0, 1]


def test_restore_many_ops_and_layers_split_launches():
    """More hits and GDN layers than one launch carries (kernel-argument
    budget: 64 layers, 96 pairs, 96 hs entries): 100 layers of which 75 are
    GDN layers and ~135 hits, so launches split over both the pairs and the
    layers (a layer chunk starting at layer 64 of the GDN list)."""
    g = wl.make_geometry(400, Hk=1, Hv=2, dk=16, dv=16, W=4, page_align=128, extra_pad=256)
    rng = wl.rng_for(41)
    n_layers = 100
    imgs = [None if l % 4 == 3 else rng.integers(0, 256, (g.num_slots, g.page_stride),
                                                dtype=np.uint8) for l in range(n_layers)]
    dp = DevicePool(g, imgs)
    perm = rng.permutation(g.num_slots)
    n = 200
    dst, pool_src = perm[:n], perm[n:]
    src = np.where(rng.random(n) < 0.25, -1, rng.choice(pool_src, n))
    req = (rng.random(n) < 0.9).astype(np.int32)
    ops = np.stack([dst, src, req], axis=1).astype(np.int32)
    hs0 = rng.integers(0, 2, n).astype(np.uint8)
    hs = to_dev(hs0)
    hits = int(((src >= 0) & (req != 0)).sum())
    n_gdn = sum(im is not None for im in imgs)
    assert hits > 96 and n_gdn > 64, (hits, n_gdn)
    log(f"restore {n} ops ({hits} hits) x {n_layers} layers ({n_gdn} GDN)")
    assert gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs) == gdn.GDN_OK
    torch.cuda.synchronize()
    ref = [None if im is None else im.copy() for im in imgs]
    h_ref = hs0.copy()
    oracle.restore(ref, g, ops, h_ref)
    assert np.array_equal(hs.cpu().numpy(), h_ref)
    for l in range(n_layers):
        if ref[l] is not None:
            assert np.array_equal(dp.host(l), ref[l]), l


@pytest.mark.parametrize("geom", ["tiny", "decode"])
def test_gather_scatter_match_oracle(geom):
    if geom == "tiny":
        g = wl.tiny_geometry(extra_pad=128)
    else:
        g = wl.decode_geometry(num_slots=24, extra_pad=4096)
    rng = wl.rng_for(42)
    img = rng.integers(0, 256, (g.num_slots, g.page_stride), dtype=np.uint8)
    dp = DevicePool(g, [img])
    idx = np.array([3, -1, 7, g.num_slots, 0, 5], np.int32)
    n = len(idx)
    sd = torch.full((n, g.ssm_region_bytes), 0x5A, dtype=torch.uint8, device="cuda")
    cd = torch.full((n, g.conv_region_bytes), 0x5A, dtype=torch.uint8, device="cuda")
    log(f"gather/scatter {geom}")
    gdn.gdn_gather_states(dp.pool, 0, to_dev(idx), n, cd, sd)
    torch.cuda.synchronize()
    rs, rc_ = oracle.gather(img, g, idx)
    assert np.array_equal(sd.cpu().numpy(), rs)
    assert np.array_equal(cd.cpu().numpy(), rc_)
    new_s = rng.integers(0, 256, rs.shape, dtype=np.uint8)
    new_c = rng.integers(0, 256, rc_.shape, dtype=np.uint8)
    gdn.gdn_scatter_states(dp.pool, 0, to_dev(idx), n, to_dev(new_c), to_dev(new_s))
    torch.cuda.synchronize()
    ref = img.copy()
    oracle.scatter(ref, g, idx, new_s, new_c)
    assert np.array_equal(dp.host(), ref)


def test_gather_unaligned_dense_rows():
    """Region sizes that are not a multiple of 16 bytes use the element path."""
    # conv-window-only pool: 2 x 10 bf16 = 40 bytes per page
    g = wl.Geometry(num_slots=6, C=10, W=3, Hk=0, Hv=0, dk=0, dv=0, page_stride=128, ssm_off=0,
                    conv_off=0)
    rng = wl.rng_for(43)
    img = rng.integers(0, 256, (g.num_slots, g.page_stride), dtype=np.uint8)
    dp = DevicePool(g, [img])
    idx = np.array([5, 1, 2], np.int32)
    cd = torch.zeros((3, g.conv_region_bytes), dtype=torch.uint8, device="cuda")
    assert g.conv_region_bytes % 16 != 0
    gdn.gdn_gather_states(dp.pool, 0, to_dev(idx), 3, cd, None)
    torch.cuda.synchronize()
    _, rc_ = oracle.gather(img, g, idx)
    assert np.array_equal(cd.cpu().numpy(), rc_)
    new_c = rng.integers(0, 256, rc_.shape, dtype=np.uint8)
    gdn.gdn_scatter_states(dp.pool, 0, to_dev(idx), 3, to_dev(new_c), None)
    torch.cuda.synchronize()
    ref = img.copy()
    oracle.scatter(ref, g, idx, np.zeros((3, 0), np.uint8), new_c)
    assert np.array_equal(dp.host(), ref)


def _layer_image(g, l):
    """Layer l's initial pool on the device, regenerated identically on demand:
    random bytes everywhere, the 4 KiB of padding after each payload included
    (every page's padding differs from every other's, so a copy that strays
    into the padding changes bytes)."""
    gen = torch.Generator(device="cuda").manual_seed(1000 + l)
    return torch.randint(0, 256, (g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda",
                         generator=gen)


@pytest.mark.slow
def test_restore_gather_scatter_full_hybrid_stack():
    """64-layer stack (every 4th layer attention-only), 48 GDN layers of 32 heads
    x 128x128 fp32 + 8192-channel windows, 1024 slots with 4 KiB of padding
    per page (random bytes), 64 ops with a quarter misses.  Every GDN layer is checked:
    the touched pages against the oracle's restore of the layer's initial
    pages, every other page unchanged.  Then, on every GDN layer, the 64 op rows
    are gathered to dense rows (against the oracle's gather) and scattered into
    64 other slots (against the oracle's scatter, padding untouched)."""
    g, linear, ops = wl.restore_workload(seed=0)
    n_layers = len(linear)
    gdn_layers = [l for l in range(n_layers) if linear[l]]
    log(f"allocating {len(gdn_layers)} x {g.pool_bytes / 2**30:.1f} GiB")
    bufs = [_layer_image(g, l) if linear[l] else None for l in range(n_layers)]
    pool = gdn.gdn_pool_create(bufs, g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                               g.W, g.Hk, g.Hv, g.dk, g.dv)
    hits = ops[:, 1] >= 0
    rng = wl.rng_for(5)
    dsts = ops[:, 0]
    used = set(dsts.tolist()) | set(ops[hits, 1].tolist())
    others = np.array([s_ for s_ in rng.permutation(g.num_slots) if s_ not in used][:64], np.int32)
    touched = np.unique(np.concatenate([dsts, ops[hits, 1], others])).astype(np.int64)
    remap = {int(s_): i for i, s_ in enumerate(touched)}
    small = dataclasses.replace(g, num_slots=len(touched))
    ops_small = np.array([[remap[d], remap[s_] if s_ >= 0 else -1, r] for d, s_, r in ops],
                         np.int32)
    t_idx = torch.from_numpy(touched).cuda()
    hs = torch.ones(len(ops), dtype=torch.uint8, device="cuda")
    log("restore 64 ops x 48 layers")
    assert gdn.gdn_restore_slots(pool, ops.tolist(), hs) == gdn.GDN_OK
    torch.cuda.synchronize()
    h = hs.cpu().numpy()
    assert h.tolist() == hits.astype(np.uint8).tolist()
    idx = torch.from_numpy(dsts.astype(np.int32)).cuda()
    idx2 = torch.from_numpy(others).cuda()
    n = len(dsts)
    cd = torch.empty((n, g.conv_region_bytes), dtype=torch.uint8, device="cuda")
    sd = torch.empty((n, g.ssm_region_bytes), dtype=torch.uint8, device="cuda")
    rev = torch.arange(n - 1, -1, -1, device="cuda")
    for l in gdn_layers:
        init = _layer_image(g, l)
        changed = torch.nonzero((bufs[l] != init).any(dim=1)).flatten().cpu().numpy()
        assert set(changed.tolist()) <= set(dsts[hits].tolist()), f"layer {l}: other pages changed"
        ref = init[t_idx].cpu().numpy()
        del init
        h = np.ones(len(ops), np.uint8)
        assert oracle.restore([ref], small, ops_small, h) == 0
        assert np.array_equal(h, hs.cpu().numpy())
        assert np.array_equal(bufs[l][t_idx].cpu().numpy(), ref), f"layer {l}: restore"
        # gather the 64 op rows
        cd.fill_(0x5A)
        sd.fill_(0x5A)
        gdn.gdn_gather_states(pool, l, idx, n, cd, sd)
        torch.cuda.synchronize()
        rs, rc_ = oracle.gather(ref, small, np.array([remap[int(d)] for d in dsts], np.int32))
        assert np.array_equal(sd.cpu().numpy(), rs), f"layer {l}: gather (state)"
        assert np.array_equal(cd.cpu().numpy(), rc_), f"layer {l}: gather (window)"
        # scatter them, in reverse order, into 64 slots no op touches
        gdn.gdn_scatter_states(pool, l, idx2, n, cd[rev].contiguous(), sd[rev].contiguous())
        torch.cuda.synchronize()
        oracle.scatter(ref, small, np.array([remap[int(s_)] for s_ in others], np.int32),
                       rs[::-1].copy(), rc_[::-1].copy())
        assert np.array_equal(bufs[l][t_idx].cpu().numpy(), ref), f"layer {l}: scatter"
        if l % 16 == 0:
            log(f"layer {l}: restore, gather and scatter match the oracle")
    log("restore, gather and scatter: all 48 GDN layers match the oracle")
    gdn.gdn_pool_destroy(pool)
    del bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(int(os.environ.get("GDN_COPY_SEEDS", "8"))))
def test_random_restore_gather_scatter_match_oracle(seed):
    r = np.random.default_rng(90_000 + seed)
    num_slots = int(r.integers(24, 121))
    if r.random() < 0.25:  # window-only pool, window bytes often not a multiple of 16
        C, W = 2 * int(r.integers(1, 20)), int(r.integers(2, 5))  # C is even
        stride = wl.round_up((W - 1) * C * 2, 16) + 16 * int(r.integers(0, 8))
        g = wl.Geometry(num_slots=num_slots, C=C, W=W, Hk=0, Hv=0, dk=0, dv=0,
                        page_stride=stride, ssm_off=0, conv_off=0)
    else:
        d = int(r.choice([16, 32]))
        Hk = int(r.integers(1, 3))
        g = wl.make_geometry(num_slots, Hk=Hk, Hv=Hk * int(r.integers(1, 3)), dk=d, dv=d,
                             W=int(r.integers(2, 5)), page_align=128,
                             extra_pad=int(r.choice([0, 16, 128, 4096])))
    n_layers = int(r.integers(1, 71))
    linear = r.random(n_layers) >= 0.3
    imgs = [r.integers(0, 256, (g.num_slots, g.page_stride), dtype=np.uint8) if lin else None
            for lin in linear]
    what = (f"copy seed {seed}: slots={num_slots} C={g.C} W={g.W} Hv={g.Hv} d={g.dk} "
            f"stride={g.page_stride} layers={n_layers} gdn={int(linear.sum())}")
    log(what)
    dp = DevicePool(g, imgs)

    # restore: distinct dst slots, src from the other slots (shared ones too), misses,
    # rows that ask for nothing, prefilled has_initial_state
    n = int(r.integers(1, min(150, num_slots // 2) + 1))
    perm = r.permutation(g.num_slots).astype(np.int32)
    dst, others = perm[:n], perm[n:]
    src = np.where(r.random(n) < 0.25, -1, r.choice(others, n)).astype(np.int32)
    req = (r.random(n) < 0.85).astype(np.int32)
    ops = np.stack([dst, src, req], axis=1).astype(np.int32)
    hs0 = r.integers(0, 2, n).astype(np.uint8)
    hs = to_dev(hs0)
    rc = gdn.gdn_restore_slots(dp.pool, ops.tolist(), hs)
    torch.cuda.synchronize()
    ref = [None if im is None else im.copy() for im in imgs]
    h_ref = hs0.copy()
    want_rc = oracle.restore(ref, g, ops, h_ref)
    assert rc == (gdn.GDN_WARN_COLD_FALLBACK if want_rc else gdn.GDN_OK), what
    assert np.array_equal(hs.cpu().numpy(), h_ref), what
    for l in range(n_layers):
        if ref[l] is not None:
            assert np.array_equal(dp.host(l), ref[l]), f"{what}: restore layer {l}"
    if not linear.any():
        return

    # gather then scatter on one GDN layer: out-of-range rows, dense rows at an
    # offset of 0, 2 or 4 bytes (the element path when not 16-byte aligned)
    layer = int(r.choice(np.flatnonzero(linear)))
    m = int(r.integers(1, 40))
    idx = r.integers(-2, g.num_slots + 2, m).astype(np.int32)
    ssm_b, conv_b = g.ssm_region_bytes, g.conv_region_bytes
    off_c = int(r.choice([0, 2]))
    off_s = int(r.choice([0, 4])) if ssm_b else 0
    cbuf = torch.full((m * conv_b + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((m * ssm_b + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    cd = cbuf[off_c:off_c + m * conv_b]
    sd = sbuf[off_s:off_s + m * ssm_b] if ssm_b else None
    gdn.gdn_gather_states(dp.pool, layer, to_dev(idx), m, cd, sd)
    torch.cuda.synchronize()
    pool_now = ref[layer]
    rs, rcd = oracle.gather(pool_now, g, idx)
    assert np.array_equal(cd.cpu().numpy().reshape(m, conv_b), rcd), f"{what}: gather window"
    if ssm_b:
        assert np.array_equal(sd.cpu().numpy().reshape(m, ssm_b), rs), f"{what}: gather state"
    # the bytes around the dense rows are untouched
    assert (cbuf[:off_c].cpu().numpy() == 0x5A).all() and \
        (cbuf[off_c + m * conv_b:].cpu().numpy() == 0x5A).all(), what
    new_s = r.integers(0, 256, rs.shape, dtype=np.uint8)
    new_c = r.integers(0, 256, rcd.shape, dtype=np.uint8)
    cd.copy_(torch.from_numpy(new_c.reshape(-1)).cuda())
    if ssm_b:
        sd.copy_(torch.from_numpy(new_s.reshape(-1)).cuda())
    # scatter needs distinct in-range rows; repeated slots keep the last writer
    # undefined, so the scatter uses the first occurrence of each slot only
    keep = np.zeros(m, bool)
    seen = set()
    for i, s_ in enumerate(idx.tolist()):
        if s_ not in seen:
            keep[i] = True
            seen.add(s_)
    sidx = np.where(keep, idx, -1).astype(np.int32)
    gdn.gdn_scatter_states(dp.pool, layer, to_dev(sidx), m, cd, sd)
    torch.cuda.synchronize()
    oracle.scatter(pool_now, g, sidx, new_s, new_c)
    assert np.array_equal(dp.host(layer), pool_now), f"{what}: scatter"
