"""Continuation at scale on the GPU (through the C-ABI).

24 GDN layers of 32 v-heads x 128x128 fp32 in one 512-slot pool with 4 KiB of
sentinel padding per page.  64 sequences of 1000 tokens each run
  X: 1000 tokens straight from a cold start, and
  A -> B: 768 tokens (a block-aligned checkpoint, block size 256), a
          cross-layer restore of every A slot into a fresh B slot, then the
          remaining 232 tokens on B,
while 192 decode rows on slots of their own take one decode step on every
layer beside each of the four phases.  Odd layers use the long-memory gate
(alpha = exp(-0.01 softplus(z))) so that the final state depends on the
restored one.

Checked:
  - B's outputs for tokens 768..999 and B's final pages equal X's bit for bit
    (every layer), and B's pages right after the restore equal A's;
  - the straight run against the oracle (8 sequences on layer 0 and 8 on
    layer 23: every output and the final pages);
  - the decode rows against the oracle after their four steps (layers 0, 23);
  - padding and the slots no phase names are unchanged.
Inputs are drawn on the device from seeded generators (the host oracle gets
copies of the parts it checks).
"""
import dataclasses

import numpy as np
import pytest
import torch

import hybrid_linear_attention_slot_amd as gdn
import oracle
import workloads as wl
from gpu_util import check_outputs, check_pages, log

pytestmark = pytest.mark.gpu

N_LAYERS = 24
N_SEQ = 64
SEQ_LEN = 1000
SPLIT = 768
N_DEC = 192
ORACLE_LAYERS = (0, 23)
ORACLE_SEQS = 8


def _np(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def test_continuation_at_scale_with_decode_rows():
    g = wl.decode_geometry(num_slots=512, extra_pad=4096)
    rng = wl.rng_for(5)
    perm = rng.permutation(g.num_slots).astype(np.int32)
    X, A, B = perm[:N_SEQ], perm[N_SEQ:2 * N_SEQ], perm[2 * N_SEQ:3 * N_SEQ]
    D = perm[3 * N_SEQ:3 * N_SEQ + N_DEC]
    unused = perm[3 * N_SEQ + N_DEC:]
    conv = [wl.draw_conv_params(rng, g.C, g.W, bias=(l % 3 == 0)) for l in range(N_LAYERS)]
    long_mem = [l % 2 == 1 for l in range(N_LAYERS)]

    log(f"continuation: allocating {N_LAYERS} x {g.pool_bytes / 2**30:.2f} GiB")
    bufs = []
    for l in range(N_LAYERS):
        gen = wl.device_generator(5, l, 0)
        b = torch.randint(0, 256, (g.num_slots, g.page_stride), dtype=torch.uint8,
                          device="cuda", generator=gen)
        b[:, g.conv_off + g.conv_region_bytes:] = wl.PAD_BYTE
        wl.device_fill_nan(b, g, np.concatenate([X, A]))
        wl.device_fill_warm(b, g, D, gen)
        bufs.append(b)
    pool = gdn.gdn_pool_create(bufs, g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                               g.W, g.Hk, g.Hv, g.dk, g.dv)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(  # noqa: E731
        a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    cw = [dev(c[0]) for c in conv]
    cb = [None if c[1] is None else dev(c[1]) for c in conv]
    unused_t = torch.from_numpy(unused.astype(np.int64)).cuda()
    unused_before = [bufs[l][unused_t].clone() for l in ORACLE_LAYERS]
    d_t = torch.from_numpy(D.astype(np.int64)).cuda()
    d_pages0 = {l: _np(bufs[l][d_t]) for l in ORACLE_LAYERS}

    def seq_inputs(l):
        gen = wl.device_generator(5, l, 1)
        x = wl.device_x(gen, N_SEQ * SEQ_LEN, g.C)
        a, b = wl.device_gates(gen, N_SEQ * SEQ_LEN, g.Hv, long_mem[l])
        return x, a, b

    def dec_inputs(l, phase):
        gen = wl.device_generator(5, l, 2, phase)
        x = wl.device_x(gen, N_DEC, g.C)
        a, b = wl.device_gates(gen, N_DEC, g.Hv, long_mem[l])
        return x, a, b

    def tokens(t, t0, t1):  # rows [t0, t1) of every sequence, contiguous
        return t.view(N_SEQ, SEQ_LEN, *t.shape[1:])[:, t0:t1].reshape(-1, *t.shape[1:]) \
            .contiguous()

    def prefill(l, x, a, b, slots, hs, seg_len):
        out = torch.empty((x.shape[0], g.Hv, g.dv), dtype=torch.int16, device="cuda")
        cu = torch.arange(N_SEQ + 1, dtype=torch.int32, device="cuda") * seg_len
        args = gdn.make_step_args(x, cw[l], cb[l], a, b, dev(slots),
                                  dev(np.full(N_SEQ, hs, np.uint8)), out, 1.0, 1e-6)
        assert gdn.gdn_prefill_varlen(pool, l, N_SEQ, cu, seg_len, x.shape[0], args) == gdn.GDN_OK
        return out

    dec_out = {l: [] for l in ORACLE_LAYERS}

    def decode_phase(phase):
        for l in range(N_LAYERS):
            x, a, b = dec_inputs(l, phase)
            out = torch.empty((N_DEC, g.Hv, g.dv), dtype=torch.int16, device="cuda")
            args = gdn.make_step_args(x, cw[l], cb[l], a, b, dev(D),
                                      dev(np.ones(N_DEC, np.uint8)), out, 1.0, 1e-6)
            assert gdn.gdn_decode_step(pool, l, N_DEC, args) == gdn.GDN_OK
            if l in dec_out:
                dec_out[l].append(out)

    # phase 1: X straight
    log("phase 1: 64 x 1000 tokens straight on every layer")
    tail_x, full_x = [], {}
    for l in range(N_LAYERS):
        x, a, b = seq_inputs(l)
        out = prefill(l, x, a, b, X, 0, SEQ_LEN)
        tail_x.append(tokens(out, SPLIT, SEQ_LEN))
        if l in ORACLE_LAYERS:
            full_x[l] = out
    decode_phase(0)
    # phase 2: A, first 768 tokens
    log("phase 2: 64 x 768 tokens on the A slots")
    for l in range(N_LAYERS):
        x, a, b = seq_inputs(l)
        prefill(l, tokens(x, 0, SPLIT), tokens(a, 0, SPLIT), tokens(b, 0, SPLIT), A, 0, SPLIT)
    decode_phase(1)
    a_t = torch.from_numpy(A.astype(np.int64)).cuda()
    b_t = torch.from_numpy(B.astype(np.int64)).cuda()
    x_t = torch.from_numpy(X.astype(np.int64)).cuda()
    a_pages = [bufs[l][a_t].clone() for l in range(N_LAYERS)]
    # phase 3: restore A -> B on every layer
    log("phase 3: restore 64 ops over 24 layers")
    hs = torch.zeros(N_SEQ, dtype=torch.uint8, device="cuda")
    rc = gdn.gdn_restore_slots(pool, [(int(d), int(s), 1) for d, s in zip(B, A)], hs)
    assert rc == gdn.GDN_OK
    torch.cuda.synchronize()
    assert hs.cpu().numpy().tolist() == [1] * N_SEQ
    pay = g.conv_off + g.conv_region_bytes
    for l in range(N_LAYERS):
        got_b = bufs[l][b_t]
        assert torch.equal(got_b[:, :pay], a_pages[l][:, :pay]), f"layer {l}: restore payload"
        assert bool((got_b[:, pay:] == wl.PAD_BYTE).all()), f"layer {l}: restore touched padding"
        assert torch.equal(bufs[l][a_t], a_pages[l]), f"layer {l}: restore changed its source"
    decode_phase(2)
    # phase 4: B, tokens 768..999
    log("phase 4: 64 x 232 tokens on the B slots")
    for l in range(N_LAYERS):
        x, a, b = seq_inputs(l)
        out = prefill(l, tokens(x, SPLIT, SEQ_LEN), tokens(a, SPLIT, SEQ_LEN),
                      tokens(b, SPLIT, SEQ_LEN), B, 1, SEQ_LEN - SPLIT)
        assert torch.equal(out, tail_x[l]), f"layer {l}: restored continuation differs"
        assert torch.equal(bufs[l][b_t], bufs[l][x_t]), f"layer {l}: final pages differ"
    decode_phase(3)
    torch.cuda.synchronize()
    log("GPU straight == restored continuation on all 24 layers (bit-exact)")

    # oracle: the straight run on a sample of sequences, and the decode rows
    oracle.set_threads(16)
    for l in ORACLE_LAYERS:
        x, a, b = seq_inputs(l)
        sel = np.arange(ORACLE_SEQS) * (N_SEQ // ORACLE_SEQS)
        xs = _np(x.view(N_SEQ, SEQ_LEN, g.C)[sel].reshape(-1, g.C))
        as_ = _np(a.view(N_SEQ, SEQ_LEN, g.Hv)[sel].reshape(-1, g.Hv))
        bs_ = _np(b.view(N_SEQ, SEQ_LEN, g.Hv)[sel].reshape(-1, g.Hv))
        sub = dataclasses.replace(g, num_slots=ORACLE_SEQS)
        ref = np.full((ORACLE_SEQS, g.page_stride), wl.PAD_BYTE, np.uint8)
        cu = np.arange(ORACLE_SEQS + 1, dtype=np.int32) * SEQ_LEN
        log(f"oracle: layer {l}, {ORACLE_SEQS} sequences x {SEQ_LEN} tokens")
        o64, _ = oracle.gdn_layer(ref, sub, cu, np.arange(ORACLE_SEQS, dtype=np.int32),
                                  np.zeros(ORACLE_SEQS, np.uint8), xs, conv[l][0], conv[l][1],
                                  as_, bs_)
        got = _np(full_x[l]).reshape(N_SEQ, SEQ_LEN, g.Hv, g.dv)[sel]
        e = check_outputs(got.reshape(-1, g.Hv, g.dv), o64, f"straight layer {l}")
        sel_slots = torch.from_numpy(X[sel].astype(np.int64)).cuda()
        e_s = check_pages(sub, _np(bufs[l][sel_slots]), ref, what=f"straight layer {l}")
        log(f"layer {l}: worst rel err out {e:.2e} state {e_s:.2e}")
        # decode rows: four steps from the initial pages
        dref = d_pages0[l].copy()
        dsub = dataclasses.replace(g, num_slots=N_DEC)
        loc = np.arange(N_DEC, dtype=np.int32)
        for phase in range(4):
            x, a, b = dec_inputs(l, phase)
            o64, _ = oracle.decode(dref, dsub, loc, np.ones(N_DEC, np.uint8), _np(x), conv[l][0],
                                   conv[l][1], _np(a), _np(b))
            check_outputs(_np(dec_out[l][phase]), o64, f"decode rows layer {l} step {phase}")
        check_pages(dsub, _np(bufs[l][d_t]), dref, what=f"decode rows layer {l}")
    for i, l in enumerate(ORACLE_LAYERS):
        assert torch.equal(bufs[l][unused_t], unused_before[i]), f"layer {l}: unused slots"
    gdn.gdn_pool_destroy(pool)
    del bufs
    torch.cuda.empty_cache()
