"""Seeded random configurations against the oracle: head size, k-heads, v-heads
per k-head, conv width, page padding, ragged lengths (empty and one-token
sequences included), warm/cold rows, a padding row (slot out of range), conv
bias and q scale are drawn per case, for the varlen prefill and the decode
step.  Each case is small; together they cover combinations the fixed cases
do not."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DevicePool, check_outputs, check_pages, log, run_decode, run_prefill, u16

pytestmark = pytest.mark.gpu


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
@pytest.mark.parametrize("seed", range(10))
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
