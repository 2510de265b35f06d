"""The bench's algorithmic byte counts (the numerator of its GB/s figures and
of the roofline) against an independent count: the sizes of the arrays a step
must read and write, and the payload regions of the pages it touches."""
import numpy as np
import pytest

import bench
import workloads as wl


def counted_bytes(inp):
    """Every input array once, every output once, each named page's payload
    read when the row starts warm and written always."""
    g = inp.geom
    payload = g.ssm_region_bytes + g.conv_region_bytes
    arrays = [inp.x, inp.conv_w, inp.alpha, inp.beta, inp.state_indices, inp.has_initial_state]
    if inp.conv_b is not None:
        arrays.append(inp.conv_b)
    out_bytes = inp.total_tokens * g.Hv * g.dv * 2  # bf16 outputs
    warm = int(np.count_nonzero(inp.has_initial_state))
    return sum(a.nbytes for a in arrays) + out_bytes + (warm + inp.num_seqs) * payload


@pytest.mark.parametrize("bias", [False, True])
def test_decode_bytes_match_the_arrays(bias):
    g = wl.make_geometry(16, Hk=2, Hv=4, dk=32, dv=32, W=4, page_align=128, extra_pad=4096)
    rng = wl.rng_for(5)
    rows = 9
    hs = (rng.random(rows) < 0.6).astype(np.uint8)
    inp = wl.step_inputs(g, rng, [1] * rows, rng.permutation(16)[:rows], hs, bias=bias)
    assert bench.decode_bytes(inp) == counted_bytes(inp)


@pytest.mark.parametrize("bias", [False, True])
def test_prefill_bytes_match_the_arrays(bias):
    g = wl.make_geometry(16, Hk=1, Hv=2, dk=64, dv=64, W=3, page_align=128)
    rng = wl.rng_for(6)
    lens = [37, 1, 0, 64, 5]
    hs = np.array([1, 0, 1, 1, 0], np.uint8)
    inp = wl.step_inputs(g, rng, lens, rng.permutation(16)[:5], hs, bias=bias)
    # the per-sequence offsets are read too (n + 1 int32)
    assert bench.prefill_bytes(inp) == counted_bytes(inp) + inp.cu_seqlens.nbytes


def test_full_size_decode_bytes():
    """The decode workload's figure quoted in the bench line."""
    inp, _ = wl.decode_workload(seed=0)
    assert bench.decode_bytes(inp) == counted_bytes(inp) == 1_060_259_072
