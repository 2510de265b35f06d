"""Helpers for the GPU parity tests: device pools built from host page images,
calls through the C-ABI binding, and the comparisons against the oracle.

Tolerances (applied per state tile and per output vector):
  state  : max |S_gpu - S_ref| <= 1e-4 * max |S_ref| over each (slot, head) tile
  output : max |o_gpu - o_ref| <= 2e-2 * max |o_ref| + 1e-6 over each (token, head)
  window, padding, untouched pages, restore / gather / scatter: bit-exact
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import hybrid_linear_attention_slot_amd as gdn
import workloads as wl

STATE_RTOL = 1e-4
OUT_RTOL = 2e-2
OUT_ATOL = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DevicePool:
    """One device buffer per layer (None = attention-only) + the pool handle."""

    def __init__(self, g: wl.Geometry, images):
        self.g = g
        self.bufs = [None if im is None else to_dev(im.reshape(g.num_slots, g.page_stride))
                     for im in images]
        self.pool = gdn.gdn_pool_create(self.bufs, g.num_slots, g.page_stride, g.conv_off,
                                        g.ssm_off, g.C, g.W, g.Hk, g.Hv, g.dk, g.dv)

    def host(self, layer: int = 0) -> np.ndarray:
        return self.bufs[layer].cpu().numpy()


def step_tensors(inp: wl.StepInputs):
    g = inp.geom
    t = dict(x=to_dev(inp.x), conv_w=to_dev(inp.conv_w),
             conv_b=None if inp.conv_b is None else to_dev(inp.conv_b),
             alpha=to_dev(inp.alpha), beta=to_dev(inp.beta),
             state_indices=to_dev(inp.state_indices),
             has_initial_state=to_dev(inp.has_initial_state),
             cu=to_dev(inp.cu_seqlens))
    t["out"] = torch.full((inp.total_tokens, g.Hv, g.dv), 0x7FC0, dtype=torch.int16,
                          device="cuda")  # NaN sentinel: every output must be written
    return t


def args_of(t, inp):
    return gdn.make_step_args(t["x"], t["conv_w"], t["conv_b"], t["alpha"], t["beta"],
                              t["state_indices"], t["has_initial_state"], t["out"],
                              inp.scale, inp.eps)


def run_prefill(dp: DevicePool, layer: int, inp: wl.StepInputs, t=None):
    t = t or step_tensors(inp)
    rc = gdn.gdn_prefill_varlen(dp.pool, layer, inp.num_seqs, t["cu"], inp.max_seqlen,
                                inp.total_tokens, args_of(t, inp))
    assert rc == gdn.GDN_OK
    return t


def run_decode(dp: DevicePool, layer: int, inp: wl.StepInputs, t=None):
    assert (np.diff(inp.cu_seqlens) == 1).all()
    t = t or step_tensors(inp)
    rc = gdn.gdn_decode_step(dp.pool, layer, inp.num_seqs, args_of(t, inp))
    assert rc == gdn.GDN_OK
    return t


def check_outputs(o16_gpu: np.ndarray, o64_ref: np.ndarray, what=""):
    o = wl.bf16_bits_to_f32(o16_gpu).astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite outputs"
    ref_max = np.abs(o64_ref).max(axis=-1)
    err = np.abs(o - o64_ref).max(axis=-1)
    bad = err > OUT_RTOL * ref_max + OUT_ATOL
    assert not bad.any(), (f"{what}: {bad.sum()} output vectors off; worst rel "
                           f"{(err / np.maximum(ref_max, 1e-30)).max():.3e}")
    return float((err / np.maximum(ref_max, 1e-30)).max())


def check_pages(g: wl.Geometry, got: np.ndarray, ref: np.ndarray, slots=None, what=""):
    """Pages in `slots` (default: all): window and padding bit-exact, state within
    tolerance per head tile; every other page bit-exact."""
    slots = set(range(g.num_slots)) if slots is None else set(int(s) for s in slots)
    worst = 0.0
    for s in range(g.num_slots):
        a, b = got[s], ref[s]
        if s not in slots:
            assert np.array_equal(a, b), f"{what}: untouched page {s} changed"
            continue
        sreg = slice(g.ssm_off, g.ssm_off + g.ssm_region_bytes)
        mask = np.ones(g.page_stride, bool)
        mask[sreg] = False
        assert np.array_equal(a[mask], b[mask]), f"{what}: window/padding of page {s} differs"
        sa = a[sreg].view(np.float32).reshape(g.Hv, -1).astype(np.float64)
        sb = b[sreg].view(np.float32).reshape(g.Hv, -1).astype(np.float64)
        assert np.isfinite(sa).all() == np.isfinite(sb).all()
        if not np.isfinite(sb).all():
            assert np.array_equal(a[sreg], b[sreg])
            continue
        err = np.abs(sa - sb).max(axis=1)
        mx = np.abs(sb).max(axis=1)
        assert (err <= STATE_RTOL * mx + 1e-30).all(), (
            f"{what}: state of page {s} off, worst rel {(err / np.maximum(mx, 1e-30)).max():.3e}")
        worst = max(worst, float((err / np.maximum(mx, 1e-30)).max()))
    return worst
