"""Seeded synthetic inputs for the slot-indexed Gated DeltaNet state path.

This module only draws numbers and lays bytes out; it holds none of the
method's arithmetic (no conv, no norm, no delta rule, no copy semantics).
Both the CPU oracle and the HIP path consume what it produces, so the two
sides always see the same bytes.

Distributions (the configurations fix x, alpha and beta; the rest is a plain
choice of scale):
  x (pre-conv mixed q|k|v input)   ~ N(0, 1), rounded to bf16
  conv weights                     ~ U(-1/2, 1/2), bf16, layout [C][W]
  conv bias (optional)             ~ U(-1/2, 1/2), bf16
  beta                             = sigmoid(z),         z ~ N(0, 1), fp32
  alpha                            = exp(-softplus(z)),  z ~ N(0, 1), fp32
  alpha (long-memory variant)      = exp(-0.01 softplus(z))
  warm recurrent state S           ~ N(0, sigma_s), fp32
  warm conv window                 ~ N(0, 1), bf16
  pages of rows that start cold    payload filled with NaN (a read would show)
  page padding                     filled with the sentinel byte 0xA5

Rounding fp32 -> bf16 of the drawn inputs uses torch's CPU conversion; it is
input preparation, not part of what is being checked.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

PAD_BYTE = 0xA5


# ---------------------------------------------------------------------------
# Geometry of one page-strided slot pool (one cache group of one layer).
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Geometry:
    num_slots: int
    C: int            # conv channels (= 2*Hk*dk + Hv*dv for a GDN layer)
    W: int            # conv taps; the window keeps W-1 past inputs
    Hk: int
    Hv: int
    dk: int
    dv: int
    page_stride: int  # bytes between consecutive slots
    ssm_off: int      # byte offset of the recurrent-state region in a page
    conv_off: int     # byte offset of the conv-window region in a page

    @property
    def ssm_region_bytes(self) -> int:
        return self.Hv * self.dk * self.dv * 4

    @property
    def conv_region_bytes(self) -> int:
        return (self.W - 1) * self.C * 2

    @property
    def pool_bytes(self) -> int:
        return self.num_slots * self.page_stride


def round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def make_geometry(num_slots, Hk, Hv, dk, dv, W=4, C=None, page_align=128,
                  extra_pad=0) -> Geometry:
    """State region first (keeps it 16-byte aligned), conv window right after;
    the page is the payload rounded up to `page_align`, plus `extra_pad`."""
    if C is None:
        C = 2 * Hk * dk + Hv * dv
    ssm = Hv * dk * dv * 4
    conv = (W - 1) * C * 2
    payload = ssm + conv
    stride = round_up(payload, page_align) + extra_pad
    return Geometry(num_slots=num_slots, C=C, W=W, Hk=Hk, Hv=Hv, dk=dk, dv=dv,
                    page_stride=stride, ssm_off=0, conv_off=round_up(ssm, 16))


# ---------------------------------------------------------------------------
# Elementary draws
# ---------------------------------------------------------------------------
def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_x(rng, n_tok, C):
    return to_bf16_bits(rng.standard_normal((n_tok, C), dtype=np.float32))


def draw_conv_params(rng, C, W, bias: bool):
    w = to_bf16_bits(rng.uniform(-0.5, 0.5, size=(C, W)).astype(np.float32))
    b = to_bf16_bits(rng.uniform(-0.5, 0.5, size=(C,)).astype(np.float32)) if bias else None
    return w, b


def draw_gates(rng, n_tok, Hv, long_memory=False):
    za = rng.standard_normal((n_tok, Hv))
    zb = rng.standard_normal((n_tok, Hv))
    softplus = np.logaddexp(0.0, za)
    alpha = np.exp(-(0.01 if long_memory else 1.0) * softplus).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    return alpha, beta


# ---------------------------------------------------------------------------
# Pool images (host byte arrays [num_slots, page_stride])
# ---------------------------------------------------------------------------
def empty_pool_image(g: Geometry) -> np.ndarray:
    return np.full((g.num_slots, g.page_stride), PAD_BYTE, dtype=np.uint8)


def fill_page_warm(img: np.ndarray, g: Geometry, slot: int, rng, sigma_s: float):
    if g.Hv > 0:
        s = (rng.standard_normal(g.Hv * g.dk * g.dv, dtype=np.float32) * np.float32(sigma_s))
        img[slot, g.ssm_off:g.ssm_off + g.ssm_region_bytes] = s.view(np.uint8)
    win = to_bf16_bits(rng.standard_normal(((g.W - 1) * g.C,), dtype=np.float32))
    img[slot, g.conv_off:g.conv_off + g.conv_region_bytes] = win.view(np.uint8)


def fill_page_nan(img: np.ndarray, g: Geometry, slot: int):
    if g.Hv > 0:
        img[slot, g.ssm_off:g.ssm_off + g.ssm_region_bytes] = (
            np.full(g.Hv * g.dk * g.dv, np.nan, dtype=np.float32).view(np.uint8))
    img[slot, g.conv_off:g.conv_off + g.conv_region_bytes] = (
        np.full((g.W - 1) * g.C, 0x7FC0, dtype=np.uint16).view(np.uint8))


def make_pool_image(g: Geometry, rng, warm_slots, nan_slots, sigma_s=0.1,
                    other="random") -> np.ndarray:
    """Pages in `warm_slots` get N(0, sigma_s) state and N(0,1) windows, pages in
    `nan_slots` get NaN payloads, every other page gets random bytes (it must
    come out untouched); padding is the sentinel byte."""
    img = empty_pool_image(g)
    warm = set(int(s) for s in warm_slots)
    nan = set(int(s) for s in nan_slots)
    for s in range(g.num_slots):
        if s in warm:
            fill_page_warm(img, g, s, rng, sigma_s)
        elif s in nan:
            fill_page_nan(img, g, s)
        elif other == "random":
            for off, n in ((g.ssm_off, g.ssm_region_bytes), (g.conv_off, g.conv_region_bytes)):
                img[s, off:off + n] = rng.integers(0, 256, size=n, dtype=np.uint8)
    return img


# ---------------------------------------------------------------------------
# Per-configuration recipes
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class StepInputs:
    """Inputs of one decode step or one varlen prefill over one GDN layer."""
    geom: Geometry
    x: np.ndarray                 # bf16 bits [T, C]
    conv_w: np.ndarray            # bf16 bits [C, W]
    conv_b: Optional[np.ndarray]  # bf16 bits [C] or None
    alpha: np.ndarray             # fp32 [T, Hv]
    beta: np.ndarray              # fp32 [T, Hv]
    state_indices: np.ndarray     # int32 [N]
    has_initial_state: np.ndarray  # uint8 [N]
    cu_seqlens: np.ndarray        # int32 [N+1]
    scale: float = 1.0
    eps: float = 1e-6

    @property
    def num_seqs(self) -> int:
        return int(self.state_indices.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        d = np.diff(self.cu_seqlens)
        return int(d.max()) if d.size else 0


def step_inputs(g: Geometry, rng, lengths, state_indices, hs, bias=False,
                long_memory=False, conv=None) -> StepInputs:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    if conv is None:
        conv = draw_conv_params(rng, g.C, g.W, bias)
    x = draw_x(rng, T, g.C)
    alpha, beta = draw_gates(rng, T, g.Hv, long_memory)
    return StepInputs(geom=g, x=x, conv_w=conv[0], conv_b=conv[1], alpha=alpha, beta=beta,
                      state_indices=np.asarray(state_indices, dtype=np.int32),
                      has_initial_state=np.asarray(hs, dtype=np.uint8), cu_seqlens=cu)


def tiny_geometry(extra_pad=0) -> Geometry:
    """1 GDN layer, Hv=2, Hk=1, dk=dv=16, C=64, W=4, 8 slots, 128-byte pages."""
    return make_geometry(8, Hk=1, Hv=2, dk=16, dv=16, W=4, page_align=128, extra_pad=extra_pad)


def decode_geometry(num_slots=1024, extra_pad=0) -> Geometry:
    """32 v-heads, 16 k-heads, dk=dv=128, C=8192, W=4; pages padded to 4 KiB."""
    return make_geometry(num_slots, Hk=16, Hv=32, dk=128, dv=128, W=4, page_align=4096,
                         extra_pad=extra_pad)


def prefill_geometry(num_slots=64) -> Geometry:
    """16 v-heads, 8 k-heads, dk=dv=128, C=4096, W=4; pages padded to 4 KiB."""
    return make_geometry(num_slots, Hk=8, Hv=16, dk=128, dv=128, W=4, page_align=4096)


def decode_workload(seed=0, rows=256, num_slots=1024, warm_frac=0.9, extra_pad=0,
                    sigma_s=0.1):
    """One decode step: `rows` rows of one token, state_indices a random
    permutation prefix, has_initial_state ~ Bernoulli(warm_frac). Returns
    (StepInputs, pages) where `pages` is the host image of the referenced
    pages only ([rows, page_stride]; row r <-> slot state_indices[r])."""
    g = decode_geometry(num_slots, extra_pad)
    rng = rng_for(seed)
    idx = rng.permutation(num_slots)[:rows].astype(np.int32)
    hs = (rng.random(rows) < warm_frac).astype(np.uint8)
    sub = dataclasses.replace(g, num_slots=rows)
    pages = empty_pool_image(sub)
    for r in range(rows):
        if hs[r]:
            fill_page_warm(pages, sub, r, rng, sigma_s)
        else:
            fill_page_nan(pages, sub, r)
    inp = step_inputs(g, rng, [1] * rows, idx, hs)
    return inp, pages


def prefill_workload(seed=0, num_seqs=8, lmin=512, lmax=4096, num_slots=64, sigma_s=0.1,
                     lengths=None):
    """Varlen recurrent prefill: lengths ~ U{lmin..lmax}; the first half of the
    rows start warm, the second half cold (NaN pages)."""
    g = prefill_geometry(num_slots)
    rng = rng_for(seed)
    if lengths is None:
        lengths = rng.integers(lmin, lmax + 1, size=num_seqs)
    idx = rng.permutation(num_slots)[:num_seqs].astype(np.int32)
    hs = np.array([1 if n < num_seqs // 2 else 0 for n in range(num_seqs)], dtype=np.uint8)
    img = make_pool_image(g, rng, warm_slots=idx[hs == 1], nan_slots=idx[hs == 0],
                          sigma_s=sigma_s)
    inp = step_inputs(g, rng, lengths, idx, hs)
    return inp, img


def restore_workload(seed=0, num_layers=64, attn_every=4, n_ops=64, miss_frac=0.25,
                     num_slots=1024):
    """Restore ops over a hybrid stack: layer l is attention-only iff
    l % attn_every == attn_every-1. dst slots distinct, src drawn from the
    slots that are not a dst, a `miss_frac` share of ops have src = -1.
    Returns (geometry, linear-layer mask, ops [n,3] = (dst, src, requested))."""
    g = decode_geometry(num_slots, extra_pad=4096)
    rng = rng_for(seed)
    linear = np.array([(l % attn_every) != attn_every - 1 for l in range(num_layers)])
    perm = rng.permutation(num_slots)
    dst = perm[:n_ops]
    pool_src = perm[n_ops:]
    src = rng.choice(pool_src, size=n_ops, replace=True)
    miss = rng.random(n_ops) < miss_frac
    src = np.where(miss, -1, src)
    ops = np.stack([dst, src, np.ones(n_ops, dtype=np.int64)], axis=1).astype(np.int32)
    return g, linear, ops


# ---------------------------------------------------------------------------
# Device-side draws for workloads too large to draw on the host (the
# continuation run at scale).  Same distributions as above, drawn with a
# seeded torch generator on the GPU; the oracle receives host copies of the
# parts it checks.
# ---------------------------------------------------------------------------
def device_generator(*seed_parts):
    import torch
    s = 0
    for p in seed_parts:
        s = (s * 1_000_003 + int(p)) % (1 << 62)
    return torch.Generator(device="cuda").manual_seed(s)


def device_x(gen, n_tok, C):
    """x ~ N(0,1) rounded to bf16 (RNE); returned as an int16 tensor of bf16 bits."""
    import torch
    return torch.randn((n_tok, C), generator=gen, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16).view(torch.int16)


def device_gates(gen, n_tok, Hv, long_memory=False):
    import torch
    za = torch.randn((n_tok, Hv), generator=gen, device="cuda", dtype=torch.float64)
    zb = torch.randn((n_tok, Hv), generator=gen, device="cuda", dtype=torch.float64)
    alpha = torch.exp(-(0.01 if long_memory else 1.0) * torch.nn.functional.softplus(za))
    beta = torch.sigmoid(zb)
    return alpha.to(torch.float32).contiguous(), beta.to(torch.float32).contiguous()


def device_fill_warm(buf, g: Geometry, slots, gen, sigma_s=0.1):
    """Warm payloads for `slots` of a device pool buffer [num_slots, page_stride]:
    state ~ N(0, sigma_s) fp32, window ~ N(0,1) bf16."""
    import torch
    idx = torch.as_tensor(np.asarray(slots, np.int64), device="cuda")
    n = idx.numel()
    s = torch.randn((n, g.ssm_region_bytes // 4), generator=gen, device="cuda") * sigma_s
    w = torch.randn((n, g.conv_region_bytes // 2), generator=gen, device="cuda")
    w = w.to(torch.bfloat16)
    buf[idx, g.ssm_off:g.ssm_off + g.ssm_region_bytes] = s.view(torch.uint8)
    buf[idx, g.conv_off:g.conv_off + g.conv_region_bytes] = w.view(torch.uint8)


def device_fill_nan(buf, g: Geometry, slots):
    import torch
    idx = torch.as_tensor(np.asarray(slots, np.int64), device="cuda")
    s = torch.full((idx.numel(), g.ssm_region_bytes // 4), float("nan"), device="cuda")
    w = torch.full((idx.numel(), g.conv_region_bytes // 2), 0x7FC0, dtype=torch.int16,
                   device="cuda")
    buf[idx, g.ssm_off:g.ssm_off + g.ssm_region_bytes] = s.view(torch.uint8)
    buf[idx, g.conv_off:g.conv_off + g.conv_region_bytes] = w.view(torch.uint8)
