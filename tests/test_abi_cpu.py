"""The C-ABI library on the host (no GPU): it loads, exports every function
the headers in include/ declare, and validates arguments before any launch.

Fake device addresses are used; every call below fails validation (or only
builds host metadata) and never touches device memory."""
import ctypes as C
import os
import re

import pytest

import hybrid_linear_attention_slot_amd as gdn
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced on the host


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 20
    L = gdn.lib()
    for n in names:
        assert hasattr(L, n), n
    # and the binding offers a Python function of the same name for each
    for n in names:
        assert callable(getattr(gdn, n)), n


def pool_for(g, layers=1, attention=(), **over):
    kw = dict(num_slots=g.num_slots, page_stride_bytes=g.page_stride,
              conv_offset_bytes=g.conv_off, ssm_offset_bytes=g.ssm_off, conv_channels=g.C,
              conv_width=g.W, num_k_heads=g.Hk, num_v_heads=g.Hv, head_k_dim=g.dk,
              head_v_dim=g.dv)
    kw.update(over)
    bases = [None if l in attention else FAKE + l * (1 << 32) for l in range(layers)]
    return gdn.gdn_pool_create(bases, **kw)


def test_pool_create_and_describe():
    g = wl.decode_geometry(num_slots=1024)
    p = pool_for(g, layers=8, attention=(3, 7))
    ssm, conv = gdn.gdn_pool_region_bytes(p)
    assert ssm == 32 * 128 * 128 * 4 and conv == 3 * 8192 * 2
    assert ssm + conv == 2_146_304 == g.page_stride  # payload is exactly 524 pages of 4 KiB
    text = gdn.gdn_pool_describe(p)
    assert "layers=8 (linear=6, attention-only=2)" in text
    assert "page_stride=2146304B" in text
    assert "attention-only layers: 3 7" in text
    gdn.gdn_pool_destroy(p)


@pytest.mark.parametrize("dk,W,mask", [
    (128, 4, gdn.GDN_STEP_DECODE | gdn.GDN_STEP_PREFILL),
    (16, 2, gdn.GDN_STEP_DECODE | gdn.GDN_STEP_PREFILL),
    (64, 3, gdn.GDN_STEP_DECODE | gdn.GDN_STEP_PREFILL),
    (48, 4, 0),    # a head size without a compiled kernel
    (128, 5, 0),   # a conv width without one
])
def test_step_support_matches_the_compiled_kernels(dk, W, mask):
    g = wl.make_geometry(8, Hk=1, Hv=2, dk=dk, dv=dk, W=W, page_align=128)
    p = pool_for(g)
    assert gdn.gdn_pool_step_support(p) == mask
    gdn.gdn_pool_destroy(p)


def test_block_stride_example_descriptor():
    # conv-window-only pool of the worked example: 48 bf16 in a 128-byte page
    p = gdn.gdn_pool_create([FAKE], num_slots=4, page_stride_bytes=128, conv_offset_bytes=0,
                            ssm_offset_bytes=0, conv_channels=16, conv_width=4, num_k_heads=0,
                            num_v_heads=0, head_k_dim=0, head_v_dim=0)
    assert gdn.gdn_pool_region_bytes(p) == (0, 96)
    assert gdn.gdn_pool_step_support(p) == 0  # no recurrent state: copies only
    assert "slot stride 64 elements" in gdn.gdn_pool_describe(p)


@pytest.mark.parametrize("over,code", [
    (dict(page_stride_bytes=2_146_304 + 8), gdn.GDN_EALIGN),
    (dict(conv_offset_bytes=2_097_160), gdn.GDN_EALIGN),
    (dict(page_stride_bytes=2_146_304 - 4096), gdn.GDN_ERANGE),
    (dict(conv_channels=8190), gdn.GDN_EINVAL),
    (dict(num_k_heads=5), gdn.GDN_EINVAL),
    (dict(conv_width=9), gdn.GDN_EINVAL),
    (dict(num_slots=0), gdn.GDN_ERANGE),
    (dict(conv_offset_bytes=1024), gdn.GDN_EOVERLAP),
])
def test_pool_create_rejects(over, code):
    g = wl.decode_geometry(num_slots=16)
    with pytest.raises(gdn.GdnError) as e:
        pool_for(g, **over)
    assert e.value.code == code
    assert gdn.gdn_last_error()


def test_pool_create_rejects_misaligned_base():
    g = wl.tiny_geometry()
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_pool_create([FAKE + 8], g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                            g.W, g.Hk, g.Hv, g.dk, g.dv)
    assert e.value.code == gdn.GDN_EALIGN


@pytest.mark.parametrize("ops,code", [
    ([(0, 3, 1), (0, 4, 1)], gdn.GDN_EOVERLAP),     # duplicate dst
    ([(0, 3, 1), (3, 5, 1)], gdn.GDN_EOVERLAP),     # src of one hit is another's dst
    ([(0, 8, 1)], gdn.GDN_ERANGE),                  # src out of range
    ([(-1, 2, 1)], gdn.GDN_ERANGE),                 # dst out of range
])
def test_restore_validation(ops, code):
    p = pool_for(wl.tiny_geometry(), layers=2)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_restore_slots(p, ops, FAKE, stream=0)
    assert e.value.code == code


def test_restore_ignores_unrequested_and_miss_slots_in_validation():
    # an unrequested op with an out-of-range slot and a zero-op call are fine
    p = pool_for(wl.tiny_geometry(), layers=1)
    assert gdn.gdn_restore_slots(p, [], FAKE, stream=0) == gdn.GDN_OK


def step_args(**over):
    kw = dict(x=FAKE, conv_w=FAKE, conv_b=None, alpha=FAKE, beta=FAKE, state_indices=FAKE,
              has_initial_state=FAKE, out=FAKE)
    kw.update(over)
    return gdn.make_step_args(**kw)


def test_step_validation():
    g = wl.decode_geometry(num_slots=16)
    p = pool_for(g, layers=4, attention=(3,))
    a = step_args()
    for fn in (lambda l, a: gdn.gdn_decode_step(p, l, 4, a, stream=0),
               lambda l, a: gdn.gdn_prefill_varlen(p, l, 2, FAKE, 8, 16, a, stream=0)):
        with pytest.raises(gdn.GdnError) as e:
            fn(3, a)       # attention-only layer
        assert e.value.code == gdn.GDN_ERANGE
        with pytest.raises(gdn.GdnError) as e:
            fn(4, a)       # no such layer
        assert e.value.code == gdn.GDN_ERANGE
        with pytest.raises(gdn.GdnError) as e:
            fn(0, step_args(x=None))
        assert e.value.code == gdn.GDN_EINVAL
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_decode_step(p, 0, -1, a, stream=0)
    assert e.value.code == gdn.GDN_EINVAL
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_decode_step(p, 0, 4, step_args(conv_w=FAKE + 2), stream=0)
    assert e.value.code == gdn.GDN_EALIGN
    for over in (dict(x=FAKE + 2), dict(out=FAKE + 4), dict(conv_b=FAKE + 2)):
        with pytest.raises(gdn.GdnError) as e:
            gdn.gdn_prefill_varlen(p, 0, 2, FAKE, 8, 16, step_args(**over), stream=0)
        assert e.value.code == gdn.GDN_EALIGN
    # zero rows / zero tokens are no-ops that launch nothing
    assert gdn.gdn_decode_step(p, 0, 0, a, stream=0) == gdn.GDN_OK
    assert gdn.gdn_prefill_varlen(p, 0, 0, FAKE, 0, 0, a, stream=0) == gdn.GDN_OK
    # ... and may name no buffer at all (empty tensors have no address)
    none = gdn.make_step_args(*[None] * 8)
    assert gdn.gdn_decode_step(p, 0, 0, none, stream=0) == gdn.GDN_OK
    assert gdn.gdn_prefill_varlen(p, 0, 3, None, 0, 0, none, stream=0) == gdn.GDN_OK
    assert gdn.gdn_prefill_varlen_checkpoint(p, 0, 0, None, 0, 0, none, None, None,
                                             stream=0) == gdn.GDN_OK
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_prefill_varlen(p, 0, 2, None, 8, 16, a, stream=0)
    assert e.value.code == gdn.GDN_EINVAL
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_prefill_varlen_checkpoint(p, 0, 2, FAKE, 8, 16, a, None, FAKE, stream=0)
    assert e.value.code == gdn.GDN_EINVAL


def test_step_unsupported_geometry():
    g = wl.make_geometry(4, Hk=1, Hv=1, dk=48, dv=48, W=4)
    p = pool_for(g)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_decode_step(p, 0, 1, step_args(), stream=0)
    assert e.value.code == gdn.GDN_EUNSUPPORTED
    g = wl.make_geometry(4, Hk=1, Hv=2, dk=16, dv=16, W=6)
    p = pool_for(g)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_prefill_varlen(p, 0, 1, FAKE, 4, 4, step_args(), stream=0)
    assert e.value.code == gdn.GDN_EUNSUPPORTED


def test_gather_scatter_validation():
    p = pool_for(wl.tiny_geometry(), layers=2, attention=(1,))
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_gather_states(p, 1, FAKE, 2, FAKE, FAKE, stream=0)
    assert e.value.code == gdn.GDN_ERANGE
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_scatter_states(p, 0, None, 2, FAKE, FAKE, stream=0)
    assert e.value.code == gdn.GDN_EINVAL
    assert gdn.gdn_gather_states(p, 0, FAKE, 0, FAKE, FAKE, stream=0) == gdn.GDN_OK
    # argument order (conv_dense, ssm_dense): bf16 rows 2-byte, fp32 rows 4-byte aligned
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_gather_states(p, 0, FAKE, 2, FAKE + 2, FAKE + 2, stream=0)
    assert e.value.code == gdn.GDN_EALIGN
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_scatter_states(p, 0, FAKE, 2, FAKE + 1, FAKE, stream=0)
    assert e.value.code == gdn.GDN_EALIGN
    # the state buffer may be NULL only when the pool has no state region
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_gather_states(p, 0, FAKE, 2, FAKE, None, stream=0)
    assert e.value.code == gdn.GDN_EINVAL
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_gather_states(p, 0, FAKE, 2, None, FAKE, stream=0)
    assert e.value.code == gdn.GDN_EINVAL


class _FakeGpuTensor:
    """Stands in for a GPU tensor in the binding's argument checks (no GPU here)."""
    is_cuda = True
    device = "cuda:0"

    def __init__(self, elem, contiguous=True):
        self._elem, self._contiguous = elem, contiguous
        self.dtype = f"{elem}-byte"

    def is_contiguous(self):
        return self._contiguous

    def element_size(self):
        return self._elem

    def data_ptr(self):
        return 0x10000


def test_binding_refuses_host_noncontiguous_and_wrong_width_tensors():
    """A host tensor's address would reach a kernel as a device address: the
    binding refuses it (and non-contiguous or wrong-width tensors) before any
    call into the library."""
    import torch
    ok = dict(x=_FakeGpuTensor(2), conv_w=_FakeGpuTensor(2), conv_b=None,
              alpha=_FakeGpuTensor(4), beta=_FakeGpuTensor(4),
              state_indices=_FakeGpuTensor(4), has_initial_state=_FakeGpuTensor(1),
              out=_FakeGpuTensor(2))
    gdn.make_step_args(**ok)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.make_step_args(**dict(ok, x=torch.zeros(8, dtype=torch.int16)))
    with pytest.raises(ValueError, match="contiguous"):
        gdn.make_step_args(**dict(ok, out=_FakeGpuTensor(2, contiguous=False)))
    with pytest.raises(ValueError, match="4-byte"):
        gdn.make_step_args(**dict(ok, alpha=_FakeGpuTensor(2)))
    with pytest.raises(ValueError, match="1-byte"):
        gdn.make_step_args(**dict(ok, has_initial_state=_FakeGpuTensor(4)))
