"""Python binding of libgdn (the slot-indexed Gated DeltaNet state library).

Argument marshalling only: every function forwards to the C-ABI entry point
of the same name (include/gdn.h), which validates and enqueues gfx950 kernels
on the given stream.  Device buffers may be given as torch tensors (their
data_ptr() is used; a tensor that is not a contiguous GPU tensor of the
expected element size is refused here, before any kernel could read a host
address) or as integer addresses, which are passed on unchecked.  The library must have been
built (`python -m hybrid_linear_attention_slot_amd.build`); there is no
fallback: loading fails loudly when libgdn.so is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK = 0
GDN_WARN_COLD_FALLBACK = 1
GDN_EINVAL = -1
GDN_ERANGE = -2
GDN_EOVERLAP = -3
GDN_EALIGN = -4
GDN_EUNSUPPORTED = -5
GDN_EHIP = -6
GDN_ENOSLOT = -7
GDN_ESTATE = -8
GDN_EIO = -9
GDN_ECORRUPT = -10
GDN_ENOMEM = -11
GDN_STEP_DECODE = 1   # gdn_pool_step_support bits
GDN_STEP_PREFILL = 2

ERROR_NAMES = {GDN_EINVAL: "GDN_EINVAL", GDN_ERANGE: "GDN_ERANGE", GDN_EOVERLAP: "GDN_EOVERLAP",
               GDN_EALIGN: "GDN_EALIGN", GDN_EUNSUPPORTED: "GDN_EUNSUPPORTED",
               GDN_EHIP: "GDN_EHIP", GDN_ENOSLOT: "GDN_ENOSLOT", GDN_ESTATE: "GDN_ESTATE",
               GDN_EIO: "GDN_EIO", GDN_ECORRUPT: "GDN_ECORRUPT", GDN_ENOMEM: "GDN_ENOMEM"}

GDN_SLOT_FREE, GDN_SLOT_LIVE, GDN_SLOT_CHECKPOINT, GDN_SLOT_RESERVED = 0, 1, 2, 3


class GdnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class gdn_pool_desc(C.Structure):
    _fields_ = [("num_layers", C.c_int32),
                ("layer_base", C.POINTER(C.c_void_p)),
                ("num_slots", C.c_int64),
                ("page_stride_bytes", C.c_int64),
                ("conv_offset_bytes", C.c_int64),
                ("ssm_offset_bytes", C.c_int64),
                ("conv_channels", C.c_int32),
                ("conv_width", C.c_int32),
                ("num_k_heads", C.c_int32),
                ("num_v_heads", C.c_int32),
                ("head_k_dim", C.c_int32),
                ("head_v_dim", C.c_int32)]


class gdn_restore_op(C.Structure):
    _fields_ = [("dst_slot", C.c_int32), ("src_slot", C.c_int32), ("requested", C.c_int32)]


class gdn_step_args(C.Structure):
    _fields_ = [("x", C.c_void_p), ("conv_w", C.c_void_p), ("conv_b", C.c_void_p),
                ("alpha", C.c_void_p), ("beta", C.c_void_p), ("state_indices", C.c_void_p),
                ("has_initial_state", C.c_void_p), ("out", C.c_void_p),
                ("scale", C.c_float), ("l2_eps", C.c_float)]


class gdn_slot_request(C.Structure):
    _fields_ = [("seq_id", C.c_int64), ("n_kv_cache_tokens", C.c_int64),
                ("n_tokens_after_step", C.c_int64), ("restore_prefix_hash", C.c_uint64),
                ("save_prefix_hash", C.c_uint64)]


class gdn_linear_state_op(C.Structure):
    _fields_ = [("linear_state_id", C.c_int32), ("restore_src_slot_id", C.c_int32),
                ("save_dst_slot_id", C.c_int32), ("has_initial_state", C.c_int32),
                ("restore_prefix_hash", C.c_uint64), ("save_prefix_hash", C.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class gdn_snapshot_info(C.Structure):
    _fields_ = [("key", C.c_uint64), ("position", C.c_int64), ("num_linear_layers", C.c_int32),
                ("conv_channels", C.c_int32), ("conv_width", C.c_int32),
                ("num_k_heads", C.c_int32), ("num_v_heads", C.c_int32),
                ("head_k_dim", C.c_int32), ("head_v_dim", C.c_int32),
                ("window_bytes", C.c_int64), ("state_bytes", C.c_int64),
                ("payload_bytes", C.c_int64), ("payload_crc", C.c_uint32)]


_lib = None


def lib() -> C.CDLL:
    """The loaded libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hybrid_linear_attention_slot_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.gdn_pool_create.argtypes = [C.POINTER(gdn_pool_desc), C.POINTER(C.c_void_p)]
        L.gdn_pool_create.restype = C.c_int
        L.gdn_pool_destroy.argtypes = [p]
        L.gdn_pool_destroy.restype = None
        L.gdn_pool_region_bytes.argtypes = [p, C.POINTER(i64), C.POINTER(i64)]
        L.gdn_pool_region_bytes.restype = C.c_int
        L.gdn_pool_step_support.argtypes = [p]
        L.gdn_pool_step_support.restype = C.c_int
        L.gdn_pool_describe.argtypes = [p, C.c_char_p, C.c_size_t]
        L.gdn_pool_describe.restype = C.c_int
        L.gdn_restore_slots.argtypes = [p, C.POINTER(gdn_restore_op), i32, p, p]
        L.gdn_restore_slots.restype = C.c_int
        L.gdn_gather_states.argtypes = [p, i32, p, i32, p, p, p]
        L.gdn_gather_states.restype = C.c_int
        L.gdn_scatter_states.argtypes = [p, i32, p, i32, p, p, p]
        L.gdn_scatter_states.restype = C.c_int
        L.gdn_decode_step.argtypes = [p, i32, i32, C.POINTER(gdn_step_args), p]
        L.gdn_decode_step.restype = C.c_int
        L.gdn_prefill_varlen.argtypes = [p, i32, i32, p, i32, i64, C.POINTER(gdn_step_args), p]
        L.gdn_prefill_varlen.restype = C.c_int
        L.gdn_prefill_varlen_checkpoint.argtypes = [p, i32, i32, p, i32, i64,
                                                    C.POINTER(gdn_step_args), p, p, p]
        L.gdn_prefill_varlen_checkpoint.restype = C.c_int
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = C.c_char_p
        u64 = C.c_uint64
        L.gdn_slots_create.argtypes = [i32, i32, C.POINTER(C.c_void_p)]
        L.gdn_slots_destroy.argtypes = [p]
        L.gdn_slots_destroy.restype = None
        L.gdn_slots_add_sequence.argtypes = [p, i64, C.POINTER(i32)]
        L.gdn_slots_remove_sequence.argtypes = [p, i64]
        L.gdn_slots_resolve.argtypes = [p, C.POINTER(gdn_slot_request), i32,
                                        C.POINTER(gdn_linear_state_op)]
        L.gdn_slots_commit.argtypes = [p]
        L.gdn_slots_abort.argtypes = [p]
        L.gdn_slots_restore_ops.argtypes = [C.POINTER(gdn_linear_state_op), i32,
                                            C.POINTER(gdn_restore_op)]
        L.gdn_slots_slot_info.argtypes = [p, i32, C.POINTER(i32), C.POINTER(i64), C.POINTER(u64),
                                          C.POINTER(i32)]
        L.gdn_slots_sequence_info.argtypes = [p, i64, C.POINTER(i32), C.POINTER(i32)]
        L.gdn_slots_lookup.argtypes = [p, u64]
        L.gdn_slots_lookup.restype = i32
        L.gdn_slots_counts.argtypes = [p, C.POINTER(i32)]
        L.gdn_crc32c.argtypes = [C.c_uint32, p, C.c_size_t]
        L.gdn_crc32c.restype = C.c_uint32
        L.gdn_snapshot_save.argtypes = [p, i32, u64, i64, C.c_char_p, p]
        L.gdn_snapshot_save.restype = C.c_int
        L.gdn_snapshot_load.argtypes = [p, i32, C.c_char_p, u64, C.POINTER(i64), i32, p]
        L.gdn_snapshot_load.restype = C.c_int
        L.gdn_snapshot_read_info.argtypes = [C.c_char_p, C.POINTER(gdn_snapshot_info)]
        L.gdn_snapshot_read_info.restype = C.c_int
        for f in ("gdn_slots_create", "gdn_slots_add_sequence", "gdn_slots_remove_sequence",
                  "gdn_slots_resolve", "gdn_slots_commit", "gdn_slots_abort",
                  "gdn_slots_restore_ops", "gdn_slots_slot_info", "gdn_slots_sequence_info",
                  "gdn_slots_counts"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _addr(t, elem: int = 0, name: str = "buffer") -> Optional[int]:
    """Device address of `t`: None, an int (unchecked), or a torch tensor that
    must be a contiguous GPU tensor (with `elem`-byte elements when elem > 0)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got one on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem and t.element_size() != elem:
        raise ValueError(f"{name} must have {elem}-byte elements (got {t.dtype})")
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(rc: int) -> int:
    if rc < 0:
        raise GdnError(rc, gdn_last_error())
    return rc


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


class Pool:
    """Owner of a gdn_pool handle (host metadata only).  Holds references to
    the layer buffers it was created from, so that tensors passed in stay
    allocated while the pool can still name them."""

    def __init__(self, handle: int, desc: gdn_pool_desc, bases, tensors):
        self.handle = handle
        self.desc = desc
        self._bases = bases
        self._tensors = tensors

    def close(self):
        if self.handle:
            lib().gdn_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gdn_pool_create(layer_base: Sequence, num_slots: int, page_stride_bytes: int,
                    conv_offset_bytes: int, ssm_offset_bytes: int, conv_channels: int,
                    conv_width: int, num_k_heads: int, num_v_heads: int, head_k_dim: int,
                    head_v_dim: int) -> Pool:
    """layer_base: per layer a device buffer (tensor or address) of num_slots
    pages, or None for an attention-only layer."""
    bases = (C.c_void_p * len(layer_base))(*[_addr(b, 0, f"layer_base[{i}]")
                                             for i, b in enumerate(layer_base)])
    d = gdn_pool_desc(len(layer_base), C.cast(bases, C.POINTER(C.c_void_p)), num_slots,
                      page_stride_bytes, conv_offset_bytes, ssm_offset_bytes, conv_channels,
                      conv_width, num_k_heads, num_v_heads, head_k_dim, head_v_dim)
    h = C.c_void_p()
    _check(lib().gdn_pool_create(C.byref(d), C.byref(h)))
    return Pool(h.value, d, bases, list(layer_base))


def gdn_pool_destroy(pool: Pool) -> None:
    pool.close()


def gdn_pool_region_bytes(pool: Pool):
    s, c = C.c_int64(), C.c_int64()
    _check(lib().gdn_pool_region_bytes(pool.handle, C.byref(s), C.byref(c)))
    return s.value, c.value


def gdn_pool_step_support(pool: Pool) -> int:
    """Mask of GDN_STEP_DECODE / GDN_STEP_PREFILL for the pool's geometry."""
    return _check(lib().gdn_pool_step_support(pool.handle))


def gdn_pool_describe(pool: Pool) -> str:
    n = _check(lib().gdn_pool_describe(pool.handle, None, 0))
    buf = C.create_string_buffer(n + 1)
    _check(lib().gdn_pool_describe(pool.handle, buf, n + 1))
    return buf.value.decode()


def gdn_restore_slots(pool: Pool, ops, has_initial_state, stream=None) -> int:
    """ops: sequence of (dst_slot, src_slot, requested) for batch rows 0..n-1.
    Returns GDN_OK or GDN_WARN_COLD_FALLBACK."""
    ops = [tuple(int(v) for v in op) for op in ops]
    arr = (gdn_restore_op * max(1, len(ops)))(*[gdn_restore_op(*op) for op in ops])
    return _check(lib().gdn_restore_slots(pool.handle, arr, len(ops),
                                          _addr(has_initial_state, 1, "has_initial_state"),
                                          _stream(stream)))


def gdn_gather_states(pool: Pool, layer: int, idx, n: int, conv_dense, ssm_dense,
                      stream=None) -> int:
    """Dense buffers may be tensors of any element width (their bytes are
    the bf16 window rows and the fp32 state rows)."""
    return _check(lib().gdn_gather_states(pool.handle, layer, _addr(idx, 4, "idx"), n,
                                          _addr(conv_dense, 0, "conv_dense"),
                                          _addr(ssm_dense, 0, "ssm_dense"), _stream(stream)))


def gdn_scatter_states(pool: Pool, layer: int, idx, n: int, conv_dense, ssm_dense,
                       stream=None) -> int:
    return _check(lib().gdn_scatter_states(pool.handle, layer, _addr(idx, 4, "idx"), n,
                                           _addr(conv_dense, 0, "conv_dense"),
                                           _addr(ssm_dense, 0, "ssm_dense"), _stream(stream)))


def make_step_args(x, conv_w, conv_b, alpha, beta, state_indices, has_initial_state, out,
                   scale=1.0, l2_eps=1e-6) -> gdn_step_args:
    """The returned struct keeps references to the tensors it names, so that
    temporaries passed here stay allocated as long as the struct lives."""
    a = gdn_step_args(_addr(x, 2, "x"), _addr(conv_w, 2, "conv_w"), _addr(conv_b, 2, "conv_b"),
                      _addr(alpha, 4, "alpha"), _addr(beta, 4, "beta"),
                      _addr(state_indices, 4, "state_indices"),
                      _addr(has_initial_state, 1, "has_initial_state"), _addr(out, 2, "out"),
                      float(scale), float(l2_eps))
    a._keep = (x, conv_w, conv_b, alpha, beta, state_indices, has_initial_state, out)
    return a


def gdn_decode_step(pool: Pool, layer: int, rows: int, args: gdn_step_args, stream=None) -> int:
    return _check(lib().gdn_decode_step(pool.handle, layer, rows, C.byref(args),
                                        _stream(stream)))


def gdn_prefill_varlen(pool: Pool, layer: int, num_seqs: int, cu_seqlens, max_seqlen: int,
                       total_tokens: int, args: gdn_step_args, stream=None) -> int:
    return _check(lib().gdn_prefill_varlen(pool.handle, layer, num_seqs,
                                           _addr(cu_seqlens, 4, "cu_seqlens"),
                                           max_seqlen, total_tokens, C.byref(args),
                                           _stream(stream)))


def gdn_prefill_varlen_checkpoint(pool: Pool, layer: int, num_seqs: int, cu_seqlens,
                                  max_seqlen: int, total_tokens: int, args: gdn_step_args,
                                  ckpt_slot, ckpt_len, stream=None) -> int:
    return _check(lib().gdn_prefill_varlen_checkpoint(
        pool.handle, layer, num_seqs, _addr(cu_seqlens, 4, "cu_seqlens"), max_seqlen,
        total_tokens, C.byref(args), _addr(ckpt_slot, 4, "ckpt_slot"),
        _addr(ckpt_len, 4, "ckpt_len"), _stream(stream)))


# ---------------------------------------------------------------------------
# Host-side slot manager of the prefix cache (include/gdn_slots.h)
# ---------------------------------------------------------------------------
class SlotManager:
    """Owner of a gdn_slot_manager handle."""

    def __init__(self, handle: int):
        self.handle = handle

    def close(self):
        if self.handle:
            lib().gdn_slots_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gdn_slots_create(num_slots: int, block_size: int) -> SlotManager:
    h = C.c_void_p()
    _check(lib().gdn_slots_create(num_slots, block_size, C.byref(h)))
    return SlotManager(h.value)


def gdn_slots_destroy(m: SlotManager) -> None:
    m.close()


def gdn_slots_add_sequence(m: SlotManager, seq_id: int) -> int:
    s = C.c_int32()
    _check(lib().gdn_slots_add_sequence(m.handle, seq_id, C.byref(s)))
    return s.value


def gdn_slots_remove_sequence(m: SlotManager, seq_id: int) -> None:
    _check(lib().gdn_slots_remove_sequence(m.handle, seq_id))


def gdn_slots_resolve(m: SlotManager, rows) -> list:
    """rows: sequence of (seq_id, n_kv_cache_tokens, n_tokens_after_step,
    restore_prefix_hash, save_prefix_hash).  Returns the ops as dicts."""
    rows = [tuple(int(v) for v in r) for r in rows]
    n = len(rows)
    arr = (gdn_slot_request * max(1, n))(*[gdn_slot_request(*r) for r in rows])
    ops = (gdn_linear_state_op * max(1, n))()
    _check(lib().gdn_slots_resolve(m.handle, arr, n, ops))
    return [ops[i].as_dict() for i in range(n)]


def gdn_slots_commit(m: SlotManager) -> None:
    _check(lib().gdn_slots_commit(m.handle))


def gdn_slots_abort(m: SlotManager) -> None:
    _check(lib().gdn_slots_abort(m.handle))


def gdn_slots_restore_ops(ops) -> list:
    """ops: the dicts gdn_slots_resolve returned; returns (dst, src, requested) tuples."""
    n = len(ops)
    arr = (gdn_linear_state_op * max(1, n))(
        *[gdn_linear_state_op(**{f: o[f] for f, _ in gdn_linear_state_op._fields_}) for o in ops])
    out = (gdn_restore_op * max(1, n))()
    _check(lib().gdn_slots_restore_ops(arr, n, out))
    return [(out[i].dst_slot, out[i].src_slot, out[i].requested) for i in range(n)]


def gdn_slots_slot_info(m: SlotManager, slot: int):
    k, o, h, p = C.c_int32(), C.c_int64(), C.c_uint64(), C.c_int32()
    _check(lib().gdn_slots_slot_info(m.handle, slot, C.byref(k), C.byref(o), C.byref(h),
                                     C.byref(p)))
    return k.value, o.value, h.value, p.value


def gdn_slots_sequence_info(m: SlotManager, seq_id: int):
    s, i = C.c_int32(), C.c_int32()
    _check(lib().gdn_slots_sequence_info(m.handle, seq_id, C.byref(s), C.byref(i)))
    return s.value, i.value


def gdn_slots_lookup(m: SlotManager, prefix_hash: int) -> int:
    return int(lib().gdn_slots_lookup(m.handle, prefix_hash))


def gdn_slots_counts(m: SlotManager) -> list:
    c = (C.c_int32 * 4)()
    _check(lib().gdn_slots_counts(m.handle, c))
    return list(c)


# ---------------------------------------------------------------------------
# State snapshots on disk (include/gdn_snapshot.h)
# ---------------------------------------------------------------------------
def gdn_crc32c(data: bytes, crc: int = 0) -> int:
    buf = C.create_string_buffer(bytes(data), len(data))
    return int(lib().gdn_crc32c(crc, buf, len(data)))


def gdn_snapshot_save(pool: Pool, slot: int, key: int, position: int, path: str,
                      stream=None) -> None:
    _check(lib().gdn_snapshot_save(pool.handle, slot, key, position, os.fsencode(path),
                                   _stream(stream)))


def gdn_snapshot_load(pool: Pool, slot: int, path: str, key: int, drop_damaged: bool = False,
                      stream=None) -> int:
    """Returns the stored position."""
    pos = C.c_int64()
    _check(lib().gdn_snapshot_load(pool.handle, slot, os.fsencode(path), key, C.byref(pos),
                                   1 if drop_damaged else 0, _stream(stream)))
    return pos.value


def gdn_snapshot_read_info(path: str) -> dict:
    info = gdn_snapshot_info()
    _check(lib().gdn_snapshot_read_info(os.fsencode(path), C.byref(info)))
    return {f: getattr(info, f) for f, _ in gdn_snapshot_info._fields_}
