"""Thin ctypes binding of libpkv (include/pkv.h).

Argument marshalling only: every step of the decode path runs in libpkv's
host code and HIP kernels. Module-level functions carry the C names; `Pool`
bundles them for convenience. Device buffers are torch tensors on the pool's
device (torch is used for device memory and streams only). There is no
fallback: if libpkv.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; PKV_LIB names another build of the same C ABI (the
# host-only sanitizer build the CPU tests make).
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OOM = -2
PKV_ERR_NO_FREE_BLOCK = -3
PKV_ERR_UNKNOWN_SEQ = -4
PKV_ERR_SEQ_EXISTS = -5
PKV_ERR_DEVICE = -6
PKV_ERR_UNSUPPORTED = -7
STATUS_NAMES = {
    0: "PKV_OK", -1: "PKV_ERR_INVALID_ARG", -2: "PKV_ERR_OOM", -3: "PKV_ERR_NO_FREE_BLOCK",
    -4: "PKV_ERR_UNKNOWN_SEQ", -5: "PKV_ERR_SEQ_EXISTS", -6: "PKV_ERR_DEVICE",
    -7: "PKV_ERR_UNSUPPORTED",
}

PKV_F32, PKV_F16, PKV_BF16, PKV_I8 = 0, 1, 2, 3
PKV_DECODE_SEPARATE_MERGE = 1
PKV_DECODE_FUSED_MERGE = 2
PKV_DECODE_VALU_CONTRACTION = 4  # comparison variant: both contractions on the vector ALUs
MERGE_COUNTER_BYTES = 65536  # PKV_MERGE_COUNTER_BYTES: the arrival-counter prefix of every workspace
PKV_BATCH_ADMISSION, PKV_BATCH_LONGEST_FIRST = 0, 1

# Every symbol include/pkv.h declares, with its ctypes signature.
_i32, _i64, _u64, _sz, _f32, _vp = C.c_int32, C.c_int64, C.c_uint64, C.c_size_t, C.c_float, C.c_void_p


class pkv_pool_config(C.Structure):
    _fields_ = [
        ("num_layers", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
        ("block_size", _i32), ("num_blocks", _i32), ("kv_dtype", C.c_int),
        ("initial_free_order", _vp), ("device_arena", _vp), ("arena_bytes", _sz),
        ("host_only", _i32), ("layer_kv_dtype", _vp), ("seal_on_full", _i32),
    ]


class pkv_stats(C.Structure):
    _fields_ = [("free_blocks", _i64), ("used_blocks", _i64), ("shared_blocks", _i64),
                ("cow_copies", _i64), ("num_seqs", _i64), ("total_blocks", _i64)]


PKV_EV_ADMIT, PKV_EV_EOS, PKV_EV_MAX_LENGTH, PKV_EV_PREEMPT, PKV_EV_WAIT = 1, 2, 3, 4, 5


class pkv_sched_config(C.Structure):
    _fields_ = [("max_batch", _i32), ("max_model_len", _i32), ("reserve_blocks", _i32), ("batch_order", _i32)]


class pkv_event(C.Structure):
    _fields_ = [("request", _i64), ("kind", _i32), ("pad_", _i32)]


class pkv_step_plan(C.Structure):
    _fields_ = [
        ("num_seqs", _i32), ("max_blocks", _i32), ("max_context_len", _i32), ("num_prefill", _i32),
        ("prefill_total", _i32), ("num_events", _i32),
        ("seqs", C.POINTER(_i64)), ("slots", C.POINTER(_i64)), ("block_tables", C.POINTER(_i32)),
        ("context_lens", C.POINTER(_i32)), ("prefill_seqs", C.POINTER(_i64)),
        ("prefill_first", C.POINTER(_i32)), ("prefill_tokens", C.POINTER(_i32)),
        ("prefill_slots", C.POINTER(_i64)), ("events", C.POINTER(pkv_event)),
    ]


class pkv_sched_stats(C.Structure):
    _fields_ = [("waiting", _i64), ("running", _i64), ("admitted", _i64), ("finished_eos", _i64),
                ("finished_max_length", _i64), ("preempted", _i64), ("generated", _i64),
                ("used_blocks", _i64), ("total_blocks", _i64), ("paused", _i32), ("pad_", _i32)]


SIGNATURES = {
    "pkv_pool_required_bytes": (_sz, [_vp]),
    "pkv_pool_create": (C.c_int, [_vp, _vp]),
    "pkv_pool_destroy": (None, [_vp]),
    "pkv_seq_allocate": (C.c_int, [_vp, _i64, _i32, _vp]),
    "pkv_seq_append_slots": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _vp]),
    "pkv_seq_fork": (C.c_int, [_vp, _i64, _i64]),
    "pkv_seq_free": (C.c_int, [_vp, _i64]),
    "pkv_seq_block_table": (C.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "pkv_seq_length": (C.c_int, [_vp, _i64, _vp]),
    "pkv_seq_order_longest_first": (C.c_int, [_vp, _vp, _i32, _vp]),
    "pkv_pool_stats": (C.c_int, [_vp, _vp]),
    "pkv_pool_free_queue": (C.c_int, [_vp, _vp, _i32, _vp]),
    "pkv_append_kv": (C.c_int, [_vp, _i32, _vp, _vp, C.c_int, _vp, _i32, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32, _i32]),
    "pkv_decode_auto_partition": (_i32, [_vp, _i32, _i32, _i32]),
    "pkv_decode_plan": (C.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pkv_decode_attention": (C.c_int, [_vp, _i32, _vp, C.c_int, _i32, _vp, _i32, _vp, _i32, _i32,
                                       _f32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "pkv_decode_step": (C.c_int, [_vp, _i32, _vp, _vp, _vp, C.c_int, _i32, _vp, _i32, _vp, _i32, _i32,
                                  _f32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "pkv_decode_step_noalloc": (C.c_int, [_vp, _i32, _vp, _vp, _vp, C.c_int, _i32, _vp, _i32, _vp, _i32, _i32,
                                          _f32, _i32, _i32, _vp, _vp]),
    "pkv_read_blocks": (C.c_int, [_vp, _i32, _vp, _i32, _vp, _vp]),
    "pkv_stream_read": (C.c_int, [_vp, _sz, _i32, _vp, _vp]),
    "pkv_sched_create": (C.c_int, [_vp, _vp, _vp]),
    "pkv_sched_destroy": (None, [_vp]),
    "pkv_sched_submit": (C.c_int, [_vp, _i64, _i32, _i32, _i64]),
    "pkv_sched_step": (C.c_int, [_vp, _vp, _i32, _vp, _vp]),
    "pkv_sched_get_stats": (C.c_int, [_vp, _vp]),
    "pkv_read_tail_blocks": (C.c_int, [_vp, _i32, _vp, _i32, _vp]),
    "pkv_prefill_attention": (C.c_int, [_vp, _i32, _vp, C.c_int, _i32, _vp, _i32, _vp, _i32, _vp, _i32, _i32,
                                        _f32, _i32, _vp, _vp, _sz, _vp]),
    "pkv_prefill_plan": (C.c_int, [_vp, C.c_int, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "pkv_kv_bytes": (_u64, [_u64] * 6),
    "pkv_last_error": (C.c_char_p, []),
}

_lib = None


def lib() -> C.CDLL:
    """Load libpkv.so (built in-tree by build.py). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run paged_kv_cache_62_amd.build.build() first")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(st: int) -> int:
    if st != PKV_OK:
        raise PkvError(st, lib().pkv_last_error().decode(errors="replace"))
    return st


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def _torch_dtype_code(t) -> int:
    import torch
    m = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


# ------------------------------------------------------- the C names ----
def pkv_pool_required_bytes(cfg: pkv_pool_config) -> int:
    return int(lib().pkv_pool_required_bytes(C.byref(cfg)))


def pkv_pool_create(cfg: pkv_pool_config) -> C.c_void_p:
    h = _vp()
    _check(lib().pkv_pool_create(C.byref(cfg), C.byref(h)))
    return h


def pkv_pool_destroy(h) -> None:
    lib().pkv_pool_destroy(h)


def pkv_seq_allocate(h, seq: int, n_tokens: int, want_slots: bool = True) -> np.ndarray:
    slots = np.zeros(max(n_tokens, 1), dtype=np.int64)
    _check(lib().pkv_seq_allocate(h, seq, n_tokens, _np_ptr(slots) if want_slots else None))
    return slots[:n_tokens]


def pkv_seq_append_slots(h, seqs, n_new, stream=None, out=None) -> np.ndarray:
    """Slots of the appended tokens; `out` (int64, contiguous, at least that
    many entries) receives them in place when given."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int64)
    n_new = np.ascontiguousarray(n_new, dtype=np.int32)
    total = int(n_new.sum()) if n_new.size else 0
    if out is None:
        out = np.zeros(max(total, 1), dtype=np.int64)
    assert out.dtype == np.int64 and out.flags.c_contiguous and out.size >= total
    _check(lib().pkv_seq_append_slots(h, _np_ptr(seqs), len(seqs), _np_ptr(n_new),
                                      _np_ptr(out), stream))
    return out[:total]


def pkv_seq_fork(h, parent: int, child: int) -> None:
    _check(lib().pkv_seq_fork(h, parent, child))


def pkv_seq_free(h, seq: int) -> None:
    _check(lib().pkv_seq_free(h, seq))


def pkv_seq_block_table(h, seqs, max_blocks: int, table=None, lens=None):
    """Block tables [n][max_blocks] (pad -1) and lengths [n]; `table` and
    `lens` (int32, contiguous) receive them in place when given."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int64)
    if table is None:
        table = np.zeros((len(seqs), max_blocks), dtype=np.int32)
    if lens is None:
        lens = np.zeros(len(seqs), dtype=np.int32)
    assert table.dtype == np.int32 and table.flags.c_contiguous and table.size >= len(seqs) * max_blocks
    assert lens.dtype == np.int32 and lens.flags.c_contiguous and lens.size >= len(seqs)
    _check(lib().pkv_seq_block_table(h, _np_ptr(seqs), len(seqs), max_blocks, _np_ptr(table),
                                     _np_ptr(lens)))
    return table, lens


def pkv_seq_length(h, seq: int) -> int:
    out = C.c_int64()
    _check(lib().pkv_seq_length(h, seq, C.byref(out)))
    return int(out.value)


def pkv_seq_order_longest_first(h, seqs) -> np.ndarray:
    """The sequence ids sorted by current length, longest first (stable)."""
    seqs = np.ascontiguousarray(seqs, dtype=np.int64)
    out = np.empty_like(seqs)
    _check(lib().pkv_seq_order_longest_first(h, _np_ptr(seqs), len(seqs), _np_ptr(out)))
    return out


def pkv_pool_stats(h) -> dict:
    s = pkv_stats()
    _check(lib().pkv_pool_stats(h, C.byref(s)))
    return {k: int(getattr(s, k)) for k, _ in pkv_stats._fields_}


def pkv_pool_free_queue(h, cap: int) -> np.ndarray:
    out = np.zeros(cap, dtype=np.int32)
    n = C.c_int32()
    _check(lib().pkv_pool_free_queue(h, _np_ptr(out), cap, C.byref(n)))
    return out[: n.value]


def pkv_append_kv(h, layer: int, k, v, slot_mapping, stream=None) -> None:
    """k, v: device tensors [n][Hkv][d] (fp32/fp16/bf16); slot_mapping: int64 device tensor."""
    assert k.is_contiguous() and v.is_contiguous() and slot_mapping.is_contiguous()
    assert k.dtype == v.dtype and k.shape == v.shape and slot_mapping.dtype.itemsize == 8
    n = int(slot_mapping.numel())
    assert k.shape[0] == n
    _check(lib().pkv_append_kv(h, layer, _vp(k.data_ptr()), _vp(v.data_ptr()), _torch_dtype_code(k),
                               _vp(slot_mapping.data_ptr()), n, _stream_ptr(stream)))


def pkv_decode_workspace_bytes(h, num_seqs, num_q_heads, max_context_len, partition_tokens=0) -> int:
    return int(lib().pkv_decode_workspace_bytes(h, num_seqs, num_q_heads, max_context_len,
                                                partition_tokens))


def pkv_decode_auto_partition(h, num_seqs, num_q_heads, max_context_len) -> int:
    return int(lib().pkv_decode_auto_partition(h, num_seqs, num_q_heads, max_context_len))


def pkv_decode_plan(h, num_seqs, max_context_len, partition_tokens=0, flags=0):
    """(partition tokens, partitions per sequence, fused merge 0/1) of a decode call."""
    T, P, fused = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().pkv_decode_plan(h, num_seqs, max_context_len, partition_tokens, flags, C.byref(T),
                                 C.byref(P), C.byref(fused)))
    return T.value, P.value, fused.value


def pkv_decode_attention(h, layer, q, block_tables, context_lens, max_context_len, softmax_scale,
                         out, workspace=None, partition_tokens=0, stream=None, flags=0) -> None:
    """q: [B][Hq][d] device tensor; block_tables [B][max_blocks] int32; context_lens [B] int32;
    out: [B][Hq][d] float32; workspace: zero-initialised uint8 device tensor or None."""
    assert q.is_contiguous() and block_tables.is_contiguous() and context_lens.is_contiguous()
    assert out.is_contiguous() and out.dtype.itemsize == 4
    B, hq, _ = q.shape
    ws_ptr = _vp(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib().pkv_decode_attention(
        h, layer, _vp(q.data_ptr()), _torch_dtype_code(q), hq, _vp(block_tables.data_ptr()),
        int(block_tables.shape[1]), _vp(context_lens.data_ptr()), B, int(max_context_len),
        float(softmax_scale), int(partition_tokens), int(flags), _vp(out.data_ptr()), ws_ptr, ws_bytes,
        _stream_ptr(stream)))


def pkv_decode_step(h, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                    softmax_scale, out, workspace=None, partition_tokens=0, stream=None, flags=0) -> None:
    """q: [B][Hq][d]; k_new, v_new: [B][Hkv][d] in q's dtype (the token at position
    context_lens[s]-1 of each sequence); other arguments as pkv_decode_attention."""
    for t in (q, k_new, v_new, block_tables, context_lens, out):
        assert t.is_contiguous()
    assert k_new.dtype == q.dtype and v_new.dtype == q.dtype and out.dtype.itemsize == 4
    B, hq, _ = q.shape
    assert k_new.shape[0] == B and v_new.shape == k_new.shape
    ws_ptr = _vp(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib().pkv_decode_step(
        h, layer, _vp(q.data_ptr()), _vp(k_new.data_ptr()), _vp(v_new.data_ptr()), _torch_dtype_code(q), hq,
        _vp(block_tables.data_ptr()), int(block_tables.shape[1]), _vp(context_lens.data_ptr()), B,
        int(max_context_len), float(softmax_scale), int(partition_tokens), int(flags), _vp(out.data_ptr()),
        ws_ptr, ws_bytes, _stream_ptr(stream)))


def pkv_decode_step_noalloc(h, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                            softmax_scale, out, partition_tokens=0, stream=None, flags=0) -> None:
    """pkv_decode_step with the library's own scratch as the workspace (it
    allocates nothing); arguments as pkv_decode_step without the workspace."""
    for t in (q, k_new, v_new, block_tables, context_lens, out):
        assert t.is_contiguous()
    assert k_new.dtype == q.dtype and v_new.dtype == q.dtype and out.dtype.itemsize == 4
    B, hq, _ = q.shape
    assert k_new.shape[0] == B and v_new.shape == k_new.shape
    _check(lib().pkv_decode_step_noalloc(
        h, layer, _vp(q.data_ptr()), _vp(k_new.data_ptr()), _vp(v_new.data_ptr()), _torch_dtype_code(q), hq,
        _vp(block_tables.data_ptr()), int(block_tables.shape[1]), _vp(context_lens.data_ptr()), B,
        int(max_context_len), float(softmax_scale), int(partition_tokens), int(flags), _vp(out.data_ptr()),
        _stream_ptr(stream)))


def pkv_read_blocks(h, layer: int, blocks, num_kv_heads: int, block_size: int, head_dim: int,
                    kv_dtype: int):
    """Host copy of blocks in canonical order: codes [n][2][Hkv][bs][d], scales [n][2][Hkv]."""
    blocks = np.ascontiguousarray(blocks, dtype=np.int32)
    dt = np.int8 if kv_dtype == PKV_I8 else np.uint16
    codes = np.zeros((len(blocks), 2, num_kv_heads, block_size, head_dim), dtype=dt)
    scales = np.zeros((len(blocks), 2, num_kv_heads), dtype=np.float32)
    _check(lib().pkv_read_blocks(h, layer, _np_ptr(blocks), len(blocks), _np_ptr(codes),
                                 _np_ptr(scales)))
    return codes, scales


def pkv_stream_read(buf, workgroups: int, sink, stream=None) -> None:
    """Measurement: stream-read the device tensor `buf` (all its bytes) with
    `workgroups` workgroups; sink: uint32 device tensor of workgroups * 256."""
    assert buf.is_contiguous() and sink.numel() >= workgroups * 256 and sink.element_size() == 4
    _check(lib().pkv_stream_read(_vp(buf.data_ptr()), int(buf.numel() * buf.element_size()), int(workgroups),
                                 _vp(sink.data_ptr()), _stream_ptr(stream)))


def pkv_kv_bytes(L, H, d, s, B, nbytes) -> int:
    return int(lib().pkv_kv_bytes(L, H, d, s, B, nbytes))


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode(errors="replace")


# ------------------------------------------------------------ Pool ----
class Pool:
    """A block pool: host allocator plus (unless host_only) the device cache,
    whose arena is a torch uint8 tensor owned by this object."""

    def __init__(self, num_layers, num_kv_heads, head_dim, block_size, num_blocks, kv_dtype,
                 initial_free_order=None, host_only=False, device="cuda", layer_kv_dtypes=None,
                 seal_on_full=False):
        """layer_kv_dtypes: optional per-layer PKV_F16 / PKV_I8 (kv_dtype is then the
        default the automatic decode plan follows)."""
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.block_size, self.num_blocks, self.kv_dtype = block_size, num_blocks, kv_dtype
        self.layer_kv_dtypes = ([kv_dtype] * num_layers if layer_kv_dtypes is None
                                else [int(x) for x in layer_kv_dtypes])
        assert len(self.layer_kv_dtypes) == num_layers
        self._order = (None if initial_free_order is None
                       else np.ascontiguousarray(initial_free_order, dtype=np.int32))
        self._ldt = (None if layer_kv_dtypes is None
                     else np.ascontiguousarray(self.layer_kv_dtypes, dtype=np.int32))
        cfg = pkv_pool_config(num_layers, num_kv_heads, head_dim, block_size, num_blocks, kv_dtype,
                              None if self._order is None else _np_ptr(self._order), None, 0,
                              1 if host_only else 0, None if self._ldt is None else _np_ptr(self._ldt),
                              1 if seal_on_full else 0)
        self.seal_on_full = bool(seal_on_full)
        self.arena = None
        if not host_only:
            import torch
            nbytes = pkv_pool_required_bytes(cfg)
            if nbytes == 0:
                raise PkvError(PKV_ERR_INVALID_ARG, pkv_last_error())
            self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
            cfg.device_arena = _vp(self.arena.data_ptr())
            cfg.arena_bytes = nbytes
        self.h = pkv_pool_create(cfg)
        self._scheds = weakref.WeakSet()  # schedulers over this pool: closed before it

    def close(self):
        if getattr(self, "h", None):
            for sched in list(getattr(self, "_scheds", ())):
                sched.close()  # it frees its running sequences' blocks through the pool
            pkv_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown: module globals may already be gone
            pass

    # allocator
    def allocate(self, seq, n_tokens):
        return pkv_seq_allocate(self.h, seq, n_tokens)

    def append_slots(self, seqs, n_new, stream=None, out=None):
        sp = None
        if self.arena is not None:
            sp = _stream_ptr(stream)
        return pkv_seq_append_slots(self.h, seqs, n_new, sp, out)

    def fork(self, parent, child):
        pkv_seq_fork(self.h, parent, child)

    def free(self, seq):
        pkv_seq_free(self.h, seq)

    def block_table(self, seqs, max_blocks, table=None, lens=None):
        return pkv_seq_block_table(self.h, seqs, max_blocks, table, lens)

    def length(self, seq):
        return pkv_seq_length(self.h, seq)

    def order_longest_first(self, seqs):
        return pkv_seq_order_longest_first(self.h, seqs)

    def stats(self):
        return pkv_pool_stats(self.h)

    def free_queue(self):
        return pkv_pool_free_queue(self.h, self.num_blocks)

    # device
    def append_kv(self, layer, k, v, slot_mapping, stream=None):
        pkv_append_kv(self.h, layer, k, v, slot_mapping, stream)

    def workspace_bytes(self, num_seqs, num_q_heads, max_context_len, partition_tokens=0):
        return pkv_decode_workspace_bytes(self.h, num_seqs, num_q_heads, max_context_len,
                                          partition_tokens)

    def auto_partition(self, num_seqs, num_q_heads, max_context_len):
        return pkv_decode_auto_partition(self.h, num_seqs, num_q_heads, max_context_len)

    def decode_plan(self, num_seqs, max_context_len, partition_tokens=0, flags=0):
        return pkv_decode_plan(self.h, num_seqs, max_context_len, partition_tokens, flags)

    def decode(self, layer, q, block_tables, context_lens, max_context_len, softmax_scale,
               out=None, workspace=None, partition_tokens=0, stream=None, flags=0):
        """workspace, if given, must have been zero-filled before its first use."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = self.workspace_bytes(q.shape[0], q.shape[1], max_context_len, partition_tokens)
            workspace = torch.zeros(max(nb, 1), dtype=torch.uint8, device=q.device)
        pkv_decode_attention(self.h, layer, q, block_tables, context_lens, max_context_len,
                             softmax_scale, out, workspace, partition_tokens, stream, flags)
        return out

    def decode_step(self, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                    softmax_scale, out=None, workspace=None, partition_tokens=0, stream=None, flags=0):
        """Append each sequence's new token (rows k_new, v_new) and decode, in one launch."""
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = self.workspace_bytes(q.shape[0], q.shape[1], max_context_len, partition_tokens)
            workspace = torch.zeros(max(nb, 1), dtype=torch.uint8, device=q.device)
        pkv_decode_step(self.h, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                        softmax_scale, out, workspace, partition_tokens, stream, flags)
        return out

    def decode_step_noalloc(self, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                            softmax_scale, out, partition_tokens=0, stream=None, flags=0):
        """pkv_decode_step on the library's own scratch: no workspace, nothing allocated."""
        pkv_decode_step_noalloc(self.h, layer, q, k_new, v_new, block_tables, context_lens, max_context_len,
                                softmax_scale, out, partition_tokens, stream, flags)
        return out

    def prefill_plan(self, q_dtype, num_q_heads, num_seqs, max_query_len, max_context_len, piece_tokens=0,
                     waves=False):
        """(piece tokens, pieces, workspace bytes) of pkv_prefill_attention for these sizes,
        and the wavefronts per workgroup as a fourth entry with waves=True."""
        T, n, nb, w = _i32(), _i32(), _sz(), _i32()
        _check(lib().pkv_prefill_plan(self.h, int(q_dtype), int(num_q_heads), int(num_seqs), int(max_query_len),
                                      int(max_context_len), int(piece_tokens), C.byref(T), C.byref(n),
                                      C.byref(nb), C.byref(w)))
        return (T.value, n.value, nb.value, w.value) if waves else (T.value, n.value, nb.value)

    def prefill(self, layer, q, query_start, max_query_len, block_tables, context_lens, softmax_scale,
                max_context_len, out=None, workspace=None, piece_tokens=0, stream=None):
        """Causal attention of each sequence's last q_len cached tokens (q rows packed by
        sequence, query_start [B+1] int32 on the device) -- pkv_prefill_attention. A
        workspace of the planned size is allocated when none is given."""
        import torch
        for t in (q, query_start, block_tables, context_lens):
            assert t.is_contiguous()
        assert query_start.dtype == torch.int32 and block_tables.dtype == torch.int32
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        assert out.is_contiguous() and out.dtype == torch.float32 and out.shape == q.shape
        B = int(context_lens.shape[0])
        if workspace is None and B > 0:
            nb = self.prefill_plan(_torch_dtype_code(q), q.shape[1], B, max_query_len, max_context_len,
                                   piece_tokens)[2]
            workspace = torch.zeros(nb, dtype=torch.uint8, device=q.device) if nb > 0 else None
        ws_ptr = _vp(workspace.data_ptr()) if workspace is not None else None
        ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
        _check(lib().pkv_prefill_attention(
            self.h, layer, _vp(q.data_ptr()), _torch_dtype_code(q), int(q.shape[1]), _vp(query_start.data_ptr()),
            int(max_query_len), _vp(block_tables.data_ptr()), int(block_tables.shape[1]),
            _vp(context_lens.data_ptr()), B, int(max_context_len), float(softmax_scale), int(piece_tokens),
            _vp(out.data_ptr()), ws_ptr, ws_bytes, _stream_ptr(stream)))
        return out

    def read_tail_blocks(self, layer, blocks):
        """FP16 staging tiles (seal_on_full pools): [n][2][Hkv][bs][d] binary16 bits."""
        blocks = np.ascontiguousarray(blocks, dtype=np.int32)
        out = np.zeros((len(blocks), 2, self.num_kv_heads, self.block_size, self.head_dim), dtype=np.uint16)
        _check(lib().pkv_read_tail_blocks(self.h, layer, _np_ptr(blocks), len(blocks), _np_ptr(out)))
        return out

    def read_blocks(self, layer, blocks):
        return pkv_read_blocks(self.h, layer, blocks, self.num_kv_heads, self.block_size,
                               self.head_dim, self.layer_kv_dtypes[layer])


# ------------------------------------------------------- Scheduler ----
def _arr(ptr, n, dtype):
    if n <= 0:
        return np.zeros(0, dtype=dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)


class Scheduler:
    """Continuous-batching step scheduler over a Pool (pkv_sched_* in
    include/pkv.h). step() returns the plan as numpy copies."""

    def __init__(self, pool: Pool, max_batch: int, max_model_len: int, reserve_blocks: int = 1,
                 batch_order: int = 0):
        self.pool = pool
        cfg = pkv_sched_config(max_batch, max_model_len, reserve_blocks, batch_order)
        h = _vp()
        _check(lib().pkv_sched_create(pool.h, C.byref(cfg), C.byref(h)))
        self.h = h
        pool._scheds.add(self)

    def close(self):
        if getattr(self, "h", None):
            lib().pkv_sched_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, request: int, prompt_len: int, max_new_tokens: int, prefix_seq: int = -1):
        _check(lib().pkv_sched_submit(self.h, request, prompt_len, max_new_tokens, prefix_seq))

    def step(self, eos=(), stream=None) -> dict:
        eos = np.ascontiguousarray(list(eos), dtype=np.int64)
        plan = pkv_step_plan()
        sp = _stream_ptr(stream) if self.pool.arena is not None else None
        _check(lib().pkv_sched_step(self.h, _np_ptr(eos) if eos.size else None, int(eos.size),
                                    C.byref(plan), sp))
        n, mb = plan.num_seqs, plan.max_blocks
        ev = [(int(plan.events[i].request), int(plan.events[i].kind)) for i in range(plan.num_events)]
        return {
            "seqs": _arr(plan.seqs, n, np.int64),
            "slots": _arr(plan.slots, n, np.int64),
            "block_tables": _arr(plan.block_tables, n * mb, np.int32).reshape(n, mb),
            "context_lens": _arr(plan.context_lens, n, np.int32),
            "max_blocks": mb,
            "max_context_len": int(plan.max_context_len),
            "prefill_seqs": _arr(plan.prefill_seqs, plan.num_prefill, np.int64),
            "prefill_first": _arr(plan.prefill_first, plan.num_prefill, np.int32),
            "prefill_tokens": _arr(plan.prefill_tokens, plan.num_prefill, np.int32),
            "prefill_slots": _arr(plan.prefill_slots, plan.prefill_total, np.int64),
            "events": ev,
        }

    def stats(self) -> dict:
        st = pkv_sched_stats()
        _check(lib().pkv_sched_get_stats(self.h, C.byref(st)))
        return {k: int(getattr(st, k)) for k, _ in pkv_sched_stats._fields_ if k != "pad_"}
