"""Python binding of liboasis (ctypes): argument marshalling only.

Every step of the decode hot path runs in the HIP kernels of liboasis.so;
this module turns torch tensors into device pointers and streams into
hipStream_t values and checks return codes.  PyTorch provides device memory
and streams.  The library must be built (``python -m
lookahead_sparse_kv_oasis_amd.build`` or ``__graft_entry__.build()``); a
missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# OASIS_LIBRARY names another build of the same library (the host-sanitized
# one that tests/test_sanitizers.py runs the host-side tests against).
LIB_PATH = os.environ.get("OASIS_LIBRARY") or os.path.join(_PKG, "liboasis.so")

OASIS_OK, OASIS_E_INVAL, OASIS_E_NOMEM, OASIS_E_HIP = 0, -1, -2, -3
OASIS_E_CAPACITY, OASIS_E_STATE, OASIS_E_NONFINITE, OASIS_E_DEVICE = -4, -5, -6, -7
OASIS_F32, OASIS_BF16 = 0, 1

TIME = dict(append=1, score=2, topk=4, select=8, gather=16, attn=32, combine=64, all=127)

BUF = dict(SUMMARY=0, SLOTS=1, HOST_KV=2, SCORES=3, IDS=4, SLOT_BLOCK=5, BLOCK_SLOT=6,
           LAST_USED=7, FETCH_BLOCK=8, FETCH_SLOT=9, ATT_BLOCK=10, ATT_SLOT=11, COUNTS=12)

EXPORTS = [
    "oasis_create", "oasis_create_shared", "oasis_destroy", "oasis_load_prefix",
    "oasis_set_state", "oasis_decode_layers", "oasis_decode_layers_ahead",
    "oasis_append_kv", "oasis_predict", "oasis_topk_from_scores", "oasis_select_and_fetch",
    "oasis_evict", "oasis_evict_attended", "oasis_get_state", "oasis_sparse_attn",
    "oasis_sparse_attn_noalloc", "oasis_sparse_attn_verify", "oasis_buffer_bytes", "oasis_read", "oasis_get_stats",
    "oasis_check", "oasis_set_timing", "oasis_set_timing_period",
    "oasis_set_score_topk_fusion", "oasis_set_fetch_in_attention",
    "oasis_set_attention_beside_copy", "oasis_set_attend_all_resident", "oasis_get_timing",
    "oasis_get_dims", "oasis_tokens",
    "oasis_copy_stream", "oasis_stream_create_cus", "oasis_stream_destroy",
    "oasis_stream_read", "oasis_kv_bytes_per_token", "oasis_cap_from_ratio",
    "oasis_strerror",
    "oasis_last_error",
]


class OasisError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class oasis_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_drafts", ctypes.c_int32),
                ("slots_per_head", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64)]


class oasis_attn_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
                 "list_stride", "slots_per_head", "reserved")]


class oasis_layer_io(ctypes.Structure):
    _fields_ = [("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("drafts", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class oasis_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("steps", "hits", "misses", "fetched", "attended", "bytes_fetched", "tokens",
                 "fetch_fused")]


class oasis_timing(ctypes.Structure):
    _fields_ = [(f"ms_{n}", ctypes.c_double) for n in
                ("append", "score", "topk", "select", "gather", "attn", "combine")] + \
               [(f"n_{n}", ctypes.c_int64) for n in
                ("append", "score", "topk", "select", "gather", "attn", "combine")]


_lib = None


def lib():
    """Load liboasis.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run lookahead_sparse_kv_oasis_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        H = ctypes.c_void_p
        sig = {
            "oasis_create": (ctypes.c_int, [ctypes.POINTER(oasis_layout), i32, i32, f32,
                                            ctypes.POINTER(ctypes.c_void_p)]),
            "oasis_create_shared": (ctypes.c_int, [ctypes.POINTER(oasis_layout), i32, i32, f32,
                                                   H, ctypes.POINTER(ctypes.c_void_p)]),
            "oasis_decode_layers": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.POINTER(oasis_layer_io), i32, i32, i32,
                                                   vp, vp]),
            "oasis_decode_layers_ahead": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p),
                                                         ctypes.POINTER(oasis_layer_io), i32, i32,
                                                         i32, i32, vp, vp, vp]),
            "oasis_destroy": (ctypes.c_int, [H]),
            "oasis_load_prefix": (ctypes.c_int, [H, vp, vp, i64, vp]),
            "oasis_set_state": (ctypes.c_int, [H, vp, vp]),
            "oasis_append_kv": (ctypes.c_int, [H, vp, vp, vp]),
            "oasis_predict": (ctypes.c_int, [H, vp, vp, i32, vp, vp, vp]),
            "oasis_topk_from_scores": (ctypes.c_int, [H, vp, vp, vp]),
            "oasis_select_and_fetch": (ctypes.c_int, [H, i32, vp, vp]),
            "oasis_evict": (ctypes.c_int, [H, vp, vp, i32, vp]),
            "oasis_evict_attended": (ctypes.c_int, [H, vp, ctypes.c_double, vp]),
            "oasis_get_state": (ctypes.c_int, [H, vp, vp, vp, vp, vp]),
            "oasis_sparse_attn": (ctypes.c_int, [H, vp, vp, vp]),
            "oasis_sparse_attn_verify": (ctypes.c_int, [H, vp, vp, i32, vp, vp, vp, vp]),
            "oasis_sparse_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(oasis_attn_desc), vp, vp,
                                                         vp, vp, vp, i64, vp, vp]),
            "oasis_buffer_bytes": (i64, [H, i32]),
            "oasis_read": (ctypes.c_int, [H, i32, i64, i64, vp]),
            "oasis_get_stats": (ctypes.c_int, [H, ctypes.POINTER(oasis_stats)]),
            "oasis_check": (ctypes.c_int, [H]),
            "oasis_set_timing": (ctypes.c_int, [H, i32]),
            "oasis_set_timing_period": (ctypes.c_int, [H, i32]),
            "oasis_set_score_topk_fusion": (ctypes.c_int, [H, i32]),
            "oasis_set_fetch_in_attention": (ctypes.c_int, [H, i32]),
            "oasis_set_attention_beside_copy": (ctypes.c_int, [H, i32]),
            "oasis_set_attend_all_resident": (ctypes.c_int, [H, i32]),
            "oasis_get_timing": (ctypes.c_int, [H, ctypes.POINTER(oasis_timing)]),
            "oasis_get_dims": (ctypes.c_int, [H, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                              ctypes.POINTER(i64), ctypes.POINTER(i32)]),
            "oasis_tokens": (i64, [H]),
            "oasis_copy_stream": (vp, [H]),
            "oasis_stream_read": (ctypes.c_int, [vp, i64, vp, i32, vp]),
            "oasis_stream_create_cus": (ctypes.c_int, [i32, i32, ctypes.POINTER(ctypes.c_void_p)]),
            "oasis_stream_destroy": (ctypes.c_int, [vp]),
            "oasis_kv_bytes_per_token": (ctypes.c_uint64, [i32, i32, i32, i32]),
            "oasis_cap_from_ratio": (i32, [f32, i32]),
            "oasis_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "oasis_last_error": (ctypes.c_char_p, [H]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    """Device (or host) address of a tensor / array, or None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be contiguous")
        return t.ctypes.data
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# oasis_select_and_fetch's copy argument: the handle's own placement of the copy
COPY_DEFAULT = ctypes.c_void_p(-1).value


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes) -> int:
    return int(lib().oasis_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def stream_read(buf, sink, workgroups: int, stream=None) -> None:
    """oasis_stream_read: one streaming read of the device tensor `buf`;
    sink (uint32 / int32 device tensor of `workgroups` entries) receives the
    per-workgroup XOR of the words read."""
    nbytes = buf.numel() * buf.element_size()
    rc = lib().oasis_stream_read(_ptr(buf), nbytes, _ptr(sink), workgroups, _stream(stream))
    if rc != OASIS_OK:
        raise OasisError(rc, "oasis_stream_read")


def stream_create_cus(first_cu: int, n_cus: int) -> int:
    """oasis_stream_create_cus: a HIP stream (as an int handle, for
    torch.cuda.ExternalStream) whose kernels run on CUs [first_cu, first_cu +
    n_cus) only; release it with stream_destroy."""
    s = ctypes.c_void_p()
    rc = lib().oasis_stream_create_cus(first_cu, n_cus, ctypes.byref(s))
    if rc != OASIS_OK:
        raise OasisError(rc, "oasis_stream_create_cus")
    return s.value


def stream_destroy(stream: int) -> None:
    rc = lib().oasis_stream_destroy(stream)
    if rc != OASIS_OK:
        raise OasisError(rc, "oasis_stream_destroy")


def sparse_attn_noalloc(desc: oasis_attn_desc, q, slots, att_block, att_slot, counts,
                        tokens: int, out, stream=None) -> int:
    """oasis_sparse_attn_noalloc on device tensors; returns the status."""
    return lib().oasis_sparse_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(slots),
                                           _ptr(att_block), _ptr(att_slot), _ptr(counts),
                                           int(tokens), _ptr(out), _stream(stream))


def cap_from_ratio(ratio, k_blocks) -> int:
    return int(lib().oasis_cap_from_ratio(ratio, k_blocks))


class Oasis:
    """One layer's handle.  Methods mirror the C-ABI calls of the same name."""

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim, dtype, max_drafts,
                 max_tokens, block_size=16, budget_tokens=2048, fetch_ratio=0.02,
                 slots_per_head=0, share_host_with: "Oasis | None" = None,
                 compute_units=0):
        """share_host_with: another handle whose host KV this layer reuses
        (oasis_create_shared); otherwise oasis_create.  compute_units: the
        layout field of that name (0: every CU)."""
        L = lib()
        self.layout = oasis_layout(batch, num_q_heads, num_kv_heads, head_dim, dtype,
                                   max_drafts, slots_per_head, compute_units, max_tokens)
        h = ctypes.c_void_p()
        if share_host_with is None:
            rc = L.oasis_create(ctypes.byref(self.layout), block_size, budget_tokens,
                                fetch_ratio, ctypes.byref(h))
            what = "oasis_create"
        else:
            rc = L.oasis_create_shared(ctypes.byref(self.layout), block_size, budget_tokens,
                                       fetch_ratio, share_host_with.h, ctypes.byref(h))
            what = "oasis_create_shared"
        if rc != OASIS_OK:
            raise OasisError(rc, f"{what}: " + L.oasis_strerror(rc).decode())
        self.h = h
        k, s, nb, bs = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
        L.oasis_get_dims(h, ctypes.byref(k), ctypes.byref(s), ctypes.byref(nb), ctypes.byref(bs))
        self.k_blocks, self.slots, self.nb_max, self.block_size = k.value, s.value, nb.value, bs.value
        self.batch, self.q_heads, self.kv_heads, self.head_dim = (batch, num_q_heads,
                                                                  num_kv_heads, head_dim)
        self.dtype = dtype

    # -- plumbing
    def _check(self, rc, what):
        if rc != OASIS_OK:
            L = lib()
            raise OasisError(rc, f"{what}: {L.oasis_strerror(rc).decode()}: "
                                 f"{L.oasis_last_error(self.h).decode()}")

    def close(self):
        if getattr(self, "h", None):
            lib().oasis_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- C-ABI calls
    def oasis_load_prefix(self, k_host: np.ndarray | None, v_host: np.ndarray | None,
                          length: int, stream=None):
        """k_host = v_host = None: start over from the prompt already in the host KV."""
        self._check(lib().oasis_load_prefix(self.h, _ptr(k_host), _ptr(v_host), length,
                                            _stream(stream)), "oasis_load_prefix")

    def oasis_set_state(self, slot_block: np.ndarray, last_used: np.ndarray):
        sb = np.ascontiguousarray(slot_block, np.int32)
        lu = np.ascontiguousarray(last_used, np.int32)
        self._check(lib().oasis_set_state(self.h, _ptr(sb), _ptr(lu)), "oasis_set_state")

    def oasis_append_kv(self, k, v, stream=None):
        self._check(lib().oasis_append_kv(self.h, _ptr(k), _ptr(v), _stream(stream)),
                    "oasis_append_kv")

    def oasis_predict(self, q, drafts, n_drafts, block_ids=None, scores=None, stream=None):
        self._check(lib().oasis_predict(self.h, _ptr(q), _ptr(drafts), n_drafts,
                                        _ptr(block_ids), _ptr(scores), _stream(stream)),
                    "oasis_predict")

    def oasis_topk_from_scores(self, scores, block_ids=None, stream=None):
        self._check(lib().oasis_topk_from_scores(self.h, _ptr(scores), _ptr(block_ids),
                                                 _stream(stream)), "oasis_topk_from_scores")

    def oasis_select_and_fetch(self, cap=-1, stream=None, copy=None):
        """copy: the stream of the host -> HBM copy; None leaves it where the
        handle puts it (inside the next attention by default)."""
        cp = COPY_DEFAULT if copy is None else _stream(copy)
        self._check(lib().oasis_select_and_fetch(self.h, cap, _stream(stream), cp),
                    "oasis_select_and_fetch")

    def oasis_evict_attended(self, draws, fraction: float, stream=None):
        """draws: float64 device tensor [B][Hkv][K]."""
        self._check(lib().oasis_evict_attended(self.h, _ptr(draws), float(fraction),
                                               _stream(stream)), "oasis_evict_attended")

    def oasis_get_state(self) -> dict:
        """slot_block, last_used [units][S]; fetch_list [units][K][2]; fetch_n
        [units]; attended [units][K] (host arrays)."""
        u = self.batch * self.kv_heads
        sb = np.empty((u, self.slots), np.int32)
        lu = np.empty((u, self.slots), np.int32)
        fl = np.empty((u, self.k_blocks, 2), np.int32)
        fn = np.empty(u, np.int32)
        at = np.empty((u, self.k_blocks), np.int32)
        self._check(lib().oasis_get_state(self.h, _ptr(sb), _ptr(lu), _ptr(fl), _ptr(fn),
                                          _ptr(at)), "oasis_get_state")
        return dict(slot_block=sb, last_used=lu, fetch_list=fl, fetch_n=fn, attended=at)

    def oasis_evict(self, blocks: np.ndarray, counts: np.ndarray, stream=None):
        blocks = np.ascontiguousarray(blocks, np.int32)
        counts = np.ascontiguousarray(counts, np.int32)
        self._check(lib().oasis_evict(self.h, _ptr(blocks), _ptr(counts), blocks.shape[-1],
                                      _stream(stream)), "oasis_evict")

    def oasis_sparse_attn(self, q, out, stream=None):
        self._check(lib().oasis_sparse_attn(self.h, _ptr(q), _ptr(out), _stream(stream)),
                    "oasis_sparse_attn")

    def oasis_sparse_attn_verify(self, q, drafts, n_drafts, k_drafts, v_drafts, out,
                                 stream=None):
        self._check(lib().oasis_sparse_attn_verify(self.h, _ptr(q), _ptr(drafts), n_drafts,
                                                   _ptr(k_drafts), _ptr(v_drafts), _ptr(out),
                                                   _stream(stream)),
                    "oasis_sparse_attn_verify")

    def oasis_check(self):
        self._check(lib().oasis_check(self.h), "oasis_check")

    def oasis_get_stats(self) -> dict:
        s = oasis_stats()
        self._check(lib().oasis_get_stats(self.h, ctypes.byref(s)), "oasis_get_stats")
        return {n: getattr(s, n) for n, _ in oasis_stats._fields_}

    def oasis_set_timing(self, mask=TIME["all"]):
        """mask: OR of TIME values (0 = off)."""
        self._check(lib().oasis_set_timing(self.h, int(mask)), "oasis_set_timing")

    def oasis_set_fetch_in_attention(self, on: bool):
        """Copy fetched blocks inside the next attention (True) or with the
        gather kernel on the copy stream right after the select (False)."""
        self._check(lib().oasis_set_fetch_in_attention(self.h, int(bool(on))),
                    "oasis_set_fetch_in_attention")

    def oasis_set_attention_beside_copy(self, on: bool):
        """Attend to the held blocks while a copy on another stream runs."""
        self._check(lib().oasis_set_attention_beside_copy(self.h, int(bool(on))),
                    "oasis_set_attention_beside_copy")

    def oasis_set_score_topk_fusion(self, on: bool):
        """Fuse score, top-K and select into one kernel (when the shape allows)."""
        self._check(lib().oasis_set_score_topk_fusion(self.h, int(bool(on))),
                    "oasis_set_score_topk_fusion")

    def oasis_set_attend_all_resident(self, on: bool):
        """Attend every block held after the step instead of the selected ones."""
        self._check(lib().oasis_set_attend_all_resident(self.h, int(bool(on))),
                    "oasis_set_attend_all_resident")

    def oasis_set_timing_period(self, period: int):
        """Time one launch in `period` of each timed kernel class."""
        self._check(lib().oasis_set_timing_period(self.h, int(period)), "oasis_set_timing_period")

    def oasis_get_timing(self) -> dict:
        t = oasis_timing()
        self._check(lib().oasis_get_timing(self.h, ctypes.byref(t)), "oasis_get_timing")
        return {n: getattr(t, n) for n, _ in oasis_timing._fields_}

    def oasis_tokens(self) -> int:
        return int(lib().oasis_tokens(self.h))

    def oasis_copy_stream(self) -> int:
        return lib().oasis_copy_stream(self.h)

    # -- inspection
    def read(self, which: str, dtype=np.int32) -> np.ndarray:
        code = BUF[which]
        n = int(lib().oasis_buffer_bytes(self.h, code))
        if n < 0:
            self._check(n, "oasis_buffer_bytes")
        out = np.empty(n // np.dtype(dtype).itemsize, dtype=dtype)
        self._check(lib().oasis_read(self.h, code, 0, n, out.ctypes.data), "oasis_read")
        return out

    def read_range(self, which: str, offset: int, nbytes: int, dtype=np.uint8) -> np.ndarray:
        out = np.empty(nbytes // np.dtype(dtype).itemsize, dtype=dtype)
        self._check(lib().oasis_read(self.h, BUF[which], offset, nbytes, out.ctypes.data),
                    "oasis_read")
        return out


class LayerStep:
    """Argument block of oasis_decode_layers for a fixed list of layer handles.

    set(l, ...) stores the device pointers of layer l's inputs and output;
    run() issues one decode step over all layers."""

    def __init__(self, layers):
        self.layers = list(layers)
        n = len(self.layers)
        self._h = (ctypes.c_void_p * n)(*[x.h for x in self.layers])
        self._io = (oasis_layer_io * n)()

    def set(self, l, k_new, v_new, q, drafts, out):
        io = self._io[l]
        io.k_new, io.v_new = _ptr(k_new), _ptr(v_new)
        io.q, io.drafts, io.out = _ptr(q), _ptr(drafts), _ptr(out)

    def run(self, n_drafts, cap, stream=None, side=None):
        """side=None runs every layer on `stream` in order; a different stream
        overlaps prediction/selection with attention."""
        st = _stream(stream)
        sd = st if side is None else _stream(side)
        rc = lib().oasis_decode_layers(self._h, self._io, len(self.layers), n_drafts, cap, st, sd)
        if rc != OASIS_OK:
            self.layers[0]._check(rc, "oasis_decode_layers")

    def run_ahead(self, n_drafts, cap, stream, side, xfer, cap_correct=0):
        """oasis_decode_layers_ahead: the lookahead ordering on three streams
        (cap_correct > 0: with decode-time miss correction)."""
        rc = lib().oasis_decode_layers_ahead(self._h, self._io, len(self.layers), n_drafts, cap,
                                             cap_correct, _stream(stream), _stream(side),
                                             _stream(xfer))
        if rc != OASIS_OK:
            self.layers[0]._check(rc, "oasis_decode_layers_ahead")
