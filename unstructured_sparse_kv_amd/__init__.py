"""Python binding of libmustafar.so (MUSTAFAR hot path on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensor.data_ptr()) and streams.  The
names mirror the C ABI in include/mustafar.h.  Importing raises when the
library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmustafar.so")

MUSTAFAR_OK = 0
MUSTAFAR_EINVAL = -1
MUSTAFAR_EUNSUPPORTED = -2
MUSTAFAR_ENODEV = -3
MUSTAFAR_ELAUNCH = -4
MUSTAFAR_ENOSPACE = -5
STATUS_APPEND_FULL = 1
STATUS_BAD_OFFSETS = 2
HEAD_DIM = 128
MAX_HEAD_KEEP = 128

# Every symbol include/mustafar.h declares.
EXPORTS = (
    "mustafar_status_str", "mustafar_keep_from_sparsity", "mustafar_kv_alloc_bytes",
    "mustafar_kv_used_bytes", "mustafar_prune_compress", "mustafar_append_token",
    "mustafar_decode_auto_splits", "mustafar_decode_workspace_bytes",
    "mustafar_decode_workspace_init", "mustafar_decode_attn", "mustafar_decode_attn_valu",
    "mustafar_decode_step", "mustafar_dense_decode_attn", "mustafar_probe_stream_read",
    "mustafar_prune_compress_24", "mustafar_decode_attn_24", "mustafar_prune_compress_channel",
    "mustafar_decode_step_noalloc",
)
NOALLOC_SCRATCH_BYTES = 8 << 20


class KVStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("keep", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("bitmaps", ctypes.c_void_p), ("values", ctypes.c_void_p), ("tile_offsets", ctypes.c_void_p),
        ("head_keep", ctypes.c_void_p),
    ]


class MustafarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # Load torch's HIP runtime first: libmustafar.so then binds to that same
        # libamdhip64 (matching soname) instead of pulling in a second runtime.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        KVP = ctypes.POINTER(KVStruct)
        sig = {
            "mustafar_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "mustafar_keep_from_sparsity": (ctypes.c_int, [ctypes.c_double, I32]),
            "mustafar_kv_alloc_bytes": (ctypes.c_int, [KVP, ctypes.POINTER(U64), ctypes.POINTER(U64),
                                                       ctypes.POINTER(U64)]),
            "mustafar_kv_used_bytes": (ctypes.c_int, [KVP, P, ctypes.POINTER(I64)]),
            "mustafar_prune_compress": (ctypes.c_int, [KVP, P, I64, P, P]),
            "mustafar_append_token": (ctypes.c_int, [KVP, KVP, P, P, P, P, P]),
            "mustafar_decode_auto_splits": (ctypes.c_int, [I32, I32, I32]),
            "mustafar_decode_workspace_bytes": (ctypes.c_int, [I32, I32, I32, I32, I32, I32,
                                                               ctypes.POINTER(U64)]),
            "mustafar_decode_workspace_init": (ctypes.c_int, [P, U64, P]),
            "mustafar_decode_attn": (ctypes.c_int, [P, I32, KVP, KVP, P, I32, ctypes.c_float, I32, P,
                                                    P, U64, P]),
            "mustafar_decode_attn_valu": (ctypes.c_int, [P, I32, KVP, KVP, P, I32, ctypes.c_float,
                                                         I32, P, P, U64, P]),
            "mustafar_decode_step": (ctypes.c_int, [P, I32, KVP, KVP, P, P, P, P, I32, ctypes.c_float,
                                                    I32, P, P, U64, P]),
            "mustafar_decode_step_noalloc": (ctypes.c_int, [P, I32, KVP, KVP, P, P, P, P, I32,
                                                            ctypes.c_float, I32, P, P]),
            "mustafar_dense_decode_attn": (ctypes.c_int, [P, I32, P, P, I32, I32, I32, I64, P, I32,
                                                          ctypes.c_float, I32, P, P, U64, P]),
            "mustafar_probe_stream_read": (ctypes.c_int, [P, U64, P, P]),
            "mustafar_prune_compress_24": (ctypes.c_int, [KVP, P, I64, P, P]),
            "mustafar_prune_compress_channel": (ctypes.c_int, [KVP, P, I64, P, P]),
            "mustafar_decode_attn_24": (ctypes.c_int, [P, I32, KVP, KVP, P, I32, ctypes.c_float, I32,
                                                       P, P, U64, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().mustafar_status_str(int(status)).decode()


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise MustafarError(fn, rc)
    return rc


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def keep_from_sparsity(sparsity: float, head_dim: int = HEAD_DIM) -> int:
    return _check("mustafar_keep_from_sparsity", lib().mustafar_keep_from_sparsity(sparsity, head_dim))


def decode_auto_splits(batch: int, num_kv_heads: int, max_seq_len: int) -> int:
    return _check("mustafar_decode_auto_splits",
                  lib().mustafar_decode_auto_splits(batch, num_kv_heads, max_seq_len))


class CompressedKV:
    """One compressed tensor (key or value cache of one layer) in device memory.

    With head_keep (a sequence of num_kv_heads ints), kv head h keeps head_keep[h]
    values per row and `keep` is their maximum (pass keep=None to take it)."""

    def __init__(self, batch: int, num_kv_heads: int, keep, capacity: int, device="cuda",
                 head_keep=None):
        import numpy as np
        import torch
        self.head_keep = None
        if head_keep is not None:
            self.head_keep = np.ascontiguousarray(np.asarray(head_keep, dtype=np.int32))
            if keep is None:
                keep = int(self.head_keep.max())
        self.s = KVStruct(batch, num_kv_heads, HEAD_DIM, keep, capacity, None, None, None,
                          None if self.head_keep is None else self.head_keep.ctypes.data)
        nb, nv, no = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        _check("mustafar_kv_alloc_bytes", lib().mustafar_kv_alloc_bytes(
            ctypes.byref(self.s), ctypes.byref(nb), ctypes.byref(nv), ctypes.byref(no)))
        self.bitmaps = torch.zeros(nb.value // 8, dtype=torch.int64, device=device)
        self.values = torch.zeros(nv.value // 2, dtype=torch.int16, device=device)
        self.tile_offsets = torch.zeros(no.value // 4, dtype=torch.int32, device=device)
        self.s.bitmaps = self.bitmaps.data_ptr()
        self.s.values = self.values.data_ptr()
        self.s.tile_offsets = self.tile_offsets.data_ptr()
        self.batch, self.num_kv_heads, self.keep, self.capacity = batch, num_kv_heads, keep, capacity

    @property
    def ref(self):
        return ctypes.byref(self.s)

    def used_bytes(self, seq_lens_host) -> int:
        import numpy as np
        seq = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
        out = ctypes.c_int64()
        _check("mustafar_kv_used_bytes", lib().mustafar_kv_used_bytes(
            self.ref, seq.ctypes.data_as(ctypes.c_void_p), ctypes.byref(out)))
        return out.value

    def views(self):
        """(bitmaps [B][H][cap][2] int64, values, tile_offsets [B][H][cap/64+1] int32); values is
        [B][H][cap*keep] int16, or [B][cap*sum(head_keep)] with per-head keep."""
        B, H, cap, k = self.batch, self.num_kv_heads, self.capacity, self.keep
        if self.head_keep is None:
            vals = self.values[:B * H * cap * k].view(B, H, cap * k)
        else:
            S = int(self.head_keep.sum())
            vals = self.values[:B * cap * S].view(B, cap * S)
        return (self.bitmaps.view(B, H, cap, 2), vals, self.tile_offsets.view(B, H, cap // 64 + 1))


def prune_compress(dst: CompressedKV, dense, seq_lens, stream=None) -> None:
    """dense: [B][H][t_stride][128] fp16 contiguous (device); seq_lens int32 [B] (device)."""
    assert dense.is_contiguous() and dense.shape[-1] == HEAD_DIM
    _check("mustafar_prune_compress", lib().mustafar_prune_compress(
        dst.ref, dense.data_ptr(), dense.shape[2], seq_lens.data_ptr(), _stream(stream)))


def prune_compress_channel(dst: CompressedKV, dense, seq_lens, stream=None) -> None:
    """Channel-wise pruning: per full 64-row tile each channel keeps dst.keep/2 rows."""
    assert dense.is_contiguous() and dense.shape[-1] == HEAD_DIM
    _check("mustafar_prune_compress_channel", lib().mustafar_prune_compress_channel(
        dst.ref, dense.data_ptr(), dense.shape[2], seq_lens.data_ptr(), _stream(stream)))


def prune_compress_24(dst: CompressedKV, dense, seq_lens, stream=None) -> None:
    """2:4 comparator: dense [B][H][t_stride][128] fp16 -> dst (keep 64)."""
    assert dense.is_contiguous() and dense.shape[-1] == HEAD_DIM
    _check("mustafar_prune_compress_24", lib().mustafar_prune_compress_24(
        dst.ref, dense.data_ptr(), dense.shape[2], seq_lens.data_ptr(), _stream(stream)))


def append_token(k: CompressedKV, v: CompressedKV, k_new, v_new, seq_lens, status=None,
                 stream=None) -> None:
    """k_new / v_new: [B][H][128] fp16 (device); seq_lens int32 [B] advanced in place."""
    assert k_new.is_contiguous() and v_new.is_contiguous()
    _check("mustafar_append_token", lib().mustafar_append_token(
        k.ref, v.ref, k_new.data_ptr(), v_new.data_ptr(), seq_lens.data_ptr(), _ptr(status),
        _stream(stream)))


def workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, splits=0) -> int:
    out = ctypes.c_uint64()
    _check("mustafar_decode_workspace_bytes", lib().mustafar_decode_workspace_bytes(
        batch, num_q_heads, num_kv_heads, HEAD_DIM, max_seq_len, splits, ctypes.byref(out)))
    return out.value


def make_workspace(batch, num_q_heads, num_kv_heads, max_seq_len, splits=0, device="cuda",
                   stream=None):
    """Allocate and initialise a decode workspace (uint8 tensor)."""
    import torch
    n = workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len, splits)
    ws = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=device)
    _check("mustafar_decode_workspace_init", lib().mustafar_decode_workspace_init(
        ws.data_ptr(), ws.numel(), _stream(stream)))
    return ws


def decode_attn(q, k: CompressedKV, v: CompressedKV, seq_lens, max_seq_len: int, scale: float,
                out, workspace, splits: int = 0, stream=None) -> None:
    """q, out: [B][Hq][128] fp16 (device).  Matrix-core kernel."""
    assert q.is_contiguous() and out.is_contiguous()
    _check("mustafar_decode_attn", lib().mustafar_decode_attn(
        q.data_ptr(), q.shape[1], k.ref, v.ref, seq_lens.data_ptr(), max_seq_len, scale, splits,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def decode_attn_valu(q, k: CompressedKV, v: CompressedKV, seq_lens, max_seq_len: int,
                     scale: float, out, workspace, splits: int = 0, stream=None) -> None:
    """Same as decode_attn, vector-unit kernel."""
    assert q.is_contiguous() and out.is_contiguous()
    _check("mustafar_decode_attn_valu", lib().mustafar_decode_attn_valu(
        q.data_ptr(), q.shape[1], k.ref, v.ref, seq_lens.data_ptr(), max_seq_len, scale, splits,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def decode_attn_24(q, k: CompressedKV, v: CompressedKV, seq_lens, max_seq_len: int, scale: float,
                   out, workspace, splits: int = 0, stream=None) -> None:
    """Same as decode_attn over 2:4 caches (from prune_compress_24), 2:4 kernel."""
    assert q.is_contiguous() and out.is_contiguous()
    _check("mustafar_decode_attn_24", lib().mustafar_decode_attn_24(
        q.data_ptr(), q.shape[1], k.ref, v.ref, seq_lens.data_ptr(), max_seq_len, scale, splits,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def decode_step(q, k: CompressedKV, v: CompressedKV, k_new, v_new, seq_lens, max_seq_len: int,
                scale: float, out, workspace, status=None, splits: int = 0, stream=None) -> None:
    """Fused append + decode: k_new / v_new [B][Hkv][128] fp16 become row seq_lens[b],
    the attention covers it, seq_lens advances (device tensors)."""
    assert q.is_contiguous() and out.is_contiguous()
    assert k_new.is_contiguous() and v_new.is_contiguous()
    _check("mustafar_decode_step", lib().mustafar_decode_step(
        q.data_ptr(), q.shape[1], k.ref, v.ref, k_new.data_ptr(), v_new.data_ptr(),
        seq_lens.data_ptr(), _ptr(status), max_seq_len, scale, splits, out.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))


def decode_step_noalloc(q, k: CompressedKV, v: CompressedKV, k_new, v_new, seq_lens,
                        max_seq_len: int, scale: float, out, status=None, splits: int = 0,
                        stream=None) -> None:
    """decode_step without a workspace: the split partials go to the library's own
    device scratch array (calls on one device must not overlap in time)."""
    assert q.is_contiguous() and out.is_contiguous()
    assert k_new.is_contiguous() and v_new.is_contiguous()
    _check("mustafar_decode_step_noalloc", lib().mustafar_decode_step_noalloc(
        q.data_ptr(), q.shape[1], k.ref, v.ref, k_new.data_ptr(), v_new.data_ptr(),
        seq_lens.data_ptr(), _ptr(status), max_seq_len, scale, splits, out.data_ptr(),
        _stream(stream)))


def dense_decode_attn(q, k, v, seq_lens, max_seq_len: int, scale: float, out, workspace,
                      splits: int = 0, stream=None) -> None:
    """q, out: [B][Hq][128]; k, v: [B][Hkv][t_stride][128] fp16 (device)."""
    assert q.is_contiguous() and out.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    B, Hkv, t_stride, d = k.shape
    _check("mustafar_dense_decode_attn", lib().mustafar_dense_decode_attn(
        q.data_ptr(), q.shape[1], k.data_ptr(), v.data_ptr(), B, Hkv, d, t_stride,
        seq_lens.data_ptr(), max_seq_len, scale, splits, out.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(stream)))


def probe_stream_read(buf, sink, stream=None) -> None:
    nbytes = buf.numel() * buf.element_size() // 4096 * 4096
    _check("mustafar_probe_stream_read", lib().mustafar_probe_stream_read(
        buf.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)))
