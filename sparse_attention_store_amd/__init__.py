"""Python binding of libdsa, the gfx950 DSA decode/prefill path.

Thin ctypes marshalling over the C ABI declared in include/dsa.h: each
function checks tensor dtypes/devices/shapes, passes device pointers, the
dims struct and the current HIP stream, and raises DsaError on a non-zero
status.  With prepare=True a function returns a Bound call instead: the
checks and the argument conversion happen once, and each call of it only
launches (a decode loop calls its steps many times on the same buffers).  Every step of the path runs in the library's HIP kernels; PyTorch
only provides device memory and streams.  There is no fallback: if the
shared library is missing, importing any entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32 = 0
DSA_BF16 = 1


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    """Mirror of dsa_dims (indexer + MLA geometry)."""
    _fields_ = [
        ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
        ("kpool", ctypes.c_int32), ("index_topk", ctypes.c_int32),
        ("out_width", ctypes.c_int32), ("mla_heads", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32), ("row_bytes", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
    ]

    @classmethod
    def of(cls, d) -> "Dims":
        """Build from any object with the same attribute names."""
        return cls(int(d.idx_heads), int(d.idx_dim), int(d.kpool), int(d.index_topk),
                   int(d.out_width), int(d.mla_heads), int(d.latent_dim), int(d.row_bytes),
                   float(d.ln_eps))

    @property
    def select_k(self) -> int:
        return self.index_topk // self.kpool


class _Seqs(ctypes.Structure):
    _fields_ = [("first_valid", ctypes.c_void_p), ("row_base", ctypes.c_void_p),
                ("tok_base", ctypes.c_void_p), ("pool_base", ctypes.c_void_p)]


@dataclass
class Seqs:
    """Per-sequence layout as device tensors (int32 first_valid, int64 bases)."""
    first_valid: torch.Tensor
    row_base: torch.Tensor
    tok_base: torch.Tensor
    pool_base: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.first_valid.shape[0])

    def _c(self) -> _Seqs:
        for name, t, dt in (("first_valid", self.first_valid, torch.int32),
                            ("row_base", self.row_base, torch.int64),
                            ("tok_base", self.tok_base, torch.int64),
                            ("pool_base", self.pool_base, torch.int64)):
            _check(t, dt, name)
        return _Seqs(self.first_valid.data_ptr(), self.row_base.data_ptr(),
                     self.tok_base.data_ptr(), self.pool_base.data_ptr())


class _PagedSeqs(ctypes.Structure):
    _fields_ = [("first_valid", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int32)]


@dataclass
class PagedSeqs:
    """Per-sequence layout of paged caches: int32 first_valid [B] and the int32
    block table [B, stride] (physical block of each 256-position block)."""
    first_valid: torch.Tensor
    block_table: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.first_valid.shape[0])

    def _c(self) -> _PagedSeqs:
        _check(self.first_valid, torch.int32, "first_valid")
        _check(self.block_table, torch.int32, "block_table")
        if self.block_table.dim() != 2 or self.block_table.shape[0] != self.num_seqs:
            raise ValueError("block_table must be [num_seqs, stride]")
        return _PagedSeqs(self.first_valid.data_ptr(), self.block_table.data_ptr(), int(self.block_table.shape[1]))


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_store_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        DP, SP, PP = ctypes.POINTER(Dims), ctypes.POINTER(_Seqs), ctypes.POINTER(_PagedSeqs)
        sig = {
            "dsa_abi_version": (ctypes.c_int, []),
            "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "dsa_store_int8": (ctypes.c_int, [DP, P, ctypes.c_int, I64, I64, P, P, I64, P]),
            "dsa_index_pools": (ctypes.c_int, [DP, P, P, ctypes.c_int, P, P, SP, I32, P, P, I32, P, P]),
            "dsa_append_tokens": (ctypes.c_int, [DP, ctypes.c_int, P, I64, I64, P, P, I64, P, P, P, P, SP, I32,
                                                 P, P, I32, P, P]),
            "dsa_index_scores": (ctypes.c_int, [DP, P, P, P, SP, I32, P, P, I32, I32, P, P]),
            "dsa_topk_workspace_bytes": (SZ, [DP, I32, I32]),
            "dsa_topk_select": (ctypes.c_int, [DP, P, I32, SP, I32, P, P, I32, P, P, SZ, P]),
            "dsa_topk_select_expand": (ctypes.c_int, [DP, P, I32, SP, I32, P, P, I32, P, P, P, SZ, P]),
            "dsa_expand_selection": (ctypes.c_int, [DP, P, SP, I32, P, P, I32, P, P]),
            "dsa_sparse_mla_workspace_bytes": (SZ, [DP, I32, I32]),
            "dsa_sparse_mla": (ctypes.c_int, [DP, P, ctypes.c_int, P, I64, P, I32, F, P, ctypes.c_int, P, I32,
                                              P, SZ, P]),
            "dsa_index_scores_select_workspace_bytes": (SZ, [DP, I32, I32]),
            "dsa_index_scores_select": (ctypes.c_int, [DP, P, P, P, SP, I32, P, P, I32, I32, P, P, P, P, SZ, P]),
            "dsa_index_scores_groups": (ctypes.c_int, [DP, P, P, P, SP, I32, P, P, I32, I32, P, P, SZ, P]),
            "dsa_topk_select_groups": (ctypes.c_int, [DP, P, I32, SP, I32, P, P, I32, P, P, P, SZ, P]),
            "dsa_append_scores_groups": (ctypes.c_int, [DP, ctypes.c_int, P, I64, I64, P, P, I64, P, P, P, P, P, P,
                                                        I32, P, P, P, SP, I32, P, P, I32, I32, P, P, SZ, P]),
            "dsa_topk_sparse_mla": (ctypes.c_int, [DP, P, I32, SP, I32, P, P, I32, P, P, P, SZ, P, ctypes.c_int, P,
                                                   I64, F, P, ctypes.c_int, P, I32, P, SZ, P]),
            "dsa_time_next_scoring_launch": (ctypes.c_int, [P, P]),
            "dsa_decode_step_workspace_bytes": (SZ, [DP, I32, I32]),
            "dsa_decode_step_status": (ctypes.c_int, [P, SZ, P]),
            "dsa_index_pools_int8": (ctypes.c_int, [DP, P, P, ctypes.c_int, P, P, SP, I32, P, P, I32, P, P, P, P]),
            "dsa_index_scores_int8": (ctypes.c_int, [DP, P, P, P, P, SP, I32, P, P, I32, I32, P, P]),
            "dsa_index_scores_groups_int8": (ctypes.c_int, [DP, P, P, P, P, SP, I32, P, P, I32, I32, P, P, SZ, P]),
            "dsa_append_scores_groups_int8": (ctypes.c_int, [DP, ctypes.c_int, P, I64, I64, P, P, I64, P, P, P, P, P,
                                                             P, I32, P, P, P, P, SP, I32, P, P, I32, I32, P, P, SZ,
                                                             P]),
            "dsa_append_scores_groups_shared": (ctypes.c_int, [DP, ctypes.c_int, P, I64, I64, P, P, I64, P, P, P, P, P,
                                                               P, I32, P, P, P, P, SP, I32, P, P, I32, I32, P, P, SZ,
                                                               I32, P]),
            "dsa_index_pools_paged": (ctypes.c_int, [DP, P, P, ctypes.c_int, P, P, PP, I32, P, P, I32, P, P]),
            "dsa_index_scores_groups_paged": (ctypes.c_int, [DP, P, P, P, PP, I32, P, P, I32, I32, P, P, SZ, P]),
            "dsa_topk_select_groups_paged": (ctypes.c_int, [DP, P, I32, PP, I32, P, P, I32, P, P, P, SZ, P]),
            "dsa_index_select_chunked_workspace_bytes": (SZ, [DP, I32, I32]),
            "dsa_index_select_chunked": (ctypes.c_int, [DP, P, P, P, SP, I32, P, P, I32, I32, I32, P, P, P, SZ, P]),
            "dsa_sparse_mla_noalloc_scratch_bytes": (SZ, []),
            "dsa_sparse_mla_noalloc": (ctypes.c_int, [DP, P, ctypes.c_int, P, I64, P, I32, F, P, ctypes.c_int, P,
                                                      I32, P]),
            "dsa_decode_step": (ctypes.c_int, [DP, P, P, P, SP, I32, P, P, I32, I32, P, ctypes.c_int, P, I64, F,
                                               P, ctypes.c_int, P, P, P, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _raise(fn: str, st: int):
    if st != 0:
        raise DsaError(fn, st, lib().dsa_status_string(st).decode())


class Bound:
    """A validated call whose C arguments were converted once (prepare=True):
    calling it only launches, on the stream that was current when it was
    prepared, with the buffers it was prepared with."""
    __slots__ = ("_name", "_fn", "_args")

    def __init__(self, name: str, args):
        fn = getattr(lib(), name)
        self._name, self._fn = name, fn
        conv = []
        for a, t in zip(args, fn.argtypes):
            conv.append(a if isinstance(a, (ctypes._SimpleCData, ctypes.Structure)) or type(a).__name__ == "CArgObject"
                        else t(a))
        self._args = tuple(conv)

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            _raise(self._name, st)


def _call(name: str, prepare: bool, *args):
    if prepare:
        return Bound(name, args)
    _raise(name, getattr(lib(), name)(*args))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def abi_version() -> int:
    return lib().dsa_abi_version()


def status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def store_int8(dims: Dims, latent: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor, stream=None, prepare: bool = False):
    """Quantise latent rows [n, D] (bf16/fp32) into INT8 rows of cache [rows, row_bytes] at slots."""
    if latent.dim() != 2 or (latent.shape[0] > 0 and latent.stride(1) != 1):
        raise ValueError("latent must be [n, D] with unit stride in D")
    if latent.dtype not in (torch.bfloat16, torch.float32) or not latent.is_cuda:
        raise TypeError("latent must be a bf16/fp32 device tensor")
    _check(slots, torch.int64, "slots")
    _check(cache, torch.int8, "cache")
    if slots.numel() != latent.shape[0]:
        raise ValueError("slots must have one entry per latent row")
    return _call("dsa_store_int8", prepare, 
        ctypes.byref(dims), latent.data_ptr(), _dt(latent), latent.shape[0], latent.stride(0),
        slots.data_ptr(), cache.data_ptr(), cache.shape[0], _stream(stream))


def index_pools(dims: Dims, k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                seqs: Seqs, pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int,
                pools: torch.Tensor, stream=None, prepare: bool = False):
    """Build pools [pool_begin[b], pool_end[b]) of each sequence into pools (bf16 [*, idx_dim])."""
    if k.dtype != gate.dtype:
        raise TypeError("k and gate must share a dtype")
    for name, t in (("k", k), ("gate", gate)):
        _check(t, k.dtype, name)
    _check(ln_w, torch.float32, "ln_w")
    _check(ln_b, torch.float32, "ln_b")
    _check(pool_begin, torch.int32, "pool_begin")
    _check(pool_end, torch.int32, "pool_end")
    _check(pools, torch.bfloat16, "pools")
    return _call("dsa_index_pools", prepare, 
        ctypes.byref(dims), k.data_ptr(), gate.data_ptr(), _dt(k), ln_w.data_ptr(), ln_b.data_ptr(),
        ctypes.byref(seqs._c()), seqs.num_seqs, pool_begin.data_ptr(), pool_end.data_ptr(),
        int(max_pools), pools.data_ptr(), _stream(stream))


def append_tokens(dims: Dims, latent: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor,
                  k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor, seqs: Seqs,
                  pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int, pools: torch.Tensor,
                  stream=None, prepare: bool = False):
    """store_int8(latent, slots, cache) and index_pools(k, gate, ...) in one launch (one dtype for all)."""
    if latent.dim() != 2 or (latent.shape[0] > 0 and latent.stride(1) != 1):
        raise ValueError("latent must be [n, D] with unit stride in D")
    if latent.dtype not in (torch.bfloat16, torch.float32) or not latent.is_cuda:
        raise TypeError("latent must be a bf16/fp32 device tensor")
    _check(slots, torch.int64, "slots")
    _check(cache, torch.int8, "cache")
    if slots.numel() != latent.shape[0]:
        raise ValueError("slots must have one entry per latent row")
    for name, t in (("k", k), ("gate", gate)):
        _check(t, latent.dtype, name)
    _check(ln_w, torch.float32, "ln_w")
    _check(ln_b, torch.float32, "ln_b")
    _check(pool_begin, torch.int32, "pool_begin")
    _check(pool_end, torch.int32, "pool_end")
    _check(pools, torch.bfloat16, "pools")
    return _call("dsa_append_tokens", prepare, 
        ctypes.byref(dims), _dt(latent), latent.data_ptr(), latent.shape[0], latent.stride(0), slots.data_ptr(),
        cache.data_ptr(), cache.shape[0], k.data_ptr(), gate.data_ptr(), ln_w.data_ptr(), ln_b.data_ptr(),
        ctypes.byref(seqs._c()), seqs.num_seqs, pool_begin.data_ptr(), pool_end.data_ptr(), int(max_pools),
        pools.data_ptr(), _stream(stream))


def index_scores(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor, seqs: Seqs,
                 q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor, stream=None, prepare: bool = False):
    """scores [T, stride] (fp32) from q_idx [T, Hi, Di] (bf16), w [T, Hi] (fp32), pools (bf16)."""
    _check(q_idx, torch.bfloat16, "q_idx")
    _check(w, torch.float32, "w")
    _check(pools, torch.bfloat16, "pools")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    _check(scores, torch.float32, "scores")
    T = q_pos.shape[0]
    if scores.dim() != 2 or scores.shape[0] != T:
        raise ValueError("scores must be [T, stride]")
    return _call("dsa_index_scores", prepare, 
        ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(), pools.data_ptr(), ctypes.byref(seqs._c()),
        seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), T, scores.shape[1], scores.data_ptr(),
        _stream(stream))


def topk_workspace_bytes(dims: Dims, T: int, score_stride: int) -> int:
    return int(lib().dsa_topk_workspace_bytes(ctypes.byref(dims), int(T), int(score_stride)))


def topk_workspace(dims: Dims, T: int, score_stride: int, device="cuda") -> torch.Tensor | None:
    """A scratch workspace of the required size (None when no workspace is needed)."""
    n = topk_workspace_bytes(dims, T, score_stride)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def topk_select(dims: Dims, scores: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                pool_ids: torch.Tensor, workspace: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """pool_ids [T, select_k] (int32): ascending selected pool ids, -1 padded."""
    _check(scores, torch.float32, "scores")
    _check(pool_ids, torch.int32, "pool_ids")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    T = q_pos.shape[0]
    ws_bytes = 0
    if workspace is not None:
        _check(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return _call("dsa_topk_select", prepare, 
        ctypes.byref(dims), scores.data_ptr(), scores.shape[1], ctypes.byref(seqs._c()), seqs.num_seqs,
        q_seq.data_ptr(), q_pos.data_ptr(), T, pool_ids.data_ptr(), _ptr(workspace), ws_bytes,
        _stream(stream))


def topk_select_expand(dims: Dims, scores: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                       indices: torch.Tensor, pool_ids: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """Top-k selection written straight as index lists [T, out_width] (and pool ids if given)."""
    _check(scores, torch.float32, "scores")
    _check(indices, torch.int32, "indices")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    T = q_pos.shape[0]
    ws_bytes = 0
    if workspace is not None:
        _check(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return _call("dsa_topk_select_expand", prepare, 
        ctypes.byref(dims), scores.data_ptr(), scores.shape[1], ctypes.byref(seqs._c()), seqs.num_seqs,
        q_seq.data_ptr(), q_pos.data_ptr(), T, _ptr(pool_ids), indices.data_ptr(), _ptr(workspace), ws_bytes,
        _stream(stream))


def expand_selection(dims: Dims, pool_ids: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor,
                     q_pos: torch.Tensor, indices: torch.Tensor, stream=None, prepare: bool = False):
    """indices [T, out_width] (int32) from pool_ids [T, select_k]."""
    _check(pool_ids, torch.int32, "pool_ids")
    _check(indices, torch.int32, "indices")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    return _call("dsa_expand_selection", prepare, 
        ctypes.byref(dims), pool_ids.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs,
        q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0], indices.data_ptr(), _stream(stream))


def sparse_mla_workspace_bytes(dims: Dims, T: int, num_splits: int = 0) -> int:
    return int(lib().dsa_sparse_mla_workspace_bytes(ctypes.byref(dims), int(T), int(num_splits)))


def sparse_mla(dims: Dims, q: torch.Tensor, cache: torch.Tensor, indices: torch.Tensor, scale: float,
               out: torch.Tensor, lse: torch.Tensor | None = None, num_splits: int = 0,
               workspace: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """out [T, H, D] = sparse NoPE MLA of q [T, H, D] over the INT8 rows listed in indices [T, W]."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    _check(q, q.dtype, "q")
    _check(cache, torch.int8, "cache")
    _check(indices, torch.int32, "indices")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    _check(out, out.dtype, "out")
    if lse is not None:
        _check(lse, torch.float32, "lse")
    T = q.shape[0]
    ws_bytes = 0
    if workspace is not None:
        _check(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return _call("dsa_sparse_mla", prepare, 
        ctypes.byref(dims), q.data_ptr(), _dt(q), cache.data_ptr(), cache.shape[0], indices.data_ptr(),
        T, float(scale), out.data_ptr(), _dt(out), _ptr(lse), int(num_splits), _ptr(workspace), ws_bytes,
        _stream(stream))


def sparse_mla_noalloc_scratch_bytes() -> int:
    return int(lib().dsa_sparse_mla_noalloc_scratch_bytes())


def sparse_mla_noalloc(dims: Dims, q: torch.Tensor, cache: torch.Tensor, indices: torch.Tensor, scale: float,
                       out: torch.Tensor, lse: torch.Tensor | None = None, num_splits: int = 0, stream=None,
                       prepare: bool = False):
    """sparse_mla with its split partials in the library's fixed device array (no workspace)."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    _check(q, q.dtype, "q")
    _check(cache, torch.int8, "cache")
    _check(indices, torch.int32, "indices")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    _check(out, out.dtype, "out")
    if lse is not None:
        _check(lse, torch.float32, "lse")
    return _call("dsa_sparse_mla_noalloc", prepare,
                 ctypes.byref(dims), q.data_ptr(), _dt(q), cache.data_ptr(), cache.shape[0], indices.data_ptr(),
                 q.shape[0], float(scale), out.data_ptr(), _dt(out), _ptr(lse), int(num_splits), _stream(stream))


def index_pools_int8(dims: Dims, k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                     seqs: Seqs, pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int,
                     codes: torch.Tensor, scales: torch.Tensor, pools_f32: torch.Tensor | None = None, stream=None,
                     prepare: bool = False):
    """Pools [pool_begin, pool_end) of each sequence as INT8 code rows [*, Di] and fp32 scales [*]."""
    if k.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("k must be bf16 or fp32")
    _check(k, k.dtype, "k")
    _check(gate, k.dtype, "gate")
    _check(ln_w, torch.float32, "ln_w")
    _check(ln_b, torch.float32, "ln_b")
    _check(pool_begin, torch.int32, "pool_begin")
    _check(pool_end, torch.int32, "pool_end")
    _check(codes, torch.int8, "codes")
    _check(scales, torch.float32, "scales")
    if pools_f32 is not None:
        _check(pools_f32, torch.float32, "pools_f32")
    return _call("dsa_index_pools_int8", prepare, ctypes.byref(dims), k.data_ptr(), gate.data_ptr(), _dt(k),
                 ln_w.data_ptr(), ln_b.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, pool_begin.data_ptr(),
                 pool_end.data_ptr(), int(max_pools), codes.data_ptr(), scales.data_ptr(), _ptr(pools_f32),
                 _stream(stream))


def index_scores_int8(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                      seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor, stream=None,
                      prepare: bool = False):
    """scores [T, stride] over INT8 pools (codes [*, Di] int8, scales [*] fp32)."""
    for t, dt, n in ((q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"), (codes, torch.int8, "codes"),
                     (scales, torch.float32, "scales"), (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"),
                     (scores, torch.float32, "scores")):
        _check(t, dt, n)
    return _call("dsa_index_scores_int8", prepare, ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(),
                 codes.data_ptr(), scales.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(),
                 q_pos.data_ptr(), q_seq.shape[0], scores.shape[1], scores.data_ptr(), _stream(stream))


def index_scores_groups_int8(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, codes: torch.Tensor,
                             scales: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                             scores: torch.Tensor, workspace: torch.Tensor, stream=None, prepare: bool = False):
    """index_scores_int8 that also keeps each 64-pool group's best pools in the workspace."""
    for t, dt, n in ((q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"), (codes, torch.int8, "codes"),
                     (scales, torch.float32, "scales"), (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"),
                     (scores, torch.float32, "scores")):
        _check(t, dt, n)
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_index_scores_groups_int8", prepare, ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(),
                 codes.data_ptr(), scales.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(),
                 q_pos.data_ptr(), q_seq.shape[0], scores.shape[1], scores.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), _stream(stream))


def append_scores_groups_int8(dims: Dims, latent: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor,
                              k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                              pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int, codes: torch.Tensor,
                              scales: torch.Tensor, q_idx: torch.Tensor, w: torch.Tensor, seqs: Seqs,
                              q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor, workspace: torch.Tensor,
                              stream=None, prepare: bool = False):
    """The new tokens (INT8 rows; pools in the INT8 form) and the scoring pass with group lists, one launch."""
    for t, dt, n in ((latent, torch.bfloat16, "latent"), (slots, torch.int64, "slots"), (cache, torch.int8, "cache"),
                     (k, torch.bfloat16, "k"), (gate, torch.bfloat16, "gate"), (ln_w, torch.float32, "ln_w"),
                     (ln_b, torch.float32, "ln_b"), (pool_begin, torch.int32, "pool_begin"),
                     (pool_end, torch.int32, "pool_end"), (codes, torch.int8, "codes"),
                     (scales, torch.float32, "scales"), (q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"),
                     (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"), (scores, torch.float32, "scores")):
        _check(t, dt, n)
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_append_scores_groups_int8", prepare, ctypes.byref(dims), DSA_BF16, latent.data_ptr(),
                 latent.shape[0], latent.stride(0), slots.data_ptr(), cache.data_ptr(), cache.shape[0], k.data_ptr(),
                 gate.data_ptr(), ln_w.data_ptr(), ln_b.data_ptr(), pool_begin.data_ptr(), pool_end.data_ptr(),
                 int(max_pools), codes.data_ptr(), scales.data_ptr(), q_idx.data_ptr(), w.data_ptr(),
                 ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), q_seq.shape[0],
                 scores.shape[1], scores.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), _stream(stream))


def append_scores_groups_shared(dims: Dims, latent: torch.Tensor | None, slots: torch.Tensor | None,
                                cache: torch.Tensor | None, k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor,
                                ln_b: torch.Tensor, pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int,
                                pools: torch.Tensor, pool_scales: torch.Tensor | None, q_idx: torch.Tensor,
                                w: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                                scores: torch.Tensor, workspace: torch.Tensor, share: int, stream=None,
                                prepare: bool = False):
    """New tokens and scoring with group lists where runs of up to `share`
    consecutive queries of one sequence read its pools once (pools bf16, or
    INT8 codes when pool_scales is given)."""
    for t, dt, nm in ((k, torch.bfloat16, "k"), (gate, torch.bfloat16, "gate"), (ln_w, torch.float32, "ln_w"),
                      (ln_b, torch.float32, "ln_b"), (pool_begin, torch.int32, "pool_begin"),
                      (pool_end, torch.int32, "pool_end"), (q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"),
                      (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"), (scores, torch.float32, "scores")):
        _check(t, dt, nm)
    _check(pools, torch.int8 if pool_scales is not None else torch.bfloat16, "pools")
    if pool_scales is not None:
        _check(pool_scales, torch.float32, "pool_scales")
    _check(workspace, workspace.dtype, "workspace")
    n = 0 if latent is None else latent.shape[0]
    if n:
        _check(latent, torch.bfloat16, "latent")
        _check(slots, torch.int64, "slots")
        _check(cache, torch.int8, "cache")
    return _call("dsa_append_scores_groups_shared", prepare, ctypes.byref(dims), DSA_BF16, _ptr(latent) if n else None,
                 n, latent.stride(0) if n else 0, _ptr(slots) if n else None, _ptr(cache) if n else None,
                 cache.shape[0] if n else 0, k.data_ptr(), gate.data_ptr(), ln_w.data_ptr(), ln_b.data_ptr(),
                 pool_begin.data_ptr(), pool_end.data_ptr(), int(max_pools), pools.data_ptr(), _ptr(pool_scales),
                 q_idx.data_ptr(), w.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(),
                 q_pos.data_ptr(), q_seq.shape[0], scores.shape[1], scores.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), int(share), _stream(stream))


def index_pools_paged(dims: Dims, k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                      seqs: PagedSeqs, pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int,
                      pools: torch.Tensor, stream=None, prepare: bool = False):
    """index_pools over paged caches (k, gate and pools rows through the block table)."""
    if k.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("k must be bf16 or fp32")
    _check(k, k.dtype, "k")
    _check(gate, k.dtype, "gate")
    for t, dt, nm in ((ln_w, torch.float32, "ln_w"), (ln_b, torch.float32, "ln_b"),
                      (pool_begin, torch.int32, "pool_begin"), (pool_end, torch.int32, "pool_end"),
                      (pools, torch.bfloat16, "pools")):
        _check(t, dt, nm)
    return _call("dsa_index_pools_paged", prepare, ctypes.byref(dims), k.data_ptr(), gate.data_ptr(), _dt(k),
                 ln_w.data_ptr(), ln_b.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, pool_begin.data_ptr(),
                 pool_end.data_ptr(), int(max_pools), pools.data_ptr(), _stream(stream))


def index_scores_groups_paged(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor,
                              seqs: PagedSeqs, q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor,
                              workspace: torch.Tensor, stream=None, prepare: bool = False):
    """index_scores_groups over paged pools."""
    for t, dt, nm in ((q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"), (pools, torch.bfloat16, "pools"),
                      (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"), (scores, torch.float32, "scores")):
        _check(t, dt, nm)
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_index_scores_groups_paged", prepare, ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(),
                 pools.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(),
                 q_seq.shape[0], scores.shape[1], scores.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), _stream(stream))


def topk_select_groups_paged(dims: Dims, scores: torch.Tensor, seqs: PagedSeqs, q_seq: torch.Tensor,
                             q_pos: torch.Tensor, indices: torch.Tensor, workspace: torch.Tensor,
                             pool_ids: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """topk_select_groups writing the index list as physical rows of paged caches."""
    for t, dt, nm in ((scores, torch.float32, "scores"), (q_seq, torch.int32, "q_seq"), (q_pos, torch.int32, "q_pos"),
                      (indices, torch.int32, "indices")):
        _check(t, dt, nm)
    _check(workspace, workspace.dtype, "workspace")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    return _call("dsa_topk_select_groups_paged", prepare, ctypes.byref(dims), scores.data_ptr(), scores.shape[1],
                 ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), q_seq.shape[0],
                 _ptr(pool_ids), indices.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), _stream(stream))


def index_select_chunked_workspace(dims: Dims, chunk: int, score_stride: int, device="cuda") -> torch.Tensor:
    n = int(lib().dsa_index_select_chunked_workspace_bytes(ctypes.byref(dims), int(chunk), int(score_stride)))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def index_select_chunked(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor, seqs: Seqs,
                         q_seq: torch.Tensor, q_pos: torch.Tensor, score_stride: int, chunk: int,
                         indices: torch.Tensor, workspace: torch.Tensor, pool_ids: torch.Tensor | None = None,
                         stream=None, prepare: bool = False):
    """Scores, top-k and expansion of many queries, `chunk` queries at a time
    through a bounded scoring workspace (the scores are not kept)."""
    _check(q_idx, torch.bfloat16, "q_idx")
    _check(w, torch.float32, "w")
    _check(pools, torch.bfloat16, "pools")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    _check(indices, torch.int32, "indices")
    _check(workspace, workspace.dtype, "workspace")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    return _call("dsa_index_select_chunked", prepare, ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(),
                 pools.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(),
                 q_seq.shape[0], int(score_stride), int(chunk), _ptr(pool_ids), indices.data_ptr(),
                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))


def index_scores_select_workspace(dims: Dims, T: int, score_stride: int, device="cuda") -> torch.Tensor | None:
    n = int(lib().dsa_index_scores_select_workspace_bytes(ctypes.byref(dims), int(T), int(score_stride)))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def index_scores_select(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor, seqs: Seqs,
                        q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor, indices: torch.Tensor,
                        pool_ids: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """index_scores then topk_select_expand (decode batches: one scoring pass that also keeps group lists)."""
    _check(q_idx, torch.bfloat16, "q_idx")
    _check(w, torch.float32, "w")
    _check(pools, torch.bfloat16, "pools")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    _check(scores, torch.float32, "scores")
    _check(indices, torch.int32, "indices")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    ws_bytes = 0
    if workspace is not None:
        _check(workspace, workspace.dtype, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return _call("dsa_index_scores_select", prepare, 
        ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(), pools.data_ptr(), ctypes.byref(seqs._c()),
        seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0], scores.shape[1], scores.data_ptr(),
        _ptr(pool_ids), indices.data_ptr(), _ptr(workspace), ws_bytes, _stream(stream))


def index_scores_groups(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor, seqs: Seqs,
                        q_seq: torch.Tensor, q_pos: torch.Tensor, scores: torch.Tensor, workspace: torch.Tensor,
                        stream=None, prepare: bool = False):
    """Decode scoring pass that also keeps each 64-pool group's best pools in `workspace`."""
    for name, t, dt in (("q_idx", q_idx, torch.bfloat16), ("w", w, torch.float32), ("pools", pools, torch.bfloat16),
                        ("q_seq", q_seq, torch.int32), ("q_pos", q_pos, torch.int32),
                        ("scores", scores, torch.float32)):
        _check(t, dt, name)
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_index_scores_groups", prepare, 
        ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(), pools.data_ptr(), ctypes.byref(seqs._c()),
        seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0], scores.shape[1], scores.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))


def append_scores_groups(dims: Dims, latent: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor,
                         k: torch.Tensor, gate: torch.Tensor, ln_w: torch.Tensor, ln_b: torch.Tensor,
                         pool_begin: torch.Tensor, pool_end: torch.Tensor, max_pools: int, pools: torch.Tensor,
                         q_idx: torch.Tensor, w: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                         scores: torch.Tensor, workspace: torch.Tensor, stream=None, prepare: bool = False):
    """append_tokens then index_scores_groups (one launch for bf16 new tokens)."""
    if latent.dim() != 2 or (latent.shape[0] > 0 and latent.stride(1) != 1):
        raise ValueError("latent must be [n, D] with unit stride in D")
    if latent.dtype not in (torch.bfloat16, torch.float32) or not latent.is_cuda:
        raise TypeError("latent must be a bf16/fp32 device tensor")
    _check(slots, torch.int64, "slots")
    _check(cache, torch.int8, "cache")
    if slots.numel() != latent.shape[0]:
        raise ValueError("slots must have one entry per latent row")
    for name, t in (("k", k), ("gate", gate)):
        _check(t, latent.dtype, name)
    for name, t, dt in (("ln_w", ln_w, torch.float32), ("ln_b", ln_b, torch.float32),
                        ("pool_begin", pool_begin, torch.int32), ("pool_end", pool_end, torch.int32),
                        ("pools", pools, torch.bfloat16), ("q_idx", q_idx, torch.bfloat16), ("w", w, torch.float32),
                        ("q_seq", q_seq, torch.int32), ("q_pos", q_pos, torch.int32),
                        ("scores", scores, torch.float32)):
        _check(t, dt, name)
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_append_scores_groups", prepare,
        ctypes.byref(dims), _dt(latent), latent.data_ptr(), latent.shape[0], latent.stride(0), slots.data_ptr(),
        cache.data_ptr(), cache.shape[0], k.data_ptr(), gate.data_ptr(), ln_w.data_ptr(), ln_b.data_ptr(),
        pool_begin.data_ptr(), pool_end.data_ptr(), int(max_pools), pools.data_ptr(), q_idx.data_ptr(),
        w.data_ptr(), ctypes.byref(seqs._c()), seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0],
        scores.shape[1], scores.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream))


def topk_select_groups(dims: Dims, scores: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                       indices: torch.Tensor, workspace: torch.Tensor, pool_ids: torch.Tensor | None = None,
                       stream=None, prepare: bool = False):
    """Selection and expansion from the group lists index_scores_groups left in `workspace`."""
    _check(scores, torch.float32, "scores")
    _check(indices, torch.int32, "indices")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    _check(workspace, workspace.dtype, "workspace")
    return _call("dsa_topk_select_groups", prepare, 
        ctypes.byref(dims), scores.data_ptr(), scores.shape[1], ctypes.byref(seqs._c()), seqs.num_seqs,
        q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0], _ptr(pool_ids), indices.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))


def topk_sparse_mla(dims: Dims, scores: torch.Tensor, seqs: Seqs, q_seq: torch.Tensor, q_pos: torch.Tensor,
                    indices: torch.Tensor, select_workspace: torch.Tensor, q: torch.Tensor, cache: torch.Tensor,
                    scale: float, out: torch.Tensor, lse: torch.Tensor | None = None, num_splits: int = 0,
                    mla_workspace: torch.Tensor | None = None, pool_ids: torch.Tensor | None = None,
                    stream=None, prepare: bool = False):
    """topk_select_groups then sparse_mla over its list (the attention launch makes the selection itself)."""
    _check(scores, torch.float32, "scores")
    _check(indices, torch.int32, "indices")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    if pool_ids is not None:
        _check(pool_ids, torch.int32, "pool_ids")
    _check(select_workspace, select_workspace.dtype, "select_workspace")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    _check(q, q.dtype, "q")
    _check(cache, torch.int8, "cache")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    _check(out, out.dtype, "out")
    if lse is not None:
        _check(lse, torch.float32, "lse")
    ws_bytes = 0
    if mla_workspace is not None:
        _check(mla_workspace, mla_workspace.dtype, "mla_workspace")
        ws_bytes = mla_workspace.numel() * mla_workspace.element_size()
    return _call("dsa_topk_sparse_mla", prepare,
        ctypes.byref(dims), scores.data_ptr(), scores.shape[1], ctypes.byref(seqs._c()), seqs.num_seqs,
        q_seq.data_ptr(), q_pos.data_ptr(), q_pos.shape[0], _ptr(pool_ids), indices.data_ptr(),
        select_workspace.data_ptr(), select_workspace.numel() * select_workspace.element_size(),
        q.data_ptr(), _dt(q), cache.data_ptr(), cache.shape[0], float(scale), out.data_ptr(), _dt(out),
        _ptr(lse), int(num_splits), _ptr(mla_workspace), ws_bytes, _stream(stream))


def time_next_scoring_launch(start_event, stop_event):
    """The next append_scores_groups scoring launch on this thread records the two
    (already created) torch.cuda.Events around the kernel itself."""
    st = lib().dsa_time_next_scoring_launch(start_event.cuda_event, stop_event.cuda_event)
    if st:
        raise DsaError("dsa_time_next_scoring_launch", st, "")


def decode_step_workspace_bytes(dims: Dims, T: int, score_stride: int) -> int:
    """Workspace of dsa_decode_step (0 when the geometry is not supported)."""
    return int(lib().dsa_decode_step_workspace_bytes(ctypes.byref(dims), int(T), int(score_stride)))


def decode_step_workspace(dims: Dims, T: int, score_stride: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for dsa_decode_step (reusable across calls)."""
    n = decode_step_workspace_bytes(dims, T, score_stride)
    if n == 0:
        raise DsaError("dsa_decode_step_workspace_bytes", -7, "geometry not supported")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def decode_step_error(workspace: torch.Tensor, stream=None) -> int:
    """dsa_decode_step_status: 0 when no wait inside a launch that used this
    workspace timed out, else the DSA_ERR_TIMEOUT status (synchronises the stream)."""
    _check(workspace, workspace.dtype, "workspace")
    return int(lib().dsa_decode_step_status(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))


def decode_step(dims: Dims, q_idx: torch.Tensor, w: torch.Tensor, pools: torch.Tensor, seqs: Seqs,
                q_seq: torch.Tensor, q_pos: torch.Tensor, score_stride: int, q: torch.Tensor, cache: torch.Tensor,
                scale: float, out: torch.Tensor, workspace: torch.Tensor, lse: torch.Tensor | None = None,
                pool_ids: torch.Tensor | None = None, indices: torch.Tensor | None = None, stream=None, prepare: bool = False):
    """One launch: scores, top-k, expansion and sparse MLA for a decode batch."""
    _check(q_idx, torch.bfloat16, "q_idx")
    _check(w, torch.float32, "w")
    _check(pools, torch.bfloat16, "pools")
    _check(q_seq, torch.int32, "q_seq")
    _check(q_pos, torch.int32, "q_pos")
    _check(q, torch.bfloat16, "q")
    _check(cache, torch.int8, "cache")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or fp32")
    _check(out, out.dtype, "out")
    _check(workspace, workspace.dtype, "workspace")
    for name, t in (("lse", lse), ("pool_ids", pool_ids), ("indices", indices)):
        if t is not None:
            _check(t, torch.float32 if name == "lse" else torch.int32, name)
    T = q_pos.shape[0]
    return _call("dsa_decode_step", prepare, 
        ctypes.byref(dims), q_idx.data_ptr(), w.data_ptr(), pools.data_ptr(), ctypes.byref(seqs._c()),
        seqs.num_seqs, q_seq.data_ptr(), q_pos.data_ptr(), T, int(score_stride), q.data_ptr(), DSA_BF16,
        cache.data_ptr(), cache.shape[0], float(scale), out.data_ptr(), _dt(out), _ptr(lse), _ptr(pool_ids),
        _ptr(indices), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))


__all__ = [
    "DSA_F32", "DSA_BF16", "DsaError", "Dims", "Seqs", "lib", "abi_version", "status_string",
    "store_int8", "index_pools", "index_scores", "topk_workspace_bytes", "topk_workspace",
    "topk_select", "topk_select_expand", "expand_selection", "sparse_mla_workspace_bytes", "sparse_mla",
    "index_scores_select_workspace", "index_scores_select", "index_scores_groups", "topk_select_groups",
    "decode_step_workspace_bytes", "decode_step_workspace", "decode_step_error", "decode_step",
    "sparse_mla_noalloc_scratch_bytes", "sparse_mla_noalloc", "index_select_chunked_workspace",
    "index_select_chunked", "index_pools_int8", "index_scores_int8", "index_scores_groups_int8",
    "append_scores_groups_int8", "append_scores_groups_shared", "PagedSeqs", "index_pools_paged",
    "index_scores_groups_paged", "topk_select_groups_paged",
]
