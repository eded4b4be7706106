"""ctypes binding of libcsa2.so: argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
checks tensor dtypes/devices/shapes, passes ``data_ptr()`` values and the
current HIP stream, and turns status codes into exceptions.  PyTorch is used
for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

PAGE_TOKENS = 64
WINDOW = 128
NOALLOC_SCRATCH_BYTES = 64 << 20       # fixed scratch of sparse_decode_noalloc, per device

_c_i32 = ctypes.c_int32
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t


class CacheStruct(ctypes.Structure):
    _fields_ = [
        ("pages", _c_vp),
        ("page_table", _c_vp),
        ("num_pages", _c_i32),
        ("max_pages_per_seq", _c_i32),
        ("batch", _c_i32),
        ("head_dim", _c_i32),
        ("idx_dim", _c_i32),
    ]


class Csa2Error(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libcsa2.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Csa2Error(
                f"{LIB_PATH} is missing: build it with `python -m fp4_compressed_sparse_csa2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(CacheStruct)
        sig = {
            "csa2_page_bytes": (_c_sz, [_c_i32, _c_i32]),
            "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "csa2_workspace_init": (ctypes.c_int, [_c_vp, _c_sz, _c_vp]),
            "csa2_stream_read": (ctypes.c_int, [_c_vp, _c_sz, _c_vp, _c_vp]),
            "csa2_quantize_append": (ctypes.c_int, [P, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
            "csa2_index_topk_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32]),
            "csa2_index_topk": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp,
                                               _c_vp, _c_vp, _c_sz, _c_vp]),
            "csa2_reindex_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32]),
            "csa2_reindex": (ctypes.c_int, [P, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_vp,
                                            _c_vp, _c_vp, _c_sz, _c_vp]),
            "csa2_sparse_decode_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
            "csa2_sparse_decode": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, ctypes.c_float, _c_vp,
                                                  _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                                  _c_vp]),
            "csa2_sparse_decode_noalloc": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, ctypes.c_float,
                                                          _c_vp, _c_vp, _c_i32, _c_vp, _c_vp,
                                                          _c_vp, _c_vp]),
            "csa2_index_topk_range": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, _c_i32, _c_i32,
                                                     _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                                     _c_vp]),
            "csa2_topk_merge_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32]),
            "csa2_topk_merge": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_i32,
                                               _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
            "csa2_lse_merge": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                              _c_vp, _c_vp]),
            "csa2_append_index_topk": (ctypes.c_int, [P, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp,
                                                      _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp,
                                                      _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
            "csa2_store_key_scales": (ctypes.c_int, [P, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]),
            "csa2_validate_selection": (ctypes.c_int, [P, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp,
                                                       _c_vp]),
            "csa2_validate_window": (ctypes.c_int, [P, _c_vp, _c_vp, _c_vp, _c_vp]),
            "csa2_index_topk_range_scaled": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,
                                                            _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                                            _c_vp, _c_sz, _c_vp]),
            "csa2_topk_merge_values": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                                      _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                                      _c_vp]),
            "csa2_store_key_scales_e4m3": (ctypes.c_int, [P, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp,
                                                          _c_vp]),
            "csa2_index_topk_scaled": (ctypes.c_int, [P, _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,
                                                      _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                                      _c_vp]),
            "csa2_reindex_scaled": (ctypes.c_int, [P, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32,
                                                   _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().csa2_status_string(status).decode()
        raise Csa2Error(f"{what}: {msg} ({status})")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _as_u16(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensors are passed by their bit patterns."""
    return t.view(torch.uint16) if t.dtype == torch.bfloat16 else t


def page_bytes(head_dim: int, idx_dim: int) -> int:
    n = lib().csa2_page_bytes(head_dim, idx_dim)
    if n == 0:
        raise Csa2Error(f"unsupported head_dim={head_dim} / idx_dim={idx_dim}")
    return int(n)


class Cache:
    """One owner layer's global state: the page pool and the page table.

    pages       uint8 [num_pages, page_bytes(D, Di)] on the GPU
    page_table  int32 [batch, max_pages_per_seq] on the same GPU
    """

    def __init__(self, pages: torch.Tensor, page_table: torch.Tensor, head_dim: int, idx_dim: int):
        pb = page_bytes(head_dim, idx_dim)
        _need(pages, "pages", torch.uint8)
        if pages.dim() != 2 or pages.shape[1] != pb:
            raise ValueError(f"pages must be [num_pages, {pb}]")
        _need(page_table, "page_table", torch.int32, pages.device)
        if page_table.dim() != 2:
            raise ValueError("page_table must be [batch, max_pages_per_seq]")
        self.pages, self.page_table = pages, page_table
        self.head_dim, self.idx_dim = head_dim, idx_dim
        self.batch, self.max_pages = page_table.shape
        self.device = pages.device
        self.struct = CacheStruct(pages.data_ptr(), page_table.data_ptr(), pages.shape[0],
                                  self.max_pages, self.batch, head_dim, idx_dim)

    @staticmethod
    def allocate(batch: int, max_pages_per_seq: int, num_pages: int, head_dim: int, idx_dim: int,
                 page_table: torch.Tensor, device) -> "Cache":
        pages = torch.zeros((num_pages, page_bytes(head_dim, idx_dim)), dtype=torch.uint8,
                            device=device)
        return Cache(pages, page_table.to(device=device, dtype=torch.int32).contiguous(), head_dim,
                     idx_dim)


class Workspace:
    """A zero-initialised workspace that grows on demand.

    The library keeps per-sequence control words at the start of a workspace
    and returns them to zero at the end of every call, but where the scratch
    that follows them begins depends on the call's batch and kind.  So the
    buffer is zeroed again whenever it is handed to a call of another kind
    (Full-layer selection, Reindex, Top-K merge, decode) or another batch
    size, and whenever it grows."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf = None
        self.key = None

    def get(self, nbytes: int, kind: str = "", batch: int = 0) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            workspace_init(self.buf)
        elif self.key != (kind, batch):
            workspace_init(self.buf)
        self.key = (kind, batch)
        return self.buf


def workspace_init(ws: torch.Tensor) -> None:
    _check(lib().csa2_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream(ws.device)), "csa2_workspace_init")


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """One read of every byte of the contiguous device tensor buf (a multiple
    of 16 bytes), XOR-folded into sink (int32 [1]): the read-only bandwidth
    reference a benchmark times beside the method's calls."""
    if not buf.is_contiguous():
        raise Csa2Error("stream_read: buf must be contiguous")
    _need(sink, "sink", torch.int32, buf.device, (1,))
    _check(lib().csa2_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                  sink.data_ptr(), _stream(buf.device)), "csa2_stream_read")


def quantize_append(cache: Cache, x: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                    keys: torch.Tensor | None = None, swa: torch.Tensor | None = None) -> None:
    """Quantise tokens x (bf16 [n, D]) into the cache at (seq, pos); optional
    int8 indexer keys [n, Di] and window ring swa (bf16 [B, 128, D])."""
    x = _as_u16(x)
    n = x.shape[0]
    dev = cache.device
    _need(x, "x", torch.uint16, dev, (n, cache.head_dim))
    _need(seq, "seq", torch.int32, dev, (n,))
    _need(pos, "pos", torch.int32, dev, (n,))
    if keys is not None:
        _need(keys, "keys", torch.int8, dev, (n, cache.idx_dim))
    if swa is not None:
        swa = _as_u16(swa)
        _need(swa, "swa", torch.uint16, dev, (cache.batch, WINDOW, cache.head_dim))
    _check(lib().csa2_quantize_append(ctypes.byref(cache.struct), n, x.data_ptr(), _ptr(keys),
                                      seq.data_ptr(), pos.data_ptr(), _ptr(swa), _stream(dev)),
           "csa2_quantize_append")


def index_topk(cache: Cache, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor, K: int,
               ws: Workspace, out_idx: torch.Tensor | None = None,
               out_count: torch.Tensor | None = None, out_scores: torch.Tensor | None = None):
    """Full layer: indexer scores + deterministic Top-K.  Returns (idx [B, K], count [B])."""
    dev, B = cache.device, cache.batch
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.int32, dev, (B, max_ctx))
    nbytes = lib().csa2_index_topk_workspace_size(B, max_ctx, K)
    if nbytes == 0:
        raise Csa2Error(f"index_topk: unsupported sizes B={B} max_ctx={max_ctx} K={K}")
    w = ws.get(nbytes, "topk", B)
    _check(lib().csa2_index_topk(ctypes.byref(cache.struct), ctx_len.data_ptr(), max_ctx,
                                 q_idx.data_ptr(), K, out_idx.data_ptr(), out_count.data_ptr(),
                                 _ptr(out_scores), w.data_ptr(), w.numel(), _stream(dev)),
           "csa2_index_topk")
    return out_idx, out_count


def append_index_topk(cache: Cache, x: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                      keys: torch.Tensor | None, swa: torch.Tensor | None, ctx_len: torch.Tensor,
                      max_ctx: int, q_idx: torch.Tensor, K: int, ws: Workspace,
                      out_idx: torch.Tensor | None = None, out_count: torch.Tensor | None = None,
                      out_scores: torch.Tensor | None = None):
    """quantize_append of decode tokens (each inside its sequence's window)
    and the Full layer's index_topk in one call.  Returns (idx [B, K], count [B])."""
    x = _as_u16(x)
    n = x.shape[0]
    dev, B = cache.device, cache.batch
    _need(x, "x", torch.uint16, dev, (n, cache.head_dim))
    _need(seq, "seq", torch.int32, dev, (n,))
    _need(pos, "pos", torch.int32, dev, (n,))
    if keys is not None:
        _need(keys, "keys", torch.int8, dev, (n, cache.idx_dim))
    if swa is not None:
        swa = _as_u16(swa)
        _need(swa, "swa", torch.uint16, dev, (B, WINDOW, cache.head_dim))
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.int32, dev, (B, max_ctx))
    nbytes = lib().csa2_index_topk_workspace_size(B, max_ctx, K)
    if nbytes == 0:
        raise Csa2Error(f"append_index_topk: unsupported sizes B={B} max_ctx={max_ctx} K={K}")
    w = ws.get(nbytes, "topk", B)
    _check(lib().csa2_append_index_topk(ctypes.byref(cache.struct), n, x.data_ptr(), _ptr(keys),
                                        seq.data_ptr(), pos.data_ptr(), _ptr(swa),
                                        ctx_len.data_ptr(), max_ctx, q_idx.data_ptr(), K,
                                        out_idx.data_ptr(), out_count.data_ptr(),
                                        _ptr(out_scores), w.data_ptr(), w.numel(), _stream(dev)),
           "csa2_append_index_topk")
    return out_idx, out_count


def reindex(cache: Cache, q_idx: torch.Tensor, pool: torch.Tensor, pool_count: torch.Tensor,
            K: int, ws: Workspace, out_idx: torch.Tensor | None = None,
            out_count: torch.Tensor | None = None, out_scores: torch.Tensor | None = None):
    """Reindex layer over the owner's pool [B, P].  Returns (idx [B, K], count [B])."""
    dev, B = cache.device, cache.batch
    P = pool.shape[1]
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    _need(pool, "pool", torch.int32, dev, (B, P))
    _need(pool_count, "pool_count", torch.int32, dev, (B,))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.int32, dev, (B, P))
    nbytes = lib().csa2_reindex_workspace_size(B, P, K)
    if nbytes == 0:
        raise Csa2Error(f"reindex: unsupported sizes B={B} P={P} K={K}")
    w = ws.get(nbytes, "reindex", B)
    _check(lib().csa2_reindex(ctypes.byref(cache.struct), q_idx.data_ptr(), pool.data_ptr(),
                              pool_count.data_ptr(), P, K, out_idx.data_ptr(),
                              out_count.data_ptr(), _ptr(out_scores), w.data_ptr(), w.numel(),
                              _stream(dev)),
           "csa2_reindex")
    return out_idx, out_count


def _decode_args(cache: Cache, ctx_len, q, idx, idx_count, swa, out, lse, want_lse):
    dev, B, D = cache.device, cache.batch, cache.head_dim
    q = _as_u16(q)
    swa = None if swa is None else _as_u16(swa)
    H = q.shape[1]
    K = idx.shape[1]
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q, "q", torch.uint16, dev, (B, H, D))
    _need(idx, "idx", torch.int32, dev, (B, K))
    _need(idx_count, "idx_count", torch.int32, dev, (B,))
    if swa is not None:
        _need(swa, "swa", torch.uint16, dev, (B, WINDOW, D))
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, (B, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, (B, H))
    return q, swa, H, K, out, lse


def sparse_decode(cache: Cache, ctx_len: torch.Tensor, q: torch.Tensor, softmax_scale: float,
                  idx: torch.Tensor, idx_count: torch.Tensor, swa: torch.Tensor | None,
                  ws: Workspace, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, want_lse: bool = True):
    """Merged sparse attention.  q bf16 [B, H, D]; idx int32 [B, K]; swa bf16
    [B, 128, D], or None for no window rows (a context shard without the
    tail).  Returns (out fp32 [B, H, D], lse fp32 [B, H] or None)."""
    q, swa, H, K, out, lse = _decode_args(cache, ctx_len, q, idx, idx_count, swa, out, lse,
                                          want_lse)
    B, D = cache.batch, cache.head_dim
    nbytes = lib().csa2_sparse_decode_workspace_size(B, H, D, K)
    if nbytes == 0:
        raise Csa2Error(f"sparse_decode: unsupported sizes B={B} H={H} D={D} K={K}")
    w = ws.get(nbytes, "decode", B)
    _check(lib().csa2_sparse_decode(ctypes.byref(cache.struct), ctx_len.data_ptr(), H,
                                    q.data_ptr(), float(softmax_scale), idx.data_ptr(),
                                    idx_count.data_ptr(), K, _ptr(swa), out.data_ptr(),
                                    _ptr(lse), w.data_ptr(), w.numel(), _stream(cache.device)),
           "csa2_sparse_decode")
    return out, lse


def sparse_decode_noalloc(cache: Cache, ctx_len: torch.Tensor, q: torch.Tensor,
                          softmax_scale: float, idx: torch.Tensor, idx_count: torch.Tensor,
                          swa: torch.Tensor | None, out: torch.Tensor, lse: torch.Tensor | None):
    """sparse_decode on the library's fixed per-device scratch: no workspace,
    and the caller passes the outputs (lse may be None), so the call
    allocates nothing.  Calls that overlap in time on one device race on the
    scratch.  Returns (out, lse)."""
    q, swa, H, K, out, lse = _decode_args(cache, ctx_len, q, idx, idx_count, swa, out, lse,
                                          False)
    _check(lib().csa2_sparse_decode_noalloc(ctypes.byref(cache.struct), ctx_len.data_ptr(), H,
                                            q.data_ptr(), float(softmax_scale), idx.data_ptr(),
                                            idx_count.data_ptr(), K, _ptr(swa), out.data_ptr(),
                                            _ptr(lse), _stream(cache.device)),
           "csa2_sparse_decode_noalloc")
    return out, lse


# ------------------------------------------------------------------ validation
SEL_BAD_LENGTH, SEL_BAD_COUNT, SEL_BAD_POSITION, SEL_BAD_PAGE, SEL_NOT_ASCENDING = 1, 2, 4, 8, 16


def validate_selection(cache: Cache, ctx_len: torch.Tensor, idx: torch.Tensor,
                       idx_count: torch.Tensor) -> torch.Tensor:
    """Contract-violation bits (SEL_*) of sparse_decode's selection inputs,
    per sequence: int32 [B] on the GPU, 0 where the inputs are valid."""
    dev, B = cache.device, cache.batch
    K = idx.shape[1]
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(idx, "idx", torch.int32, dev, (B, K))
    _need(idx_count, "idx_count", torch.int32, dev, (B,))
    flags = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(lib().csa2_validate_selection(ctypes.byref(cache.struct), ctx_len.data_ptr(),
                                         idx.data_ptr(), idx_count.data_ptr(), K, flags.data_ptr(),
                                         _stream(dev)),
           "csa2_validate_selection")
    return flags


WIN_NOT_F16, WIN_NOT_FINITE = 1, 2


def validate_window(cache: Cache, ctx_len: torch.Tensor, swa: torch.Tensor) -> torch.Tensor:
    """Window-ring check bits (WIN_*) per sequence: int32 [B] on the GPU, 0
    where every live slot is finite and exact in fp16."""
    dev, B = cache.device, cache.batch
    swa = _as_u16(swa)
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(swa, "swa", torch.uint16, dev, (B, WINDOW, cache.head_dim))
    flags = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(lib().csa2_validate_window(ctypes.byref(cache.struct), ctx_len.data_ptr(),
                                      swa.data_ptr(), flags.data_ptr(), _stream(dev)),
           "csa2_validate_window")
    return flags


# ------------------------------------------------------------------ key scales
def key_scales_for(cache: Cache) -> torch.Tensor:
    """A zeroed per-token key-scale array (float32 [num_pages, 64]) for cache."""
    return torch.zeros((cache.pages.shape[0], PAGE_TOKENS), dtype=torch.float32,
                       device=cache.device)


def store_key_scales(cache: Cache, scale: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                     key_scales: torch.Tensor) -> None:
    """Write the key scales of tokens at (seq, pos) into key_scales
    [num_pages, 64] through the page table: fp32 scales, or E4M3 bytes
    (uint8, decoded exactly)."""
    dev = cache.device
    n = scale.shape[0]
    e4m3 = scale.dtype == torch.uint8
    _need(scale, "scale", torch.uint8 if e4m3 else torch.float32, dev, (n,))
    _need(seq, "seq", torch.int32, dev, (n,))
    _need(pos, "pos", torch.int32, dev, (n,))
    _need(key_scales, "key_scales", torch.float32, dev, (cache.pages.shape[0], PAGE_TOKENS))
    fn = lib().csa2_store_key_scales_e4m3 if e4m3 else lib().csa2_store_key_scales
    _check(fn(ctypes.byref(cache.struct), n, scale.data_ptr(), seq.data_ptr(), pos.data_ptr(),
              key_scales.data_ptr(), _stream(dev)),
           "csa2_store_key_scales" + ("_e4m3" if e4m3 else ""))


def index_topk_scaled(cache: Cache, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor,
                      key_scales: torch.Tensor, K: int, ws: Workspace,
                      out_idx: torch.Tensor | None = None, out_count: torch.Tensor | None = None,
                      out_values: torch.Tensor | None = None,
                      out_sel_values: torch.Tensor | None = None):
    """Full layer ranked by v_p = fl32(s_p * score_p).  Returns (idx [B, K],
    count [B], values of the selected [B, K] or None)."""
    dev, B = cache.device, cache.batch
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    _need(key_scales, "key_scales", torch.float32, dev, (cache.pages.shape[0], PAGE_TOKENS))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    if out_values is not None:
        _need(out_values, "out_values", torch.float32, dev, (B, max_ctx))
    if out_sel_values is not None:
        _need(out_sel_values, "out_sel_values", torch.float32, dev, (B, K))
    nbytes = lib().csa2_index_topk_workspace_size(B, max_ctx, K)
    if nbytes == 0:
        raise Csa2Error(f"index_topk_scaled: unsupported sizes B={B} max_ctx={max_ctx} K={K}")
    w = ws.get(nbytes, "topk", B)
    _check(lib().csa2_index_topk_scaled(ctypes.byref(cache.struct), ctx_len.data_ptr(), max_ctx,
                                        q_idx.data_ptr(), key_scales.data_ptr(), K,
                                        out_idx.data_ptr(), out_count.data_ptr(),
                                        _ptr(out_values), _ptr(out_sel_values), w.data_ptr(),
                                        w.numel(), _stream(dev)),
           "csa2_index_topk_scaled")
    return out_idx, out_count, out_sel_values


def reindex_scaled(cache: Cache, q_idx: torch.Tensor, key_scales: torch.Tensor,
                   pool: torch.Tensor, pool_count: torch.Tensor, K: int, ws: Workspace,
                   out_idx: torch.Tensor | None = None, out_count: torch.Tensor | None = None,
                   out_values: torch.Tensor | None = None):
    """Reindex layer ranked by the scaled values of the pool [B, P] entries.
    Returns (idx [B, K], count [B])."""
    dev, B = cache.device, cache.batch
    P = pool.shape[1]
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    _need(key_scales, "key_scales", torch.float32, dev, (cache.pages.shape[0], PAGE_TOKENS))
    _need(pool, "pool", torch.int32, dev, (B, P))
    _need(pool_count, "pool_count", torch.int32, dev, (B,))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    if out_values is not None:
        _need(out_values, "out_values", torch.float32, dev, (B, P))
    nbytes = lib().csa2_reindex_workspace_size(B, P, K)
    if nbytes == 0:
        raise Csa2Error(f"reindex_scaled: unsupported sizes B={B} P={P} K={K}")
    w = ws.get(nbytes, "reindex", B)
    _check(lib().csa2_reindex_scaled(ctypes.byref(cache.struct), q_idx.data_ptr(),
                                     key_scales.data_ptr(), pool.data_ptr(),
                                     pool_count.data_ptr(), P, K, out_idx.data_ptr(),
                                     out_count.data_ptr(), _ptr(out_values), w.data_ptr(),
                                     w.numel(), _stream(dev)),
           "csa2_reindex_scaled")
    return out_idx, out_count


# ------------------------------------------------------------------ sharding
def index_topk_range(cache: Cache, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor,
                     K: int, p_begin: int, p_end: int, ws: Workspace,
                     out_idx: torch.Tensor | None = None, out_count: torch.Tensor | None = None,
                     out_sel_scores: torch.Tensor | None = None):
    """Full-layer selection over candidates p_begin <= p < min(p_end, L-128)
    (p_begin a multiple of 64).  Returns (idx [B, K], count [B], scores of the
    selected [B, K])."""
    dev, B = cache.device, cache.batch
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_sel_scores is None:
        out_sel_scores = torch.empty((B, K), dtype=torch.int32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    _need(out_sel_scores, "out_sel_scores", torch.int32, dev, (B, K))
    nbytes = lib().csa2_index_topk_workspace_size(B, max_ctx, K)
    if nbytes == 0:
        raise Csa2Error(f"index_topk_range: unsupported sizes B={B} max_ctx={max_ctx} K={K}")
    w = ws.get(nbytes, "topk", B)
    _check(lib().csa2_index_topk_range(ctypes.byref(cache.struct), ctx_len.data_ptr(), max_ctx,
                                       q_idx.data_ptr(), K, p_begin, p_end, out_idx.data_ptr(),
                                       out_count.data_ptr(), out_sel_scores.data_ptr(),
                                       w.data_ptr(), w.numel(), _stream(dev)),
           "csa2_index_topk_range")
    return out_idx, out_count, out_sel_scores


def topk_merge(idx: torch.Tensor, scores: torch.Tensor, counts: torch.Tensor, K: int,
               ws: Workspace, out_idx: torch.Tensor | None = None,
               out_count: torch.Tensor | None = None, out_sel_scores: torch.Tensor | None = None):
    """Top-K of shard selections: idx int32 [n, B, K_in] (ascending,
    disjoint, parts in ascending position order), their scores (int32, or
    float32 values of the scaled indexer) [n, B, K_in], counts int32 [n, B].
    Returns (idx [B, K], count [B], scores or values [B, K])."""
    n, B, K_in = idx.shape
    dev = idx.device
    values = scores.dtype == torch.float32
    sdt = torch.float32 if values else torch.int32
    _need(idx, "idx", torch.int32, dev, (n, B, K_in))
    _need(scores, "scores", sdt, dev, (n, B, K_in))
    _need(counts, "counts", torch.int32, dev, (n, B))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_sel_scores is None:
        out_sel_scores = torch.empty((B, K), dtype=sdt, device=dev)
    _need(out_sel_scores, "out_sel_scores", sdt, dev, (B, K))
    nbytes = lib().csa2_topk_merge_workspace_size(B, n, K_in, K)
    if nbytes == 0:
        raise Csa2Error(f"topk_merge: unsupported sizes n={n} B={B} K_in={K_in} K={K}")
    w = ws.get(nbytes, "merge", B)
    fn = lib().csa2_topk_merge_values if values else lib().csa2_topk_merge
    _check(fn(B, n, K_in, idx.data_ptr(), scores.data_ptr(), counts.data_ptr(), K,
              out_idx.data_ptr(), out_count.data_ptr(), out_sel_scores.data_ptr(), w.data_ptr(),
              w.numel(), _stream(dev)),
           "csa2_topk_merge" + ("_values" if values else ""))
    return out_idx, out_count, out_sel_scores


def index_topk_range_scaled(cache: Cache, ctx_len: torch.Tensor, max_ctx: int,
                            q_idx: torch.Tensor, key_scales: torch.Tensor, K: int, p_begin: int,
                            p_end: int, ws: Workspace, out_idx: torch.Tensor | None = None,
                            out_count: torch.Tensor | None = None,
                            out_sel_values: torch.Tensor | None = None):
    """Scaled Full-layer selection over candidates p_begin <= p < min(p_end,
    L-128).  Returns (idx [B, K], count [B], values of the selected [B, K])."""
    dev, B = cache.device, cache.batch
    _need(ctx_len, "ctx_len", torch.int32, dev, (B,))
    _need(q_idx, "q_idx", torch.int8, dev, (B, cache.idx_dim))
    _need(key_scales, "key_scales", torch.float32, dev, (cache.pages.shape[0], PAGE_TOKENS))
    if out_idx is None:
        out_idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B,), dtype=torch.int32, device=dev)
    if out_sel_values is None:
        out_sel_values = torch.empty((B, K), dtype=torch.float32, device=dev)
    _need(out_idx, "out_idx", torch.int32, dev, (B, K))
    _need(out_count, "out_count", torch.int32, dev, (B,))
    _need(out_sel_values, "out_sel_values", torch.float32, dev, (B, K))
    nbytes = lib().csa2_index_topk_workspace_size(B, max_ctx, K)
    if nbytes == 0:
        raise Csa2Error(f"index_topk_range_scaled: unsupported sizes B={B} max_ctx={max_ctx} K={K}")
    w = ws.get(nbytes, "topk", B)
    _check(lib().csa2_index_topk_range_scaled(ctypes.byref(cache.struct), ctx_len.data_ptr(),
                                              max_ctx, q_idx.data_ptr(), key_scales.data_ptr(), K,
                                              p_begin, p_end, out_idx.data_ptr(),
                                              out_count.data_ptr(), out_sel_values.data_ptr(),
                                              w.data_ptr(), w.numel(), _stream(dev)),
           "csa2_index_topk_range_scaled")
    return out_idx, out_count, out_sel_values


def lse_merge(outs: torch.Tensor, lses: torch.Tensor, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None):
    """Merge attention parts: outs fp32 [n, B, H, D], lses fp32 [n, B, H].
    Returns (out [B, H, D], lse [B, H])."""
    n, B, H, D = outs.shape
    dev = outs.device
    _need(outs, "outs", torch.float32, dev, (n, B, H, D))
    _need(lses, "lses", torch.float32, dev, (n, B, H))
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, (B, H, D))
    _need(lse, "lse", torch.float32, dev, (B, H))
    _check(lib().csa2_lse_merge(n, B, H, D, outs.data_ptr(), lses.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), _stream(dev)), "csa2_lse_merge")
    return out, lse


# ------------------------------------------------------------------ replay
def restore_window(cache: Cache, swa: torch.Tensor, tokens: torch.Tensor, lens) -> None:
    """Rebuild a layer's window ring after it was dropped, from the bf16 tokens
    of the last min(L_b, 128) positions of every sequence: tokens [B, 128, D]
    (bf16), row j of sequence b holding position L_b - 128 + j (rows of
    positions below 0 are ignored); lens: the host lengths L_b.  The tokens
    are re-appended with csa2_quantize_append (window ring written, indexer
    keys untouched); their FP4 rows are rewritten with the bytes they already
    hold, since the quantisation is a function of the token alone."""
    dev, B, D = cache.device, cache.batch, cache.head_dim
    tokens = _as_u16(tokens)
    _need(tokens, "tokens", torch.uint16, dev, (B, WINDOW, D))
    lens = [int(v) for v in lens]
    if len(lens) != B:
        raise ValueError(f"lens must hold {B} lengths")
    rows, seq, pos = [], [], []
    for b, L in enumerate(lens):
        w = min(max(L, 0), WINDOW)
        if w:
            rows.append(tokens[b, WINDOW - w:])
            seq.append(torch.full((w,), b, dtype=torch.int32, device=dev))
            pos.append(torch.arange(L - w, L, dtype=torch.int32, device=dev))
    if rows:
        quantize_append(cache, torch.cat(rows).contiguous(), torch.cat(seq), torch.cat(pos),
                        swa=swa)

