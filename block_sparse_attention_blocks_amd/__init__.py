"""Python binding of libbsattn: selected-block attention on MI355X (gfx950).

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI of ``include/bsattn.h``; PyTorch provides device
memory and the stream. There is no fallback of any kind: if the library is
missing, importing this package fails, and a failing call raises
``BsAttnError`` with the library's own description (vllm-omni PR #8335,
Purpose: an error of the attention provider reaches the caller; it is never
answered by running dense attention instead or by repeating K/V heads).

Tensors: q ``[B, q_len, Hq, D]``, k / v ``[B, kv_len, Hkv, D]``, bf16 on the
GPU, last dimension contiguous. ``layout`` is a mapping with the integer
fields of ``attn_shape`` (batch, num_q_heads, num_kv_heads, head_dim,
block_q, block_k, q_len, q_valid, kv_prefix_len, kv_prefix_valid, kv_len,
kv_suffix_valid) and optionally ``scale``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# Which build of the library to load: the release build next to this file
# unless BSATTN_LIBRARY names another (the tests use it for the list-checking
# and host-sanitized builds).
LIB_PATH = os.environ.get("BSATTN_LIBRARY") or os.path.join(_HERE, "libbsattn.so")

ATTN_OK = 0
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "LAUNCH", 5: "DEVICE",
                6: "SELF_TEST"}


class BsAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{STATUS_NAMES.get(status, status)}] {message}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("q_len", ctypes.c_int32), ("q_valid", ctypes.c_int32),
        ("kv_prefix_len", ctypes.c_int32), ("kv_prefix_valid", ctypes.c_int32),
        ("kv_len", ctypes.c_int32), ("kv_suffix_valid", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("softmax_scale", ctypes.c_float),
    ]


class AttnStrategy(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("dense_steps", ctypes.c_int32),
        ("sparse_layers", ctypes.c_uint64), ("sparsity_pct", ctypes.c_int32),
    ]


EXPORTS = ("attn_keep_blocks", "attn_select_workspace_size", "attn_select_blocks",
           "attn_select_blocks_noalloc", "attn_block_sparse_fwd", "attn_dense_fwd", "attn_dense_causal_fwd",
           "attn_strategy_is_sparse", "attn_strategy_workspace_size", "attn_strategy_fwd",
           "attn_strategy_warmup", "attn_query_support", "attn_self_test", "attn_last_error",
           "attn_version")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
            "g.build()' or python block_sparse_attention_blocks_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SH = ctypes.POINTER(AttnShape)
    lib.attn_keep_blocks.argtypes = [I32, I32, I32]
    lib.attn_keep_blocks.restype = I32
    lib.attn_select_workspace_size.argtypes = [SH]
    lib.attn_select_workspace_size.restype = SZ
    lib.attn_select_blocks.argtypes = [SH, P, P, I32, P, P, I32, P, SZ, P]
    lib.attn_select_blocks.restype = I32
    lib.attn_select_blocks_noalloc.argtypes = [SH, P, P, I32, P, P, I32, P]
    lib.attn_select_blocks_noalloc.restype = I32
    lib.attn_block_sparse_fwd.argtypes = [SH, P, P, P, P, P, I32, P, P, P]
    lib.attn_block_sparse_fwd.restype = I32
    lib.attn_dense_fwd.argtypes = [SH, P, P, P, P, P, P]
    lib.attn_dense_fwd.restype = I32
    lib.attn_dense_causal_fwd.argtypes = [SH, P, P, P, P, P, P]
    lib.attn_dense_causal_fwd.restype = I32
    ST = ctypes.POINTER(AttnStrategy)
    lib.attn_strategy_is_sparse.argtypes = [ST, I32, I32]
    lib.attn_strategy_is_sparse.restype = I32
    lib.attn_strategy_workspace_size.argtypes = [SH, ST]
    lib.attn_strategy_workspace_size.restype = SZ
    lib.attn_strategy_fwd.argtypes = [SH, ST, I32, I32, P, P, P, P, P, P, SZ, P]
    lib.attn_strategy_fwd.restype = I32
    lib.attn_strategy_warmup.argtypes = [SH, ST, P, P, P, P, P, SZ, P]
    lib.attn_strategy_warmup.restype = I32
    lib.attn_query_support.argtypes = [SH]
    lib.attn_query_support.restype = I32
    lib.attn_self_test.argtypes = []
    lib.attn_self_test.restype = I32
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def version() -> str:
    return lib.attn_version().decode()


def last_error() -> str:
    return lib.attn_last_error().decode()


def _check(status: int):
    if status != ATTN_OK:
        raise BsAttnError(status, last_error())


def self_test() -> None:
    """Start-up check on the current device (attn_self_test): a tiny
    selection and dense, sparse and causal attention run compared with the
    values their inputs fix. Raises BsAttnError naming the device, the check
    and the library version on any difference."""
    _check(lib.attn_self_test())


_FIELDS = ("batch", "num_q_heads", "num_kv_heads", "head_dim", "block_q", "block_k", "q_len",
           "q_valid", "kv_prefix_len", "kv_prefix_valid", "kv_len", "kv_suffix_valid")


def make_shape(layout, q=None, k=None, v=None, out=None) -> AttnShape:
    """attn_shape from a layout mapping; strides from the tensors given
    (contiguous [B, L, H, D] strides where a tensor is not given)."""
    s = AttnShape()
    for f in _FIELDS:
        setattr(s, f, int(layout[f]))
    d = int(layout["head_dim"])
    hq, hkv = int(layout["num_q_heads"]), int(layout["num_kv_heads"])

    def strides(t, length, heads):
        if t is not None:
            if t.stride(-1) != 1:
                raise ValueError("the last (head_dim) dimension must be contiguous")
            return t.stride(0), t.stride(1), t.stride(2)
        return length * heads * d, heads * d, d

    s.q_stride[:] = strides(q, int(layout["q_len"]), hq)
    s.k_stride[:] = strides(k, int(layout["kv_len"]), hkv)
    s.v_stride[:] = strides(v, int(layout["kv_len"]), hkv)
    s.o_stride[:] = strides(out, int(layout["q_len"]), hq)
    scale = layout.get("scale") if hasattr(layout, "get") else None
    s.softmax_scale = float(scale) if scale is not None else 0.0
    return s


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_kind(t, name, dtype, shape=None, seq_dim=None):
    """Type, dtype and shape; with ``seq_dim``, that dimension may hold more
    entries than the layout uses (rows past the layout are never touched)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is None:
        return
    got = tuple(t.shape)
    ok = len(got) == len(shape) and all(
        g >= w if i == seq_dim else g == w for i, (g, w) in enumerate(zip(got, shape)))
    if not ok:
        need = "at least " if seq_dim is not None else ""
        raise ValueError(f"{name} has shape {got}, the layout needs {tuple(shape)}"
                         + (f" ({need}{shape[seq_dim]} along dim {seq_dim})" if seq_dim is not None else ""))


def _check_device(t, name, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_operands(layout, q, k=None, v=None, out=None, block_idx=None, block_cnt=None):
    """dtype, exact shape and device of every tensor a call reads or writes:
    the library sees only pointers and strides, so a tensor smaller than the
    layout says would be read or written out of bounds. Shapes are checked
    before devices."""
    import torch
    b, d = int(layout["batch"]), int(layout["head_dim"])
    hq, hkv = int(layout["num_q_heads"]), int(layout["num_kv_heads"])
    lq, lk = int(layout["q_len"]), int(layout["kv_len"])
    nq, _, _ = num_blocks(layout)
    # [B, L, H, D] tensors may hold more rows than the layout's length
    named = [(q, "q", torch.bfloat16, (b, lq, hq, d), 1), (k, "k", torch.bfloat16, (b, lk, hkv, d), 1),
             (v, "v", torch.bfloat16, (b, lk, hkv, d), 1),
             (out, "out", torch.bfloat16, (b, lq, hq, d), 1)]
    if block_idx is not None:
        if not isinstance(block_idx, torch.Tensor) or block_idx.dim() != 4 or block_idx.shape[-1] < 1:
            raise ValueError("block_idx must be an int32 tensor [B, Hq, NQ, row] with row >= 1")
        named.append((block_idx, "block_idx", torch.int32, (b, hq, nq, int(block_idx.shape[-1])), None))
    named.append((block_cnt, "block_cnt", torch.int32, (b, hq, nq), None))
    present = [x for x in named if x[0] is not None]
    for t, n, dt, shp, sd in present:
        _check_kind(t, n, dt, shp, sd)
    for t, n, _, _, _ in present:
        _check_device(t, n, q.device)
    for t, n in ((block_idx, "block_idx"), (block_cnt, "block_cnt")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")


def keep_blocks(n_kv_blocks: int, n_protected: int, sparsity_pct: int) -> int:
    """Kept blocks per row for a target sparsity (protected blocks included)."""
    k = lib.attn_keep_blocks(n_kv_blocks, n_protected, sparsity_pct)
    if k < 0:
        raise ValueError("need 0 <= n_protected <= n_kv_blocks and 0 <= sparsity_pct <= 100")
    return k


def num_blocks(layout):
    """(NQ, NK, P) of a layout."""
    return (int(layout["q_len"]) // int(layout["block_q"]),
            int(layout["kv_len"]) // int(layout["block_k"]),
            int(layout["kv_prefix_len"]) // int(layout["block_k"]))


def select_workspace_size(layout) -> int:
    n = lib.attn_select_workspace_size(ctypes.byref(make_shape(layout)))
    if n == 0:
        _check(lib.attn_query_support(ctypes.byref(make_shape(layout))))
    return n


def select_blocks(q, k, layout, keep: int, idx_row_stride=None, *, block_idx=None,
                  block_cnt=None, workspace=None, stream=None):
    """Per-query-head KV-block indices and counts (attn_select_blocks).
    Returns (block_idx [B,Hq,NQ,stride] int32, block_cnt [B,Hq,NQ] int32)."""
    import torch
    _check_operands(layout, q, k, block_idx=block_idx, block_cnt=block_cnt)
    shape = make_shape(layout, q=q, k=k)
    nq, nk, _ = num_blocks(layout)
    stride = int(keep if idx_row_stride is None else idx_row_stride)
    stride = max(stride, 1)
    b, hq = int(layout["batch"]), int(layout["num_q_heads"])
    if block_idx is not None and int(block_idx.shape[-1]) != stride:
        raise ValueError(f"block_idx rows hold {int(block_idx.shape[-1])} entries, "
                         f"idx_row_stride is {stride}")
    if block_idx is None:
        block_idx = torch.empty((b, hq, nq, stride), dtype=torch.int32, device=q.device)
    if block_cnt is None:
        block_cnt = torch.empty((b, hq, nq), dtype=torch.int32, device=q.device)
    ws_bytes = lib.attn_select_workspace_size(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _check(lib.attn_select_blocks(ctypes.byref(shape), _ptr(q), _ptr(k), int(keep),
                                  _ptr(block_idx), _ptr(block_cnt), stride, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream)))
    return block_idx, block_cnt


# Bytes of the library's own selector scratch (attn_select_blocks_noalloc).
SELECT_STATIC_WORKSPACE_BYTES = 64 << 20


def select_blocks_noalloc(q, k, layout, keep: int, idx_row_stride=None, *, block_idx=None,
                          block_cnt=None, stream=None):
    """attn_select_blocks_noalloc: the selector with the library's fixed
    scratch array instead of a caller workspace (nothing is allocated by the
    library; the outputs are allocated here unless given). Calls that overlap
    on one device race on that array."""
    import torch
    _check_operands(layout, q, k, block_idx=block_idx, block_cnt=block_cnt)
    shape = make_shape(layout, q=q, k=k)
    nq, _, _ = num_blocks(layout)
    stride = max(int(keep if idx_row_stride is None else idx_row_stride), 1)
    b, hq = int(layout["batch"]), int(layout["num_q_heads"])
    if block_idx is not None and int(block_idx.shape[-1]) != stride:
        raise ValueError(f"block_idx rows hold {int(block_idx.shape[-1])} entries, "
                         f"idx_row_stride is {stride}")
    if block_idx is None:
        block_idx = torch.empty((b, hq, nq, stride), dtype=torch.int32, device=q.device)
    if block_cnt is None:
        block_cnt = torch.empty((b, hq, nq), dtype=torch.int32, device=q.device)
    _check(lib.attn_select_blocks_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), int(keep),
                                          _ptr(block_idx), _ptr(block_cnt), stride,
                                          _stream_handle(stream)))
    return block_idx, block_cnt


def block_sparse_attention(q, k, v, block_idx, block_cnt, layout, *, out=None, return_lse=False,
                           stream=None):
    """Attention over the selected blocks (attn_block_sparse_fwd)."""
    import torch
    if block_idx is None or block_cnt is None:
        raise ValueError("block_idx and block_cnt are required")
    _check_operands(layout, q, k, v, out, block_idx, block_cnt)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = None
    if return_lse:
        lse = torch.empty((int(layout["batch"]), int(layout["num_q_heads"]), int(layout["q_len"])),
                          dtype=torch.float32, device=q.device)
    shape = make_shape(layout, q=q, k=k, v=v, out=out)
    _check(lib.attn_block_sparse_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(block_idx), _ptr(block_cnt), int(block_idx.shape[-1]),
                                     _ptr(out), _ptr(lse), _stream_handle(stream)))
    return (out, lse) if return_lse else out


def dense_attention(q, k, v, layout, *, causal=False, out=None, return_lse=False, stream=None):
    """Dense attention through the same kernel (attn_dense_fwd), or, with
    ``causal``, causal dense attention bottom-right aligned over the real
    tokens (attn_dense_causal_fwd)."""
    import torch
    _check_operands(layout, q, k, v, out)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = None
    if return_lse:
        lse = torch.empty((int(layout["batch"]), int(layout["num_q_heads"]), int(layout["q_len"])),
                          dtype=torch.float32, device=q.device)
    shape = make_shape(layout, q=q, k=k, v=v, out=out)
    fn = lib.attn_dense_causal_fwd if causal else lib.attn_dense_fwd
    _check(fn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
              _stream_handle(stream)))
    return (out, lse) if return_lse else out


def make_strategy(num_layers: int, dense_steps: int, sparse_layers, sparsity_pct: int) -> AttnStrategy:
    """attn_strategy: steps [0, dense_steps) dense in every layer, then the
    layers in ``sparse_layers`` sparse at ``sparsity_pct``."""
    mask = 0
    for layer in sparse_layers:
        if not 0 <= int(layer) < 64:
            raise ValueError("layers must be in [0, 64)")
        mask |= 1 << int(layer)
    return AttnStrategy(int(num_layers), int(dense_steps), mask, int(sparsity_pct))


def strategy_is_sparse(strategy: AttnStrategy, step: int, layer: int) -> bool:
    r = lib.attn_strategy_is_sparse(ctypes.byref(strategy), int(step), int(layer))
    if r < 0:
        raise ValueError("invalid strategy or (step, layer)")
    return bool(r)


def strategy_workspace_size(layout, strategy: AttnStrategy) -> int:
    n = lib.attn_strategy_workspace_size(ctypes.byref(make_shape(layout)), ctypes.byref(strategy))
    if n == 0:
        raise ValueError("invalid layout or strategy")
    return n


def _strategy_ws(layout, strategy, workspace, device):
    import torch
    if workspace is None:
        workspace = torch.empty(strategy_workspace_size(layout, strategy), dtype=torch.uint8,
                                device=device)
    return workspace, workspace.numel() * workspace.element_size()


def strategy_forward(q, k, v, layout, strategy: AttnStrategy, step: int, layer: int, *, out=None,
                     return_lse=False, workspace=None, stream=None):
    """The attention of (step, layer) under ``strategy`` (attn_strategy_fwd):
    dense, or selection + block-sparse attention."""
    import torch
    _check_operands(layout, q, k, v, out)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = None
    if return_lse:
        lse = torch.empty((int(layout["batch"]), int(layout["num_q_heads"]), int(layout["q_len"])),
                          dtype=torch.float32, device=q.device)
    ws, nbytes = _strategy_ws(layout, strategy, workspace, q.device)
    shape = make_shape(layout, q=q, k=k, v=v, out=out)
    _check(lib.attn_strategy_fwd(ctypes.byref(shape), ctypes.byref(strategy), int(step), int(layer),
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                 _stream_handle(stream)))
    return (out, lse) if return_lse else out


def strategy_warmup(q, k, v, layout, strategy: AttnStrategy, *, out=None, workspace=None,
                    stream=None):
    """Run every kind of call the strategy makes once (attn_strategy_warmup)."""
    import torch
    _check_operands(layout, q, k, v, out)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    ws, nbytes = _strategy_ws(layout, strategy, workspace, q.device)
    shape = make_shape(layout, q=q, k=k, v=v, out=out)
    _check(lib.attn_strategy_warmup(ctypes.byref(shape), ctypes.byref(strategy), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(out), _ptr(ws), nbytes, _stream_handle(stream)))


def query_support(layout):
    """(status, message) of attn_query_support for a layout."""
    st = lib.attn_query_support(ctypes.byref(make_shape(layout)))
    return st, (last_error() if st else "")


def pad_segments(q_gen, k_prefix, v_prefix, k_gen, v_gen, block_q: int, block_k: int, scale=None):
    """Request preparation (vllm-omni PR #8335, Purpose: the shared layer owns
    protected prefixes and suffix padding): pad the query stream to block_q and
    each key/value segment to block_k on its own (diffusers cosmos_parallel.py,
    shard_cosmos3_sequence), and return (q, k, v, layout). Inputs are
    [B, L, H, D] bf16 GPU tensors; k_prefix/v_prefix may have length 0."""
    import torch
    b, lg, hq, d = q_gen.shape
    lp, hkv = k_prefix.shape[1], k_prefix.shape[2]

    def up(n, m):
        return ((n + m - 1) // m) * m

    ql, pl, gl = up(lg, block_q), up(lp, block_k), up(k_gen.shape[1], block_k)
    q = torch.zeros((b, ql, hq, d), dtype=q_gen.dtype, device=q_gen.device)
    q[:, :lg] = q_gen
    k = torch.zeros((b, pl + gl, hkv, d), dtype=k_gen.dtype, device=k_gen.device)
    v = torch.zeros_like(k)
    k[:, :lp] = k_prefix
    v[:, :lp] = v_prefix
    k[:, pl:pl + k_gen.shape[1]] = k_gen
    v[:, pl:pl + v_gen.shape[1]] = v_gen
    layout = dict(batch=b, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_q=block_q,
                  block_k=block_k, q_len=ql, q_valid=lg, kv_prefix_len=pl, kv_prefix_valid=lp,
                  kv_len=pl + gl, kv_suffix_valid=k_gen.shape[1], scale=scale)
    return q, k, v, layout


__all__ = ["BsAttnError", "AttnShape", "AttnStrategy", "EXPORTS", "LIB_PATH", "lib", "version",
           "last_error", "make_shape", "keep_blocks", "num_blocks", "select_workspace_size",
           "select_blocks", "select_blocks_noalloc", "SELECT_STATIC_WORKSPACE_BYTES", "block_sparse_attention", "dense_attention", "make_strategy",
           "strategy_is_sparse", "strategy_workspace_size", "strategy_forward",
           "strategy_warmup", "query_support", "self_test", "pad_segments"]
