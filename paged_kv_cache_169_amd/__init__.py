"""Python binding of libkvcache.so (include/kvcache.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. PyTorch supplies device memory (tensors) and streams; functions
take tensors, check that they live on the GPU with the right dtype and
shape, and pass their data pointers to the C functions of the same name.

The library must have been built (``__graft_entry__.build()``); importing
this package raises if it is missing. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVCACHE_LIB may name another build of the library (same ABI)
LIB_PATH = os.environ.get("KVCACHE_LIB", os.path.join(_PKG, "libkvcache.so"))

KV_OK, KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_ERR_HIP, KV_ERR_TABLE = 0, -1, -2, -3, -4, -5
KV_F32, KV_BF16, KV_INT4 = 0, 1, 2
BLOCK = 16
KV_NOALLOC_SCRATCH_BYTES = 64 << 20  # the device array of kv_decode_step_noalloc
(KV_REGION_K, KV_REGION_V, KV_REGION_KQ, KV_REGION_KS, KV_REGION_KM, KV_REGION_VQ, KV_REGION_VS,
 KV_REGION_VM, KV_REGION_KTAIL) = range(9)
KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA = 0, 1, 2
KV_SCHED_AUTO, KV_SCHED_SPLIT, KV_SCHED_BALANCED = 0, 1, 2

_DTYPES = {"f32": KV_F32, "bf16": KV_BF16, "int4": KV_INT4}


class KVError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kv_status_string(status)} ({status})")
        self.status = status


class kv_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class kv_attn_opts(ctypes.Structure):
    _fields_ = [("split_blocks", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("window", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("events", ctypes.c_void_p * 3)]


KV_MAX_PREFIX_GROUPS = 256


class kv_prefix_groups(ctypes.Structure):
    _fields_ = [("n_groups", ctypes.c_int32), ("group_start", ctypes.POINTER(ctypes.c_int32)),
                ("prefix_blocks", ctypes.POINTER(ctypes.c_int32))]


def prefix_groups(group_start, prefix_blocks):
    """kv_prefix_groups over host copies of the two lists; the arrays are kept
    alive on the returned record (attribute _keep)."""
    gs = (ctypes.c_int32 * len(group_start))(*[int(x) for x in group_start])
    pb = (ctypes.c_int32 * max(1, len(prefix_blocks)))(*[int(x) for x in prefix_blocks])
    g = kv_prefix_groups(len(prefix_blocks), gs, pb)
    g._keep = (gs, pb)
    return g


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I32, _SZ, _F, _D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_double


def _decl(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_kv_status_string = _decl("kv_status_string", ctypes.c_char_p, [_I32])
_kv_abi_version = _decl("kv_abi_version", _I32, [])
_kv_pool_required_bytes = _decl("kv_pool_required_bytes", _SZ, [ctypes.POINTER(kv_pool_desc)])
_kv_pool_create = _decl("kv_pool_create", _I32, [ctypes.POINTER(kv_pool_desc), _P, _SZ, ctypes.POINTER(_P)])
_kv_pool_destroy = _decl("kv_pool_destroy", _I32, [_P])
_kv_pool_region = _decl("kv_pool_region", _I32, [_P, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)])
_kv_pool_get_desc = _decl("kv_pool_get_desc", _I32, [_P, ctypes.POINTER(kv_pool_desc)])
_kv_append = _decl("kv_append", _I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _P])
_kv_append_tokens = _decl("kv_append_tokens", _I32, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P])
_paged_decode_attention_workspace_bytes = _decl(
    "paged_decode_attention_workspace_bytes", _SZ, [_P, _I32, _I32, _I32, ctypes.POINTER(kv_attn_opts)])
_paged_decode_attention = _decl(
    "paged_decode_attention", _I32,
    [_P, _P, _P, _I32, _F, _P, _I32, _P, _P, _I32, _I32, _P, _SZ, ctypes.POINTER(kv_attn_opts), _P])
_paged_decode_attention_shared_workspace_bytes = _decl(
    "paged_decode_attention_shared_workspace_bytes", _SZ,
    [_P, _I32, _I32, _I32, ctypes.POINTER(kv_prefix_groups), ctypes.POINTER(kv_attn_opts)])
_paged_decode_attention_shared = _decl(
    "paged_decode_attention_shared", _I32,
    [_P, _P, _P, _I32, _F, _P, _I32, _P, _I32, _I32, ctypes.POINTER(kv_prefix_groups), _P, _SZ,
     ctypes.POINTER(kv_attn_opts), _P])
_paged_multi_token_attention_workspace_bytes = _decl(
    "paged_multi_token_attention_workspace_bytes", _SZ, [_P, _I32, _I32, _I32, _I32, ctypes.POINTER(kv_attn_opts)])
_paged_multi_token_attention = _decl(
    "paged_multi_token_attention", _I32,
    [_P, _P, _P, _I32, _I32, _F, _P, _I32, _P, _P, _I32, _I32, _P, _SZ, ctypes.POINTER(kv_attn_opts), _P])
_kv_decode_step = _decl(
    "kv_decode_step", _I32,
    [_P, _P, _P, _P, _P, _I32, _I32, _F, _P, _I32, _P, _P, _I32, _I32, _P, _SZ, ctypes.POINTER(kv_attn_opts), _P])
_kv_decode_step_noalloc = _decl(
    "kv_decode_step_noalloc", _I32,
    [_P, _P, _P, _P, _P, _I32, _I32, _F, _P, _I32, _P, _P, _I32, _I32, ctypes.POINTER(kv_attn_opts), _P])
_kv_quantize_int4 = _decl("kv_quantize_int4", _I32, [_P, _P, _P, _I32, _P, _P, _I32, _P])
_rope_rerotate = _decl("rope_rerotate", _I32, [_P, _P, _I32, _I32, _I32, _F, _I32, _P])
_kv_block_bytes = _decl("kv_block_bytes", _SZ, [_P])
_kv_copy_blocks = _decl("kv_copy_blocks", _I32, [_P, _P, _P, _I32, _P])
_kv_layer_window = _decl("kv_layer_window", _I32, [_P, _I32, _I32, _P])
_kv_window_released_blocks = _decl("kv_window_released_blocks", _I32, [_P, _I32, _I32, _P, _P])
_kv_gather_blocks = _decl("kv_gather_blocks", _I32, [_P, _P, _I32, _P, _SZ, _P])
_kv_scatter_blocks = _decl("kv_scatter_blocks", _I32, [_P, _P, _I32, _P, _SZ, _P])
_kv_token_deviation = _decl("kv_token_deviation", _I32, [_P, _P, _I32, _I32, _P, _P, _I32, _P, _P, _P, _P])
_kv_topk_select = _decl("kv_topk_select", _I32, [_P, _P, _P, _I32, _P, _P])
_kv_recompute_ratio = _decl("kv_recompute_ratio", _D, [_D, _D, _I32, _D])
_kv_recompute_count = _decl("kv_recompute_count", _I32, [_D, _I32])
_kv_read_probe = _decl("kv_read_probe", _I32, [_P, _SZ, _I32, _P, _P])
_kv_validate_tables = _decl("kv_validate_tables", _I32,
                            [ctypes.POINTER(kv_pool_desc), _P, _I32, _P, _I32, _I32, ctypes.POINTER(_I32)])


def lib_handle():
    """The loaded ctypes library (tests check its exports)."""
    return _lib


def kv_status_string(status: int) -> str:
    return _kv_status_string(int(status)).decode()


def kv_abi_version() -> int:
    return int(_kv_abi_version())


def _check(status: int, where: str) -> None:
    if status != KV_OK:
        raise KVError(status, where)


def make_desc(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str = "bf16",
              max_seqs: int = 0) -> kv_pool_desc:
    return kv_pool_desc(int(num_blocks), BLOCK, int(num_kv_heads), int(head_dim), int(max_seqs),
                        _DTYPES[dtype] if isinstance(dtype, str) else int(dtype))


def kv_pool_required_bytes(desc: kv_pool_desc) -> int:
    return int(_kv_pool_required_bytes(ctypes.byref(desc)))


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_ptr(t: torch.Tensor | None, name: str, dtype=None, numel=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


_REGION_DTYPE = {KV_REGION_KQ: torch.uint8, KV_REGION_VQ: torch.uint8, KV_REGION_KS: torch.float16,
                 KV_REGION_KM: torch.float16, KV_REGION_VS: torch.float16, KV_REGION_VM: torch.float16,
                 KV_REGION_KTAIL: torch.bfloat16}


class KVPool:
    """A pool bound to a torch-allocated device blob (kv_pool_create).

    Region views (``K``, ``V`` for fp32/bf16 pools; ``KQ``, ``KS``, ``KM``,
    ``VQ``, ``VS``, ``VM``, ``KTAIL`` for INT4 pools) are torch views of the
    blob with the shapes documented in include/kvcache.h."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str = "bf16",
                 max_seqs: int = 0, device="cuda", memory: torch.Tensor | None = None):
        self.desc = make_desc(num_blocks, num_kv_heads, head_dim, dtype, max_seqs)
        self.dtype = dtype
        need = kv_pool_required_bytes(self.desc)
        if need == 0:
            raise ValueError("invalid pool descriptor")
        if memory is None:
            memory = torch.empty(need + 256, dtype=torch.uint8, device=device)
        base = memory.data_ptr()
        pad = (-base) % 256
        self.memory = memory
        self.blob = memory[pad:pad + need]
        self.nbytes = need
        h = _P()
        _check(_kv_pool_create(ctypes.byref(self.desc), self.blob.data_ptr(), need, ctypes.byref(h)),
               "kv_pool_create")
        self.handle = h
        nb, nkv, d = num_blocks, num_kv_heads, head_dim
        shapes = {KV_REGION_K: (nb, nkv, BLOCK, d), KV_REGION_V: (nb, nkv, BLOCK, d),
                  KV_REGION_KQ: (nb, nkv, BLOCK, d // 2), KV_REGION_VQ: (nb, nkv, BLOCK, d // 2),
                  KV_REGION_KS: (nb, nkv, d), KV_REGION_KM: (nb, nkv, d),
                  KV_REGION_VS: (nb, nkv, BLOCK), KV_REGION_VM: (nb, nkv, BLOCK),
                  KV_REGION_KTAIL: (max_seqs, nkv, BLOCK, d)}
        names = ["K", "V", "KQ", "KS", "KM", "VQ", "VS", "VM", "KTAIL"]
        elem = {"f32": torch.float32, "bf16": torch.bfloat16}.get(dtype)
        for r, nm in enumerate(names):
            off, size = self.region(r)
            if off is None:
                setattr(self, nm, None)
                continue
            dt = _REGION_DTYPE.get(r, elem)
            view = self.blob[off:off + size].view(dt).view(shapes[r])
            setattr(self, nm, view)

    def region(self, region: int):
        off, size = _SZ(), _SZ()
        st = _kv_pool_region(self.handle, int(region), ctypes.byref(off), ctypes.byref(size))
        if st != KV_OK:
            return None, None
        return int(off.value), int(size.value)

    def get_desc(self) -> kv_pool_desc:
        d = kv_pool_desc()
        _check(_kv_pool_get_desc(self.handle, ctypes.byref(d)), "kv_pool_get_desc")
        return d

    def close(self) -> None:
        if getattr(self, "handle", None):
            _kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _i32(t, name):
    return _dev_ptr(t, name, torch.int32)


def kv_append(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, block_tables: torch.Tensor,
              seq_lens: torch.Tensor, seq_slots: torch.Tensor | None = None, stream=None) -> None:
    d = pool.desc
    B = int(seq_lens.numel())
    want = torch.float32 if d.dtype == KV_F32 else torch.bfloat16
    n = B * d.num_kv_heads * d.head_dim
    st = _kv_append(pool.handle, _dev_ptr(k_new, "k_new", want, n), _dev_ptr(v_new, "v_new", want, n),
                    _i32(block_tables, "block_tables"), int(block_tables.shape[1]), _i32(seq_lens, "seq_lens"),
                    _i32(seq_slots, "seq_slots"), B, _stream(stream))
    _check(st, "kv_append")


def kv_append_tokens(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, block_tables: torch.Tensor,
                     seq_lens: torch.Tensor, seq_slots: torch.Tensor | None = None, stream=None) -> None:
    """k_new, v_new: [batch][n_new][n_kv][head_dim]."""
    d = pool.desc
    B, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    want = torch.float32 if d.dtype == KV_F32 else torch.bfloat16
    n = B * n_new * d.num_kv_heads * d.head_dim
    if int(seq_lens.numel()) != B:
        raise ValueError("seq_lens must have one entry per sequence")
    st = _kv_append_tokens(pool.handle, _dev_ptr(k_new, "k_new", want, n), _dev_ptr(v_new, "v_new", want, n),
                           _i32(block_tables, "block_tables"), int(block_tables.shape[1]), _i32(seq_lens, "seq_lens"),
                           _i32(seq_slots, "seq_slots"), B, n_new, _stream(stream))
    _check(st, "kv_append_tokens")


def attn_opts(split_blocks: int = 0, kernel: int = 0, window: int = 0, schedule: int = 0,
              events=None) -> kv_attn_opts:
    o = kv_attn_opts(int(split_blocks), int(kernel), int(window), int(schedule))
    if events:
        for i, e in enumerate(events[:3]):
            o.events[i] = e
    return o


def paged_decode_attention_workspace_bytes(pool: KVPool, batch: int, num_q_heads: int, max_ctx: int,
                                           opts: kv_attn_opts | None = None) -> int:
    n = _paged_decode_attention_workspace_bytes(pool.handle, int(batch), int(num_q_heads), int(max_ctx),
                                                ctypes.byref(opts) if opts is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise KVError(KV_ERR_INVALID_ARG, "paged_decode_attention_workspace_bytes")
    return int(n)


def paged_decode_attention(pool: KVPool, q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                           ctx_lens: torch.Tensor, scale: float, max_ctx: int,
                           workspace: torch.Tensor | None = None, seq_slots: torch.Tensor | None = None,
                           opts: kv_attn_opts | None = None, stream=None) -> None:
    d = pool.desc
    B, n_h, hd = q.shape
    if hd != d.head_dim or tuple(out.shape) != (B, n_h, hd):
        raise ValueError("q / out shape does not match the pool")
    want = torch.float32 if d.dtype == KV_F32 else torch.bfloat16
    ws_ptr = _dev_ptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _paged_decode_attention(pool.handle, _dev_ptr(q, "q", want), _dev_ptr(out, "out", torch.float32), n_h,
                                 float(scale), _i32(block_tables, "block_tables"), int(block_tables.shape[1]),
                                 _i32(ctx_lens, "ctx_lens"), _i32(seq_slots, "seq_slots"), B, int(max_ctx),
                                 ws_ptr, ws_bytes, ctypes.byref(opts) if opts is not None else None,
                                 _stream(stream))
    _check(st, "paged_decode_attention")


def paged_decode_attention_shared_workspace_bytes(pool: KVPool, batch: int, num_q_heads: int, max_ctx: int,
                                                  groups: kv_prefix_groups, opts: kv_attn_opts | None = None) -> int:
    n = _paged_decode_attention_shared_workspace_bytes(pool.handle, int(batch), int(num_q_heads), int(max_ctx),
                                                       ctypes.byref(groups),
                                                       ctypes.byref(opts) if opts is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise KVError(KV_ERR_INVALID_ARG, "paged_decode_attention_shared_workspace_bytes")
    return int(n)


def paged_decode_attention_shared(pool: KVPool, q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                                  ctx_lens: torch.Tensor, scale: float, max_ctx: int, groups: kv_prefix_groups,
                                  workspace: torch.Tensor | None = None, opts: kv_attn_opts | None = None,
                                  stream=None) -> None:
    """paged_decode_attention with the shared prefixes of `groups`
    (prefix_groups(group_start, prefix_blocks)) read once per group."""
    d = pool.desc
    B, n_h, hd = q.shape
    if hd != d.head_dim or tuple(out.shape) != (B, n_h, hd):
        raise ValueError("q / out shape does not match the pool")
    ws_ptr = _dev_ptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _paged_decode_attention_shared(pool.handle, _dev_ptr(q, "q", torch.bfloat16),
                                        _dev_ptr(out, "out", torch.float32), n_h, float(scale),
                                        _i32(block_tables, "block_tables"), int(block_tables.shape[1]),
                                        _i32(ctx_lens, "ctx_lens"), B, int(max_ctx), ctypes.byref(groups),
                                        ws_ptr, ws_bytes, ctypes.byref(opts) if opts is not None else None,
                                        _stream(stream))
    _check(st, "paged_decode_attention_shared")


def paged_multi_token_attention_workspace_bytes(pool: KVPool, batch: int, num_q_heads: int, q_len: int,
                                                max_ctx: int, opts: kv_attn_opts | None = None) -> int:
    n = _paged_multi_token_attention_workspace_bytes(pool.handle, int(batch), int(num_q_heads), int(q_len),
                                                     int(max_ctx), ctypes.byref(opts) if opts is not None else None)
    if n == ctypes.c_size_t(-1).value:
        raise KVError(KV_ERR_INVALID_ARG, "paged_multi_token_attention_workspace_bytes")
    return int(n)


def paged_multi_token_attention(pool: KVPool, q: torch.Tensor, out: torch.Tensor, block_tables: torch.Tensor,
                                ctx_lens: torch.Tensor, scale: float, max_ctx: int,
                                workspace: torch.Tensor | None = None, seq_slots: torch.Tensor | None = None,
                                opts: kv_attn_opts | None = None, stream=None) -> None:
    """q: [batch][q_len][num_q_heads][head_dim] bf16; out the same shape, fp32."""
    d = pool.desc
    B, q_len, n_h, hd = q.shape
    if hd != d.head_dim or tuple(out.shape) != (B, q_len, n_h, hd):
        raise ValueError("q / out shape does not match the pool")
    ws_ptr = _dev_ptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _paged_multi_token_attention(pool.handle, _dev_ptr(q, "q", torch.bfloat16), _dev_ptr(out, "out", torch.float32),
                                      n_h, q_len, float(scale), _i32(block_tables, "block_tables"),
                                      int(block_tables.shape[1]), _i32(ctx_lens, "ctx_lens"),
                                      _i32(seq_slots, "seq_slots"), B, int(max_ctx), ws_ptr, ws_bytes,
                                      ctypes.byref(opts) if opts is not None else None, _stream(stream))
    _check(st, "paged_multi_token_attention")


def kv_decode_step(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, out: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_ctx: int,
                   workspace: torch.Tensor | None = None, seq_slots: torch.Tensor | None = None,
                   opts: kv_attn_opts | None = None, stream=None) -> None:
    """Append q_len tokens per sequence, then attend (see kv_decode_step in
    kvcache.h). q: [batch][num_q_heads][head_dim] (one token) or
    [batch][q_len][num_q_heads][head_dim]; k_new / v_new: [batch][n_kv][head_dim]
    or [batch][q_len][n_kv][head_dim]; out: fp32, the shape of q."""
    d = pool.desc
    if q.dim() == 3:
        B, n_h, hd = q.shape
        q_len = 1
    else:
        B, q_len, n_h, hd = q.shape
    if hd != d.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out shape does not match the pool")
    kdt = torch.float32 if d.dtype == KV_F32 else torch.bfloat16
    n = B * q_len * d.num_kv_heads * d.head_dim
    ws_ptr = _dev_ptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _kv_decode_step(pool.handle, _dev_ptr(k_new, "k_new", kdt, n), _dev_ptr(v_new, "v_new", kdt, n),
                         _dev_ptr(q, "q", kdt), _dev_ptr(out, "out", torch.float32), n_h, q_len, float(scale),
                         _i32(block_tables, "block_tables"), int(block_tables.shape[1]), _i32(seq_lens, "seq_lens"),
                         _i32(seq_slots, "seq_slots"), B, int(max_ctx), ws_ptr, ws_bytes,
                         ctypes.byref(opts) if opts is not None else None, _stream(stream))
    _check(st, "kv_decode_step")


def kv_decode_step_noalloc(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                           out: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                           max_ctx: int, seq_slots: torch.Tensor | None = None, opts: kv_attn_opts | None = None,
                           stream=None) -> None:
    """kv_decode_step with the library's own device workspace (see
    kv_decode_step_noalloc in kvcache.h); shapes as kv_decode_step."""
    d = pool.desc
    if q.dim() == 3:
        B, n_h, hd = q.shape
        q_len = 1
    else:
        B, q_len, n_h, hd = q.shape
    if hd != d.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out shape does not match the pool")
    kdt = torch.float32 if d.dtype == KV_F32 else torch.bfloat16
    n = B * q_len * d.num_kv_heads * d.head_dim
    st = _kv_decode_step_noalloc(pool.handle, _dev_ptr(k_new, "k_new", kdt, n), _dev_ptr(v_new, "v_new", kdt, n),
                                 _dev_ptr(q, "q", kdt), _dev_ptr(out, "out", torch.float32), n_h, q_len,
                                 float(scale), _i32(block_tables, "block_tables"), int(block_tables.shape[1]),
                                 _i32(seq_lens, "seq_lens"), _i32(seq_slots, "seq_slots"), B, int(max_ctx),
                                 ctypes.byref(opts) if opts is not None else None, _stream(stream))
    _check(st, "kv_decode_step_noalloc")


def kv_quantize_int4(dst: KVPool, src: KVPool, block_tables: torch.Tensor, lens: torch.Tensor,
                     seq_slots: torch.Tensor | None = None, stream=None) -> None:
    st = _kv_quantize_int4(dst.handle, src.handle, _i32(block_tables, "block_tables"), int(block_tables.shape[1]),
                           _i32(lens, "lens"), _i32(seq_slots, "seq_slots"), int(lens.numel()), _stream(stream))
    _check(st, "kv_quantize_int4")


def rope_rerotate(pool: KVPool, chunk_blocks: torch.Tensor, first_slot: int, num_tokens: int, delta: int,
                  base: float = 10000.0, style: int = 0, stream=None) -> None:
    st = _rope_rerotate(pool.handle, _i32(chunk_blocks, "chunk_blocks"), int(first_slot), int(num_tokens),
                        int(delta), float(base), int(style), _stream(stream))
    _check(st, "rope_rerotate")


def kv_block_bytes(pool: KVPool) -> int:
    return int(_kv_block_bytes(pool.handle))


def kv_layer_window(windows, layer: int) -> int:
    """Window of a 0-based layer from a per-layer list repeated cyclically."""
    w = (ctypes.c_int32 * len(windows))(*[int(x) for x in windows])
    out = ctypes.c_int32(0)
    _check(_kv_layer_window(ctypes.cast(w, ctypes.c_void_p) if len(windows) else None, len(windows), int(layer),
                            ctypes.byref(out)), "kv_layer_window")
    return int(out.value)


def kv_window_released_blocks(seq_lens: torch.Tensor, window: int, released: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """Per sequence, the leading blocks no later query can attend (-1 for a
    negative length), as an int32 device tensor."""
    B = int(seq_lens.numel())
    if released is None:
        released = torch.empty(B, dtype=torch.int32, device=seq_lens.device)
    if int(released.numel()) != B:
        raise ValueError("released must hold one entry per sequence")
    _check(_kv_window_released_blocks(_i32(seq_lens, "seq_lens"), B, int(window), _i32(released, "released"),
                                      _stream(stream)), "kv_window_released_blocks")
    return released


def kv_copy_blocks(pool: KVPool, src_blocks: torch.Tensor, dst_blocks: torch.Tensor, stream=None) -> None:
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    _check(_kv_copy_blocks(pool.handle, _i32(src_blocks, "src_blocks"), _i32(dst_blocks, "dst_blocks"), n,
                           _stream(stream)), "kv_copy_blocks")


def _buf_ptr(buffer: torch.Tensor, name: str) -> tuple[int, int]:
    """Device tensor, or pinned host tensor (mapped for the device)."""
    if not buffer.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not buffer.is_cuda and not buffer.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    return buffer.data_ptr(), buffer.numel() * buffer.element_size()


def kv_gather_blocks(pool: KVPool, blocks: torch.Tensor, buffer: torch.Tensor, stream=None) -> None:
    ptr, nbytes = _buf_ptr(buffer, "buffer")
    _check(_kv_gather_blocks(pool.handle, _i32(blocks, "blocks"), int(blocks.numel()), ptr, nbytes, _stream(stream)),
           "kv_gather_blocks")


def kv_scatter_blocks(pool: KVPool, blocks: torch.Tensor, buffer: torch.Tensor, stream=None) -> None:
    ptr, nbytes = _buf_ptr(buffer, "buffer")
    _check(_kv_scatter_blocks(pool.handle, _i32(blocks, "blocks"), int(blocks.numel()), ptr, nbytes,
                              _stream(stream)), "kv_scatter_blocks")


def kv_token_deviation(pool: KVPool, block_tables: torch.Tensor, row_seq: torch.Tensor, row_pos: torch.Tensor,
                       k_re: torch.Tensor, v_re: torch.Tensor, deviation: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """fp64 KV deviation per row (see kv_token_deviation in kvcache.h)."""
    n = int(row_seq.numel())
    if int(row_pos.numel()) != n:
        raise ValueError("row_seq and row_pos differ in length")
    want = n * pool.desc.num_kv_heads * pool.desc.head_dim
    kdt = torch.float32 if pool.desc.dtype == KV_F32 else torch.bfloat16
    if deviation is None:
        deviation = torch.empty(n, dtype=torch.float64, device=k_re.device)
    batch, max_blocks = block_tables.shape
    st = _kv_token_deviation(pool.handle, _i32(block_tables, "block_tables"), int(max_blocks), int(batch),
                             _i32(row_seq, "row_seq"), _i32(row_pos, "row_pos"), n,
                             _dev_ptr(k_re, "k_re", kdt, want), _dev_ptr(v_re, "v_re", kdt, want),
                             _dev_ptr(deviation, "deviation", torch.float64, n), _stream(stream))
    _check(st, "kv_token_deviation")
    return deviation


def kv_topk_select(values: torch.Tensor, seg_offsets: torch.Tensor, seg_k: torch.Tensor,
                   selected: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Ascending indices of each segment's seg_k largest values (see kvcache.h)."""
    n_seg = int(seg_k.numel())
    if int(seg_offsets.numel()) != n_seg + 1:
        raise ValueError("seg_offsets needs n_seg + 1 entries")
    if selected is None:
        selected = torch.full((int(values.numel()),), -1, dtype=torch.int32, device=values.device)
    st = _kv_topk_select(_dev_ptr(values, "values", torch.float64), _i32(seg_offsets, "seg_offsets"),
                         _i32(seg_k, "seg_k"), n_seg, _dev_ptr(selected, "selected", torch.int32, values.numel()),
                         _stream(stream))
    _check(st, "kv_topk_select")
    return selected


def kv_recompute_ratio(load_time: float, token_time: float, num_tokens: int, floor_ratio: float = 0.15) -> float:
    return float(_kv_recompute_ratio(float(load_time), float(token_time), int(num_tokens), float(floor_ratio)))


def kv_recompute_count(ratio: float, num_tokens: int) -> int:
    return int(_kv_recompute_count(float(ratio), int(num_tokens)))


def kv_validate_tables(desc: kv_pool_desc, block_tables, lens, appending: bool = True):
    """Host check of host copies (numpy int32 or CPU tensors). Returns
    (status, first bad row or -1)."""
    import numpy as np
    tab = np.ascontiguousarray(np.asarray(block_tables), dtype=np.int32)
    ln = np.ascontiguousarray(np.asarray(lens), dtype=np.int32)
    bad = _I32(-1)
    st = _kv_validate_tables(ctypes.byref(desc), tab.ctypes.data, int(tab.shape[1]), ln.ctypes.data,
                             int(ln.shape[0]), int(bool(appending)), ctypes.byref(bad))
    return int(st), int(bad.value)


def kv_read_probe(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, stream=None) -> None:
    """Read `buf` (a contiguous device tensor, a multiple of 4096 bytes) once:
    the read-ceiling measurement of kvcache.h."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(_kv_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), int(workgroups),
                          _dev_ptr(sink, "sink", torch.int32, 1), _stream(stream)), "kv_read_probe")


# raw entry points, for tests of the C ABI itself
raw = {
    "kv_pool_create": _kv_pool_create, "kv_pool_destroy": _kv_pool_destroy, "kv_pool_region": _kv_pool_region,
    "kv_append": _kv_append, "kv_append_tokens": _kv_append_tokens, "paged_decode_attention": _paged_decode_attention,
    "paged_decode_attention_workspace_bytes": _paged_decode_attention_workspace_bytes,
    "kv_quantize_int4": _kv_quantize_int4, "rope_rerotate": _rope_rerotate,
    "paged_multi_token_attention": _paged_multi_token_attention,
    "paged_multi_token_attention_workspace_bytes": _paged_multi_token_attention_workspace_bytes,
    "kv_block_bytes": _kv_block_bytes, "kv_copy_blocks": _kv_copy_blocks, "kv_gather_blocks": _kv_gather_blocks,
    "kv_scatter_blocks": _kv_scatter_blocks, "kv_token_deviation": _kv_token_deviation,
    "kv_topk_select": _kv_topk_select, "kv_decode_step": _kv_decode_step,
    "paged_decode_attention_shared": _paged_decode_attention_shared,
    "paged_decode_attention_shared_workspace_bytes": _paged_decode_attention_shared_workspace_bytes,
    "kv_validate_tables": _kv_validate_tables, "kv_read_probe": _kv_read_probe,
    "kv_decode_step_noalloc": _kv_decode_step_noalloc,
    "kv_layer_window": _kv_layer_window, "kv_window_released_blocks": _kv_window_released_blocks,
}
