"""The oracle: numpy-facing wrappers over ``kvoracle.c``.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It is independent
of the HIP library: it neither loads nor imports it, and the product never
imports this package.

Every function takes and returns host numpy arrays. bf16 data is carried as
``uint16`` bit patterns, fp16 scale/min as ``uint16`` bit patterns.
What each function computes, and which page passage it follows, is stated in
``kvoracle.c`` beside the C function of the same name.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvoracle.c")
# KVORACLE_LIB may name another build of kvoracle.c (used to check that the
# pins fail on a copy with a planted mistake).
_LIB = os.environ.get("KVORACLE_LIB", os.path.join(_HERE, "libkvoracle.so"))

F32, BF16, F64 = 0, 1, 3
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "f64": F64}


def build() -> str:
    """Compile kvoracle.c with gcc (IEEE arithmetic, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def _declare(L):
    L.kvo_kv_bytes.restype = _D
    L.kvo_kv_bytes.argtypes = [_D] * 5
    L.kvo_f32_to_bf16.restype = ctypes.c_uint16
    L.kvo_f32_to_bf16.argtypes = [ctypes.c_float]
    L.kvo_f32_to_f16.restype = ctypes.c_uint16
    L.kvo_f32_to_f16.argtypes = [ctypes.c_float]
    L.kvo_f16_to_f32.restype = ctypes.c_float
    L.kvo_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.kvo_append.restype = None
    L.kvo_append.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _I]
    L.kvo_attention.restype = _I
    L.kvo_attention.argtypes = [_I, _P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _I, _D, _I, _P]
    L.kvo_attention_multi.restype = _I
    L.kvo_attention_multi.argtypes = [_I, _P, _P, _I, _P, _P, _I, _P, _I, _I, _I, _I, _I, _D, _I, _P]
    L.kvo_q4_group_bf16.restype = None
    L.kvo_q4_group_bf16.argtypes = [_P, _I, _P, _P, _P]
    L.kvo_q4_group_f32.restype = None
    L.kvo_q4_group_f32.argtypes = [_P, _I, _P, _P, _P]
    L.kvo_q4_quantize_pool.restype = None
    L.kvo_q4_quantize_pool.argtypes = [_P, _P, _I, _I, _P, _I, _P, _P, _I] + [_P] * 7
    L.kvo_q4_append.restype = None
    L.kvo_q4_append.argtypes = [_P, _P, _I, _I, _P, _I, _P, _P, _I] + [_P] * 7
    L.kvo_q4_dequant.restype = None
    L.kvo_q4_dequant.argtypes = [_I, _I, _P, _I, _P, _P, _I] + [_P] * 9
    L.kvo_rope_rerotate.restype = None
    L.kvo_rope_rerotate.argtypes = [_I, _I, _I, _P, _P, _I, _I, _I, _D, _I]
    L.kvo_rope_rotate_f64.restype = None
    L.kvo_rope_rotate_f64.argtypes = [_P, _I, _D, _D, _I]
    for f in ("kvo_copy_blocks",):
        getattr(L, f).restype = None
        getattr(L, f).argtypes = [_I, _P, _P, _P, _P, _I]
    for f in ("kvo_gather_blocks", "kvo_scatter_blocks"):
        getattr(L, f).restype = None
        getattr(L, f).argtypes = [_I, _P, _P, _P, _I, _P]
    L.kvo_deviation.restype = None
    L.kvo_deviation.argtypes = [_I, _I, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P]
    L.kvo_topk.restype = None
    L.kvo_topk.argtypes = [_P, _I, _I, _P]
    L.kvo_recompute_ratio.restype = _D
    L.kvo_recompute_ratio.argtypes = [_D, _D, _I, _D]
    L.kvo_recompute_count.restype = _I
    L.kvo_recompute_count.argtypes = [_D, _I]
    L.kvo_layer_window.restype = _I
    L.kvo_layer_window.argtypes = [ctypes.c_void_p, _I, _I]
    L.kvo_window_released.restype = None
    L.kvo_window_released.argtypes = [ctypes.c_void_p, _I, _I, ctypes.c_void_p]
    L.kvo_set_threads.restype = None
    L.kvo_set_threads.argtypes = [_I]
    L.kvo_max_threads.restype = _I
    L.kvo_max_threads.argtypes = []


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported element type {a.dtype} (f32, bf16 bits as uint16, f64)")


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def kv_bytes(layers, tokens, d_h, n_kv, b) -> float:
    """M_KV = 2 L T (d_h n_kv) b (see kvo_kv_bytes)."""
    return lib().kvo_kv_bytes(layers, tokens, d_h, n_kv, b)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    f = lib().kvo_f32_to_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    f = lib().kvo_f32_to_f16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    f = lib().kvo_f16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# the hot path
# --------------------------------------------------------------------------

def append(K: np.ndarray, V: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
           tables: np.ndarray, seq_lens: np.ndarray) -> None:
    """In place: write k_new/v_new [B][n_kv][d] into their slots of the pool
    images K, V [nb][n_kv][16][d] (f32, or bf16 bits as uint16)."""
    assert K.dtype == V.dtype == k_new.dtype == v_new.dtype
    nb, n_kv, bs, d = K.shape
    tables = _i32(tables)
    seq_lens = _i32(seq_lens)
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    lib().kvo_append(K.itemsize, n_kv, d, _ptr(K), _ptr(V), _ptr(k_new), _ptr(v_new),
                     _ptr(tables), tables.shape[1], _ptr(seq_lens), len(seq_lens))


def attention(K: np.ndarray, V: np.ndarray, q: np.ndarray, tables: np.ndarray,
              ctx_lens: np.ndarray, scale: float, window: int = 0) -> np.ndarray:
    """fp64 decode attention through the block tables; returns [B][n_h][d] f64.

    K, V: [nb][n_kv][16][d] as f32, bf16 bits (uint16) or f64.
    q: [B][n_h][d] as f32 or bf16 bits.
    """
    nb, n_kv, bs, d = K.shape
    B, n_h, dq = q.shape
    assert dq == d and V.shape == K.shape and V.dtype == K.dtype
    tables = _i32(tables)
    ctx_lens = _i32(ctx_lens)
    q = np.ascontiguousarray(q)
    out = np.zeros((B, n_h, d), dtype=np.float64)
    rc = lib().kvo_attention(_dtype_of(K), _ptr(K), _ptr(V), _dtype_of(q), _ptr(q),
                             _ptr(tables), tables.shape[1], _ptr(ctx_lens), B,
                             n_h, n_kv, d, float(scale), int(window), _ptr(out))
    if rc != 0:
        raise ValueError("n_h must be a multiple of n_kv")
    return out


def attention_multi(K: np.ndarray, V: np.ndarray, q: np.ndarray, tables: np.ndarray,
                    ctx_lens: np.ndarray, scale: float, window: int = 0) -> np.ndarray:
    """Several query tokens per sequence, causal among themselves.
    q: [B][q_len][n_h][d]; returns [B][q_len][n_h][d] f64."""
    nb, n_kv, bs, d = K.shape
    B, q_len, n_h, dq = q.shape
    assert dq == d and V.shape == K.shape and V.dtype == K.dtype
    tables = _i32(tables)
    ctx_lens = _i32(ctx_lens)
    q = np.ascontiguousarray(q)
    out = np.zeros((B, q_len, n_h, d), dtype=np.float64)
    rc = lib().kvo_attention_multi(_dtype_of(K), _ptr(K), _ptr(V), _dtype_of(q), _ptr(q), _ptr(tables),
                                   tables.shape[1], _ptr(ctx_lens), B, q_len, n_h, n_kv, d, float(scale),
                                   int(window), _ptr(out))
    if rc != 0:
        raise ValueError("n_h must be a multiple of n_kv and q_len >= 1")
    return out


def q4_group(x: np.ndarray):
    """Quantize one group; x as f32 or bf16 bits. Returns (codes u8, s16, m16)."""
    x = np.ascontiguousarray(x)
    codes = np.zeros(len(x), dtype=np.uint8)
    s = ctypes.c_uint16()
    m = ctypes.c_uint16()
    if x.dtype == np.uint16:
        lib().kvo_q4_group_bf16(_ptr(x), len(x), _ptr(codes), ctypes.addressof(s), ctypes.addressof(m))
    else:
        x = x.astype(np.float32)
        lib().kvo_q4_group_f32(_ptr(x), len(x), _ptr(codes), ctypes.addressof(s), ctypes.addressof(m))
    return codes, s.value, m.value


class Q4Image:
    """Host INT4 pool image in the layout of kvoracle.c."""

    def __init__(self, num_blocks: int, n_kv: int, d: int, max_seqs: int):
        self.nb, self.n_kv, self.d, self.max_seqs = num_blocks, n_kv, d, max_seqs
        self.kq = np.zeros((num_blocks, n_kv, 16, d // 2), dtype=np.uint8)
        self.ks = np.zeros((num_blocks, n_kv, d), dtype=np.uint16)
        self.km = np.zeros((num_blocks, n_kv, d), dtype=np.uint16)
        self.vq = np.zeros((num_blocks, n_kv, 16, d // 2), dtype=np.uint8)
        self.vs = np.zeros((num_blocks, n_kv, 16), dtype=np.uint16)
        self.vm = np.zeros((num_blocks, n_kv, 16), dtype=np.uint16)
        self.kt = np.zeros((max_seqs, n_kv, 16, d), dtype=np.uint16)

    def arrays(self):
        return [self.kq, self.ks, self.km, self.vq, self.vs, self.vm, self.kt]

    def copy(self) -> "Q4Image":
        c = Q4Image.__new__(Q4Image)
        c.nb, c.n_kv, c.d, c.max_seqs = self.nb, self.n_kv, self.d, self.max_seqs
        c.kq, c.ks, c.km, c.vq, c.vs, c.vm, c.kt = [a.copy() for a in self.arrays()]
        return c


def q4_quantize_pool(img: Q4Image, Kb: np.ndarray, Vb: np.ndarray, tables, lens, slots=None) -> None:
    tables = _i32(tables)
    lens = _i32(lens)
    slots = None if slots is None else _i32(slots)
    lib().kvo_q4_quantize_pool(_ptr(np.ascontiguousarray(Kb)), _ptr(np.ascontiguousarray(Vb)),
                               img.n_kv, img.d, _ptr(tables), tables.shape[1], _ptr(lens),
                               _ptr(slots), len(lens), *[_ptr(a) for a in img.arrays()])


def q4_append(img: Q4Image, k_new: np.ndarray, v_new: np.ndarray, tables, seq_lens, slots=None) -> None:
    tables = _i32(tables)
    seq_lens = _i32(seq_lens)
    slots = None if slots is None else _i32(slots)
    lib().kvo_q4_append(_ptr(np.ascontiguousarray(k_new)), _ptr(np.ascontiguousarray(v_new)),
                        img.n_kv, img.d, _ptr(tables), tables.shape[1], _ptr(seq_lens),
                        _ptr(slots), len(seq_lens), *[_ptr(a) for a in img.arrays()])


def q4_dequant(img: Q4Image, tables, ctx_lens, slots=None):
    """Returns fp64 pool images (Kd, Vd) holding what attention reads
    (other entries are 0)."""
    tables = _i32(tables)
    ctx_lens = _i32(ctx_lens)
    slots = None if slots is None else _i32(slots)
    Kd = np.zeros((img.nb, img.n_kv, 16, img.d), dtype=np.float64)
    Vd = np.zeros_like(Kd)
    lib().kvo_q4_dequant(img.n_kv, img.d, _ptr(tables), tables.shape[1], _ptr(ctx_lens),
                         _ptr(slots), len(ctx_lens), *[_ptr(a) for a in img.arrays()],
                         _ptr(Kd), _ptr(Vd))
    return Kd, Vd


def rope_rerotate(K: np.ndarray, chunk_blocks, first_slot: int, num_tokens: int,
                  delta: int, base: float, style: int = 0) -> None:
    """In place on a K pool image (f32, or bf16 bits as uint16)."""
    nb, n_kv, bs, d = K.shape
    chunk_blocks = _i32(chunk_blocks)
    lib().kvo_rope_rerotate(_dtype_of(K), n_kv, d, _ptr(K), _ptr(chunk_blocks), int(first_slot),
                            int(num_tokens), int(delta), float(base), int(style))


def rope_rotate_f64(x: np.ndarray, delta: float, base: float, style: int = 0) -> np.ndarray:
    y = np.array(x, dtype=np.float64, copy=True)
    lib().kvo_rope_rotate_f64(_ptr(y), len(y), float(delta), float(base), int(style))
    return y


def _regions(arrays):
    """Per-block regions: each array's first axis is the block id."""
    arrs = [np.ascontiguousarray(a) for a in arrays]
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    sizes = (ctypes.c_size_t * len(arrs))(*[a.nbytes // a.shape[0] for a in arrs])
    return arrs, ptrs, sizes


def copy_blocks(arrays, src, dst) -> None:
    """In place on the given region arrays (all C-contiguous, block-major)."""
    arrs, ptrs, sizes = _regions(arrays)
    assert all(a is b for a, b in zip(arrs, arrays)), "region arrays must be C-contiguous"
    src, dst = _i32(src), _i32(dst)
    lib().kvo_copy_blocks(len(arrs), ptrs, sizes, _ptr(src), _ptr(dst), len(src))


def gather_blocks(arrays, blocks) -> np.ndarray:
    arrs, ptrs, sizes = _regions(arrays)
    blocks = _i32(blocks)
    out = np.zeros(len(blocks) * sum(sizes), dtype=np.uint8)
    lib().kvo_gather_blocks(len(arrs), ptrs, sizes, _ptr(blocks), len(blocks), _ptr(out))
    return out


def scatter_blocks(arrays, blocks, buffer: np.ndarray) -> None:
    arrs, ptrs, sizes = _regions(arrays)
    assert all(a is b for a, b in zip(arrs, arrays)), "region arrays must be C-contiguous"
    blocks = _i32(blocks)
    buffer = np.ascontiguousarray(buffer, dtype=np.uint8)
    lib().kvo_scatter_blocks(len(arrs), ptrs, sizes, _ptr(blocks), len(blocks), _ptr(buffer))


def deviation(K: np.ndarray, V: np.ndarray, tables, row_seq, row_pos, k_re: np.ndarray,
              v_re: np.ndarray) -> np.ndarray:
    """fp64 squared KV deviation of row i of k_re / v_re ([rows][n_kv][d])
    from the cached KV of token row_pos[i] of sequence row_seq[i]."""
    nb, n_kv, bs, d = K.shape
    tables = _i32(tables)
    rs, rp = _i32(row_seq), _i32(row_pos)
    k_re, v_re = np.ascontiguousarray(k_re), np.ascontiguousarray(v_re)
    assert k_re.dtype == K.dtype == v_re.dtype == V.dtype
    assert len(rs) == len(rp) == k_re.shape[0] == v_re.shape[0]
    out = np.zeros(k_re.shape[0], dtype=np.float64)
    lib().kvo_deviation(_dtype_of(K), n_kv, d, _ptr(K), _ptr(V), _ptr(tables), tables.shape[-1], _ptr(rs), _ptr(rp),
                        k_re.shape[0], _ptr(k_re), _ptr(v_re), _ptr(out))
    return out


def topk(values: np.ndarray, k: int) -> np.ndarray:
    """Rows of the k largest values (ties: lower row), in ascending order."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.zeros(min(k, len(v)), dtype=np.int32)
    lib().kvo_topk(_ptr(v), len(v), int(k), _ptr(out))
    return out


def recompute_ratio(load_time: float, token_time: float, num_tokens: int, floor_ratio: float = 0.15) -> float:
    return lib().kvo_recompute_ratio(float(load_time), float(token_time), int(num_tokens), float(floor_ratio))


def recompute_count(ratio: float, num_tokens: int) -> int:
    return lib().kvo_recompute_count(float(ratio), int(num_tokens))


def layer_window(windows, layer: int) -> int:
    """Window of a 0-based layer from a per-layer list repeated cyclically."""
    w = np.ascontiguousarray(windows, dtype=np.int32)
    return lib().kvo_layer_window(_ptr(w), len(w), int(layer))


def window_released(lens, window: int) -> np.ndarray:
    """Per sequence, the leading blocks no later query attends (-1: negative length)."""
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros(len(ln), dtype=np.int32)
    lib().kvo_window_released(_ptr(ln), len(ln), int(window), _ptr(out))
    return out


def set_threads(n: int) -> None:
    lib().kvo_set_threads(int(n))


def max_threads() -> int:
    return lib().kvo_max_threads()
