"""CPU oracle for the paged-attention read path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``paged_kv_cache_96_amd``)
never does, and this package imports nothing from it.

The arithmetic lives in ``pa_oracle.c`` (plain C, OpenMP over independent
(request, kv head) units); this module builds it with gcc twice -- the fp32
two-pass reference (``precision="f32"``, the default) and the same steps in
fp64 (``precision="f64"``, the stricter check) -- and marshals numpy arrays.
``ledger.py`` models the page pool and per-request page lists on the write
side.

Every function takes plain arrays; ``*_of(inputs)`` helpers accept any object
with the attributes of ``workloads.PagedInputs`` (duck-typed, no import).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")          # fp64 build
_LIB32 = os.path.join(_HERE, "liboracle_f32.so")    # fp32 build (-DOR_SINGLE)
_FLAGS = {_LIB: (), _LIB32: ("-DOR_SINGLE",)}
PRECISIONS = {"f64": _LIB, "f32": _LIB32}

STATUS = {0: "ok", 1: "bad shape", 2: "page id out of range", 3: "bad context length",
          4: "bad query length", 5: "out of memory"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle rejected the inputs: {STATUS.get(code, code)} (code {code})")
        self.code = code


def compile_library(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle C source into a shared library (gcc, -O2, OpenMP)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Rebuild both oracle libraries (fp64 and fp32) unconditionally."""
    for path, flags in _FLAGS.items():
        compile_library(out=path, extra_flags=flags)
    return _LIB


def lib_for(precision: str) -> str:
    """Path of the oracle library of `precision` ("f32" or "f64")."""
    if precision not in PRECISIONS:
        raise ValueError(f"precision must be one of {sorted(PRECISIONS)}")
    return PRECISIONS[precision]


_lib_cache = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load the oracle library, building it first only if it is missing."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path not in _FLAGS:
            raise FileNotFoundError(path)
        compile_library(out=path, extra_flags=_FLAGS[path])
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i = ctypes.c_int
    d = ctypes.c_double
    common = [P, P, P, P, P, P, i, i, i, i, i, i, i, i, i, i, d, i, d, d]
    lib.or_attention.argtypes = common + [i, P, P]
    lib.or_attention.restype = i
    lib.or_partials.argtypes = common + [i, i, i, P, P]
    lib.or_partials.restype = i
    lib.or_merge.argtypes = [P, P, ctypes.c_long, i, i, P]
    lib.or_merge.restype = i
    lib.or_translate.argtypes = [P, P, i, i, i, i, P]
    lib.or_translate.restype = i
    lib.or_e4m3_values.argtypes = [P, ctypes.c_long, P]
    lib.or_e4m3_values.restype = i
    _lib_cache[path] = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


_DTYPE_CODES = {"f32": 0, "bf16": 1, "fp8_e4m3": 2}


class _Prepared:
    """Contiguous copies of the inputs with the dtypes the C code expects.
    `kv_dtype` (None: the pages share `dtype`) may be "fp8_e4m3": the pages
    then hold uint8 codes whose values are scaled by k_scale / v_scale."""

    def __init__(self, query, key_pages, value_pages, block_table, context_lens,
                 query_lens, page_size, dtype, causal, scale, kv_dtype=None, k_scale=1.0,
                 v_scale=1.0):
        fp = np.float32 if dtype == "f32" else np.uint16
        kv_dtype = kv_dtype or dtype
        if kv_dtype not in _DTYPE_CODES or dtype not in ("f32", "bf16"):
            raise ValueError(f"unsupported dtype {dtype!r} / kv_dtype {kv_dtype!r}")
        kfp = {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[kv_dtype]
        self.q = np.ascontiguousarray(query, dtype=fp)
        self.kp = np.ascontiguousarray(key_pages, dtype=kfp)
        self.vp = np.ascontiguousarray(value_pages, dtype=kfp)
        self.kv_code = _DTYPE_CODES[kv_dtype]
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.bt = np.ascontiguousarray(block_table, dtype=np.int32)
        self.cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        self.ql = None if query_lens is None else np.ascontiguousarray(query_lens, dtype=np.int32)
        B, Hq, L, D = self.q.shape
        P, Hkv, ps, D2 = self.kp.shape
        if D2 != D or ps != page_size or self.vp.shape != self.kp.shape:
            raise ValueError("shape mismatch between query and pages")
        if self.bt.ndim != 2 or self.bt.shape[0] != B or self.cl.shape != (B,):
            raise ValueError("block_table / context_lens shape mismatch")
        self.dims = (B, Hq, Hkv, L, D, P, ps, self.bt.shape[1])
        self.dtype_code = 0 if dtype == "f32" else 1
        self.causal = 1 if causal else 0
        self.scale = float(scale)

    def args(self):
        B, Hq, Hkv, L, D, P, ps, mp = self.dims
        return [_ptr(self.q), _ptr(self.kp), _ptr(self.vp), _ptr(self.bt), _ptr(self.cl),
                _ptr(self.ql), B, Hq, Hkv, L, D, P, ps, mp, self.dtype_code, self.causal,
                self.scale, self.kv_code, self.k_scale, self.v_scale]


def attention(query, key_pages, value_pages, block_table, context_lens, page_size, *,
              dtype: str, causal: bool, scale: float, query_lens=None,
              nthreads: Optional[int] = None, lib_path: Optional[str] = None,
              precision: str = "f32", return_threads: bool = False,
              kv_dtype: Optional[str] = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """Paged attention by the plain definition; float64 array [B, H_q, L, D]
    holding the results of the `precision` build (`lib_path` overrides it).
    kv_dtype "fp8_e4m3": uint8 pages dequantised with k_scale / v_scale."""
    lib_path = lib_path or lib_for(precision)
    prep = _Prepared(query, key_pages, value_pages, block_table, context_lens, query_lens,
                     page_size, dtype, causal, scale, kv_dtype, k_scale, v_scale)
    B, Hq, Hkv, L, D = prep.dims[:5]
    out = np.zeros((B, Hq, L, D), dtype=np.float64)
    used = ctypes.c_int(0)
    n = nthreads if nthreads is not None else default_threads()
    rc = load(lib_path).or_attention(*prep.args(), n, ctypes.byref(used), _ptr(out))
    if rc:
        raise OracleError(rc)
    return (out, used.value) if return_threads else out


def partials(query, key_pages, value_pages, block_table, context_lens, page_size, *,
             dtype: str, causal: bool, scale: float, partition_tokens: int, num_splits: int,
             query_lens=None, nthreads: Optional[int] = None,
             lib_path: Optional[str] = None, precision: str = "f32",
             kv_dtype: Optional[str] = None, k_scale: float = 1.0,
             v_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Per-partition (o, lse) states: [B,H_q,L,S,D] and [B,H_q,L,S] (float64
    arrays of the `precision` build's results)."""
    lib_path = lib_path or lib_for(precision)
    prep = _Prepared(query, key_pages, value_pages, block_table, context_lens, query_lens,
                     page_size, dtype, causal, scale, kv_dtype, k_scale, v_scale)
    B, Hq, Hkv, L, D = prep.dims[:5]
    S = int(num_splits)
    po = np.zeros((B, Hq, L, S, D), dtype=np.float64)
    pl = np.zeros((B, Hq, L, S), dtype=np.float64)
    n = nthreads if nthreads is not None else default_threads()
    rc = load(lib_path).or_partials(*prep.args(), int(partition_tokens), S, n, _ptr(po), _ptr(pl))
    if rc:
        raise OracleError(rc)
    return po, pl


def merge(part_o: np.ndarray, part_lse: np.ndarray, lib_path: Optional[str] = None,
          precision: str = "f32") -> np.ndarray:
    """Log-sum-exp merge of partition states over the second-to-last axis."""
    lib_path = lib_path or lib_for(precision)
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    S, D = po.shape[-2], po.shape[-1]
    rows = int(np.prod(po.shape[:-2]))
    if pl.shape != po.shape[:-1]:
        raise ValueError("part_lse must have the shape of part_o without its last axis")
    out = np.zeros(po.shape[:-2] + (D,), dtype=np.float64)
    load(lib_path).or_merge(_ptr(po), _ptr(pl), rows, S, D, _ptr(out))
    return out


def translate(block_table, context_lens, page_size: int, num_pages: int,
              lib_path: Optional[str] = None) -> np.ndarray:
    """(physical page, slot) of every logical key: int32 [B, max_pages*page_size, 2]."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, mp = bt.shape
    lib_path = lib_path or _LIB
    tr = np.zeros((B, mp * page_size, 2), dtype=np.int32)
    rc = load(lib_path).or_translate(_ptr(bt), _ptr(cl), B, mp, page_size, num_pages, _ptr(tr))
    if rc:
        raise OracleError(rc)
    return tr


def e4m3_values(codes, lib_path: Optional[str] = None) -> np.ndarray:
    """Values of fp8 E4M3 codes as the C oracle decodes them (float64)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(c.shape, dtype=np.float64)
    load(lib_path or _LIB).or_e4m3_values(_ptr(c), c.size, _ptr(out))
    return out


def _kw(x):
    kw = dict(dtype=x.dtype, causal=x.causal, scale=x.scale, query_lens=x.query_lens)
    if getattr(x, "kv_dtype", None):
        kw.update(kv_dtype=x.kv_dtype, k_scale=x.k_scale, v_scale=x.v_scale)
    return kw


def attention_of(x, **kw):
    """``attention`` on an object shaped like workloads.PagedInputs."""
    return attention(x.query, x.key_pages, x.value_pages, x.block_table, x.context_lens,
                     x.page_size, **_kw(x), **kw)


def partials_of(x, partition_tokens: int, num_splits: int, **kw):
    return partials(x.query, x.key_pages, x.value_pages, x.block_table, x.context_lens,
                    x.page_size, **_kw(x), partition_tokens=partition_tokens,
                    num_splits=num_splits, **kw)


def translate_of(x, **kw):
    return translate(x.block_table, x.context_lens, x.page_size, x.num_pages, **kw)
