"""fp64 CPU oracle for the attention forward pass (Python wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may use this package; the GPU library and its Python
binding never import it.

The arithmetic lives in ``fa_oracle.c`` (plain C, fp64, built with gcc); this
module only compiles it, loads it and passes numpy buffers to it.  What the C
code computes is the plain definition of attention: S = scale * Q K^T, with
the causal mask excluding key j from query i when j > i, P = softmax(S) along
each row, O = P V ("Android Transformer Optimization: Attention and Mobile GPU
Bottlenecks", section "The Self-Attention Bottleneck Is Memory Traffic, Not
Compute"; scale as in "Flash Attention on Android: tiled SGEMM with
RenderScript", section "Architecture: tiled attention with RenderScript
BLAS").
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
_BITS = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}

def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile fa_oracle.c into a shared library with gcc (-O2, OpenMP, no
    fast-math).  src/out may name another copy of the source (the mutation
    tests build deliberately broken copies in a temporary folder)."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _prep(t, dtype):
    want = _BITS[dtype]
    t = np.ascontiguousarray(t)
    if t.dtype != want:
        raise TypeError(f"{dtype} input must be a {np.dtype(want).name} bit array, got {t.dtype}")
    return t


def _check(q, k, v, dtype):
    if dtype not in DTYPE_CODES:
        raise ValueError(f"unknown storage type {dtype!r}")
    q, k, v = (_prep(t, dtype) for t in (q, k, v))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, D] shape")
    return q, k, v


class Oracle:
    """A loaded build of fa_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.fa_oracle_forward.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                          ctypes.c_double, ctypes.c_int, vp, vp, vp, ctypes.c_int]
        lib.fa_oracle_forward.restype = ctypes.c_int
        lib.fa_oracle_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                       ctypes.c_double, ctypes.c_int, vp, vp, i64, vp, vp,
                                       ctypes.c_int]
        lib.fa_oracle_rows.restype = ctypes.c_int
        for name, arg in (("f16", ctypes.c_uint16), ("bf16", ctypes.c_uint16),
                          ("f32", ctypes.c_uint32)):
            f = getattr(lib, "fa_oracle_decode_" + name)
            f.argtypes = [arg]
            f.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    def decode(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """Storage bits -> exact fp64 values, by the oracle's own decoders."""
        flat = np.ascontiguousarray(bits).reshape(-1)
        if dtype == "f32":
            flat = flat.view(np.uint32)
        f = getattr(self.lib, "fa_oracle_decode_" + dtype)
        out = np.fromiter((f(int(x)) for x in flat), dtype=np.float64, count=flat.size)
        return out.reshape(np.shape(bits))

    def forward(self, q, k, v, dtype: str, scale: float, causal: bool, nthreads: int = 0,
                return_rowsum: bool = False, return_lse: bool = False):
        """O = softmax(scale * Q K^T [+ causal mask]) V for every (b, h), in fp64.

        q, k, v: [B, H, N, D] storage-bit arrays.  Returns O (fp64,
        [B, H, N, D]); with return_rowsum also the sum of each P row
        ([B, H, N]) and the number of threads used; with return_lse (and not
        return_rowsum) (O, lse) where lse [B, H, N] is the log-sum-exp of each
        row of scale * Q K^T over its visible keys."""
        q, k, v = _check(q, k, v, dtype)
        B, H, N, D = q.shape
        o = np.empty((B, H, N, D), dtype=np.float64)
        rs = np.empty((B, H, N), dtype=np.float64) if return_rowsum else None
        lse = np.empty((B, H, N), dtype=np.float64) if return_lse else None
        used = self.lib.fa_oracle_forward(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                          DTYPE_CODES[dtype], B, H, N, D, float(scale),
                                          int(bool(causal)), o.ctypes.data,
                                          rs.ctypes.data if rs is not None else None,
                                          lse.ctypes.data if lse is not None else None,
                                          int(nthreads))
        if used < 0:
            raise RuntimeError("oracle rejected its arguments")
        if return_rowsum:
            return (o, rs, used, lse) if return_lse else (o, rs, used)
        if return_lse:
            return o, lse
        return o

    def rows(self, q, k, v, dtype: str, scale: float, causal: bool, bh_idx, row_idx,
             nthreads: int = 0, return_threads: bool = False, return_lse: bool = False):
        """Selected output rows: row r is query row_idx[r] of flattened head
        bh_idx[r] (= b*H + h).  Returns an [nrows, D] fp64 array (with
        return_lse, also the rows' log-sum-exp, [nrows])."""
        q, k, v = _check(q, k, v, dtype)
        B, H, N, D = q.shape
        bh = np.ascontiguousarray(bh_idx, dtype=np.int64).reshape(-1)
        ri = np.ascontiguousarray(row_idx, dtype=np.int64).reshape(-1)
        if bh.size != ri.size:
            raise ValueError("bh_idx and row_idx must have the same length")
        # Group rows by head so each worker decodes a head's K and V once.
        order = np.lexsort((ri, bh))
        bh_sorted = np.ascontiguousarray(bh[order])
        ri_sorted = np.ascontiguousarray(ri[order])
        out_sorted = np.empty((bh.size, D), dtype=np.float64)
        lse_sorted = np.empty(bh.size, dtype=np.float64)
        used = self.lib.fa_oracle_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                       DTYPE_CODES[dtype], B, H, N, D, float(scale),
                                       int(bool(causal)), bh_sorted.ctypes.data,
                                       ri_sorted.ctypes.data, bh.size, out_sorted.ctypes.data,
                                       lse_sorted.ctypes.data, int(nthreads))
        if used < 0:
            raise RuntimeError("oracle rejected its arguments")
        out = np.empty_like(out_sorted)
        out[order] = out_sorted
        lse = np.empty_like(lse_sorted)
        lse[order] = lse_sorted
        if return_lse:
            return (out, lse, used) if return_threads else (out, lse)
        return (out, used) if return_threads else out


_default = None


def load() -> Oracle:
    """The oracle built from this folder's source (built on first use if no
    build exists yet)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def decode(bits, dtype):
    return load().decode(bits, dtype)


def forward(q, k, v, dtype, scale, causal, nthreads=0, return_rowsum=False, return_lse=False):
    return load().forward(q, k, v, dtype, scale, causal, nthreads, return_rowsum, return_lse)


def rows(q, k, v, dtype, scale, causal, bh_idx, row_idx, nthreads=0, return_threads=False,
         return_lse=False):
    return load().rows(q, k, v, dtype, scale, causal, bh_idx, row_idx, nthreads, return_threads,
                       return_lse)
