"""CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``liboracle.so`` (plain C, double
precision), built from ``oracle.c`` by ``oracle/build.py``; ``oracle.c`` says
what each function computes and which passage of the pages it follows.

Every function takes host numpy arrays: fp16 tensors as ``np.float16`` (their
bit patterns are what the C code reads) and int32 tables; results are float64.
``Oracle(path)`` loads another build of the same source (the tests load
copies with deliberately planted mistakes to show that the pins catch them).
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "liboracle.so"
# another build of oracle.c (e.g. with sanitizers) for get()
LIB_ENV = "PKV_ORACLE_LIB"
SOURCE_PATH = _HERE / "oracle.c"

_ERRORS = {1: "bad argument", 2: "slot or block id out of range",
           3: "duplicate slot or destination block", 4: "out of memory"}


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


class OracleError(ValueError):
    pass


class Oracle:
    def __init__(self, path: str | Path = LIB_PATH):
        path = Path(path)
        if not path.exists():
            if path == LIB_PATH:
                from .build import build
                build()
            else:
                raise FileNotFoundError(path)
        lib = ctypes.CDLL(str(path))
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = D
        lib.oracle_kv_append.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [P, P, P, P, P, I32, P, I32, I32, I32, I32,
                                      I32, I32, D, P, I64]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [P, P, P, P, P, P, I32, P, I32, I32, I32,
                                       I32, I32, I32, D, P, I64]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_copy_blocks.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32]
        lib.oracle_copy_blocks.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(rc: int, what: str):
        if rc:
            raise OracleError(f"oracle {what}: {_ERRORS.get(rc, rc)}")

    def set_threads(self, n: int):
        """Threads of the oracle's OpenMP loops; n <= 0 restores the default."""
        self.lib.oracle_set_threads(int(n))

    def half_to_double(self, bits: int) -> float:
        return self.lib.oracle_half_to_double(int(bits) & 0xFFFF)

    def kv_append(self, key, value, k_cache, v_cache, slot_mapping):
        """Writes new rows into copies of the pools; returns (k_cache, v_cache)."""
        kc = np.array(k_cache, dtype=np.float16, copy=True, order="C")
        vc = np.array(v_cache, dtype=np.float16, copy=True, order="C")
        self.kv_append_inplace(key, value, kc, vc, slot_mapping)
        return kc, vc

    def kv_append_inplace(self, key, value, k_cache, v_cache, slot_mapping):
        """Writes new rows into the given pools (C-contiguous float16 arrays,
        modified in place)."""
        key, value = _c(key, np.float16), _c(value, np.float16)
        for a in (k_cache, v_cache):
            if not (isinstance(a, np.ndarray) and a.dtype == np.float16
                    and a.flags.c_contiguous and a.flags.writeable):
                raise TypeError("pools must be writeable C-contiguous float16 arrays")
        slot = _c(slot_mapping, np.int32)
        NB, Hkv, bs, D = k_cache.shape
        T = slot.shape[0]
        if v_cache.shape != k_cache.shape:
            raise ValueError("k_cache and v_cache shapes differ")
        if key.shape != (T, Hkv, D) or value.shape != (T, Hkv, D):
            raise ValueError("key/value shape")
        rc = self.lib.oracle_kv_append(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(slot), T, Hkv, D, bs, NB)
        self._check(rc, "kv_append")

    def decode(self, q, k_cache, v_cache, block_tables, seq_lens, scale, rows=None):
        """out[s, h, :]; with ``rows`` (ids s*Hq+h) only those rows are
        computed and the others are NaN."""
        q = _c(q, np.float16)
        kc, vc = _c(k_cache, np.float16), _c(v_cache, np.float16)
        bt, sl = _c(block_tables, np.int32), _c(seq_lens, np.int32)
        S, Hq, D = q.shape
        NB, Hkv, bs, D2 = kc.shape
        if D2 != D or bt.shape[0] != S or sl.shape != (S,):
            raise ValueError("shape mismatch")
        out = np.full((S, Hq, D), np.nan, dtype=np.float64)
        rp, nr = None, 0
        if rows is not None:
            rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
            rp, nr = _ptr(rows), rows.shape[0]
        rc = self.lib.oracle_decode(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt),
                                    bt.shape[1], _ptr(sl), S, Hq, Hkv, D, bs, NB,
                                    float(scale), rp, nr)
        self._check(rc, "decode")
        return out

    def prefill(self, q, cu_q_lens, k_cache, v_cache, block_tables, seq_lens,
                scale, rows=None):
        """out[token, h, :] for packed chunk rows; ``rows`` = ids token*Hq+h."""
        q = _c(q, np.float16)
        cu = _c(cu_q_lens, np.int32)
        kc, vc = _c(k_cache, np.float16), _c(v_cache, np.float16)
        bt, sl = _c(block_tables, np.int32), _c(seq_lens, np.int32)
        T, Hq, D = q.shape
        NB, Hkv, bs, D2 = kc.shape
        C = sl.shape[0]
        if D2 != D or cu.shape != (C + 1,) or int(cu[-1]) != T or bt.shape[0] != C:
            raise ValueError("shape mismatch")
        out = np.full((T, Hq, D), np.nan, dtype=np.float64)
        rp, nr = None, 0
        if rows is not None:
            rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
            rp, nr = _ptr(rows), rows.shape[0]
        rc = self.lib.oracle_prefill(_ptr(out), _ptr(q), _ptr(cu), _ptr(kc), _ptr(vc),
                                     _ptr(bt), bt.shape[1], _ptr(sl), C, Hq, Hkv, D,
                                     bs, NB, float(scale), rp, nr)
        self._check(rc, "prefill")
        return out


    def copy_blocks(self, src_k, src_v, dst_k, dst_v, src_blocks, dst_blocks):
        """Copies of the destination pools with block src_blocks[i] of the
        source pools written to block dst_blocks[i]; returns (dst_k, dst_v)."""
        sk, sv = _c(src_k, np.float16), _c(src_v, np.float16)
        dk = np.array(dst_k, dtype=np.float16, copy=True, order="C")
        dv = np.array(dst_v, dtype=np.float16, copy=True, order="C")
        s, d = _c(src_blocks, np.int32), _c(dst_blocks, np.int32)
        sNB, Hkv, bs, D = sk.shape
        dNB = dk.shape[0]
        if sv.shape != sk.shape or dv.shape != dk.shape or dk.shape[1:] != sk.shape[1:] \
                or s.shape != d.shape or s.ndim != 1:
            raise ValueError("shape mismatch")
        rc = self.lib.oracle_copy_blocks(_ptr(sk), _ptr(sv), _ptr(dk), _ptr(dv), _ptr(s),
                                         _ptr(d), s.shape[0], Hkv, D, bs, sNB, dNB)
        self._check(rc, "copy_blocks")
        return dk, dv


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from oracle.c, or the build $PKV_ORACLE_LIB names."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get(LIB_ENV) or LIB_PATH)
    return _default


def half_to_double(bits):
    return get().half_to_double(bits)


def kv_append(*a, **k):
    return get().kv_append(*a, **k)


def decode(*a, **k):
    return get().decode(*a, **k)


def prefill(*a, **k):
    return get().prefill(*a, **k)


def copy_blocks(*a, **k):
    return get().copy_blocks(*a, **k)
