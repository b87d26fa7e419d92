"""Plain CPU oracle for paged decode attention (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library and never imports it.

  oracle.c          binary64 decode attention through block tables, the slot
                    scatter (reshape_and_cache), the whole-block copy
                    (copy_blocks) and the block move between two pools
                    (swap_blocks); the same for pools of OCP E4M3 codes with a
                    scale per (block, KV head) (decode_fp8, reshape_and_cache_fp8,
                    fp8_value, fp8_encode); causal attention of several query
                    tokens per sequence (multi_query); built here with gcc,
                    single-threaded.
  alloc_model.py    the block allocator (free list, reference counts, fork,
                    append with copy-on-write, free) in plain Python.
  place.py          helpers that build pools and tables with the model allocator
                    and the oracle's scatter/copy, for a workload batch.

Sources: the four pages on vLLM's PagedAttention — "PagedAttention" concept
report (compassingai.com) §5 (block table, base + offset addressing), §6
(reference counts, copy-on-write), §8 (dot product, softmax, weighted sum of
values; outer loop over blocks, inner over tokens), §11 (free list); "vLLM
PagedAttention 技术深度解析" (kwkr.cn) §1.2.2 (allocation flow) and §1.3.2
(sharing); the KV-cache/paging tutorial (wmrh.cn) "KV cache" and "paged
attention" parts (newest token's K/V computed at the step; shared blocks with
reference counts 2 and 3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
_STATUS = {0: "ok", 1: "bad argument", 2: "index out of range", 3: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(mutant: int = 0, out: Optional[str] = None) -> str:
    """Compile oracle.c with gcc (-O2, strict IEEE, no fast-math). Returns the path."""
    out = out or _LIB
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-lm", "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _needs_build(path: str) -> bool:
    return not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Optional[str] = None):
        # ORACLE_LIBRARY: another build of oracle.c (the sanitizer build of the tests)
        path = path or os.environ.get("ORACLE_LIBRARY") or _LIB
        if path == _LIB and _needs_build(path):
            build()
        self._lib = ctypes.CDLL(path)
        vp, i32p, dp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
        ci, cd = ctypes.c_int, ctypes.c_double
        self._lib.oracle_decode.argtypes = [dp, vp, vp, vp, i32p, ci, i32p, ci, ci, ci, ci, ci, ci, cd, ci]
        self._lib.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, i32p, ci, ci, ci, ci, ci, ci]
        self._lib.oracle_copy_blocks.argtypes = [vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci]
        self._lib.oracle_swap_blocks.argtypes = [vp, vp, vp, vp, i32p, i32p, ci, ci, ci, ci, ci, ci,
                                                 ci]
        self._lib.oracle_load.argtypes = [vp, ctypes.c_int64, ci]
        self._lib.oracle_load.restype = cd
        fp = ctypes.POINTER(ctypes.c_float)
        self._lib.oracle_decode_fp8.argtypes = [dp, vp, vp, vp, fp, fp, i32p, ci, i32p, ci, ci, ci,
                                                ci, ci, ci, cd, ci]
        self._lib.oracle_reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, fp, fp, i32p, ci, ci,
                                                           ci, ci, ci, ci]
        self._lib.oracle_multi_query.argtypes = [dp, vp, vp, vp, i32p, ci, i32p, i32p, ci, ci, ci, ci,
                                                 ci, ci, cd, ci]
        self._lib.oracle_multi_query.restype = ctypes.c_int
        self._lib.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        self._lib.oracle_fp8_value.restype = cd
        self._lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
        self._lib.oracle_fp8_encode.restype = ctypes.c_uint8
        for f in ("oracle_decode", "oracle_reshape_and_cache", "oracle_copy_blocks",
                  "oracle_swap_blocks", "oracle_decode_fp8", "oracle_reshape_and_cache_fp8"):
            getattr(self._lib, f).restype = ctypes.c_int

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError(f"{what}: {_STATUS.get(rc, rc)}")

    @staticmethod
    def _i32(a) -> np.ndarray:
        return np.ascontiguousarray(a, dtype=np.int32)

    def load(self, arr: np.ndarray, dtype: str) -> np.ndarray:
        """Decode stored values to float64 with the oracle's own decoder."""
        a = np.ascontiguousarray(arr)
        out = np.empty(a.size, np.float64)
        for i in range(a.size):
            out[i] = self._lib.oracle_load(a.ctypes.data, i, DTYPE_CODE[dtype])
        return out.reshape(a.shape)

    def decode(self, query, key_cache, value_cache, block_tables, context_lens, scale: float,
               dtype: str, num_kv_heads: Optional[int] = None) -> np.ndarray:
        """out[S][H_q][d] in float64.  Pools are [num_blocks][H_kv][B][d]."""
        q = np.ascontiguousarray(query)
        kc = np.ascontiguousarray(key_cache)
        vc = np.ascontiguousarray(value_cache)
        bt = self._i32(block_tables)
        cl = self._i32(context_lens)
        S, Hq, d = q.shape
        nb, Hkv, B, d2 = kc.shape
        assert d2 == d and vc.shape == kc.shape and bt.shape[0] == S and cl.shape == (S,)
        if num_kv_heads is not None:
            assert num_kv_heads == Hkv
        out = np.zeros((S, Hq, d), np.float64)
        rc = self._lib.oracle_decode(
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), q.ctypes.data, kc.ctypes.data,
            vc.ctypes.data, bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), bt.shape[1],
            cl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), S, Hq, Hkv, d, B, nb, float(scale),
            DTYPE_CODE[dtype])
        self._check(rc, "oracle_decode")
        return out

    @staticmethod
    def _f32(a) -> np.ndarray:
        return np.ascontiguousarray(a, dtype=np.float32)

    def fp8_value(self, codes) -> np.ndarray:
        """E4M3 codes (uint8) -> float64 values."""
        c = np.asarray(codes, np.uint8)
        return np.array([self._lib.oracle_fp8_value(int(x)) for x in c.ravel()],
                        np.float64).reshape(c.shape)

    def fp8_encode(self, y) -> np.ndarray:
        """float32 numbers -> nearest E4M3 codes (ties to even, saturating)."""
        y = np.asarray(y, np.float32)
        return np.array([self._lib.oracle_fp8_encode(float(x)) for x in y.ravel()],
                        np.uint8).reshape(y.shape)

    def decode_fp8(self, query, key_cache, value_cache, k_scales, v_scales, block_tables,
                   context_lens, scale: float, qdtype: str) -> np.ndarray:
        """Decode over E4M3 pools (uint8 [num_blocks][H_kv][B][d]) with float32 scales
        [num_blocks][H_kv]; query f16 / bf16 [S][H_q][d].  Returns float64."""
        q = np.ascontiguousarray(query)
        kc = np.ascontiguousarray(key_cache, dtype=np.uint8)
        vc = np.ascontiguousarray(value_cache, dtype=np.uint8)
        ks, vs = self._f32(k_scales), self._f32(v_scales)
        bt = self._i32(block_tables)
        cl = self._i32(context_lens)
        S, Hq, d = q.shape
        nb, Hkv, B, d2 = kc.shape
        assert d2 == d and vc.shape == kc.shape and ks.shape == (nb, Hkv) and vs.shape == ks.shape
        out = np.zeros((S, Hq, d), np.float64)
        fp = ctypes.POINTER(ctypes.c_float)
        rc = self._lib.oracle_decode_fp8(
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), q.ctypes.data, kc.ctypes.data,
            vc.ctypes.data, ks.ctypes.data_as(fp), vs.ctypes.data_as(fp),
            bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), bt.shape[1],
            cl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), S, Hq, Hkv, d, B, nb, float(scale),
            DTYPE_CODE[qdtype])
        self._check(rc, "oracle_decode_fp8")
        return out

    def reshape_and_cache_fp8(self, key, value, key_cache, value_cache, k_scales, v_scales,
                              slot_mapping, src_dtype: str):
        """In-place scatter of key/value [N][H_kv][d] (src_dtype) into E4M3 pools."""
        k = np.ascontiguousarray(key)
        v = np.ascontiguousarray(value)
        sm = self._i32(slot_mapping)
        assert key_cache.dtype == np.uint8 and value_cache.dtype == np.uint8
        assert key_cache.flags.c_contiguous and value_cache.flags.c_contiguous
        ks, vs = self._f32(k_scales), self._f32(v_scales)
        nb, Hkv, B, d = key_cache.shape
        N = sm.shape[0]
        assert k.shape == (N, Hkv, d) and v.shape == k.shape and ks.shape == (nb, Hkv)
        fp = ctypes.POINTER(ctypes.c_float)
        rc = self._lib.oracle_reshape_and_cache_fp8(
            k.ctypes.data, v.ctypes.data, key_cache.ctypes.data, value_cache.ctypes.data,
            ks.ctypes.data_as(fp), vs.ctypes.data_as(fp),
            sm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), N, Hkv, d, B, nb,
            DTYPE_CODE[src_dtype])
        self._check(rc, "oracle_reshape_and_cache_fp8")

    def multi_query(self, query, key_cache, value_cache, block_tables, context_lens, query_start,
                    scale: float, dtype: str) -> np.ndarray:
        """Causal attention of several query tokens per sequence (the last n_s positions
        of each context).  query [T][H_q][d], query_start int32 [S+1].  Returns float64."""
        q = np.ascontiguousarray(query)
        kc = np.ascontiguousarray(key_cache)
        vc = np.ascontiguousarray(value_cache)
        bt, cl, qs = self._i32(block_tables), self._i32(context_lens), self._i32(query_start)
        T, Hq, d = q.shape
        nb, Hkv, B, d2 = kc.shape
        S = cl.shape[0]
        assert d2 == d and vc.shape == kc.shape and qs.shape == (S + 1,) and qs[-1] == T
        out = np.zeros((T, Hq, d), np.float64)
        p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        rc = self._lib.oracle_multi_query(
            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), q.ctypes.data, kc.ctypes.data,
            vc.ctypes.data, p32(bt), bt.shape[1], p32(cl), p32(qs), S, Hq, Hkv, d, B, nb,
            float(scale), DTYPE_CODE[dtype])
        self._check(rc, "oracle_multi_query")
        return out

    def reshape_and_cache(self, key, value, key_cache, value_cache, slot_mapping, dtype: str):
        """In-place scatter of key/value [N][H_kv][d] into the pools."""
        k = np.ascontiguousarray(key)
        v = np.ascontiguousarray(value)
        sm = self._i32(slot_mapping)
        assert key_cache.flags.c_contiguous and value_cache.flags.c_contiguous
        nb, Hkv, B, d = key_cache.shape
        N = sm.shape[0]
        assert k.shape == (N, Hkv, d) and v.shape == k.shape
        rc = self._lib.oracle_reshape_and_cache(
            k.ctypes.data, v.ctypes.data, key_cache.ctypes.data, value_cache.ctypes.data,
            sm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), N, Hkv, d, B, nb, DTYPE_CODE[dtype])
        self._check(rc, "oracle_reshape_and_cache")

    def copy_blocks(self, key_cache, value_cache, src, dst, dtype: str):
        """In-place whole-block copies src[i] -> dst[i] in both pools."""
        s = self._i32(src)
        t = self._i32(dst)
        assert key_cache.flags.c_contiguous and value_cache.flags.c_contiguous
        nb, Hkv, B, d = key_cache.shape
        rc = self._lib.oracle_copy_blocks(
            key_cache.ctypes.data, value_cache.ctypes.data,
            s.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(s), Hkv, d, B, nb,
            DTYPE_CODE[dtype])
        self._check(rc, "oracle_copy_blocks")

    def swap_blocks(self, src_k, src_v, dst_k, dst_v, src, dst, dtype: str):
        """In-place whole-block moves src pools[src[i]] -> dst pools[dst[i]]."""
        s_ = self._i32(src)
        t = self._i32(dst)
        for a in (src_k, src_v, dst_k, dst_v):
            assert a.flags.c_contiguous
        ns, Hkv, B, d = src_k.shape
        nd = dst_k.shape[0]
        assert dst_k.shape[1:] == (Hkv, B, d)
        rc = self._lib.oracle_swap_blocks(
            src_k.ctypes.data, src_v.ctypes.data, dst_k.ctypes.data, dst_v.ctypes.data,
            s_.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(s_), Hkv, d, B, ns, nd,
            DTYPE_CODE[dtype])
        self._check(rc, "oracle_swap_blocks")


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def build_mutant(mutant: int) -> Oracle:
    """An oracle with one planted mistake (tests of the pins only)."""
    d = tempfile.mkdtemp(prefix="oracle_mutant_")
    return Oracle(build(mutant, os.path.join(d, f"liboracle_m{mutant}.so")))
