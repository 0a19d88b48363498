"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It imports nothing
from the HIP library's package and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "oracle.c"
DEFAULT_LIB = HERE / "liboracle.so"
CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


SANITIZED_LIB = HERE / "liboracle_asan.so"
# The sanitizer build uses ROCm's clang, so that it shares one AddressSanitizer runtime with
# the library's sanitizer build (paged_kv_cache_27_amd/build.py); OpenMP from its libomp.
CLANG = "/opt/rocm/llvm/bin/clang"


def build(out: Path | str = DEFAULT_LIB, mutation: int = 0, sanitize: bool = False) -> Path:
    """Compile oracle.c with gcc (IEEE fp64, no contraction, OpenMP).  sanitize: with clang
    under AddressSanitizer and UndefinedBehaviorSanitizer instead (default output
    liboracle_asan.so), for the CPU test suite run against it."""
    if sanitize:
        out = Path(out) if Path(out) != DEFAULT_LIB else SANITIZED_LIB
        cmd = [CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", f"-DORACLE_MUTATION={int(mutation)}", str(SOURCE), "-o",
               str(out) + ".tmp", "-lm"]
    else:
        out = Path(out)
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", f"-DORACLE_MUTATION={int(mutation)}", str(SOURCE), "-o",
               str(out) + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(str(out) + ".tmp", out)
    return out


class Oracle:
    def __init__(self, path: Path | str | None = None):
        # PKV_ORACLE_LIB selects another build (the sanitizer build, for instance)
        path = Path(path if path is not None else os.environ.get("PKV_ORACLE_LIB", DEFAULT_LIB))
        if not path.exists():
            build(path)
        self.lib = lib = ctypes.CDLL(str(path))
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_fp8_to_f64.restype = ctypes.c_double
        lib.oracle_fp8_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_f32_to_fp8.restype = ctypes.c_uint8
        lib.oracle_f32_to_fp8.argtypes = [ctypes.c_float]
        lib.oracle_kv_bytes.restype = ctypes.c_int64
        lib.oracle_kv_bytes.argtypes = [ctypes.c_int64] * 5
        lib.oracle_slot_mapping.restype = ctypes.c_int
        lib.oracle_slot_mapping.argtypes = [_i32p, _i32p, ctypes.c_int64, _i32p, ctypes.c_int32,
                                            ctypes.c_int32, _i64p]
        lib.oracle_kv_write.restype = ctypes.c_int
        lib.oracle_kv_write.argtypes = [_i64p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_float]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                      ctypes.c_int32, _i32p, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_int64, _f64p, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.c_int]
        lib.oracle_decode_window.restype = ctypes.c_int
        lib.oracle_decode_window.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_int64,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                             ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, _f64p,
                                             ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, _i32p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       _i32p, ctypes.c_int32, _i32p, ctypes.c_float, _f64p, ctypes.c_int]
        lib.oracle_copy_blocks.restype = ctypes.c_int
        lib.oracle_copy_blocks.argtypes = [_i32p, _i32p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_int64]
        lib.oracle_swap_blocks.restype = ctypes.c_int
        lib.oracle_swap_blocks.argtypes = [_i32p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int]
        lib.oracle_mutation.restype = ctypes.c_int
        self.mutation = lib.oracle_mutation()

    # -- codecs (vectorised over numpy arrays by plain loops: these are small) --
    def bf16_to_f64(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16)
        return np.array([self.lib.oracle_bf16_to_f64(int(b)) for b in bits.ravel()]).reshape(bits.shape)

    def f16_to_f64(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16)
        return np.array([self.lib.oracle_f16_to_f64(int(b)) for b in bits.ravel()]).reshape(bits.shape)

    def fp8_to_f64(self, codes) -> np.ndarray:
        codes = np.asarray(codes, dtype=np.uint8)
        return np.array([self.lib.oracle_fp8_to_f64(int(c)) for c in codes.ravel()]).reshape(codes.shape)

    def f32_to_fp8(self, x) -> np.ndarray:
        x = np.asarray(x, dtype=np.float32)
        return np.array([self.lib.oracle_f32_to_fp8(float(v)) for v in x.ravel()],
                        dtype=np.uint8).reshape(x.shape)

    def kv_bytes(self, T, L, H_kv, d_h, b) -> int:
        return int(self.lib.oracle_kv_bytes(T, L, H_kv, d_h, b))

    # -- the step --
    def slot_mapping(self, seq_ids, positions, block_tables, block_size) -> np.ndarray:
        seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        out = np.empty(seq_ids.size, dtype=np.int64)
        rc = self.lib.oracle_slot_mapping(seq_ids, positions, seq_ids.size, bt, bt.shape[1],
                                          block_size, out)
        if rc:
            raise ValueError(f"oracle_slot_mapping failed: {rc}")
        return out

    def kv_write(self, slots, k, v, src_dtype, k_cache, v_cache, cache_dtype, k_scale=1.0,
                 v_scale=1.0) -> None:
        slots = np.ascontiguousarray(slots, dtype=np.int64)
        k = np.ascontiguousarray(k)
        v = np.ascontiguousarray(v)
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        nb, hkv, bs, d = k_cache.shape
        assert k.shape == (slots.size, hkv, d) and v.shape == k.shape
        rc = self.lib.oracle_kv_write(slots, slots.size, k.ctypes.data, v.ctypes.data,
                                      CODES[src_dtype], k_cache.ctypes.data, v_cache.ctypes.data,
                                      nb, bs, hkv, d, CODES[cache_dtype], k_scale, v_scale)
        if rc:
            raise ValueError(f"oracle_kv_write failed: {rc}")

    def prefill(self, q, q_dtype, cu_q, k_cache, v_cache, cache_dtype, block_tables, context_lens,
                scale, k_scale=1.0, v_scale=1.0, threads=1):
        """Causal attention of each sequence's last cu_q[s+1]-cu_q[s] tokens (rows of q,
        [rows][H_q][d_h]) over its paged context.  Returns [rows][H_q][d_h] fp64."""
        q = np.ascontiguousarray(q)
        rows, hq, d = q.shape
        nb, hkv, bs, d2 = k_cache.shape
        assert d == d2
        cu = np.ascontiguousarray(cu_q, dtype=np.int32)
        assert cu[-1] == rows
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        out = np.zeros((rows, hq, d), dtype=np.float64)
        rc = self.lib.oracle_prefill(q.ctypes.data, CODES[q_dtype], cu.size - 1, hq, cu, k_cache.ctypes.data,
                                     v_cache.ctypes.data, CODES[cache_dtype], k_scale, v_scale, bs, hkv, d,
                                     bt, bt.shape[1], cl, scale, out, threads)
        if rc:
            raise ValueError(f"oracle_prefill failed: {rc}")
        return out

    def copy_blocks(self, src, dst, k_cache, v_cache) -> None:
        """Copy-on-write: block src[i] -> block dst[i] in both caches (in place)."""
        src = np.ascontiguousarray(src, dtype=np.int32)
        dst = np.ascontiguousarray(dst, dtype=np.int32)
        assert src.shape == dst.shape and k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        nb = k_cache.shape[0]
        rc = self.lib.oracle_copy_blocks(src, dst, src.size, k_cache.ctypes.data, v_cache.ctypes.data,
                                         nb, k_cache.nbytes // nb)
        if rc:
            raise ValueError(f"oracle_copy_blocks failed: {rc}")

    def swap_out(self, ids, k_cache, v_cache):
        """Blocks ids[i] of each cache as rows of new contiguous arrays (K, V)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        nb = k_cache.shape[0]
        kb = np.zeros((ids.size,) + k_cache.shape[1:], dtype=k_cache.dtype)
        vb = np.zeros_like(kb)
        rc = self.lib.oracle_swap_blocks(ids, ids.size, k_cache.ctypes.data, v_cache.ctypes.data,
                                         kb.ctypes.data, vb.ctypes.data, nb, k_cache.nbytes // nb, 0)
        if rc:
            raise ValueError(f"oracle_swap_blocks failed: {rc}")
        return kb, vb

    def swap_in(self, ids, k_buf, v_buf, k_cache, v_cache) -> None:
        """Rows i of the contiguous arrays back into blocks ids[i] (in place)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k_buf = np.ascontiguousarray(k_buf)
        v_buf = np.ascontiguousarray(v_buf)
        nb = k_cache.shape[0]
        rc = self.lib.oracle_swap_blocks(ids, ids.size, k_cache.ctypes.data, v_cache.ctypes.data,
                                         k_buf.ctypes.data, v_buf.ctypes.data, nb, k_cache.nbytes // nb, 1)
        if rc:
            raise ValueError(f"oracle_swap_blocks failed: {rc}")

    def decode(self, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens,
               scale, k_scale=1.0, v_scale=1.0, pairs=None, threads=1, count_bytes=False,
               window=0, sinks=0):
        """Attention of every (or each listed) (sequence, query head) pair; with
        window > 0 only over the last `window` tokens plus the first `sinks`."""
        q = np.ascontiguousarray(q)
        n, hq, d = q.shape
        nb, hkv, bs, d2 = k_cache.shape
        assert d == d2
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        if pairs is None:
            npairs, pptr = n * hq, None
        else:
            pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
            npairs, pptr = pairs.shape[0], pairs.ctypes.data
        out = np.zeros((npairs, d), dtype=np.float64)
        nbytes = ctypes.c_int64(0)
        rc = self.lib.oracle_decode_window(q.ctypes.data, CODES[q_dtype], n, hq, k_cache.ctypes.data,
                                           v_cache.ctypes.data, CODES[cache_dtype], k_scale, v_scale,
                                           nb, bs, hkv, d, bt, bt.shape[1], cl, int(window),
                                           int(sinks), scale, pptr, npairs, out,
                                           ctypes.byref(nbytes), threads)
        if rc:
            raise ValueError(f"oracle_decode failed: {rc}")
        if pairs is None:
            out = out.reshape(n, hq, d)
        return (out, nbytes.value) if count_bytes else out


_default = None


def get_oracle() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
