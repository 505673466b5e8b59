"""CPU oracle for paged MLA decode -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP path: ``oracle.c`` is compiled on its own with
gcc, and this module only marshals numpy arrays into it.

Functions:
  * ``decode(w, sel=None)`` -- fp64 reference outputs (out, lse) for a
    ``workloads.Workload``; ``sel`` restricts it to a list of flat query indices
    ``(b * s_q + s) * h_q + h`` so large workloads can be checked by sampling.
  * ``schedule(seqlens, rows, num_parts)`` -- the independent twin of the
    split-KV partition (tile metadata and cumulative split counts).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def _compile(out_path: str, defines=()) -> str:
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall"]
    cmd += [f"-D{d}" for d in defines]
    cmd += ["-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    global _default
    if force or not os.path.exists(_LIB_PATH):
        _compile(_LIB_PATH)
        _default = None
    return _LIB_PATH


def build_mutant(mutant: int, out_dir: str) -> "Oracle":
    """A copy of the oracle with one planted mistake (see ORACLE_MUTANT in oracle.c);
    used only to show that the pins in tests/ reject it."""
    path = os.path.join(out_dir, f"liboracle_mutant{mutant}.so")
    _compile(path, [f"ORACLE_MUTANT={int(mutant)}"])
    return Oracle(path)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        LL = ctypes.c_longlong
        lib.oracle_decode.argtypes = [P, P, LL, P, I, P, I, I, I, I, I, I, I, I,
                                      ctypes.c_double, P, LL, P, P]
        lib.oracle_decode.restype = I
        lib.oracle_schedule.argtypes = [P, I, I, I, P, P]
        lib.oracle_schedule.restype = I
        lib.oracle_tile_rows.argtypes = [I]
        lib.oracle_tile_rows.restype = I
        lib.oracle_num_threads.restype = I
        lib.oracle_set_threads.argtypes = [I]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def decode(self, w, sel: Optional[Sequence[int]] = None, causal: Optional[bool] = None,
               scale: Optional[float] = None):
        """fp64 (out [n, dv], lse [n]) for workload ``w`` (all queries, or ``sel``)."""
        q = np.ascontiguousarray(w.q, dtype=np.uint16)
        kc = np.ascontiguousarray(w.kcache, dtype=np.uint16)
        bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
        sl = np.ascontiguousarray(w.cache_seqlens, dtype=np.int32)
        total = w.batch * w.s_q * w.h_q
        if sel is None:
            n = total
            sel_arr = None
        else:
            sel_arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
            n = int(sel_arr.shape[0])
        out = np.zeros((n, w.dv), dtype=np.float64)
        lse = np.zeros(n, dtype=np.float64)
        rc = self.lib.oracle_decode(
            _ptr(q), _ptr(kc), kc.shape[0], _ptr(bt), bt.shape[1], _ptr(sl),
            w.batch, w.s_q, w.h_q, w.h_kv, w.d_qk, w.dv, w.page,
            int(w.causal if causal is None else causal),
            float(w.scale if scale is None else scale),
            _ptr(sel_arr) if sel_arr is not None else None, n, _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("block_table references a page outside the cache")
        return out, lse

    def tile_rows(self, rows: int) -> int:
        return int(self.lib.oracle_tile_rows(int(rows)))

    def schedule(self, seqlens, rows: int, num_parts: int):
        """Twin of the split-KV partition: (tile_metadata [P, 8], num_splits [b+1])."""
        sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
        b = int(sl.shape[0])
        md = np.zeros((num_parts, 8), dtype=np.int32)
        ns = np.zeros(b + 1, dtype=np.int32)
        rc = self.lib.oracle_schedule(_ptr(sl), b, int(rows), int(num_parts), _ptr(md), _ptr(ns))
        if rc != 0:
            raise ValueError("invalid schedule arguments")
        return md, ns


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _default = Oracle(_LIB_PATH)
    return _default


def decode(w, sel=None, causal=None, scale=None):
    return default().decode(w, sel=sel, causal=causal, scale=scale)


def schedule(seqlens, rows: int, num_parts: int):
    return default().schedule(seqlens, rows, num_parts)


def tile_rows(rows: int) -> int:
    return default().tile_rows(rows)


def num_threads() -> int:
    return default().num_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)
