"""CPU oracle for the sparse MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never loads it, and it
never loads the HIP library.

The arithmetic lives in ``moe_oracle.c`` (plain float64 loops, OpenMP over
tokens); this module only marshals numpy arrays through ctypes. Every
function follows the passage cited in the C source:

* ``router_logits``   -- router linear (MoE paragraph of the mini-sglang
  chapter-7 guide; "Linear layers" on "The op layer" page).
* ``select_topk``     -- softmax over all experts, top-k in torch.topk order,
  optional norm_topk_prob renormalisation.
* ``align``           -- tokens grouped by expert (fused-backend paragraph),
  each group padded to block_m with the sentinel T*k.
* ``expert_gate_up``, ``expert_down``, ``expert_mlp`` -- one expert's gated
  MLP and its two halves (GatedMLP on the "Models and weight loading" page).
* ``combine``         -- the weighted sum of a token's k expert outputs.
* ``fused_add_rmsnorm`` -- the residual add + RMSNorm that precedes the MLP
  ("The op layer" page: reference ops and "RMSNorm and the residual").
* ``moe_layer``       -- the whole layer, one token at a time.

All of these are pinned by the tests in ``tests/test_oracle_*.py`` (brute
force, library cross-checks, closed forms and invariants); nothing here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIB names another build (the host-sanitizer test build).
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")


class OracleLib:
    """ctypes view of one build of the oracle library (the default build, or
    a test's deliberately mutated copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_router_logits.argtypes = [p, p, p, i64, i64, i64, p]
        lib.oracle_router_logits.restype = None
        lib.oracle_select_topk.argtypes = [p, i64, i64, i64, ci, p, p]
        lib.oracle_select_topk.restype = None
        lib.oracle_align.argtypes = [p, i64, i64, i64, i64, i64, p, p, p]
        lib.oracle_align.restype = i64
        lib.oracle_expert_mlp.argtypes = [p, p, p, i64, i64, p, p]
        lib.oracle_expert_mlp.restype = None
        lib.oracle_expert_gate_up.argtypes = [p, p, i64, i64, p]
        lib.oracle_expert_gate_up.restype = None
        lib.oracle_expert_down.argtypes = [p, p, i64, i64, p]
        lib.oracle_expert_down.restype = None
        lib.oracle_combine.argtypes = [p, p, i64, i64, p]
        lib.oracle_combine.restype = None
        lib.oracle_moe_layer.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ci, p, i64, p, p, p]
        lib.oracle_moe_layer.restype = None
        lib.oracle_fused_add_rmsnorm.argtypes = [p, p, p, i64, i64, ctypes.c_double, ci]
        lib.oracle_fused_add_rmsnorm.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ci
        lib.oracle_set_threads.argtypes = [ci]
        lib.oracle_set_threads.restype = None
        self.path = path
        self._lib = lib

    def max_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self._lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        """Threads for the oracle's later parallel loops (for timing runs)."""
        self._lib.oracle_set_threads(int(n))

    def router_logits(self, x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
        """fp64 logits [T, E] from bf16 x [T, H] and w_router [E, H] (+ fp32 bias [E])."""
        x, w_router = _u16(x), _u16(w_router)
        T, H = x.shape
        E = w_router.shape[0]
        assert w_router.shape == (E, H)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        out = np.empty((T, E), dtype=np.float64)
        self._lib.oracle_router_logits(x.ctypes.data, w_router.ctypes.data, _ptr(b), T, H, E, out.ctypes.data)
        return out

    def select_topk(self, logits: np.ndarray, k: int, norm_topk_prob: bool = True):
        """(ids int32 [T, k], weights fp64 [T, k]) from logits [T, E] (any float
        dtype, widened exactly to fp64)."""
        lg = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = lg.shape
        if not 1 <= k <= E:
            raise ValueError("need 1 <= k <= E")
        ids = np.empty((T, k), dtype=np.int32)
        w = np.empty((T, k), dtype=np.float64)
        self._lib.oracle_select_topk(lg.ctypes.data, T, E, k, int(bool(norm_topk_prob)), ids.ctypes.data,
                                     w.ctypes.data)
        return ids, w

    def align(self, ids: np.ndarray, E: int, block_m: int, cap: Optional[int] = None):
        """Expert-grouped permutation. Returns (sorted_ids [cap], block_expert
        [cap/block_m], counts [E], num_padded)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, k = ids.shape
        if ids.size and (ids.min() < 0 or ids.max() >= E):
            raise ValueError("expert id out of range")
        if cap is None:
            cap = align_capacity(T, k, E, block_m)
        sorted_ids = np.empty(cap, dtype=np.int32)
        block_expert = np.empty(cap // block_m, dtype=np.int32)
        counts = np.empty(E, dtype=np.int32)
        npad = self._lib.oracle_align(ids.ctypes.data, T, k, E, block_m, cap, sorted_ids.ctypes.data,
                                      block_expert.ctypes.data, counts.ctypes.data)
        if npad < 0:
            raise ValueError("capacity too small")
        return sorted_ids, block_expert, counts, int(npad)

    def expert_mlp(self, x: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
        """One expert's gated MLP on fp64 rows x [n, H]; w13_e [2I, H], w2_e [H, I] bf16."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
        w13_e, w2_e = _u16(w13_e), _u16(w2_e)
        H = x.shape[1]
        I = w2_e.shape[1]
        assert w13_e.shape == (2 * I, H) and w2_e.shape == (H, I)
        out = np.empty_like(x)
        act = np.empty(I, dtype=np.float64)
        for r in range(x.shape[0]):
            self._lib.oracle_expert_mlp(x[r].ctypes.data, w13_e.ctypes.data, w2_e.ctypes.data, H, I,
                                        act.ctypes.data, out[r].ctypes.data)
        return out

    def expert_gate_up(self, x: np.ndarray, w13_e: np.ndarray) -> np.ndarray:
        """silu(gate) * up of one expert for fp64 rows x [n, H]; w13_e [2I, H] bf16 -> [n, I]."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float64)
        w13_e = _u16(w13_e)
        H = x.shape[1]
        I = w13_e.shape[0] // 2
        assert w13_e.shape == (2 * I, H)
        out = np.empty((x.shape[0], I), dtype=np.float64)
        for r in range(x.shape[0]):
            self._lib.oracle_expert_gate_up(x[r].ctypes.data, w13_e.ctypes.data, H, I, out[r].ctypes.data)
        return out

    def expert_down(self, act: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
        """Down projection of one expert for fp64 rows act [n, I]; w2_e [H, I] bf16 -> [n, H]."""
        act = np.ascontiguousarray(np.atleast_2d(act), dtype=np.float64)
        w2_e = _u16(w2_e)
        H, I = w2_e.shape
        assert act.shape[1] == I
        out = np.empty((act.shape[0], H), dtype=np.float64)
        for r in range(act.shape[0]):
            self._lib.oracle_expert_down(act[r].ctypes.data, w2_e.ctypes.data, H, I, out[r].ctypes.data)
        return out

    def combine(self, y: np.ndarray, w: np.ndarray) -> np.ndarray:
        """out [T, H] = sum_j w[t, j] * y[t, j, :] for y [T, k, H], w [T, k] (fp64)."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        T, k, H = y.shape
        assert w.shape == (T, k)
        out = np.empty((T, H), dtype=np.float64)
        for t in range(T):
            self._lib.oracle_combine(y[t].ctypes.data, w[t].ctypes.data, k, H, out[t].ctypes.data)
        return out

    def fused_add_rmsnorm(self, x: np.ndarray, residual: Optional[np.ndarray], weight: np.ndarray,
                          eps: float = 1e-6):
        """(normalized x, new residual) as bf16 bits, [T, H] each; residual
        None is the first layer (the residual is x itself)."""
        xo = _u16(x).copy()
        T, H = xo.shape
        ro = np.empty_like(xo) if residual is None else _u16(residual).copy()
        w = _u16(weight)
        assert w.shape == (H,) and ro.shape == (T, H)
        self._lib.oracle_fused_add_rmsnorm(xo.ctypes.data, ro.ctypes.data, w.ctypes.data, T, H, float(eps),
                                           int(residual is not None))
        return xo, ro

    def moe_layer(self, x, w_router, w13, w2, k: int, norm_topk_prob: bool = True, bias=None,
                  tokens: Optional[Sequence[int]] = None):
        """The whole layer in fp64 for the listed tokens (default: all).
        Returns (out [n, H] fp64, ids [n, k] int32, weights [n, k] fp64)."""
        x, w_router, w13, w2 = _u16(x), _u16(w_router), _u16(w13), _u16(w2)
        T, H = x.shape
        E = w_router.shape[0]
        I = w2.shape[2]
        assert w_router.shape == (E, H) and w13.shape == (E, 2 * I, H) and w2.shape == (E, H, I)
        if not 1 <= k <= E:
            raise ValueError("need 1 <= k <= E")
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        n = T if tok is None else tok.shape[0]
        if tok is not None and n and (tok.min() < 0 or tok.max() >= T):
            raise IndexError("token index out of range")
        out = np.empty((n, H), dtype=np.float64)
        ids = np.empty((n, k), dtype=np.int32)
        w = np.empty((n, k), dtype=np.float64)
        self._lib.oracle_moe_layer(x.ctypes.data, w_router.ctypes.data, _ptr(b), w13.ctypes.data, w2.ctypes.data,
                                   T, H, E, k, I, int(bool(norm_topk_prob)), _ptr(tok), n, out.ctypes.data,
                                   ids.ctypes.data, w.ctypes.data)
        return out, ids, w


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    """Rows sufficient for any routing: T*k real rows plus at most block_m-1
    pad rows for each non-empty expert, rounded up to block_m."""
    n = T * k
    c = n + min(E, n) * (block_m - 1)
    return (c + block_m - 1) // block_m * block_m


def build(force: bool = False) -> str:
    """Compile the oracle with gcc -O2 (no fast-math), OpenMP."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


_default: Optional[OracleLib] = None


def default() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = OracleLib(_LIB_PATH)
    return _default


def router_logits(*a, **kw):
    return default().router_logits(*a, **kw)


def select_topk(*a, **kw):
    return default().select_topk(*a, **kw)


def align(*a, **kw):
    return default().align(*a, **kw)


def expert_mlp(*a, **kw):
    return default().expert_mlp(*a, **kw)


def expert_gate_up(*a, **kw):
    return default().expert_gate_up(*a, **kw)


def expert_down(*a, **kw):
    return default().expert_down(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def fused_add_rmsnorm(*a, **kw):
    return default().fused_add_rmsnorm(*a, **kw)


def moe_layer(*a, **kw):
    return default().moe_layer(*a, **kw)
