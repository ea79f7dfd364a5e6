"""CPU oracle for the sigmoid group-limited MoE gate and its dispatch.

TEST INFRASTRUCTURE ONLY.  This package is the float64 checker that the HIP
library is compared against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library (``sigmoid_group_limited_amd``) and imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain loops, float64, OpenMP over
tokens); this module only compiles it with gcc and marshals numpy arrays.

Sources the steps follow (page title, then the part of the page):
  * DeepSeek-V3.2-Exp · Normalize weights -- the "Code" excerpt (Gate forward)
    and the equation for G_i;
  * Kimi K2 · Normalize weights -- the "Code" excerpt (gate forward) and the
    equation for G_i;
  * AI Engineer Exhaustive · DeepSeek-V3 MoE Router -- "How it works"
    (eq. for s_{i,t}, eq. for g'_{i,t} and g_{i,t}, the bias and the
    node-limited routing paragraphs, the route_scale paragraph);
  * Kimi K2 · Add shared output -- the "Code" excerpt, first lines of
    moe_infer (counts, argsort, row gather).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

OK = 0
EINVAL = -1


def compile_oracle(source: str = SOURCE, output: str = LIBRARY,
                   strict: bool = True) -> str:
    """Compile ``source`` into a shared library at ``output`` with gcc
    (warnings are errors when ``strict``)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall"]
    cmd += ["-Werror"] if strict else []
    cmd += [source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def _needs_build(output: str, source: str) -> bool:
    return (not os.path.exists(output)
            or os.path.getmtime(output) < os.path.getmtime(source))


@dataclass
class Scores:
    affinity: np.ndarray  # float64 [T, E]: s (sigmoid or softmax of the logits)
    choice: np.ndarray    # float64 [T, E]: v = s + bias (v = s without a bias)
    group: np.ndarray     # float64 [T, G]: group scores (empty when G == 1)


@dataclass
class GateResult:
    weights: np.ndarray   # float64 [T, K]
    indices: np.ndarray   # int32   [T, K]
    margins: np.ndarray   # float64 [T, 2]: (v_K - v_K+1, gs_KG - gs_KG+1)
    scores: Scores | None = None   # the float64 scores the selection ranked


@dataclass
class DispatchResult:
    counts: np.ndarray    # int32 [E]
    offsets: np.ndarray   # int32 [E+1]
    perm: np.ndarray      # int32 [T*K]


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """ctypes view of one compiled copy of ``oracle.c``."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        P = ctypes.POINTER
        lib.oracle_num_threads.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_logits.restype = None
        lib.oracle_logits.argtypes = [P(ctypes.c_uint16), P(ctypes.c_float),
                                      i64, i64, i64, P(dbl)]
        lib.oracle_select.restype = i32
        lib.oracle_select.argtypes = [P(dbl), P(ctypes.c_float), i64, i64,
                                      i32, i32, i32, dbl, i32, i32, i32, i32,
                                      dbl, P(dbl), P(ctypes.c_int32), P(dbl)]
        lib.oracle_scores.restype = i32
        lib.oracle_scores.argtypes = [P(dbl), P(ctypes.c_float), i64, i64, i32, i32,
                                      P(dbl), P(dbl), P(dbl)]
        lib.oracle_gate.restype = i32
        lib.oracle_gate.argtypes = [P(ctypes.c_uint16), P(ctypes.c_float),
                                    P(ctypes.c_float), i64, i64, i64, i32,
                                    i32, i32, dbl, i32, i32, i32, i32, dbl,
                                    P(dbl), P(ctypes.c_int32), P(dbl)]
        lib.oracle_dispatch.restype = i32
        lib.oracle_dispatch.argtypes = [P(ctypes.c_int32), i64, i32, i64,
                                        P(ctypes.c_int32), P(ctypes.c_int32),
                                        P(ctypes.c_int32)]
        lib.oracle_gather_rows.restype = i32
        lib.oracle_gather_rows.argtypes = [P(ctypes.c_uint16), i64, i64, i32,
                                           P(ctypes.c_int32), i64,
                                           P(ctypes.c_uint16)]
        lib.oracle_ep_send_splits.restype = i32
        lib.oracle_ep_send_splits.argtypes = [P(ctypes.c_int32), i64, i32,
                                              P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.oracle_ep_regroup.restype = i32
        lib.oracle_ep_regroup.argtypes = [P(ctypes.c_int32), i32, i64,
                                          P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.oracle_ep_dedup.restype = i32
        lib.oracle_ep_dedup.argtypes = [P(ctypes.c_int32), i64, i32, i64, i32,
                                        P(ctypes.c_int32), P(ctypes.c_int32),
                                        P(ctypes.c_int32), P(ctypes.c_int32)]
        lib.oracle_combine.restype = i32
        lib.oracle_combine.argtypes = [P(ctypes.c_uint16), i64, P(dbl),
                                       P(ctypes.c_int32), i64, i32, i64,
                                       P(dbl), P(ctypes.c_uint16)]
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def logits(self, x_bf16: np.ndarray, W: np.ndarray) -> np.ndarray:
        """float64 logits [T, E] of bfloat16 bits x [T, d] and float32 W [E, d]."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.float32)
        T, d = x.shape
        E, d2 = W.shape
        if d != d2:
            raise ValueError("x and W disagree on d")
        out = np.empty((T, E), dtype=np.float64)
        self.lib.oracle_logits(_ptr(x, ctypes.c_uint16), _ptr(W, ctypes.c_float),
                               T, d, E, _ptr(out, ctypes.c_double))
        return out

    @staticmethod
    def _bias_ptr(bias, E):
        if bias is None:
            return None, ctypes.POINTER(ctypes.c_float)()
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.shape != (E,):
            raise ValueError("bias must have shape [E]")
        return b, _ptr(b, ctypes.c_float)

    def select(self, logits: np.ndarray, bias: np.ndarray | None, n_group: int,
               topk_group: int, top_k: int, route_scale: float,
               order: int = 0, score_func: int = 0, renorm: int = 0,
               mask_zero: int = 0, denom_eps: float = 0.0,
               with_scores: bool = False) -> GateResult:
        """Gate steps after the logits, from float64 logits [T, E].
        bias=None selects the no-bias variant (group score = group max);
        score_func 0 sigmoid / 1 softmax; renorm 0 auto / 1 on / 2 off;
        mask_zero fills dropped groups with 0.0 instead of -inf.
        with_scores also returns the float64 scores that were ranked."""
        L = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = L.shape
        b, bp = self._bias_ptr(bias, E)
        w = np.empty((T, top_k), dtype=np.float64)
        idx = np.empty((T, top_k), dtype=np.int32)
        m = np.empty((T, 2), dtype=np.float64)
        rc = self.lib.oracle_select(_ptr(L, ctypes.c_double), bp,
                                    T, E, n_group, topk_group, top_k,
                                    float(route_scale), order, score_func, renorm,
                                    mask_zero, float(denom_eps),
                                    _ptr(w, ctypes.c_double),
                                    _ptr(idx, ctypes.c_int32),
                                    _ptr(m, ctypes.c_double))
        if rc != OK:
            raise ValueError(f"oracle_select rejected the configuration (rc={rc})")
        sc = self.scores(L, bias, n_group, score_func) if with_scores else None
        return GateResult(w, idx, m, sc)

    def scores(self, logits: np.ndarray, bias: np.ndarray | None, n_group: int,
               score_func: int = 0) -> Scores:
        """Affinities, choice scores and group scores (steps 2-4) from
        float64 logits [T, E]; the same code the selection runs."""
        L = np.ascontiguousarray(logits, dtype=np.float64)
        T, E = L.shape
        b, bp = self._bias_ptr(bias, E)
        s = np.empty((T, E), dtype=np.float64)
        v = np.empty((T, E), dtype=np.float64)
        G = n_group
        gs = np.empty((T, G if G > 1 else 0), dtype=np.float64)
        gsp = _ptr(gs, ctypes.c_double) if G > 1 else ctypes.POINTER(ctypes.c_double)()
        rc = self.lib.oracle_scores(_ptr(L, ctypes.c_double), bp, T, E, G, score_func,
                                    _ptr(s, ctypes.c_double), _ptr(v, ctypes.c_double), gsp)
        if rc != OK:
            raise ValueError(f"oracle_scores rejected the configuration (rc={rc})")
        return Scores(s, v, gs)

    def gate(self, x_bf16: np.ndarray, W: np.ndarray, bias: np.ndarray | None,
             n_group: int, topk_group: int, top_k: int, route_scale: float,
             order: int = 0, score_func: int = 0, renorm: int = 0,
             mask_zero: int = 0, denom_eps: float = 0.0,
             with_scores: bool = False) -> GateResult:
        """Whole gate from bfloat16 bits x [T, d], float32 W [E, d], bias [E]
        (or None); options as in select()."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        W = np.ascontiguousarray(W, dtype=np.float32)
        T, d = x.shape
        E, d2 = W.shape
        if d != d2:
            raise ValueError("shape mismatch between x and W")
        b, bp = self._bias_ptr(bias, E)
        w = np.empty((T, top_k), dtype=np.float64)
        idx = np.empty((T, top_k), dtype=np.int32)
        m = np.empty((T, 2), dtype=np.float64)
        rc = self.lib.oracle_gate(_ptr(x, ctypes.c_uint16), _ptr(W, ctypes.c_float),
                                  bp, T, d, E, n_group,
                                  topk_group, top_k, float(route_scale), order,
                                  score_func, renorm, mask_zero, float(denom_eps),
                                  _ptr(w, ctypes.c_double),
                                  _ptr(idx, ctypes.c_int32),
                                  _ptr(m, ctypes.c_double))
        if rc != OK:
            raise ValueError(f"oracle_gate rejected the configuration (rc={rc})")
        sc = self.scores(self.logits(x, W), bias, n_group, score_func) if with_scores else None
        return GateResult(w, idx, m, sc)

    def dispatch(self, indices: np.ndarray, n_experts: int) -> DispatchResult:
        """Counts, offsets and the stable expert-major permutation."""
        idx = np.ascontiguousarray(indices, dtype=np.int32)
        T, K = idx.shape
        counts = np.empty(n_experts, dtype=np.int32)
        offsets = np.empty(n_experts + 1, dtype=np.int32)
        perm = np.empty(T * K, dtype=np.int32)
        rc = self.lib.oracle_dispatch(_ptr(idx, ctypes.c_int32), T, K, n_experts,
                                      _ptr(counts, ctypes.c_int32),
                                      _ptr(offsets, ctypes.c_int32),
                                      _ptr(perm, ctypes.c_int32))
        if rc != OK:
            raise ValueError(f"oracle_dispatch rejected its input (rc={rc})")
        return DispatchResult(counts, offsets, perm)

    def gather_rows(self, x_bf16: np.ndarray, perm: np.ndarray, top_k: int,
                    rows: np.ndarray | None = None) -> np.ndarray:
        """out[pos] = x[perm[pos] // top_k]; ``rows`` picks a subset of pos."""
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        T, d = x.shape
        p = np.ascontiguousarray(perm if rows is None else perm[rows],
                                 dtype=np.int32)
        out = np.empty((p.shape[0], d), dtype=np.uint16)
        rc = self.lib.oracle_gather_rows(_ptr(x, ctypes.c_uint16), T, d, top_k,
                                         _ptr(p, ctypes.c_int32), p.shape[0],
                                         _ptr(out, ctypes.c_uint16))
        if rc != OK:
            raise ValueError("oracle_gather_rows: permutation entry out of range")
        return out


    def combine(self, expert_out_bf16: np.ndarray, weights: np.ndarray,
                dest: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
        """y[t] = sum_k w[t,k] * out[dest[t*K+k]] for expert outputs in
        dispatch order (bfloat16 bits [n_pos, d]).  Returns (float64 sums
        [T, d], bfloat16 bits [T, d] of the sums rounded via float32)."""
        out = np.ascontiguousarray(expert_out_bf16, dtype=np.uint16)
        w = np.ascontiguousarray(weights, dtype=np.float64)
        dst = np.ascontiguousarray(dest, dtype=np.int32).ravel()
        T, K = w.shape
        n_pos, d = out.shape
        if dst.shape != (T * K,):
            raise ValueError("dest must have T*K entries")
        y64 = np.empty((T, d), dtype=np.float64)
        y16 = np.empty((T, d), dtype=np.uint16)
        rc = self.lib.oracle_combine(_ptr(out, ctypes.c_uint16), n_pos,
                                     _ptr(w, ctypes.c_double), _ptr(dst, ctypes.c_int32),
                                     T, K, d, _ptr(y64, ctypes.c_double),
                                     _ptr(y16, ctypes.c_uint16))
        if rc != OK:
            raise ValueError("oracle_combine: dest entry out of range")
        return y64, y16


    # -- expert-parallel metadata --------------------------------------
    def ep_send_splits(self, tokens_per_expert: np.ndarray, ep_size: int):
        """(send_counts [ep_size], send_offsets [ep_size+1]): per-rank sums
        of tokens_per_expert."""
        tpe = np.ascontiguousarray(tokens_per_expert, dtype=np.int32)
        c = np.empty(ep_size, np.int32)
        off = np.empty(ep_size + 1, np.int32)
        rc = self.lib.oracle_ep_send_splits(_ptr(tpe, ctypes.c_int32), tpe.shape[0], ep_size,
                                            _ptr(c, ctypes.c_int32), _ptr(off, ctypes.c_int32))
        if rc != OK:
            raise ValueError("oracle_ep_send_splits: E not a multiple of ep_size")
        return c, off

    def ep_regroup(self, counts: np.ndarray):
        """counts [ep_size, experts_per_rank] of received rows ->
        (local_counts [experts_per_rank], regroup [n_recv])."""
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        R, per = cnt.shape
        n = int(cnt.sum())
        lc = np.empty(per, np.int32)
        rg = np.empty(max(n, 1), np.int32)
        rc = self.lib.oracle_ep_regroup(_ptr(cnt, ctypes.c_int32), R, per,
                                        _ptr(lc, ctypes.c_int32), _ptr(rg, ctypes.c_int32))
        if rc != OK:
            raise ValueError("oracle_ep_regroup rejected its input")
        return lc, rg[:n]

    def ep_dedup(self, indices: np.ndarray, n_experts: int, ep_size: int):
        """De-duplicated rank-major send list: (rank_counts, rank_offsets,
        send_tokens, pair_slot)."""
        idx = np.ascontiguousarray(indices, dtype=np.int32)
        T, K = idx.shape
        rcnt = np.empty(ep_size, np.int32)
        roff = np.empty(ep_size + 1, np.int32)
        send = np.empty(max(T * K, 1), np.int32)
        slot = np.empty(max(T * K, 1), np.int32)
        rc = self.lib.oracle_ep_dedup(_ptr(idx, ctypes.c_int32), T, K, n_experts, ep_size,
                                      _ptr(rcnt, ctypes.c_int32), _ptr(roff, ctypes.c_int32),
                                      _ptr(send, ctypes.c_int32), _ptr(slot, ctypes.c_int32))
        if rc != OK:
            raise ValueError("oracle_ep_dedup rejected its input")
        return rcnt, roff, send[:int(roff[-1])], slot[:T * K]


_DEFAULT: Oracle | None = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``oracle.c`` next to this file (compiled on
    first use, or when the source is newer than the library)."""
    global _DEFAULT
    if rebuild or _needs_build(LIBRARY, SOURCE):
        compile_oracle()
        _DEFAULT = None
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
