"""Python wrapper of the recurrent oracle (oracle/still_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's
CPU-baseline leg. It never touches a GPU and imports nothing from the HIP
path.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "still_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "liboracle.so")
_lib = None

# merge of the two branches (still_oracle.c): one normaliser, the sum of
# separately normalised branches, or the softmax branch alone
MERGES = {"one": 0, "sum": 1, "softmax_only": 2}
# routing metric (still_oracle.c): the Self-Saliency Score or one of the
# alternatives of the routing ablation; "external" takes the caller's scores
ROUTES = {"saliency": 0, "diag": 1, "qk": 2, "keynorm": 3, "uniform": 4, "external": 5}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, strict evaluation order)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_OUT_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O3", "-march=native", "-ffp-contract=off", "-fPIC",
                    "-shared", "-pthread", "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        f = lib.still_oracle_run
        P = ctypes.c_void_p
        f.argtypes = [ctypes.c_int] * 8 + [ctypes.c_double] * 2 + [P] * 5 + \
            [ctypes.c_int] + [P] * 7 + [ctypes.c_int] + [P] * 4 + [ctypes.c_int, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        g = lib.still_oracle_e4m3_rows
        g.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P]
        g.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: widen to float32 (exact for bf16)
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def units_of(B: int, Hkv: int) -> Sequence[Tuple[int, int]]:
    return [(b, kv) for b in range(B) for kv in range(Hkv)]


def prefill(q, k, v, fmap_w, gate, *, window: int, chunk: int, budget: int,
            t_max: int, eps: float = 1e-6, sm_scale: Optional[float] = None,
            units: Optional[Sequence[Tuple[int, int]]] = None,
            n_threads: int = 1, merge: str = "one",
            partials: bool = False, route: str = "saliency",
            ext_score=None, decay=None, fp8_from: int = -1) -> Dict[str, np.ndarray]:
    """Run the recurrent oracle on the listed (batch, kv head) units.

    q [B,Hq,L,d], k/v [B,Hkv,L,d], fmap_w [Hkv,d,d], gate [Hq]. Outputs
    are per unit, in the order of `units` (default: every unit, batch-major):
    y [U,G,L,d], score [U,L], sel [U,n_dec,lam], S [U,d,d], z [U,d],
    pending [U,C], n_pool [U]; with partials=True also y_sa, y_la [U,G,L,d]
    and lse_sa, lse_la [U,G,L] (each branch normalised on its own, the
    linear one without the gate; y_la = 0 and lse_la = -inf where the state
    is empty). merge: "one", "sum" or "softmax_only" (see MERGES). route:
    a key of ROUTES; ext_score [B,Hkv,L] the caller's scores for "external".
    decay [Hkv]: forget factors in (0, 1] of the linear state (key j weighted
    decay^(t - j) at query t), rounded to float32 as the caller holds them;
    None for the plain layer.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    units = list(units_of(B, Hkv) if units is None else units)
    U = len(units)
    qs = np.stack([_f32(q[b, kv * G:(kv + 1) * G]) for b, kv in units]) if U else \
        np.zeros((0, G, L, d), np.float32)
    ks = np.stack([_f32(k[b, kv]) for b, kv in units]) if U else np.zeros((0, L, d), np.float32)
    vs = np.stack([_f32(v[b, kv]) for b, kv in units]) if U else np.zeros((0, L, d), np.float32)
    Fs = np.stack([_f32(fmap_w[kv]) for _, kv in units]) if U else np.zeros((0, d, d), np.float32)
    gs = np.stack([_f32(gate[kv * G:(kv + 1) * G]) for _, kv in units]) if U else \
        np.zeros((0, G), np.float32)
    ext = None
    if ext_score is not None:
        ext = np.stack([_f32(ext_score[b, kv]) for b, kv in units]) if U else \
            np.zeros((0, L), np.float32)
    dec = None
    if decay is not None:
        d32 = _f32(decay)
        dec = np.array([d32[kv] for _, kv in units], dtype=np.float32)
    return run_units(qs, ks, vs, Fs, gs, window=window, chunk=chunk, budget=budget,
                     t_max=t_max, eps=eps, sm_scale=sm_scale, n_threads=n_threads,
                     merge=merge, partials=partials, route=route, ext=ext, decay=dec,
                     fp8_from=fp8_from)


def run_units(qs, ks, vs, Fs, gs, *, window: int, chunk: int, budget: int, t_max: int,
              eps: float = 1e-6, sm_scale: Optional[float] = None,
              n_threads: int = 1, merge: str = "one", partials: bool = False,
              route: str = "saliency", ext=None, decay=None,
              fp8_from: int = -1) -> Dict[str, np.ndarray]:
    """Run on pre-gathered per-unit arrays (see still_oracle_run); ext
    [U, L]: the caller's scores for route "external"; decay [U]: the
    units' forget factors of the linear state (float32 values), or None;
    fp8_from: queries from this position on read the kept tokens below
    their window band in E4M3 with power-of-two row scales (e4m3_rows),
    -1: never."""
    qs, ks, vs, Fs, gs = (_f32(a) for a in (qs, ks, vs, Fs, gs))
    if route == "external":
        if ext is None:
            raise ValueError("route external needs the caller's scores")
        ext = _f32(ext)
    U, G, L, d = qs.shape
    lam = min(chunk, (budget - window) // t_max) if budget >= window else 0
    n_dec = (L - 1) // chunk if L > 0 else 0
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    y = np.zeros((U, G, L, d))
    score = np.zeros((U, L))
    sel = np.full((U, n_dec, max(lam, 0)), -1, dtype=np.int32)
    S = np.zeros((U, d, d))
    z = np.zeros((U, d))
    pending = np.zeros((U, chunk))
    n_pool = np.zeros((U,), dtype=np.int32)
    part = None
    if partials:
        part = {"y_sa": np.zeros((U, G, L, d)), "lse_sa": np.zeros((U, G, L)),
                "y_la": np.zeros((U, G, L, d)), "lse_la": np.zeros((U, G, L))}
    dec64 = None
    if decay is not None:
        dec64 = np.ascontiguousarray(_f32(decay).astype(np.float64).reshape(-1))
        if dec64.shape[0] != U:
            raise ValueError("decay needs one value per unit")
    lib = _load()
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    pp = [None] * 4 if part is None else [ptr(part[n]) for n in ("y_sa", "lse_sa", "y_la", "lse_la")]
    rc = lib.still_oracle_run(U, L, d, G, window, chunk, budget, t_max, float(eps), scale,
                              ptr(qs), ptr(ks), ptr(vs), ptr(Fs), ptr(gs), int(n_threads),
                              ptr(y), ptr(score), ptr(sel), ptr(S), ptr(z), ptr(pending),
                              ptr(n_pool), MERGES[merge], *pp, ROUTES[route],
                              ptr(ext) if route == "external" else None,
                              ptr(dec64) if dec64 is not None else None, int(fp8_from))
    if rc != 0:
        raise ValueError("still_oracle_run rejected its arguments (rc=%d)" % rc)
    out = {"y": y, "score": score, "sel": sel, "S": S, "z": z, "pending": pending,
           "n_pool": n_pool, "lam": lam, "n_dec": n_dec}
    if part is not None:
        out.update(part)
    return out


def e4m3_rows(x) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rows x [n, d] (float32) as the kept pool's 8-bit store: E4M3 codes
    [n, d] uint8, scale exponents [n] (int32, scale 2^e) and the values they
    stand for [n, d] (float64). See e4m3_row in still_oracle.c."""
    x = _f32(x)
    n, d = x.shape
    codes = np.zeros((n, d), np.uint8)
    exps = np.zeros((n,), np.int32)
    values = np.zeros((n, d))
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    if _load().still_oracle_e4m3_rows(n, d, ptr(x), ptr(codes), ptr(exps), ptr(values)) != 0:
        raise ValueError("still_oracle_e4m3_rows rejected its arguments")
    return codes, exps, values
