"""fp64 CPU oracle for the activation-sparse MoE expert FFN (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
CPU-baseline leg of ``bench.py``; never by the library.  The arithmetic lives in
``oracle.c`` (plain double-precision loops, built with gcc); this module only
marshals numpy arrays.  It shares no code with the HIP path.

What each function follows is stated in ``oracle.c``; in short:
  pack_up_int2 / dequant_up   INT2 group-64 up weights (FloE review, "混合压缩策略")
  expert_forward              Algorithm 1 of the FloE review ("高效稀疏 GEMV 内核")
  route_topk                  top-k gating (MoE-Infinity review "A3";
                              MoE-Lightning review "MoE 模型架构") and the
                              per-expert token counts (MoE-Infinity review "4.3")
  layer_forward               routed + shared experts combined, sparse or dense
  ream_add / eamc_match       request-level EAM accumulation and the cosine-
                              distance nearest stored EAM (MoE-Infinity review
                              "4.3", "4.5")
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.c")

DT = {"f16": 0, "bf16": 1, "f32": 2}


def build() -> None:
    """Compile the oracle with gcc (no fused multiply-add contraction)."""
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-shared", "-o", LIB, SRC, "-lm"])


def build_sanitized(out: str) -> str:
    """The oracle under ASan + UBSan (clang, so that one sanitizer runtime
    serves it and the library's sanitizer build in the same process); loaded
    through ORACLE_LIB."""
    clang = os.environ.get("ORACLE_SAN_CC", "/opt/rocm/llvm/bin/clang")
    subprocess.check_call([clang, "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-shared-libsan", "-shared", "-o", out, SRC,
                           "-lm"])
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = LIB
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
        L = C.CDLL(path)
        P = C.c_void_p
        I = C.c_int
        L.oracle_half_to_double.restype = C.c_double
        L.oracle_half_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_double_to_half_rne.restype = C.c_uint16
        L.oracle_double_to_half_rne.argtypes = [C.c_double]
        L.oracle_double_to_bf16_rne.restype = C.c_uint16
        L.oracle_double_to_bf16_rne.argtypes = [C.c_double]
        L.oracle_pack_up_int2.argtypes = [P, I, I, P, P]
        L.oracle_dequant_up.argtypes = [P, P, I, I, P]
        L.oracle_materialize_up_bf16.argtypes = [P, P, I, I, P]
        L.oracle_expert_forward.argtypes = [P, I, I, I, I, P, P, P, P, I, C.c_float, P, P,
                                            P, P, P, I]
        L.oracle_route_topk.argtypes = [P, I, I, I, P, I, P, I, I, I, P, P, P, P, P, P]
        L.oracle_layer_forward.argtypes = [P, I, I, I, I, P, I, P, I, I, I, I, P, P, P, P, I,
                                           P, I, P, P, P, P, P, P, P]
        L.oracle_ream_add.argtypes = [P, I, I, P]
        L.oracle_pack_up_bits.argtypes = [P, I, I, I, P, P]
        L.oracle_dequant_up_bits.argtypes = [P, P, I, I, I, P]
        L.oracle_expert_forward_bits.argtypes = [I, P, I, I, I, I, P, P, P, P, I, C.c_float, P,
                                                 P, P, P, P, I]
        L.oracle_eamc_match.restype = I
        L.oracle_eamc_match.argtypes = [P, I, I, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ scalars

def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def double_to_half_rne(v: float) -> int:
    return lib().oracle_double_to_half_rne(float(v))


def double_to_bf16_rne(v: float) -> int:
    return lib().oracle_double_to_bf16_rne(float(v))


# ------------------------------------------------------------------ INT2 up

def pack_up_int2(w_t: np.ndarray):
    """fp32 up weights [f][d] (row j = column j of W^up) -> (up_q [f][d/4] u8,
    up_sz [f][d/64][2] fp16 bits)."""
    w_t = _c(w_t, np.float32)
    f, d = w_t.shape
    assert d % 64 == 0
    q = np.zeros((f, d // 4), dtype=np.uint8)
    sz = np.zeros((f, d // 64, 2), dtype=np.uint16)
    lib().oracle_pack_up_int2(_p(w_t), d, f, _p(q), _p(sz))
    return q, sz


def dequant_up(up_q: np.ndarray, up_sz: np.ndarray, d: int) -> np.ndarray:
    """-> float64 [f][d], element [j][k] = s*(q-z) for input k of channel j."""
    up_q = _c(up_q, np.uint8)
    up_sz = _c(up_sz, np.uint16)
    f = up_q.shape[0]
    out = np.empty((f, d), dtype=np.float64)
    lib().oracle_dequant_up(_p(up_q), _p(up_sz), d, f, _p(out))
    return out


def pack_up_bits(w_t: np.ndarray, bits: int):
    """Up weights at 8, 4, 2 or 1 bits per code -> (up_q [f][d*bits/8] u8,
    up_sz [f][d/64][2] fp16 bits); 2 is the INT2 format above."""
    w_t = _c(w_t, np.float32)
    f, d = w_t.shape
    assert d % 64 == 0 and bits in (1, 2, 4, 8)
    q = np.zeros((f, d * bits // 8), dtype=np.uint8)
    sz = np.zeros((f, d // 64, 2), dtype=np.uint16)
    lib().oracle_pack_up_bits(_p(w_t), d, f, bits, _p(q), _p(sz))
    return q, sz


def dequant_up_bits(up_q, up_sz, d: int, bits: int) -> np.ndarray:
    up_q = _c(up_q, np.uint8)
    up_sz = _c(up_sz, np.uint16)
    f = up_q.shape[0]
    out = np.empty((f, d), dtype=np.float64)
    lib().oracle_dequant_up_bits(_p(up_q), _p(up_sz), d, f, bits, _p(out))
    return out


def materialize_up_bf16(up_q, up_sz, d):
    up_q = _c(up_q, np.uint8)
    up_sz = _c(up_sz, np.uint16)
    f = up_q.shape[0]
    out = np.empty((f, d), dtype=np.uint16)
    lib().oracle_materialize_up_bf16(_p(up_q), _p(up_sz), d, f, _p(out))
    return out


# ------------------------------------------------------------------ expert

def expert_forward(x_bits, xdt, up_q, up_sz, gate_bits, down_bits, wdt, thr,
                   scale=None, mask_in=None, y_init=None, bits=2):
    """Algorithm 1 on T tokens.  x_bits [T][d] (uint16 bits for f16/bf16 or
    float32), up weights in the format of ``bits`` (2: INT2).  Returns (v [T][f] f64,
    mask [T][f] u8, y [T][d] f64)."""
    xa = _c(x_bits, np.float32 if xdt == "f32" else np.uint16)
    T, d = xa.shape
    up_q = _c(up_q, np.uint8)
    up_sz = _c(up_sz, np.uint16)
    f = up_q.shape[0]
    wa = np.float32 if wdt == "f32" else np.uint16
    g = _c(gate_bits, wa)
    dn = _c(down_bits, wa)
    assert g.shape == (f, d) and dn.shape == (f, d)
    v = np.empty((T, f), dtype=np.float64)
    m = np.empty((T, f), dtype=np.uint8)
    if y_init is None:
        y = np.empty((T, d), dtype=np.float64)
        acc = 0
    else:
        y = np.array(y_init, dtype=np.float64, copy=True)
        acc = 1
    sc = None if scale is None else _c(scale, np.float64)
    mi = None if mask_in is None else _c(mask_in, np.uint8)
    lib().oracle_expert_forward_bits(int(bits), _p(xa), DT[xdt], T, d, f, _p(up_q), _p(up_sz),
                                     _p(g), _p(dn), DT[wdt], C.c_float(thr), _p(sc), _p(mi),
                                     _p(v), _p(m), _p(y), acc)
    return v, m, y


# ------------------------------------------------------------------ router

def route_topk(x_bits, xdt, router_bits, rdt, E, k, renormalize=True, bias=None):
    """Returns dict(topk_idx [T][k] i32, topk_w [T][k] f64, logits [T][E] f64,
    expert_count [E], expert_offset [E+1], pair_by_expert [T*k])."""
    xa = _c(x_bits, np.float32 if xdt == "f32" else np.uint16)
    T, d = xa.shape
    ra = _c(router_bits, np.float32 if rdt == "f32" else np.uint16)
    assert ra.shape == (E, d)
    b = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lg = np.empty((T, E), dtype=np.float64)
    cnt = np.empty(E, dtype=np.int32)
    off = np.empty(E + 1, dtype=np.int32)
    pbe = np.empty(T * k, dtype=np.int32)
    lib().oracle_route_topk(_p(xa), DT[xdt], T, d, _p(ra), DT[rdt], _p(b), E, k,
                            int(bool(renormalize)), _p(idx), _p(w), _p(lg), _p(cnt), _p(off),
                            _p(pbe))
    return dict(topk_idx=idx, topk_w=w, logits=lg, expert_count=cnt, expert_offset=off,
                pair_by_expert=pbe)


# ------------------------------------------------------------------ layer

def layer_forward(x_bits, xdt, router_bits, rdt, bias, E, k, S, renormalize,
                  up_q, up_sz, gate_bits, down_bits, wdt, thr, dense=False,
                  topk_in=None, masks_in=None, dense_experts=None):
    """One MoE layer, E routed (top-k) + S shared experts at a fixed stride.
    up_q [E+S][f][d/4], up_sz [E+S][f][d/64][2], gate/down [E+S][f][d],
    thr [E+S].  dense: every expert on the dense path; dense_experts [E+S]
    (0/1): that path for the flagged experts only.  Returns (y [T][d] f64,
    topk_idx [T][k], topk_w [T][k], masks [T][k+S][f] u8)."""
    xa = _c(x_bits, np.float32 if xdt == "f32" else np.uint16)
    T, d = xa.shape
    up_q = _c(up_q, np.uint8)
    f = up_q.shape[1]
    up_sz = _c(up_sz, np.uint16)
    wa = np.float32 if wdt == "f32" else np.uint16
    g = _c(gate_bits, wa)
    dn = _c(down_bits, wa)
    ra = _c(router_bits, np.float32 if rdt == "f32" else np.uint16)
    b = None if bias is None else _c(bias, np.float32)
    th = _c(thr, np.float32)
    assert up_q.shape == (E + S, f, d // 4) and g.shape == (E + S, f, d)
    ti = None if topk_in is None else _c(topk_in, np.int32)
    mi = None if masks_in is None else _c(masks_in, np.uint8)
    de = None if dense_experts is None else _c(dense_experts, np.uint8)
    assert de is None or de.shape == (E + S,)
    y = np.empty((T, d), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    m = np.empty((T, k + S, f), dtype=np.uint8)
    lib().oracle_layer_forward(_p(xa), DT[xdt], T, d, f, _p(ra), DT[rdt], _p(b), E, k, S,
                               int(bool(renormalize)), _p(up_q), _p(up_sz), _p(g), _p(dn),
                               DT[wdt], _p(th), int(bool(dense)), _p(de), _p(ti), _p(mi), _p(y),
                               _p(idx), _p(w), _p(m))
    return y, idx, w, m


def calibrate_threshold(v_abs: np.ndarray, sparsity: float) -> np.float32:
    """Threshold that leaves ``sparsity`` of the pooled |v| values at or below
    it: the linear-interpolation quantile of |v| over the calibration tokens
    (the pages give t_ij as an input and do not say how it is placed)."""
    return np.float32(np.quantile(np.asarray(v_abs, dtype=np.float64).ravel(), sparsity))


# ------------------------------------------------------------------ EAM

def ream_add(ream: np.ndarray, layer: int, count) -> None:
    """Add one iteration's per-expert counts of ``layer`` into the request-level
    EAM ``ream`` [L][E] int32 (in place)."""
    assert ream.dtype == np.int32 and ream.flags.c_contiguous
    c = _c(count, np.int32)
    assert c.shape == (ream.shape[1],)
    lib().oracle_ream_add(_p(ream), ream.shape[1], int(layer), _p(c))


def eamc_match(eamc, query):
    """(index of the nearest stored EAM or -1, distances [n] f64)."""
    b = _c(eamc, np.int32)
    q = _c(query, np.int32).ravel()
    n, ln = b.shape
    assert q.shape == (ln,)
    dist = np.empty(n, dtype=np.float64)
    i = lib().oracle_eamc_match(_p(b), n, ln, _p(q), _p(dist))
    return int(i), dist
