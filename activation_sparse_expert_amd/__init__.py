"""Python binding of libmoeffn (activation-sparse MoE expert FFN, MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmoeffn.so``.  PyTorch provides device memory and the current
stream.  If the shared library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# MOEFFN_LIB names another build of the same sources (the sanitizer build)
LIB_PATH = os.environ.get("MOEFFN_LIB") or os.path.join(HERE, "libmoeffn.so")

MOE_F16, MOE_BF16, MOE_F32 = 0, 1, 2
PATH_SPARSE, PATH_DENSE, PATH_AUTO, PATH_MIXED = 0, 1, 2, 3
OP_EXPERT, OP_ROUTE, OP_LAYER, OP_CALIBRATE, OP_EAMC, OP_EXPERT_BITS = 0, 1, 2, 3, 4, 5

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_ALIGNMENT", -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP"}

EXPORTED = ["moe_route_topk", "moe_expert_forward_sparse", "moe_layer_forward",
            "moe_workspace_size", "moe_workspace_init", "moe_pack_up_int2",
            "moe_materialize_up_bf16", "moe_status_string", "moe_calibrate_threshold",
            "moe_eamc_match", "moe_expert_forward_sparse_bits", "moe_pack_up_bits",
            "moe_build_sources_sha256", "moe_expert_forward_sparse_noalloc",
            "moe_noalloc_scratch_bytes", "moe_materialize_up", "moe_transpose_down",
            "moe_auto_dense_min", "moe_mixed_dense_min"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class ExpertView(C.Structure):
    _fields_ = [("up_q", C.c_void_p), ("up_sz", C.c_void_p), ("gate_t", C.c_void_p),
                ("down", C.c_void_p), ("threshold", C.c_float)]


class LayerDesc(C.Structure):
    _fields_ = [("d", C.c_int), ("f", C.c_int), ("n_routed", C.c_int), ("n_shared", C.c_int),
                ("top_k", C.c_int), ("renormalize", C.c_int), ("wdt", C.c_int),
                ("router_w", C.c_void_p), ("rdt", C.c_int), ("router_bias", C.c_void_p),
                ("up_q", C.c_void_p), ("up_sz", C.c_void_p), ("gate_t", C.c_void_p),
                ("down", C.c_void_p), ("thresholds", C.c_void_p), ("up_dense", C.c_void_p),
                ("down_dense", C.c_void_p), ("density", C.c_float)]


class LayerTrace(C.Structure):
    _fields_ = [("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("logits", C.c_void_p),
                ("expert_count", C.c_void_p), ("masks", C.c_void_p), ("eam_row", C.c_void_p),
                ("mask_bits", C.c_void_p), ("nnz", C.c_void_p), ("expert_dense", C.c_void_p)]


_lib = None


def lib():
    """The loaded libmoeffn.  Raises if it has not been built, or if it was
    built from other sources than the ones in csrc/ (a stale binary)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoeffn.so not built ({LIB_PATH}); run __graft_entry__.build()")
        from .build import sources_sha256
        L = C.CDLL(LIB_PATH)
        L.moe_build_sources_sha256.restype = C.c_char_p
        L.moe_build_sources_sha256.argtypes = []
        built = L.moe_build_sources_sha256().decode()
        want = sources_sha256()
        if built != want:
            raise RuntimeError(f"libmoeffn.so is stale: built from sources {built[:16]}..., "
                               f"csrc/ now hashes to {want[:16]}...; run __graft_entry__.build()")
        P, I, Z = C.c_void_p, C.c_int, C.c_size_t
        L.moe_route_topk.restype = I
        L.moe_route_topk.argtypes = [P, I, I, I, P, I, P, I, I, I, P, P, P, P, P, P, P, Z, P]
        L.moe_expert_forward_sparse.restype = I
        L.moe_expert_forward_sparse.argtypes = [C.POINTER(ExpertView), I, I, I, P, I, I, P, I,
                                                P, I, P, P, P, P, P, Z, P]
        L.moe_layer_forward.restype = I
        L.moe_layer_forward.argtypes = [C.POINTER(LayerDesc), P, I, I, P, I, I,
                                        C.POINTER(LayerTrace), P, Z, P]
        L.moe_workspace_size.restype = Z
        L.moe_workspace_size.argtypes = [I, I, I, I, I, I, I]
        L.moe_workspace_init.restype = I
        L.moe_workspace_init.argtypes = [P, Z, P]
        L.moe_pack_up_int2.restype = I
        L.moe_pack_up_int2.argtypes = [P, I, I, I, P, P, P]
        L.moe_materialize_up_bf16.restype = I
        L.moe_materialize_up_bf16.argtypes = [P, P, I, I, P, P]
        L.moe_materialize_up.restype = I
        L.moe_materialize_up.argtypes = [P, P, I, I, I, P, P]
        L.moe_transpose_down.restype = I
        L.moe_transpose_down.argtypes = [P, I, I, I, P, P]
        L.moe_auto_dense_min.restype = I
        L.moe_auto_dense_min.argtypes = [C.POINTER(LayerDesc), I]
        L.moe_mixed_dense_min.restype = I
        L.moe_mixed_dense_min.argtypes = [C.POINTER(LayerDesc), I]
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [I]
        L.moe_calibrate_threshold.restype = I
        L.moe_calibrate_threshold.argtypes = [P, C.c_longlong, C.c_double, P, P, Z, P]
        L.moe_expert_forward_sparse_noalloc.restype = I
        L.moe_expert_forward_sparse_noalloc.argtypes = [C.POINTER(ExpertView), I, I, I, P, I, I,
                                                        P, I, P, I, P, P, P, P, P]
        L.moe_noalloc_scratch_bytes.restype = Z
        L.moe_noalloc_scratch_bytes.argtypes = []
        L.moe_expert_forward_sparse_bits.restype = I
        L.moe_expert_forward_sparse_bits.argtypes = [C.POINTER(ExpertView), I, I, I, I, P, I, I,
                                                     P, I, P, I, P, P, P, P, P, Z, P]
        L.moe_pack_up_bits.restype = I
        L.moe_pack_up_bits.argtypes = [P, I, I, I, I, P, P, P]
        L.moe_eamc_match.restype = I
        L.moe_eamc_match.argtypes = [P, I, I, P, P, P, P, Z, P]
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != 0:
        raise MoeError(st, what)


def _dt(t) -> int:
    import torch
    m = {torch.float16: MOE_F16, torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoeffn must be contiguous")
    return t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_size(op: int, T: int, d: int, f: int = 0, E: int = 1, k: int = 1, S: int = 0) -> int:
    return int(lib().moe_workspace_size(op, T, d, f, E, k, S))


def new_workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace tensor (uint8) of at least ``nbytes``."""
    import torch
    return torch.zeros(max(256, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=device)


def workspace_init(ws) -> None:
    _check(lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "moe_workspace_init")


@dataclass
class Expert:
    """One compressed expert on the device (layouts as in include/moeffn.h)."""
    up_q: "torch.Tensor"        # [f][d/4] uint8
    up_sz: "torch.Tensor"       # [f][d/64][2] int16/uint16 (fp16 bits)
    gate_t: "torch.Tensor"      # [f][d] fp16/bf16
    down: "torch.Tensor"        # [f][d] fp16/bf16
    threshold: float

    @property
    def d(self):
        return self.gate_t.shape[1]

    @property
    def f(self):
        return self.gate_t.shape[0]

    def view(self) -> ExpertView:
        return ExpertView(_ptr(self.up_q), _ptr(self.up_sz), _ptr(self.gate_t), _ptr(self.down),
                          float(self.threshold))


def expert_forward_sparse(expert: Expert, x, *, y=None, out_dtype=None, token_scale=None,
                          accumulate: bool = False, mask_out=None, v_out=None, mask_bits=None,
                          nnz=None, ws=None):
    """Algorithm 1 of the FloE review on x [T][d]; returns y [T][d].

    Optional exports: mask_out [T][f] uint8, v_out [T][f] fp32, mask_bits
    [T][f/64] int64 (bit l of word i = channel 64 i + l), nnz [T] int32."""
    import torch
    T, d = x.shape
    if y is None:
        y = torch.empty((T, d), dtype=out_dtype or torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(workspace_size(OP_EXPERT, T, d, expert.f), x.device)
    v = expert.view()
    st = lib().moe_expert_forward_sparse(
        C.byref(v), d, expert.f, _dt(expert.gate_t), _ptr(x), _dt(x), T, _ptr(token_scale),
        int(bool(accumulate)), _ptr(y), _dt(y), _ptr(mask_bits), _ptr(nnz), _ptr(mask_out),
        _ptr(v_out), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_expert_forward_sparse")
    return y


def expert_forward_sparse_noalloc(expert: Expert, x, *, y, token_scale=None,
                                  accumulate: bool = False, mask_out=None, v_out=None,
                                  mask_bits=None, nnz=None):
    """expert_forward_sparse through the allocation-free entry point: the
    library's static device scratch serves as the workspace, and the caller
    passes every output (y included), so nothing is allocated."""
    T, d = x.shape
    v = expert.view()
    st = lib().moe_expert_forward_sparse_noalloc(
        C.byref(v), d, expert.f, _dt(expert.gate_t), _ptr(x), _dt(x), T, _ptr(token_scale),
        int(bool(accumulate)), _ptr(y), _dt(y), _ptr(mask_bits), _ptr(nnz), _ptr(mask_out),
        _ptr(v_out), _stream())
    _check(st, "moe_expert_forward_sparse_noalloc")
    return y


def expert_forward_sparse_bits(expert: Expert, bits: int, x, *, y=None, out_dtype=None,
                               token_scale=None, accumulate: bool = False, mask_out=None,
                               v_out=None, mask_bits=None, nnz=None, ws=None):
    """Algorithm 1 with the up codes at ``bits`` (8, 4, 2 or 1) bits; y [T][d]."""
    import torch
    T, d = x.shape
    if y is None:
        y = torch.empty((T, d), dtype=out_dtype or torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(workspace_size(OP_EXPERT_BITS, T, d, expert.f), x.device)
    v = expert.view()
    st = lib().moe_expert_forward_sparse_bits(
        C.byref(v), int(bits), d, expert.f, _dt(expert.gate_t), _ptr(x), _dt(x), T,
        _ptr(token_scale), int(bool(accumulate)), _ptr(y), _dt(y), _ptr(mask_bits), _ptr(nnz),
        _ptr(mask_out), _ptr(v_out), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_expert_forward_sparse_bits")
    return y


def route_topk(x, router_w, k: int, *, renormalize: bool = True, bias=None, logits=False, ws=None):
    """Top-k routing and grouping; returns a dict of device tensors."""
    import torch
    T, d = x.shape
    E = router_w.shape[0]
    dev = x.device
    out = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
               topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
               expert_count=torch.empty(E, dtype=torch.int32, device=dev),
               expert_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
               pair_by_expert=torch.empty(T * k, dtype=torch.int32, device=dev))
    if logits:
        out["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if ws is None:
        ws = new_workspace(workspace_size(OP_ROUTE, T, d, 0, E, k), dev)
    st = lib().moe_route_topk(_ptr(x), _dt(x), T, d, _ptr(router_w), _dt(router_w), _ptr(bias), E,
                              k, int(bool(renormalize)), _ptr(out["topk_idx"]), _ptr(out["topk_w"]),
                              _ptr(out["expert_count"]), _ptr(out["expert_offset"]),
                              _ptr(out["pair_by_expert"]), _ptr(out.get("logits")), _ptr(ws),
                              ws.numel(), _stream())
    _check(st, "moe_route_topk")
    return out


@dataclass
class Layer:
    """One MoE layer: E routed + S shared experts at a fixed stride."""
    d: int
    f: int
    E: int
    S: int
    k: int
    renormalize: bool
    router_w: "torch.Tensor"      # [E][d]
    up_q: "torch.Tensor"          # [E+S][f][d/4]
    up_sz: "torch.Tensor"         # [E+S][f][d/64][2]
    gate_t: "torch.Tensor"        # [E+S][f][d]
    down: "torch.Tensor"          # [E+S][f][d]
    thresholds: "torch.Tensor"    # [E+S] fp32
    router_bias: Optional["torch.Tensor"] = None
    up_dense: Optional["torch.Tensor"] = None   # [E+S][f][d] in the weight type
    down_dense: Optional["torch.Tensor"] = None  # [E+S][d][f] W^down transposed
    density: float = 0.0                         # expected active fraction (AUTO, MIXED)

    def desc(self) -> LayerDesc:
        return LayerDesc(self.d, self.f, self.E, self.S, self.k, int(bool(self.renormalize)),
                         _dt(self.gate_t), _ptr(self.router_w), _dt(self.router_w),
                         _ptr(self.router_bias), _ptr(self.up_q), _ptr(self.up_sz),
                         _ptr(self.gate_t), _ptr(self.down), _ptr(self.thresholds),
                         _ptr(self.up_dense), _ptr(self.down_dense), float(self.density))

    def workspace_bytes(self, T: int) -> int:
        return workspace_size(OP_LAYER, T, self.d, self.f, self.E, self.k, self.S)

    def auto_dense_min(self, T: int) -> int:
        """MOE_PATH_AUTO's choice at T tokens: 1 when the call takes the dense
        path (every expert with tokens), 0 when it stays sparse."""
        desc = self.desc()
        return int(lib().moe_auto_dense_min(C.byref(desc), T))

    def mixed_dense_min(self, T: int) -> int:
        """Token count from which MOE_PATH_MIXED sends an expert to the dense
        path at T tokens (0: the call stays sparse)."""
        desc = self.desc()
        return int(lib().moe_mixed_dense_min(C.byref(desc), T))


def layer_forward(layer: Layer, x, *, path: int = PATH_SPARSE, y=None, out_dtype=None,
                  trace: Optional[dict] = None, ws=None):
    """Route and combine one layer on x [T][d]; returns y [T][d].

    ``trace`` may map any of topk_idx, topk_w, logits, expert_count, masks,
    mask_bits, nnz, expert_dense to preallocated device tensors that receive
    those exports,
    and eam_row to an int32 [E] device tensor that the call's per-expert counts
    are added into."""
    import torch
    T, d = x.shape
    if y is None:
        y = torch.empty((T, d), dtype=out_dtype or torch.float32, device=x.device)
    if ws is None:
        ws = new_workspace(layer.workspace_bytes(T), x.device)
    tr = None
    if trace:
        tr = LayerTrace(_ptr(trace.get("topk_idx")), _ptr(trace.get("topk_w")),
                        _ptr(trace.get("logits")), _ptr(trace.get("expert_count")),
                        _ptr(trace.get("masks")), _ptr(trace.get("eam_row")),
                        _ptr(trace.get("mask_bits")), _ptr(trace.get("nnz")),
                        _ptr(trace.get("expert_dense")))
    desc = layer.desc()
    st = lib().moe_layer_forward(C.byref(desc), _ptr(x), _dt(x), T, _ptr(y), _dt(y), path,
                                 C.byref(tr) if tr is not None else None, _ptr(ws), ws.numel(),
                                 _stream())
    _check(st, "moe_layer_forward")
    return y


def calibrate_threshold(v, q: float, *, out=None, ws=None):
    """Threshold t = linear-interpolation q-quantile of |v| over all of the
    fp32 device tensor v, computed on the GPU; returns a one-element fp32
    device tensor."""
    import torch
    if v.dtype != torch.float32 or not v.is_contiguous():
        raise ValueError("v must be a contiguous fp32 tensor")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=v.device)
    if ws is None:
        ws = new_workspace(workspace_size(OP_CALIBRATE, 1, 1), v.device)
    st = lib().moe_calibrate_threshold(_ptr(v), v.numel(), float(q), _ptr(out), _ptr(ws),
                                       ws.numel(), _stream())
    _check(st, "moe_calibrate_threshold")
    return out


def eamc_match(eamc, query, *, idx=None, dist=None, ws=None):
    """Cosine-distance nearest match of the int32 query [len] among the stored
    EAMs eamc [n][len] (both contiguous int32 device tensors, flattened L x E
    counts).  Returns (idx, dist): a one-element int32 tensor with the index
    (-1 when no stored EAM is valid) and, if ``dist`` was given or ``ws`` is
    None, the fp64 distances [n]."""
    import torch
    if eamc.dtype != torch.int32 or query.dtype != torch.int32:
        raise TypeError("eamc and query must be int32")
    if eamc.dim() != 2 or not eamc.is_contiguous() or not query.is_contiguous():
        raise ValueError("eamc must be a contiguous [n][len] tensor, query contiguous")
    n, ln = eamc.shape
    if query.numel() != ln:
        raise ValueError("query must have len entries")
    if idx is None:
        idx = torch.empty(1, dtype=torch.int32, device=eamc.device)
    if dist is None and ws is None:
        dist = torch.empty(n, dtype=torch.float64, device=eamc.device)
    st = lib().moe_eamc_match(_ptr(eamc), n, ln, _ptr(query), _ptr(idx), _ptr(dist), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream())
    _check(st, "moe_eamc_match")
    return idx, dist


def pack_up_int2(w_up_t, *, up_q=None, up_sz=None):
    """INT2 group-64 quantisation of up weights [f][d] on the device."""
    import torch
    f, d = w_up_t.shape
    if up_q is None:
        up_q = torch.empty((f, d // 4), dtype=torch.uint8, device=w_up_t.device)
    if up_sz is None:
        up_sz = torch.empty((f, d // 64, 2), dtype=torch.int16, device=w_up_t.device)
    st = lib().moe_pack_up_int2(_ptr(w_up_t), _dt(w_up_t), d, f, _ptr(up_q), _ptr(up_sz),
                                _stream())
    _check(st, "moe_pack_up_int2")
    return up_q, up_sz


def pack_up_bits(w_up_t, bits: int, *, up_q=None, up_sz=None):
    """Group-64 quantisation of up weights [f][d] to 8, 4, 2 or 1 bits on the
    device; returns (up_q [f][d*bits/8] uint8, up_sz [f][d/64][2])."""
    import torch
    f, d = w_up_t.shape
    if up_q is None:
        up_q = torch.empty((f, d * bits // 8), dtype=torch.uint8, device=w_up_t.device)
    if up_sz is None:
        up_sz = torch.empty((f, d // 64, 2), dtype=torch.int16, device=w_up_t.device)
    st = lib().moe_pack_up_bits(_ptr(w_up_t), _dt(w_up_t), d, f, int(bits), _ptr(up_q),
                                _ptr(up_sz), _stream())
    _check(st, "moe_pack_up_bits")
    return up_q, up_sz


def materialize_up(up_q, up_sz, d: int, dtype, *, out=None):
    """Dense-path up weights [f][d] = rne(s (q - z)) in dtype (torch.bfloat16
    or torch.float16)."""
    import torch
    f = up_q.shape[0]
    if out is None:
        out = torch.empty((f, d), dtype=dtype, device=up_q.device)
    st = lib().moe_materialize_up(_ptr(up_q), _ptr(up_sz), d, f, _dt(out), _ptr(out), _stream())
    _check(st, "moe_materialize_up")
    return out


def transpose_down(down, *, out=None):
    """Dense-path down weights: [n][d][f] (or [d][f]) = the transpose of each
    expert's down [f][d]."""
    import torch
    squeeze = down.dim() == 2
    dn = down.unsqueeze(0) if squeeze else down
    n, f, d = dn.shape
    if out is None:
        out = torch.empty((n, d, f), dtype=down.dtype, device=down.device)
    st = lib().moe_transpose_down(_ptr(dn), n, d, f, _ptr(out), _stream())
    _check(st, "moe_transpose_down")
    return out[0] if squeeze else out


def materialize_up_bf16(up_q, up_sz, d: int, *, out=None):
    """bf16 up weights [f][d] = bf16_rne(s (q - z)) for the dense path."""
    import torch
    f = up_q.shape[0]
    if out is None:
        out = torch.empty((f, d), dtype=torch.bfloat16, device=up_q.device)
    st = lib().moe_materialize_up_bf16(_ptr(up_q), _ptr(up_sz), d, f, _ptr(out), _stream())
    _check(st, "moe_materialize_up_bf16")
    return out
