"""The C ABI without a GPU: the library loads, exports what the header declares,
sizes workspaces, and rejects invalid requests on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

import activation_sparse_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeffn.h")


def _lib_or_skip():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoeffn.so not built")
    return moe.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_expert_forward_sparse", "moe_layer_forward"):
        assert n in names
    assert sorted(moe.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    L = _lib_or_skip()
    for n in declared_functions():
        assert hasattr(L, n), n
    # and nothing from the oracle leaks into it
    assert not hasattr(C.CDLL(moe.LIB_PATH), "oracle_expert_forward")


def test_status_strings():
    L = _lib_or_skip()
    for code in (0, -1, -2, -3, -4, -5):
        s = L.moe_status_string(code).decode()
        assert s and s != "unknown status"
    assert L.moe_status_string(7).decode() == "unknown status"


def test_workspace_sizes():
    _lib_or_skip()
    # one fp32 partial row per (token, channel tile): about 256 tiles at f=14336
    e = moe.workspace_size(moe.OP_EXPERT, 4, 4096, 14336)
    assert e >= 4 * 4096 * 4 * 200 and e % 256 == 0
    assert moe.workspace_size(moe.OP_EXPERT, 0, 4096, 14336) == 0
    assert moe.workspace_size(moe.OP_EXPERT, 4, 4096, 0) == 0
    # partial rows stay bounded for many tokens
    assert moe.workspace_size(moe.OP_EXPERT, 256, 4096, 14336) <= (256 << 20) + 4096
    assert moe.workspace_size(moe.OP_ROUTE, 16, 4096, 0, 8, 2) >= 4
    l1 = moe.workspace_size(moe.OP_LAYER, 16, 4096, 14336, 8, 2, 0)
    l2 = moe.workspace_size(moe.OP_LAYER, 32, 4096, 14336, 8, 2, 0)
    assert 0 < l1 < l2
    assert moe.workspace_size(moe.OP_LAYER, 16, 4096, 14336, 8, 9, 0) == 0   # k > E


FAKE = 0x10000          # 64 KiB-aligned fake device address; never dereferenced


def _view(**kw):
    v = dict(up_q=FAKE, up_sz=FAKE, gate_t=FAKE, down=FAKE, threshold=0.1)
    v.update(kw)
    return moe.ExpertView(v["up_q"], v["up_sz"], v["gate_t"], v["down"], v["threshold"])


def _expert(view=None, d=4096, f=14336, wdt=0, x=FAKE, xdt=0, T=1, y=FAKE, ydt=2, ws=FAKE,
            ws_bytes=1 << 26, scale=None, v_out=None, mask_bits=None, nnz=None):
    L = _lib_or_skip()
    v = view if view is not None else _view()
    return L.moe_expert_forward_sparse(C.byref(v), d, f, wdt, x, xdt, T, scale, 0, y, ydt,
                                       mask_bits, nnz, None, v_out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1),
    (dict(y=None), -1),
    (dict(T=0), -1),
    (dict(f=100), -1),                  # f % 64 != 0
    (dict(d=4128), -2),                 # d unsupported: not whole groups of 64
    (dict(d=16448), -2),                # wider than the widest geometry
    (dict(d=1000), -2),
    (dict(wdt=2), -2),                  # weights must be 16-bit
    (dict(xdt=1), -2),                  # x type differs from weight type
    (dict(ydt=7), -2),
    (dict(x=FAKE + 8), -3),             # x not 16-byte aligned
    (dict(y=FAKE + 2, ydt=2), -3),      # fp32 output not 4-byte aligned
    (dict(ws=None), -4),
    (dict(ws_bytes=1024), -4),
    (dict(ws=FAKE + 4), -3),
    (dict(mask_bits=FAKE + 4), -3),     # the bitmask is 64-bit words
    (dict(nnz=FAKE + 2), -3),
    (dict(ws_bytes=4 * 4096 * 256), -4),    # partial rows only: no room for staged masks
])
def test_expert_rejects(kw, code):
    assert _expert(**kw) == code


@pytest.mark.parametrize("field,val,code", [
    ("up_q", None, -1), ("gate_t", None, -1), ("down", None, -1), ("up_sz", None, -1),
    ("up_q", FAKE + 4, -3), ("gate_t", FAKE + 2, -3), ("down", FAKE + 8, -3), ("up_sz", FAKE + 2, -3),
])
def test_expert_rejects_weight_pointers(field, val, code):
    assert _expert(view=_view(**{field: val})) == code


def test_expert_null_view():
    L = _lib_or_skip()
    assert L.moe_expert_forward_sparse(None, 4096, 14336, 0, FAKE, 0, 1, None, 0, FAKE, 2, None,
                                       None, None, None, FAKE, 1 << 20, None) == -1


def _route(x=FAKE, xdt=0, T=4, d=4096, rw=FAKE, rdt=0, E=8, k=2, outs=True, ws=FAKE, ws_bytes=256):
    L = _lib_or_skip()
    o = FAKE if outs else None
    return L.moe_route_topk(x, xdt, T, d, rw, rdt, None, E, k, 1, o, o, o, o, o, None, ws, ws_bytes,
                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(rw=None), -1), (dict(T=0), -1), (dict(k=0), -1), (dict(k=9), -1),
    (dict(E=0), -1), (dict(E=2000, k=2), -1), (dict(outs=False), -1), (dict(ws=None), -4),
    (dict(ws_bytes=0), -4), (dict(xdt=5), -2), (dict(x=FAKE + 1), -3), (dict(T=40000, k=2), -2),
    (dict(d=60000), -2),
    (dict(d=4), -1), (dict(d=4100), -2),    # rows are read in 16-byte units: d % 8 == 0
])
def test_route_rejects(kw, code):
    assert _route(**kw) == code


def _layer_desc(**kw):
    base = dict(d=4096, f=14336, n_routed=8, n_shared=0, top_k=2, renormalize=1, wdt=0,
                router_w=FAKE, rdt=0, router_bias=None, up_q=FAKE, up_sz=FAKE, gate_t=FAKE,
                down=FAKE, thresholds=FAKE, up_dense=None, down_dense=None, density=0.0)
    base.update(kw)
    return moe.LayerDesc(*[base[n] for n, _ in moe.LayerDesc._fields_])


def _layer(desc=None, x=FAKE, xdt=0, T=4, y=FAKE, ydt=2, path=0, ws=FAKE, ws_bytes=1 << 30):
    L = _lib_or_skip()
    dsc = desc if desc is not None else _layer_desc()
    return L.moe_layer_forward(C.byref(dsc), x, xdt, T, y, ydt, path, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(T=0), -1), (dict(path=4), -1), (dict(path=-1), -1), (dict(ws=None), -4),
    (dict(path=2, ws_bytes=4096), -4),      # MOE_PATH_AUTO is a valid path: the workspace check follows
    (dict(path=3, ws_bytes=4096), -4),      # and MOE_PATH_MIXED
    (dict(ws_bytes=4096), -4), (dict(xdt=1), -2), (dict(path=1), -2),   # dense needs bf16 + up_dense
])
def test_layer_rejects(kw, code):
    assert _layer(**kw) == code


@pytest.mark.parametrize("dkw,code", [
    (dict(top_k=0), -1), (dict(top_k=9), -1), (dict(n_shared=-1), -1), (dict(thresholds=None), -1),
    (dict(up_q=None), -1), (dict(router_w=None), -1), (dict(f=1000), -1), (dict(d=3000), -2),
    (dict(thresholds=FAKE + 2), -3), (dict(gate_t=FAKE + 4), -3),
    (dict(n_shared=1100), -2),          # more than 1024 routed + shared rows per token
])
def test_layer_rejects_desc(dkw, code):
    assert _layer(desc=_layer_desc(**dkw)) == code


def test_layer_dense_shape_limits():
    d = _layer_desc(wdt=1, up_dense=FAKE, f=14336 + 64)   # f % 256 != 0 for the dense path
    assert _layer(desc=d, xdt=1, path=1) == -2
    # fp16 layers need the transposed down weights for the dense path
    assert _layer(desc=_layer_desc(wdt=0, up_dense=FAKE), path=1) == -2
    # the 256 x 256-tile kernels: d % 256 and f % 128
    d = _layer_desc(wdt=0, d=128, f=128, up_dense=FAKE, down_dense=FAKE)
    assert _layer(desc=d, path=1) == -2
    d = _layer_desc(wdt=0, up_dense=FAKE, down_dense=FAKE + 2)
    assert _layer(desc=d, path=1) == -3


@pytest.mark.parametrize("density,T,k,E,expect", [
    # tb = 4 chunks (d = 4096): a chunk of m tokens reads 5/16 + 4 (1 - (1 - rho)^m)
    # d f bytes; an expert goes dense once its chunks cost more than 6 / 2 = 3
    (0.3, 256, 2, 8, 4),       # chunks of 1..4 tokens: 1.51, 2.35, 2.94, 3.35 -> 4 tokens
    (0.1, 256, 2, 8, 7),       # 1.69 for a full chunk, + 1.40 for 3 more tokens -> 7
    (0.2, 256, 2, 8, 5),       # 2.67 + 1.11 -> 5
    (0.0, 256, 2, 8, 2),       # unset: 0.5 -> 2.31, 3.31 -> 2
    (0.1, 8, 2, 8, 6),         # tb = 2 at 2 tokens per expert: 3 x 1.07 + ... -> 6 <= 8
    (0.1, 4, 2, 8, 0),         # tb = 1: 6 tokens, more than the call has
])
def test_mixed_dense_min(density, T, k, E, expect):
    L = _lib_or_skip()
    dsc = _layer_desc(n_routed=E, top_k=k, up_dense=FAKE, down_dense=FAKE, density=density)
    assert L.moe_mixed_dense_min(C.byref(dsc), T) == expect
    # no dense weights: never
    assert L.moe_mixed_dense_min(C.byref(_layer_desc(density=density)), T) == 0


# MOE_PATH_AUTO decides per call.  The boundaries below are where a sweep of
# both pure paths on MI355X found the dense path overtaking the sparse one: the
# DeepSeek-V2-Lite-shaped layer (64 routed top-6 + 2 shared, d=2048, f=1408,
# 70% sparsity) was faster sparse at 12 tokens (78 against 93 us) and dense at
# 16 (98 against 101 us); the Mixtral-8x22B-shaped layer (8 routed top-2,
# d=6144, f=16384) sparse at 8 tokens (645 against 694 us), dense at 16 (821
# against 1013 us).
@pytest.mark.parametrize("shape,sparse_at,dense_at", [
    (dict(d=2048, f=1408, n_routed=64, n_shared=2, top_k=6, density=0.3), (1, 2, 4, 8, 12),
     (16, 64, 256, 4096)),
    (dict(d=6144, f=16384, n_routed=8, n_shared=0, top_k=2, density=0.3, wdt=1), (1, 2, 4, 8),
     (16, 32, 256)),
])
def test_auto_per_call_choice(shape, sparse_at, dense_at):
    L = _lib_or_skip()
    dsc = _layer_desc(up_dense=FAKE, down_dense=FAKE, **shape)
    for T in sparse_at:
        assert L.moe_auto_dense_min(C.byref(dsc), T) == 0, T
    for T in dense_at:
        assert L.moe_auto_dense_min(C.byref(dsc), T) == 1, T
    # without the transposed down weights the GEMM cannot run: sparse, except
    # the older bf16 kernels for whole calls from T k >= 8 E
    nodown = _layer_desc(up_dense=FAKE, **shape)
    for T in dense_at:
        old = shape.get("wdt", 0) == 1 and T * shape["top_k"] >= 8 * shape["n_routed"]
        assert L.moe_auto_dense_min(C.byref(nodown), T) == int(old), T
    # invalid arguments
    assert L.moe_auto_dense_min(None, 16) == 0
    assert L.moe_auto_dense_min(C.byref(dsc), 0) == 0
    assert L.moe_mixed_dense_min(None, 16) == 0


def test_auto_expected_bytes_limits():
    """AUTO's expected-bytes rule at its limits.  One token: an expert reads
    (5/16 + 4 rho) d f on the sparse path against 6 d f dense, so it stays
    sparse while 6 >= 2 (5/16 + 4 rho), i.e. rho <= 0.67, and goes dense at
    rho = 1 (thresholds that keep every channel).  A router that sends every
    token to every expert (k = E) is priced without the binomial; a huge call
    goes dense; and a tiny density keeps even many tokens per expert sparse
    (a chunk reads little more than the codes)."""
    L = _lib_or_skip()
    for rho, want in ((0.01, 0), (0.3, 0), (0.65, 0), (0.7, 1), (1.0, 1)):
        for E, k, S in ((8, 2, 0), (64, 6, 2), (4, 4, 1)):
            dsc = _layer_desc(n_routed=E, top_k=k, n_shared=S, up_dense=FAKE, down_dense=FAKE,
                              density=rho)
            assert L.moe_auto_dense_min(C.byref(dsc), 1) == want, (rho, E, k, S)
    dsc = _layer_desc(n_routed=4, top_k=4, n_shared=1, up_dense=FAKE, down_dense=FAKE, density=0.3)
    assert L.moe_auto_dense_min(C.byref(dsc), 64) == 1
    dsc = _layer_desc(n_routed=64, top_k=6, up_dense=FAKE, down_dense=FAKE, density=0.3)
    assert L.moe_auto_dense_min(C.byref(dsc), 10000) == 1
    # rho = 0.001, tb = 4: a chunk of four tokens reads 0.3285 d f, so about 16
    # tokens per expert cost about 4 x 0.3285 = 1.3 d f, under half of the
    # dense 6 d f: the call stays sparse; at 64 per expert (5.3) it goes dense
    dsc = _layer_desc(n_routed=8, top_k=2, up_dense=FAKE, down_dense=FAKE, density=0.001)
    assert L.moe_auto_dense_min(C.byref(dsc), 64) == 0
    assert L.moe_auto_dense_min(C.byref(dsc), 256) == 1


def test_prep_entry_points_reject():
    L = _lib_or_skip()
    assert L.moe_materialize_up(FAKE, FAKE, 4096, 8, 2, FAKE, None) == -2   # fp32 out
    assert L.moe_materialize_up(None, FAKE, 4096, 8, 0, FAKE, None) == -1
    assert L.moe_materialize_up(FAKE, FAKE, 100, 8, 0, FAKE, None) == -1
    assert L.moe_transpose_down(None, 1, 4096, 8, FAKE, None) == -1
    assert L.moe_transpose_down(FAKE, 0, 4096, 8, FAKE, None) == -1
    assert L.moe_transpose_down(FAKE, 1, 4096, 8, FAKE + 1, None) == -3


@pytest.mark.parametrize("field,val,path,code", [
    ("mask_bits", FAKE, 1, -2),         # the dense path has no masks to export
    ("nnz", FAKE, 1, -2),
    ("masks", FAKE, 1, -2),
    ("mask_bits", FAKE + 4, 0, -3),
    ("nnz", FAKE + 2, 0, -3),
])
def test_layer_trace_exports_rejected(field, val, path, code):
    L = _lib_or_skip()
    dsc = _layer_desc(wdt=1, up_dense=FAKE)
    tr = moe.LayerTrace(**{field: val})
    assert L.moe_layer_forward(C.byref(dsc), FAKE, 1, 4, FAKE, 2, path, C.byref(tr), FAKE,
                               1 << 30, None) == code


def test_expert_workspace_holds_mask_staging():
    _lib_or_skip()
    # T f bytes of staged byte masks (for the bitmask / nnz exports) follow the
    # partial rows
    a = moe.workspace_size(moe.OP_EXPERT, 1, 4096, 14336)
    assert a >= 4 * 4096 * 256 + 14336


def test_pack_and_materialize_reject():
    L = _lib_or_skip()
    assert L.moe_pack_up_int2(None, 2, 4096, 8, FAKE, FAKE, None) == -1
    assert L.moe_pack_up_int2(FAKE, 2, 100, 8, FAKE, FAKE, None) == -1
    assert L.moe_pack_up_int2(FAKE, 2, 4096, 0, FAKE, FAKE, None) == -1
    assert L.moe_pack_up_int2(FAKE, 9, 4096, 8, FAKE, FAKE, None) == -2
    assert L.moe_pack_up_int2(FAKE, 2, 4096, 8, FAKE + 4, FAKE, None) == -3
    assert L.moe_materialize_up_bf16(None, FAKE, 4096, 8, FAKE, None) == -1
    assert L.moe_materialize_up_bf16(FAKE, FAKE, 4095, 8, FAKE, None) == -1
    assert L.moe_workspace_init(None, 256, None) == -1
    assert L.moe_workspace_init(FAKE + 2, 256, None) == -3


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), -1), (dict(n=0), -1), (dict(n=1 << 31), -1), (dict(q=-0.01), -1),
    (dict(q=1.5), -1), (dict(q=float("nan")), -1), (dict(out=None), -1),
    (dict(v=FAKE + 2), -3), (dict(ws=None), -4), (dict(ws_bytes=64), -4),
])
def test_calibrate_rejects(kw, code):
    L = _lib_or_skip()
    a = dict(v=FAKE, n=1000, q=0.9, out=FAKE, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    assert L.moe_calibrate_threshold(a["v"], a["n"], a["q"], a["out"], a["ws"], a["ws_bytes"],
                                     None) == code
    assert L.moe_workspace_size(moe.OP_CALIBRATE, 1, 1, 0, 1, 1, 0) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), -1), (dict(q=None), -1), (dict(idx=None), -1), (dict(n=0), -1),
    (dict(ln=0), -1), (dict(ln=(1 << 17) + 1), -1), (dict(b=FAKE + 2), -3),
    (dict(idx=FAKE + 1), -3), (dict(dist=FAKE + 4), -3), (dict(dist=None, ws=None), -4),
    (dict(dist=None, ws_bytes=8 * 99), -4), (dict(dist=None, ws=FAKE + 8), -3),
])
def test_eamc_match_rejects(kw, code):
    L = _lib_or_skip()
    a = dict(b=FAKE, n=100, ln=256, q=FAKE, idx=FAKE, dist=FAKE, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    assert L.moe_eamc_match(a["b"], a["n"], a["ln"], a["q"], a["idx"], a["dist"], a["ws"],
                            a["ws_bytes"], None) == code
    assert L.moe_workspace_size(moe.OP_EAMC, 100, 256, 0, 0, 0, 0) >= 800
    assert L.moe_workspace_size(moe.OP_EAMC, 100, (1 << 17) + 1, 0, 0, 0, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), -1), (dict(bits=0), -1), (dict(d=6144), -2), (dict(d=8192), -2), (dict(d=1000), -2),
    (dict(d=448), -2),
    (dict(T=70000), -1), (dict(T=0), -1), (dict(d=256), -2), (dict(f=100), -1), (dict(x=None), -1),
    (dict(x=FAKE + 8), -3), (dict(ws=None), -4), (dict(ws_bytes=1024), -4), (dict(wdt=2), -2),
])
def test_expert_bits_rejects(kw, code):
    L = _lib_or_skip()
    a = dict(bits=4, d=4096, f=14336, wdt=0, x=FAKE, T=1, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    v = _view()
    assert L.moe_expert_forward_sparse_bits(C.byref(v), a["bits"], a["d"], a["f"], a["wdt"],
                                            a["x"], a["wdt"], a["T"], None, 0, FAKE, 2, None,
                                            None, None, None, a["ws"], a["ws_bytes"],
                                            None) == code
    assert L.moe_pack_up_bits(FAKE, 2, 4096, 8, 3, FAKE, FAKE, None) == -1
    assert L.moe_pack_up_bits(FAKE, 2, 100, 8, 4, FAKE, FAKE, None) == -1
    assert L.moe_pack_up_bits(FAKE, 2, 4096, 8, 4, FAKE + 8, FAKE, None) == -3
    assert moe.workspace_size(moe.OP_EXPERT_BITS, 4, 4096, 14336) >= \
        moe.workspace_size(moe.OP_EXPERT, 4, 4096, 14336)


def test_binding_refuses_a_stale_library(monkeypatch):
    _lib_or_skip()
    import activation_sparse_expert_amd.build as b
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(b, "sources_sha256", lambda: "0" * 64)
    with pytest.raises(RuntimeError, match="stale"):
        moe.lib()


def test_library_matches_its_sources():
    L = _lib_or_skip()
    import activation_sparse_expert_amd.build as b
    assert L.moe_build_sources_sha256().decode() == b.sources_sha256()


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", "/nonexistent/libmoeffn.so")
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()
