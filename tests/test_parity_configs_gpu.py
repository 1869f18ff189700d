"""GPU parity at the full sizes of the three layer workloads, on sampled
outputs the fp64 oracle computes token by token:

* a 32-layer stack of 8 Mixtral-shaped experts (d=4096, f=14336, top-2,
  80% sparsity), 64.8 GB resident, hidden state carried across layers;
* a Mixtral-8x22B-shaped layer (8 experts, d=6144, f=16384, top-2, bf16,
  256 tokens) on the dense MFMA path and on the 70%-sparse path, and at 16
  tokens under MOE_PATH_MIXED;
* a DeepSeek-V2-Lite-shaped layer (64 routed top-6 + 2 shared experts,
  d=2048, f=1408, Zipf-skewed router bias, 70% sparsity) at 1 and 64 tokens
  on the sparse path, and at 64 tokens under MOE_PATH_AUTO (the dense fp16
  MFMA call) and MOE_PATH_MIXED (per expert, on two streams).

Weights are drawn on the device (torch generator), INT2-packed by the
library's packer and held bit-exact against the oracle's packer for every
expert the oracle reads.  Routing is checked on every token, outputs and
masks on the sampled ones."""
import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import synth
from gpu_helpers import (DeviceLayer, check_layer_tokens, check_route, check_y, run_layer, say,
                         to_dev_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def route_view(tr, E):
    """The layer's exported routing as check_route expects it."""
    cnt = tr["expert_count"]
    return {"topk_idx": torch.from_numpy(tr["topk_idx"]), "topk_w": torch.from_numpy(tr["topk_w"]),
            "logits": torch.from_numpy(tr["logits"]), "expert_count": torch.from_numpy(cnt),
            "expert_offset": torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)])),
            "pair_by_expert": torch.from_numpy(np.argsort(tr["topk_idx"].ravel(), kind="stable"))}


# ------------------------------------------------------------------ 32-layer stack

@pytest.fixture(scope="module")
def stack():
    c = synth.CONFIGS[synth.CFG_STACK]
    say("drawing and packing 32 layers x 8 experts (d=4096, f=14336) on the device")
    layers = [DeviceLayer(synth.CFG_STACK, l, c["E"], 0, c["k"], c["d"], c["f"], c["wdt"],
                          c["x_scale"], c["sparsity"]) for l in range(c["L"])]
    say(f"stack resident: {torch.cuda.memory_allocated() / 1e9:.1f} GB")
    yield layers, c
    for lay in layers:
        lay.free()


@pytest.mark.parametrize("T", [1, 4, 16])
def test_stack_decode(stack, T):
    layers, c = stack
    d, E, k = c["d"], c["E"], c["k"]
    xs = synth.hidden_stream_f32(synth.CFG_STACK, c["L"], T, d, c["x_scale"])
    sampled = {0: [0], 13: list(range(min(T, 3))), 31: [T - 1]}
    nnz = []
    for l, lay in enumerate(layers):
        x_bits = synth.to_f16_bits(xs[l])
        y, tr = run_layer(lay.L, to_dev_bits(x_bits, "f16"), moe.PATH_SPARSE)
        check_route(x_bits, "f16", lay.R_bits, "f16", E, k, True, None, route_view(tr, E),
                    f"stack layer {l} router T={T}")
        nnz.append(tr["masks"].mean())
        if l in sampled:
            check_layer_tokens(lay, x_bits, y, tr, np.array(sampled[l]), False,
                               f"stack layer {l} T={T}")
    say(f"stack T={T}: realised density {np.mean(nnz):.3f} (target {1 - c['sparsity']:.2f})")
    assert abs(np.mean(nnz) - (1 - c["sparsity"])) < 0.03


# ------------------------------------------------------------------ wide bf16 layer

@pytest.fixture(scope="module")
def wide():
    c = synth.CONFIGS[synth.CFG_WIDE]
    say("drawing and packing 8 experts (d=6144, f=16384, bf16) on the device")
    lay = DeviceLayer(synth.CFG_WIDE, 0, c["E"], 0, c["k"], c["d"], c["f"], c["wdt"],
                      c["x_scale"], c["sparsity"], dense=True)
    x_bits = synth.to_bf16_bits(synth.tokens_f32(synth.CFG_WIDE, c["T"], c["d"], c["x_scale"]))
    yield lay, x_bits, c
    lay.free()


@pytest.mark.parametrize("path", [moe.PATH_DENSE, moe.PATH_SPARSE])
def test_wide_layer(wide, path):
    lay, x_bits, c = wide
    dense = path == moe.PATH_DENSE
    y, tr = run_layer(lay.L, to_dev_bits(x_bits, "bf16"), path)
    check_route(x_bits, "bf16", lay.R_bits, "bf16", c["E"], c["k"], True, None,
                route_view(tr, c["E"]), f"wide router {'dense' if dense else 'sparse'}")
    # tokens in different 64-token MFMA tiles, and the last one
    tokens = np.array([0, 77, 255]) if dense else np.array([3, 200])
    check_layer_tokens(lay, x_bits, y, tr, tokens, dense,
                       f"wide d=6144 f=16384 T=256 {'dense MFMA' if dense else '70% sparse'}")
    assert np.isfinite(y).all()


def test_wide_layer_mixed_T16(wide):
    """The wide bf16 layer at 16 tokens under MOE_PATH_MIXED (the sparse
    kernel and the 256 x 256-tile GEMM on two streams): experts with at least
    n* tokens on the dense path, the others sparse.  The flags follow n* from
    the call's counts, and y on sampled tokens matches the oracle run with the
    same per-expert paths (sparse experts fed a sparse-path call's masks)."""
    import oracle
    lay, x_all, c = wide
    T, E, k = 16, c["E"], c["k"]
    x_bits = x_all[:T]
    lay.L.density = 1.0 - c["sparsity"]
    nstar = lay.L.mixed_dense_min(T)
    assert 1 < nstar <= T
    x = to_dev_bits(x_bits, "bf16")
    flags = torch.zeros(E, dtype=torch.uint8, device="cuda")
    cnt_d = torch.empty(E, dtype=torch.int32, device="cuda")
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    y = moe.layer_forward(lay.L, x, path=moe.PATH_MIXED,
                          trace=dict(expert_dense=flags, expert_count=cnt_d, topk_idx=idx_d))
    torch.cuda.synchronize()
    cnt, fl = cnt_d.cpu().numpy(), flags.cpu().numpy()
    assert np.array_equal(fl, (cnt >= nstar).astype(np.uint8))
    assert fl.any() and not fl[cnt > 0].all(), f"not a mixed call: counts {cnt.tolist()}"
    _, tr = run_layer(lay.L, x, moe.PATH_SPARSE)
    assert np.array_equal(tr["topk_idx"], idx_d.cpu().numpy())
    tokens = np.array([0, 7, 15])
    used = set()
    for t in tokens:
        used.update(int(e) for e in tr["topk_idx"][t])
    uq, us, g, dn = lay.host_weights(used)
    y_ref, _, _, _ = oracle.layer_forward(
        x_bits[tokens], "bf16", lay.R_bits, "bf16", None, E, k, 0, True, uq, us, g, dn, "bf16",
        lay.thr, topk_in=tr["topk_idx"][tokens], masks_in=tr["masks"][tokens],
        dense_experts=fl)
    err = check_y(y.cpu().numpy()[tokens], y_ref, 2e-3, "wide d=6144 f=16384 T=16 MIXED")
    say(f"wide T=16 MIXED: n*={nstar}, dense experts {np.flatnonzero(fl).tolist()} "
        f"(counts {cnt.tolist()}), max relL2 {err:.2e}")


# ------------------------------------------------------------------ fine-grained layer

@pytest.fixture(scope="module")
def fine():
    c = synth.CONFIGS[synth.CFG_FINE]
    say("drawing and packing 64 + 2 experts (d=2048, f=1408) on the device")
    bias = synth.zipf_bias(synth.CFG_FINE, 0, c["E"], c["zipf_s"])
    lay = DeviceLayer(synth.CFG_FINE, 0, c["E"], c["S"], c["k"], c["d"], c["f"], c["wdt"],
                      c["x_scale"], c["sparsity"], bias=bias, dense=True)
    lay.L.density = 1.0 - c["sparsity"]
    yield lay, c
    lay.free()


@pytest.mark.parametrize("T", [1, 64])
def test_fine_layer(fine, T):
    lay, c = fine
    x_bits = synth.to_f16_bits(synth.tokens_f32(synth.CFG_FINE, T, c["d"], c["x_scale"]))
    y, tr = run_layer(lay.L, to_dev_bits(x_bits, "f16"), moe.PATH_SPARSE)
    check_route(x_bits, "f16", lay.R_bits, "f16", c["E"], c["k"], True, lay.bias,
                route_view(tr, c["E"]), f"fine router T={T}")
    hist = np.bincount(tr["topk_idx"].ravel(), minlength=c["E"])
    say(f"fine T={T}: experts used {int((hist > 0).sum())}/{c['E']}, max load {hist.max()}")
    tokens = np.arange(T) if T == 1 else np.array([0, 1, 31, 63])
    check_layer_tokens(lay, x_bits, y, tr, tokens, False, f"fine 64+2 T={T}")


def test_fine_layer_auto_dense_T64(fine):
    """The fine layer at 64 tokens under MOE_PATH_AUTO, which takes the dense
    fp16 MFMA path for the whole call (64-row tiles; the Zipf-hot experts and
    the shared ones in several chunks), against the oracle's dense path."""
    lay, c = fine
    T = 64
    assert lay.L.auto_dense_min(T) == 1
    x_bits = synth.to_f16_bits(synth.tokens_f32(synth.CFG_FINE, T, c["d"], c["x_scale"]))
    y, tr = run_layer(lay.L, to_dev_bits(x_bits, "f16"), moe.PATH_AUTO, want_masks=False)
    check_route(x_bits, "f16", lay.R_bits, "f16", c["E"], c["k"], True, lay.bias,
                route_view(tr, c["E"]), "fine router T=64 (AUTO)")
    check_layer_tokens(lay, x_bits, y, tr, np.array([0, 1, 31, 63]), True,
                       "fine 64+2 T=64 AUTO (dense fp16 MFMA)")


def test_fine_layer_mixed_T64(fine):
    """The fine layer at 64 tokens under MOE_PATH_MIXED: experts with at
    least n* tokens (the shared ones included) on the dense MFMA path, the
    others on the sparse kernel, the two on separate streams.  The per-expert
    flags follow n* from the call's counts, and y on sampled tokens matches
    the oracle run with the same per-expert paths (the sparse experts fed the
    masks of a sparse-path call of the same tokens)."""
    import oracle
    lay, c = fine
    T, E, S, k = 64, c["E"], c["S"], c["k"]
    nstar = lay.L.mixed_dense_min(T)
    assert 1 < nstar <= T
    x_bits = synth.to_f16_bits(synth.tokens_f32(synth.CFG_FINE, T, c["d"], c["x_scale"]))
    x = to_dev_bits(x_bits, "f16")
    flags = torch.zeros(E, dtype=torch.uint8, device="cuda")
    cnt_d = torch.empty(E, dtype=torch.int32, device="cuda")
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    y = moe.layer_forward(lay.L, x, path=moe.PATH_MIXED,
                          trace=dict(expert_dense=flags, expert_count=cnt_d, topk_idx=idx_d))
    torch.cuda.synchronize()
    cnt, fl = cnt_d.cpu().numpy(), flags.cpu().numpy()
    assert np.array_equal(fl, (cnt >= nstar).astype(np.uint8))
    assert fl.any() and not fl[cnt > 0].all(), "not a mixed call"
    _, tr = run_layer(lay.L, x, moe.PATH_SPARSE)
    assert np.array_equal(tr["topk_idx"], idx_d.cpu().numpy())
    tokens = np.array([0, 1, 31, 63])
    used = set(range(E, E + S))
    for t in tokens:
        used.update(int(e) for e in tr["topk_idx"][t])
    uq, us, g, dn = lay.host_weights(used)
    dense_experts = np.concatenate([fl, np.full(S, 1 if T >= nstar else 0, np.uint8)])
    y_ref, _, _, _ = oracle.layer_forward(
        x_bits[tokens], "f16", lay.R_bits, "f16", lay.bias, E, k, S, True, uq, us, g, dn, "f16",
        lay.thr, topk_in=tr["topk_idx"][tokens], masks_in=tr["masks"][tokens],
        dense_experts=dense_experts)
    err = check_y(y.cpu().numpy()[tokens], y_ref, 2e-3, "fine 64+2 T=64 MIXED")
    say(f"fine T=64 MIXED: n*={nstar}, {int(fl.sum())} routed experts dense, max relL2 {err:.2e}")
