"""GPU parity of the request-level EAM bookkeeping (MoE-Infinity review, "4.3":
per-layer token counts per expert, added up over a request's iterations) and
of the cosine-distance nearest stored EAM ("4.5"), through the C ABI, against
the fp64 oracle."""
import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import oracle
import synth
from gpu_helpers import DEV, say, to_dev_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# distances are formed from exact integer sums by the same fp64 operations on
# both sides; allow one rounding step of slack in case the device's square root
# or division differ in the last place
DIST_ATOL = 4e-16


def check_match(b, q, idx, dist, what):
    i_ref, d_ref = oracle.eamc_match(b, q)
    nan = np.isnan(d_ref)
    assert np.array_equal(np.isnan(dist), nan), f"{what}: NaN pattern"
    err = np.abs(dist[~nan] - d_ref[~nan]).max() if (~nan).any() else 0.0
    assert err <= DIST_ATOL, f"{what}: max |dist - oracle| {err:.3e}"
    if i_ref < 0:
        assert idx == -1, what
    else:
        # the unique answer when the runner-up is further than the slack;
        # otherwise any entry within the slack of the minimum is a valid match
        assert idx >= 0 and not nan[idx], what
        assert d_ref[idx] <= d_ref[i_ref] + 2 * DIST_ATOL, what
        srt = np.sort(d_ref[~nan])
        if len(srt) == 1 or srt[1] - srt[0] > 2 * DIST_ATOL:
            assert idx == i_ref, f"{what}: index {idx} != {i_ref}"
    say(f"{what}: n={b.shape[0]} len={b.shape[1]} idx={idx} (oracle {i_ref}) max err {err:.1e}")
    return i_ref


def gpu_match(b, q, use_ws=False):
    bd = torch.from_numpy(np.ascontiguousarray(b)).to(DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    if use_ws:
        ws = moe.new_workspace(moe.workspace_size(moe.OP_EAMC, b.shape[0], b.shape[1]))
        idx, _ = moe.eamc_match(bd, qd, ws=ws)
        torch.cuda.synchronize()
        return int(idx.item()), None
    idx, dist = moe.eamc_match(bd, qd)
    torch.cuda.synchronize()
    return int(idx.item()), dist.cpu().numpy()


# Mixtral 32 x 8, DeepSeek-V2-Lite-like 27 x 64, Arctic-like 35 x 128 (len 4480),
# and a length that is not a multiple of 4 (the 4-byte load form)
@pytest.mark.parametrize("n,L,E,k", [(1000, 32, 8, 2), (300, 27, 64, 6), (64, 35, 128, 2),
                                     (257, 3, 5, 2), (1, 32, 8, 2)])
def test_eamc_match_synthetic_collections(n, L, E, k):
    a = synth.eam_collection(90 + E, n, L, E, k)
    b, q = a[:n], a[n]
    idx, dist = gpu_match(b, q)
    i_ref = check_match(b, q, idx, dist, f"EAMC {L}x{E}")
    idx2, _ = gpu_match(b, q, use_ws=True)
    assert idx2 == idx
    # the query itself stored twice, later in the collection: distance ~0,
    # and the earlier copy wins the exact tie
    b2 = b.copy()
    j = n // 2
    b2[j] = q
    if n > 1:
        b2[-1] = q
    idx, dist = gpu_match(b2, q)
    check_match(b2, q, idx, dist, f"EAMC {L}x{E} with the query stored")
    assert idx == j or (n > 1 and dist[idx] == dist[j] and idx < j)
    if n > 1:
        assert dist[j] == dist[-1]


def test_eamc_match_unaligned_view_and_exact_ties():
    a = synth.eam_collection(95, 200, 32, 8, 2)
    flat = np.concatenate([[7], a[:200].ravel()]).astype(np.int32)
    dflat = torch.from_numpy(flat).to(DEV)
    bd = dflat[1:].view(200, 256)                 # 4-byte aligned only: the 4-byte form
    q = a[200]
    qd = torch.from_numpy(q).to(DEV)
    idx, dist = moe.eamc_match(bd, qd)
    torch.cuda.synchronize()
    check_match(a[:200], q, int(idx.item()), dist.cpu().numpy(), "EAMC unaligned view")
    # several identical rows: bit-identical distances, the lowest index chosen
    b = np.tile(a[:1], (9, 1))
    idx, dist = gpu_match(b, q)
    assert idx == 0 and np.all(dist == dist[0])


def test_eamc_match_degenerate_and_invalid_entries():
    rng = np.random.default_rng(96)
    b = rng.integers(0, 50, size=(40, 64)).astype(np.int32)
    b[3] = 0                                       # zero EAM: distance 1
    b[5, 7] = 1 << 22                              # out of range: NaN, never chosen
    b[9, 0] = -3
    q = rng.integers(0, 50, size=64).astype(np.int32)
    idx, dist = gpu_match(b, q)
    check_match(b, q, idx, dist, "EAMC invalid rows")
    assert dist[3] == 1.0 and np.isnan(dist[5]) and np.isnan(dist[9])
    # zero query: every valid distance is 1, the first valid row wins
    idx, dist = gpu_match(b, np.zeros(64, dtype=np.int32))
    check_match(b, np.zeros(64, dtype=np.int32), idx, dist, "EAMC zero query")
    assert idx == 0
    # invalid query: nothing matches
    q2 = q.copy()
    q2[1] = -1
    idx, dist = gpu_match(b, q2)
    assert idx == -1 and np.all(np.isnan(dist))
    # every stored EAM invalid
    b3 = b.copy()
    b3[:, 0] = 1 << 30
    idx, dist = gpu_match(b3, q)
    assert idx == -1 and np.all(np.isnan(dist))
    # entries at the limit: 2^22 - 1 is valid, sums stay exact
    b4 = np.full((3, 4096), (1 << 22) - 1, dtype=np.int32)
    b4[1, ::2] = 0
    q4 = np.full(4096, (1 << 22) - 1, dtype=np.int32)
    q4[1::2] = 1
    idx, dist = gpu_match(b4, q4)
    check_match(b4, q4, idx, dist, "EAMC entries at the limit")


# ------------------------------------------------------------------ rEAM rows

def test_layer_eam_row_accumulates_request_counts():
    """A request (prefill of 12 tokens, then 5 single-token decode steps) run
    through one layer with an EAM row kept across the calls: the row ends as its
    start plus every call's per-expert routed token counts."""
    from test_parity_layer_gpu import build_host_layer, device_layer
    E, S, k, d, f = 8, 1, 2, 512, 128
    experts, thr = build_host_layer(70, E, S, d, f, "f16", 0.6, 1.0)
    R_bits = synth.to_f16_bits(synth.router_f32(70, 0, E, d, std=0.5))
    L = device_layer(experts, thr, R_bits, "f16", E, S, k)
    start = np.arange(E, dtype=np.int32) * 3
    row = torch.from_numpy(start.copy()).to(DEV)
    want = start.astype(np.int64)
    for step, T in enumerate([12, 1, 1, 1, 1, 1]):
        x_bits = synth.to_f16_bits(synth.tokens_f32(71 + step, T, d, 1.0))
        tr = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=DEV),
                  topk_w=torch.empty((T, k), dtype=torch.float32, device=DEV),
                  logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
                  expert_count=torch.empty(E, dtype=torch.int32, device=DEV),
                  eam_row=row)
        moe.layer_forward(L, to_dev_bits(x_bits, "f16"), trace=tr)
        torch.cuda.synchronize()
        # the routing against the oracle (the router's logit gaps here are far
        # above fp32 rounding), the row against the GPU's own counts
        idx = tr["topk_idx"].cpu().numpy()
        cnt = np.bincount(idx.ravel(), minlength=E)
        ref = oracle.route_topk(x_bits, "f16", R_bits, "f16", E, k)
        assert np.array_equal(idx, ref["topk_idx"]), f"step {step}: routing"
        assert np.array_equal(tr["expert_count"].cpu().numpy(), cnt)
        want += cnt
        got = row.cpu().numpy()
        assert np.array_equal(got, want), f"step {step}: {got} != {want}"
    # the oracle's request-level accumulation of the same counts
    acc = np.zeros((2, E), dtype=np.int32)
    acc[1] = start
    for step, T in enumerate([12, 1, 1, 1, 1, 1]):
        x_bits = synth.to_f16_bits(synth.tokens_f32(71 + step, T, d, 1.0))
        oracle.ream_add(acc, 1, oracle.route_topk(x_bits, "f16", R_bits, "f16", E, k)["expert_count"])
    assert np.array_equal(acc[1], row.cpu().numpy())
    say(f"rEAM row after the request: {row.cpu().numpy().tolist()}")


def test_layer_eam_row_on_dense_and_auto_paths():
    """The row is added by the grouping step, which every path shares: a bf16
    layer run on the dense MFMA path and then through AUTO (which picks dense
    here) accumulates the routed counts of both calls."""
    from test_parity_layer_gpu import build_host_layer, device_layer
    T, E, S, k, d, f = 40, 4, 1, 2, 512, 256
    experts, thr = build_host_layer(72, E, S, d, f, "bf16", 0.7, 1 / 16, layer=1)
    R_bits = synth.to_bf16_bits(synth.router_f32(72, 1, E, d, std=0.5))
    L = device_layer(experts, thr, R_bits, "bf16", E, S, k, dense=True)
    row = torch.full((E,), 5, dtype=torch.int32, device=DEV)
    want = np.full(E, 5, dtype=np.int64)
    for step, path in enumerate([moe.PATH_DENSE, moe.PATH_AUTO]):
        x_bits = synth.to_bf16_bits(synth.tokens_f32(73 + step, T, d, 1.0, layer=1))
        tr = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=DEV), eam_row=row)
        moe.layer_forward(L, to_dev_bits(x_bits, "bf16"), path=path, trace=tr)
        torch.cuda.synchronize()
        idx = tr["topk_idx"].cpu().numpy()
        ref = oracle.route_topk(x_bits, "bf16", R_bits, "bf16", E, k)
        assert np.array_equal(idx, ref["topk_idx"]), f"path {path}: routing"
        want += np.bincount(idx.ravel(), minlength=E)
        got = row.cpu().numpy()
        assert np.array_equal(got, want), f"path {path}: {got} != {want}"
