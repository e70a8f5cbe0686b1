"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a figure or worked example
printed on the expert-parallelism blog page (fixtures in tests/golden/), a
closed form, a special case that reduces to a library routine, an invariant,
or brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_synth
import oracle
from dense_reference import dense_layer, swiglu, topk_mask

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ page figures


def test_page_byte_figures():
    """Section 2.1, 2.2, 2.3 and 6.3 byte counts follow from the layer shape
    the workloads use (hidden 7168, intermediate 2048, fp16, top-8)."""
    H, I, K, E = 7168, 2048, 8, 256
    exact = {
        "hidden_row_fp16_bytes": H * 2,
        "per_expert_fp16_bytes": 3 * H * I * 2,
        "routed_layer_fp16_bytes": E * 3 * H * I * 2,
        "shared_two_experts_fp16_bytes": 2 * 3 * H * I * 2,
        "dispatch_plus_combine_per_token_fp16_bytes": 2 * K * H * 2,
        "dispatch_plus_combine_per_token_fp8_bytes": 2 * K * H * 1,
        "eight_replicas_fp16_bytes": 8 * 3 * H * I * 2,
        "replica_overhead_fraction": 8 / 256,
        "experts_with_redundancy": 256 + 8,
        "experts_per_gpu_with_redundancy": (256 + 8) // 8,
        "tp_allreduce_bytes": 2 * H * 2 * 7 / 8,
    }
    g = gold("page_figures.json")
    for f in g["figures"]:
        want = f["printed"] * g["units"][f["unit"]]
        got = exact[f["name"]]
        assert abs(got - want) <= f["rel_tol"] * want + 1e-12, (f["name"], got, want)
    c2 = moe_synth.config(2)
    assert 3 * c2.H * c2.I * c2.itemsize == 88_080_384


def test_worked_example_placement():
    """Section 2.2 Step 1: top-8 {5,23,67,89,130,155,201,244} -> GPUs
    {0,0,2,2,4,4,6,7} under section 2.1's contiguous placement."""
    g = gold("worked_example_step1.json")
    got = [oracle.gpu_of_expert(e, g["E"], g["ep_size"]) for e in g["top8"]]
    assert got == g["gpu"]
    rep_off, rep_slot, slot_experts = oracle.placement(g["E"], g["ep_size"], 0)
    idx = np.array([g["top8"]], np.int32)
    slot = oracle.slot_map(idx, rep_off, rep_slot, seed=0)
    local = [e for e, s in zip(g["top8"], slot[0]) if s >= 0]
    assert local == g["local_on_gpu0"]
    assert all(slot_experts[s] == e for e, s in zip(g["top8"], slot[0]) if s >= 0)
    # each expert of the example is local on exactly the GPU the page names
    for r in range(g["ep_size"]):
        ro, rs, se = oracle.placement(g["E"], g["ep_size"], r)
        sl = oracle.slot_map(idx, ro, rs, seed=0)[0]
        assert [e for e, s in zip(g["top8"], sl) if s >= 0] == \
            [e for e, gp in zip(g["top8"], g["gpu"]) if gp == r]


def test_placement_with_replica_matches_section_6_3():
    """Section 6.3: 256 experts + 8 redundant copies = 264 physical experts,
    33 per GPU; each GPU's extra slot holds one remote hot expert."""
    total = 0
    for r in range(8):
        rep_off, rep_slot, se = oracle.placement(256, 8, r, replica_of=(r * 32 + 40) % 256)
        assert len(se) == 33
        total += len(se)
        assert rep_off[-1] == len(rep_slot) == 257
    assert total == 264


# ------------------------------------------------------------ SplitMix64


def test_splitmix64_published_vectors():
    v = gold("splitmix64_vectors.json")
    gamma = int(v["gamma"], 16)
    for n, want in enumerate(v["from_state_0"]):
        assert oracle.splitmix64((n * gamma) % 2**64) == int(want, 16)
    assert oracle.splitmix64(1234567) == v["seed_1234567_first"]


def test_replica_choice_uses_hash_of_pair_index():
    """Two replicas of expert 40 on rank 0 (home copy remote, extra slot 32):
    the pair (t, k) goes to replica splitmix64(seed ^ (t*K+k)) mod 2."""
    rep_off, rep_slot, _ = oracle.placement(256, 8, 0, replica_of=40)
    T, K, seed = 300, 8, 99
    idx = np.tile(np.array([[40, 1, 2, 3, 4, 5, 6, 7]], np.int32), (T, 1))
    idx[:, [0, 3]] = idx[:, [3, 0]]  # expert 40 at k = 3
    slot = oracle.slot_map(idx, rep_off, rep_slot, seed)
    for t in range(T):
        r = oracle.splitmix64(seed ^ (t * K + 3)) % 2
        assert slot[t, 3] == (-1 if r == 0 else 32)
    frac = (slot[:, 3] == 32).mean()
    assert 0.35 < frac < 0.65  # binomial(300, 1/2): 5 sigma
    # tok_ids reproduce the full-batch choice on a sample of tokens
    sub = np.array([7, 100, 299], np.int32)
    s2 = oracle.slot_map(idx[sub], rep_off, rep_slot, seed, tok_ids=sub)
    assert np.array_equal(s2, slot[sub])
    # a dead replica (removed from the table) sends every pair to the survivor
    rep_slot2 = rep_slot.copy()
    ro = rep_off.copy()
    lo = ro[40]
    rep_slot2 = np.delete(rep_slot2, lo)  # drop the home copy
    ro[41:] -= 1
    s3 = oracle.slot_map(idx, ro, rep_slot2, seed)
    assert np.all(s3[:, 3] == 32)


# ------------------------------------------------------------ router


def test_router_logits_permutation_closed_form():
    """Rows of W that pick one coordinate each: logits[t][e] = h[t][pi(e)]
    (+ bias).  A transposed operand or a wrong row index fails this."""
    rng = np.random.default_rng(0)
    T, H, E = 5, 40, 12
    pi = rng.permutation(H)[:E]
    W = np.zeros((E, H), np.float16)
    W[np.arange(E), pi] = 1
    h = rng.standard_normal((T, H)).astype(np.float16)
    b = rng.standard_normal(E).astype(np.float32)
    lg = oracle.router_logits(h, W, b)
    want = h.astype(np.float32)[:, pi] + b
    assert np.array_equal(lg, want)
    assert np.array_equal(oracle.router_logits(h, W), h.astype(np.float32)[:, pi])


def test_router_logits_error_bound_fp32_and_fp16():
    """fp64 sums of exactly representable products are within the fp64
    rounding bound of the exact sum; rounding to fp32 then adds at most half
    an ulp.  Exact sums come from Python integers (values scaled to ints)."""
    rng = np.random.default_rng(1)
    T, H, E = 3, 64, 7
    h = rng.standard_normal((T, H)).astype(np.float16)
    W = rng.standard_normal((E, H)).astype(np.float16)
    lg = oracle.router_logits(h, W)
    hi = (h.astype(np.float64) * 2**24).astype(np.int64)  # fp16 * 2^24 is an integer
    wi = (W.astype(np.float64) * 2**24).astype(np.int64)
    for t in range(T):
        for e in range(E):
            exact = sum(int(a) * int(c) for a, c in zip(hi[t], wi[e])) / 2.0**48
            assert abs(float(lg[t, e]) - exact) <= 0.5 * np.spacing(np.float32(abs(exact))) + 1e-12


def test_duplicate_router_rows_tie_to_lower_id():
    rng = np.random.default_rng(2)
    T, H, E, K = 16, 32, 10, 3
    W = rng.standard_normal((E, H)).astype(np.float16)
    W[7] = W[2]  # identical rows -> bit-identical logits
    h = rng.standard_normal((T, H)).astype(np.float16)
    lg = oracle.router_logits(h, W)
    assert np.array_equal(lg[:, 7], lg[:, 2])
    idx, _ = oracle.softmax_topk(lg, E)
    for t in range(T):
        assert list(idx[t]).index(2) < list(idx[t]).index(7)


def test_topk_matches_lexsort_and_softmax_closed_forms():
    rng = np.random.default_rng(3)
    T, E, K = 200, 64, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[5, 10] = lg[5, 3] = 9.0  # exact tie at the top
    idx, w = oracle.softmax_topk(lg, K)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -lg[t].astype(np.float64)))[:K]
        assert np.array_equal(idx[t], order)
    assert idx[5, 0] == 3 and idx[5, 1] == 10
    # p_e = exp(l_e) / sum exp: check against scipy's softmax on the full row
    from scipy.special import softmax
    p = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-6, atol=0)
    # K = E: the gate weights are the whole distribution
    _, wall = oracle.softmax_topk(lg, E)
    assert np.allclose(wall.astype(np.float64).sum(1), 1.0, atol=1e-6)
    # shift invariance
    _, w2 = oracle.softmax_topk(lg + np.float32(3.0), K)
    assert np.allclose(w2, w, rtol=1e-6)
    # all equal logits: ids 0..K-1, each 1/E
    idx3, w3 = oracle.softmax_topk(np.zeros((2, E), np.float32), K)
    assert np.array_equal(idx3, np.tile(np.arange(K), (2, 1)))
    assert np.allclose(w3, 1.0 / E, rtol=1e-7)
    # logits ln(1..E): p_e = (e+1) / (E(E+1)/2)
    lg4 = np.log(np.arange(1, E + 1, dtype=np.float64)).astype(np.float32)[None]
    idx4, w4 = oracle.softmax_topk(lg4, K)
    assert np.array_equal(idx4[0], np.arange(E - 1, E - 1 - K, -1))
    assert np.allclose(w4[0], (idx4[0] + 1) / (E * (E + 1) / 2), rtol=1e-6)


def test_group_limited_topk_worked_cases():
    """Group-limited routing (expert-parallelism blog page, section 八: route
    to expert groups first, then to experts): hand-worked cases."""
    # E = 8 in G = 4 groups {0,1} {2,3} {4,5} {6,7}; group scores (best logit)
    # 5, 4, 9, 1 -> keep groups 2 and 0 (M = 2); top-3 among {0,1,4,5}.
    lg = np.array([[5, 0, 4, 4, 9, -1, 1, 1]], np.float32)
    idx, w = oracle.softmax_topk(lg, 3, groups=(4, 2))
    assert idx.tolist() == [[4, 0, 1]]
    assert oracle.softmax_topk(lg, 3)[0].tolist() == [[4, 0, 2]]  # without the limit
    # the gates stay the softmax over all 8 logits
    p = np.exp(lg[0].astype(np.float64) - 9.0)
    p /= p.sum()
    assert np.allclose(w[0], p[[4, 0, 1]], rtol=1e-6, atol=0)
    # a group's score is its best logit, not its first
    lg = np.array([[1, 0, 0, 8, 2, 2, 0, 0]], np.float32)
    assert oracle.softmax_topk(lg, 2, groups=(4, 1))[0].tolist() == [[3, 2]]
    # groups 0 and 2 tie on their best logit: the lower group id is kept
    lg = np.array([[3, 1, 0, 0, 3, 2, 0, 0]], np.float32)
    assert oracle.softmax_topk(lg, 2, groups=(4, 1))[0].tolist() == [[0, 1]]


def test_group_limited_topk_against_brute_force():
    """Random logits with ties: the kept groups are the top-M of the group
    maxima (ties to the lower group), the experts are the plain top-K of
    the logits with every other group masked out, at most M groups are
    used, and M = G is the plain top-K."""
    rng = np.random.default_rng(11)
    T, E, G, M, K = 400, 64, 8, 3, 6
    gs = E // G
    lg = (rng.integers(-20, 20, (T, E)) / 4.0).astype(np.float32)  # many exact ties
    idx, w = oracle.softmax_topk(lg, K, groups=(G, M))
    i0, w0 = oracle.softmax_topk(lg, K)
    iG, wG = oracle.softmax_topk(lg, K, groups=(G, G))
    assert np.array_equal(iG, i0) and np.array_equal(wG, w0)
    for t in range(T):
        score = lg[t].reshape(G, gs).max(1)
        keep = sorted(range(G), key=lambda g: (-float(score[g]), g))[:M]
        masked = np.full(E, -np.inf, np.float32)
        for g in keep:
            masked[g * gs:(g + 1) * gs] = lg[t, g * gs:(g + 1) * gs]
        order = np.lexsort((np.arange(E), -masked.astype(np.float64)))[:K]
        assert np.array_equal(idx[t], order), t
        assert len(set((idx[t] // gs).tolist())) <= M
    from scipy.special import softmax
    p = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-6, atol=0)


def test_shared_gate_closed_forms():
    h = np.ones((3, 8), np.float32)
    assert np.all(oracle.shared_gate(h, np.zeros(8, np.float32)) == np.float32(0.5))
    w = np.zeros(8, np.float32)
    w[0] = math.log(3.0)
    assert np.allclose(oracle.shared_gate(h, w), 0.75, rtol=1e-7)
    w[0] = -math.log(3.0)
    assert np.allclose(oracle.shared_gate(h, w), 0.25, rtol=1e-7)


# ------------------------------------------------------------ dispatch


def test_dispatch_against_stable_argsort_and_invariants():
    rng = np.random.default_rng(4)
    for T, K, S, E in [(1, 1, 1, 1), (37, 4, 5, 20), (300, 8, 33, 256), (0, 8, 4, 16)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, K), np.int32)
        ro, rs, _ = oracle.placement(E, max(1, E // S), 0) if S < E else oracle.placement(E, 1, 0)
        slot = oracle.slot_map(idx, ro, rs, seed=5) if T else np.zeros((0, K), np.int32)
        slot = np.where(slot >= S, -1, slot).astype(np.int32)
        counts, offsets, perm, inv = oracle.dispatch(slot, S)
        flat = slot.reshape(-1)
        local = np.nonzero(flat >= 0)[0]
        # brute force: stable sort of local pairs by (slot, token)
        order = local[np.lexsort((local // max(K, 1), flat[local]))]
        assert np.array_equal(perm, order)
        assert np.array_equal(counts, np.bincount(flat[local], minlength=S)[:S])
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        assert counts.sum() == len(local)
        if len(local):
            assert np.array_equal(perm[inv.reshape(-1)[local]], local)
        assert np.all(inv.reshape(-1)[flat < 0] == -1)
        for s in range(S):
            toks = perm[offsets[s]:offsets[s + 1]] // K
            assert np.all(np.diff(toks) > 0)


def test_dispatch_ep_simulation_each_pair_once():
    """Eight simulated ranks of an EP=8 group: every (t, k) is local on
    exactly one rank, and the rank counts sum to T*K."""
    rng = np.random.default_rng(6)
    T, K, E = 64, 8, 256
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    seen = np.zeros((T, K), int)
    tot = 0
    for r in range(8):
        ro, rs, _ = oracle.placement(E, 8, r)
        slot = oracle.slot_map(idx, ro, rs, seed=1)
        counts, offsets, perm, inv = oracle.dispatch(slot, 32)
        seen += inv >= 0
        tot += counts.sum()
    assert np.all(seen == 1) and tot == T * K


# ------------------------------------------------------------ fp8


def test_e4m3_codec_exhaustive_and_spec_points():
    dec = oracle.e4m3_decode_table()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert np.isnan(dec[c])
            continue
        assert oracle.e4m3_encode(dec[c]) == c, hex(c)
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert dec[0x08] == 2.0**-6 and dec[0x01] == 2.0**-9
    assert dec[0x38] == 1.0
    # round half to even between neighbouring codes
    for c in range(0, 0x7E):
        mid = (np.float64(dec[c]) + np.float64(dec[c + 1])) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.float32(mid)) == want, hex(c)


def test_e4m3_encode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 30]).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_quant_rows_scale_and_error_bound():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 512)).astype(np.float16)
    x[3] = 0
    q, s = oracle.quant_e4m3_rows(x)
    dec = oracle.e4m3_decode_table()
    xf = x.astype(np.float32)
    amax = np.abs(xf).max(1)
    for r in range(6):
        if amax[r] == 0:
            assert s[r] == 0 and np.all(q[r] == 0)
            continue
        assert s[r] == np.float32(amax[r] / np.float32(448.0))
        j = np.argmax(np.abs(xf[r]))
        assert (q[r, j] & 0x7F) == 0x7E  # the row maximum maps to 448
        back = dec[q[r]].astype(np.float64) * s[r]
        # normals keep 3 mantissa bits: relative error <= 2^-4; subnormals 2^-10 * scale
        err = np.abs(back - xf[r])
        assert np.all(err <= np.maximum(np.abs(xf[r]) * 2.0**-4, 2.0**-10 * s[r] * 1.0001))


# ------------------------------------------------------------ expert FFN


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_expert_rows_match_torch_swiglu(dtype):
    """E = 1, K = 1 reduces the layer to a textbook SwiGLU FFN; torch's CPU
    F.silu and matmul in float64 give it independently."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    R, H, I = 7, 48, 24  # non-square so a transposed operand cannot pass
    x = rng.standard_normal((R, H)).astype(dtype)
    g = (rng.standard_normal((I, H)) / np.sqrt(H)).astype(dtype)
    u = (rng.standard_normal((I, H)) / np.sqrt(H)).astype(dtype)
    d = (rng.standard_normal((H, I)) / np.sqrt(I)).astype(dtype)
    y, hm = oracle.expert_rows(x.astype(np.float64), g, u, d, want_hm=True)
    X = torch.from_numpy(x.astype(np.float64))
    G, U, D = (torch.from_numpy(m.astype(np.float64)) for m in (g, u, d))
    hm_ref = torch.nn.functional.silu(X @ G.T) * (X @ U.T)
    y_ref = hm_ref.float().double() @ D.T
    assert np.allclose(hm, hm_ref.numpy(), rtol=1e-6, atol=1e-7)
    assert np.allclose(y, y_ref.numpy(), rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------ layer


def _tiny_layer_inputs(cfg):
    h = moe_synth.gen_hidden(cfg)
    wr = moe_synth.gen_router(cfg)
    bias = moe_synth.gen_router_bias(cfg)
    experts = [moe_synth.gen_expert(cfg, e) for e in range(cfg.E)]
    shared = [moe_synth.gen_shared_expert(cfg, j) for j in range(cfg.n_shared)]
    return h, wr, bias, experts, shared


def _oracle_layer(cfg, h, wr, bias, experts, shared, rank=None, replica=None, seed=0):
    ep = cfg.ep_size if rank is not None else 1
    r = rank or 0
    ro, rs, se = oracle.placement(cfg.E, ep, r, replica_of=replica)
    sh = None
    if shared:
        sh = tuple(np.ascontiguousarray(np.stack(p)) for p in zip(*shared))
    return oracle.layer_forward(
        h=h, w_router=wr[: cfg.E], bias=bias,
        w_sg=wr[cfg.E] if cfg.n_shared else None,
        slot_weights=[experts[e] for e in se], shared=sh,
        rep_off=ro, rep_slot=rs, seed=seed, K=cfg.K,
        fp8_dispatch=cfg.dispatch == "fp8"), se


def test_layer_tiny_fp32_matches_dense_bruteforce():
    cfg = moe_synth.config(1)
    h, wr, bias, experts, shared = _tiny_layer_inputs(cfg)
    res, _ = _oracle_layer(cfg, h, wr, bias, experts, shared)
    want, logits32, mask = dense_layer(h, wr[: cfg.E], bias, wr[cfg.E], experts, shared, cfg.K)
    assert np.array_equal(res["logits"], logits32)
    assert np.array_equal(np.sort(res["topk_idx"], 1), np.nonzero(mask)[1].reshape(cfg.T, cfg.K))
    assert np.allclose(res["out"], want, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("n", [2, 3, 5])
def test_layer_scaled_configs_match_dense_bruteforce(n):
    """Workloads 2, 3, 5 with their routing structure (EP share, long tail,
    replica + fp8) at small dense sizes."""
    cfg = moe_synth.scaled_config(n, T=48, H=64, I=32, E=32, K=4, seed=n + 100,
                                  ep_size=(4 if moe_synth.config(n).ep_size > 1 else 1))
    h, wr, bias, experts, shared = _tiny_layer_inputs(cfg)
    rep = moe_synth.replica_expert(cfg)
    res, se = _oracle_layer(cfg, h, wr, bias, experts, shared,
                            rank=0 if cfg.ep_size > 1 else None, replica=rep, seed=cfg.seed)
    emask = np.zeros(cfg.E, bool)
    emask[se] = True
    xo = None
    if cfg.dispatch == "fp8":
        q, s = oracle.quant_e4m3_rows(h)
        xo = oracle.e4m3_decode_table()[q] * s[:, None]
    if rep is None:
        want, _, _ = dense_layer(h, wr[: cfg.E], bias, wr[cfg.E] if cfg.n_shared else None,
                                 experts, shared, cfg.K, expert_mask=emask, x_override=xo)
        assert np.allclose(res["out"], want, rtol=2e-6, atol=1e-6)
    else:
        # with a replica the expert of the replicated id is computed here only
        # for the pairs the hash sends to the local slot
        base_mask = emask.copy()
        base_mask[rep] = False
        want, _, mask = dense_layer(h, wr[: cfg.E], bias, None, experts, None, cfg.K,
                                    expert_mask=base_mask, x_override=xo)
        rows = res["slot"] == len(se) - 1
        t_rep = np.nonzero(rows.any(1))[0]
        p = res["topk_w"][rows]
        xr = xo[t_rep]
        y = swiglu(xr, *experts[rep]).astype(np.float32).astype(np.float64)
        want[t_rep] += p[:, None].astype(np.float64) * y
        assert np.allclose(res["out"], want, rtol=2e-6, atol=1e-6)


def test_topk_equal_E_is_dense_softmax_moe():
    cfg = moe_synth.scaled_config(1, T=16, H=32, I=16, E=6, K=6, n_shared=0, seed=11)
    h, wr, bias, experts, shared = _tiny_layer_inputs(cfg)
    res, _ = _oracle_layer(cfg, h, wr, bias, experts, None)
    x = h.astype(np.float64)
    l = (x @ wr.astype(np.float64).T).astype(np.float32).astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ys = np.stack([swiglu(x, *experts[e]) for e in range(cfg.E)], 1)  # [T, E, H]
    want = np.einsum("te,teh->th", p, ys)
    assert np.allclose(res["out"], want, rtol=1e-5, atol=1e-6)
    assert np.allclose(res["topk_w"].astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_identical_experts_give_gate_sum_times_expert():
    cfg = moe_synth.scaled_config(2, T=20, H=32, I=16, E=16, K=4, ep_size=1, seed=12)
    h, wr, bias, experts, _ = _tiny_layer_inputs(cfg)
    experts = [experts[0]] * cfg.E
    res, _ = _oracle_layer(cfg, h, wr, bias, experts, None)
    y = oracle.expert_rows(h.astype(np.float64), *experts[0]).astype(np.float64)
    want = res["topk_w"].astype(np.float64).sum(1)[:, None] * y
    assert np.allclose(res["out"], want, rtol=1e-6, atol=1e-7)


def test_rank_shares_sum_to_full_routed_layer():
    """EP simulation: the 8 rank-share partial outputs sum to the full layer's
    routed output (no shared term)."""
    cfg = moe_synth.scaled_config(2, T=24, H=32, I=16, seed=13)
    h, wr, bias, experts, _ = _tiny_layer_inputs(cfg)
    full, _ = _oracle_layer(cfg, h, wr, bias, experts, None)
    tot = np.zeros_like(full["out"], dtype=np.float64)
    for r in range(8):
        part, _ = _oracle_layer(cfg, h, wr, bias, experts, None, rank=r)
        tot += part["out"]
    assert np.allclose(tot, full["out"], rtol=1e-5, atol=1e-6)


def test_long_tail_bias_gives_sixty_percent_hot_share():
    """Section 6.1: about 30% of the experts take about 60% of the tokens."""
    cfg = moe_synth.scaled_config(3, T=4096, H=256, I=8, seed=3)
    h = moe_synth.gen_hidden(cfg)
    wr = moe_synth.gen_router(cfg)[: cfg.E]
    lg = oracle.router_logits(h, wr, moe_synth.gen_router_bias(cfg))
    idx, _ = oracle.softmax_topk(lg, cfg.K)
    hot = moe_synth.gen_hot_experts(cfg)
    share = np.isin(idx, hot).mean()
    assert len(hot) == 77
    assert 0.55 <= share <= 0.65, share


def test_near_tie_detector():
    lg = np.zeros((2, 12), np.float32)
    lg[0] = np.arange(12, dtype=np.float32)
    lg[1] = np.arange(12, dtype=np.float32)
    lg[1, 11] = lg[1, 10] + np.float32(5e-6)
    assert list(oracle.near_tie_tokens(lg, 4)) == [False, True]


def test_combine_consistent_with_layer():
    """oref_combine (staged form of Steps 4-5) against the whole-layer
    oracle, which is pinned by the dense brute force above."""
    cfg = moe_synth.config(1)
    h, wr, bias, experts, shared = _tiny_layer_inputs(cfg)
    res, se = _oracle_layer(cfg, h, wr, bias, experts, shared)
    counts, offsets, perm, inv = oracle.dispatch(res["slot"], len(se))
    y = np.zeros((len(perm), cfg.H), np.float32)
    for s in range(len(se)):
        rows = perm[offsets[s]:offsets[s + 1]] // cfg.K
        if len(rows):
            y[offsets[s]:offsets[s + 1]] = oracle.expert_rows(h[rows].astype(np.float64),
                                                             *experts[se[s]])
    shy = np.stack([oracle.expert_rows(h.astype(np.float64), *s) for s in shared])
    gs = oracle.shared_gate(h, wr[cfg.E])
    out = oracle.combine(y, inv, res["topk_w"], shy, gs)
    assert np.allclose(out, res["out"], rtol=1e-6, atol=1e-7)
    assert np.array_equal(gs, res["shared_gate"])
    # no local pair and no shared term: exact zeros
    z = oracle.combine(y, np.full_like(inv, -1), res["topk_w"])
    assert np.all(z == 0)
    # a rank share that received no pair at all (P = 0 rows of y): zeros of
    # the full [T, H] shape, the row length taken from y's columns
    z0 = oracle.combine(np.zeros((0, cfg.H), np.float32), np.full_like(inv, -1),
                        res["topk_w"])
    assert z0.shape == (len(inv), cfg.H) and np.all(z0 == 0)
    # ... or, with the shared experts, exactly their gated sum
    zs = oracle.combine(np.zeros((0, cfg.H), np.float32), np.full_like(inv, -1),
                        res["topk_w"], shy, gs)
    assert np.allclose(zs, gs[:, None] * shy.sum(0), rtol=1e-6, atol=1e-7)


def test_layer_refuses_a_token_meeting_one_slot_twice():
    """A token's experts are distinct (Step 1) and a slot holds one expert,
    so a slot sees a token at most once; a table listing slot 0 under
    experts 0 and 1 breaks that for every token routed to both, and the
    oracle refuses it rather than summing the slot twice (or overrunning
    its per-slot row buffers)."""
    T, H, I, E, K = 6, 16, 8, 4, 2
    rng = np.random.default_rng(3)
    h = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    bias = np.array([50.0, 40.0, 0.0, 0.0], np.float32)  # experts 0 and 1 win every token
    ex = [tuple(rng.standard_normal(s).astype(np.float32) for s in ((I, H), (I, H), (H, I)))
          for _ in range(2)]
    kw = dict(h=h, w_router=wr, bias=bias, w_sg=None, slot_weights=ex, shared=None, seed=0,
              K=K, fp8_dispatch=False)
    ok = oracle.layer_forward(rep_off=np.arange(E + 1, dtype=np.int32),
                              rep_slot=np.array([0, 1, -1, -1], np.int32), **kw)
    assert np.all(np.sort(ok["topk_idx"], 1) == [0, 1])
    with pytest.raises(ValueError, match="one slot"):
        oracle.layer_forward(rep_off=np.arange(E + 1, dtype=np.int32),
                             rep_slot=np.array([0, 0, -1, -1], np.int32), **kw)
