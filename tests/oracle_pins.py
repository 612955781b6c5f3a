"""Pins of the QSA CPU oracle against what the pages and the mathematics fix.

Every ``pin_*`` function takes an oracle object and raises AssertionError if
the oracle disagrees with something that does not come from the oracle
itself: closed forms, brute force on tiny inputs, textbook attention
(torch's scaled_dot_product_attention in float64 on the CPU), the worked
count printed on the pages, and invariants.  The mutation battery runs all of
them against deliberately broken builds of the oracle, so each pin must be
able to fail.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS32 = float(np.finfo(np.float32).eps)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def brute_topk(s, k):
    """Block j is kept iff fewer than k candidates beat it, where i beats j
    when s_i > s_j, or s_i == s_j and i < j (lowest index wins ties)."""
    nb = len(s)
    keep = []
    for j in range(nb):
        beaten_by = sum(1 for i in range(nb) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if beaten_by < k:
            keep.append(j)
    return np.array(keep, np.int32)


def manual_token_set(sel, r, p):
    """Tokens of the selected blocks plus the incomplete tail, all <= p."""
    n = p + 1
    nb = n // r
    toks = [b * r + s for b in sel for s in range(r)] + list(range(nb * r, n))
    return np.array(sorted(toks), np.int64)


def sdpa_gated(q, K, V, gate, mask, scale=None):
    """Textbook gated GQA attention, float64 on the CPU.
    q, gate [T, Hq, D]; K, V [N, Hkv, D]; mask [T, N] bool (True = attend)."""
    q64 = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    Hq = q64.shape[1]
    Hkv = K.shape[1]
    g = Hq // Hkv
    K64 = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    V64 = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)[None]
    m = torch.from_numpy(np.asarray(mask, bool))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q64, K64.contiguous(), V64.contiguous(), attn_mask=m, scale=scale)
    o = o[0].permute(1, 0, 2).numpy()
    return o * _sig(gate)


def _dims(Hq, Hkv, D, HI, dI, r, budget):
    return dict(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_idx_heads=HI, idx_dim=dI,
                block_size=r, budget=budget, attn_scale=0.0, idx_scale=0.0)


def _rand_seq(rng, n, Hq, Hkv, D, HI, dI):
    K = (rng.standard_normal((n, Hkv, D)) * 0.7).astype(np.float32)
    V = rng.standard_normal((n, Hkv, D)).astype(np.float32)
    kI = (rng.standard_normal((n, dI)) / math.sqrt(dI)).astype(np.float32)
    q = (rng.standard_normal((n, Hq, D)) * 0.7).astype(np.float32)
    qI = rng.standard_normal((n, HI, dI)).astype(np.float32)
    w = rng.random((n, HI)).astype(np.float32)
    gate = rng.standard_normal((n, Hq, D)).astype(np.float32)
    return K, V, kI, q, qI, w, gate


# ---------------------------------------------------------------- pooling
def pin_pool_exact(o):
    """Mean of exactly representable values is exact: compare bit for bit,
    for a power-of-two block and for a block of 12; the tail is not pooled."""
    rng = np.random.default_rng(11)
    for r in (16, 12):
        n, dI = r * 5 + 7, 8
        kI = rng.integers(-64, 64, size=(n, dI)).astype(np.float32) / 16
        pooled = o.pool(kI, r)
        assert pooled.shape == (5, dI)
        ref = kI[:5 * r].astype(np.float64).reshape(5, r, dI).sum(axis=1) / r
        assert np.array_equal(pooled, ref.astype(np.float32))


def pin_pool_random(o):
    """Random keys: the fp32 block mean is within the summation error bound of
    the exact mean, and there are floor(3002/4) = 750 complete blocks (the
    LocalAI QSA-block commit, section on the context length)."""
    rng = np.random.default_rng(12)
    r, dI, n = 4, 64, 3002
    kI = (rng.standard_normal((n, dI)) / 8).astype(np.float32)
    pooled = o.pool(kI, r)
    assert pooled.shape == (750, dI)
    blk = kI[:750 * r].astype(np.float64).reshape(750, r, dI)
    ref = blk.mean(axis=1)
    bound = (r + 1) * EPS32 * np.abs(blk).sum(axis=1) / r
    assert np.all(np.abs(pooled - ref) <= bound)


# ---------------------------------------------------------------- scores
def pin_scores_onehot(o):
    """One-hot indexer queries: s_j = sum_h w_h relu(c alpha_h pooled_j[x_h])
    in closed form; one head has a negative alpha so the relu acts."""
    rng = np.random.default_rng(13)
    HI, dI, nb = 3, 16, 40
    pooled = (rng.standard_normal((nb, dI)) / 8).astype(np.float32)
    xs, alpha = [3, 7, 12], [0.5, -2.0, 4.0]
    qI = np.zeros((HI, dI), np.float32)
    for h in range(HI):
        qI[h, xs[h]] = alpha[h]
    w = np.array([0.75, 0.5, 0.25], np.float32)
    c = np.float32(1 / math.sqrt(dI))
    s = o.scores(qI, w, pooled, float(c))
    ref = sum(float(w[h]) * np.maximum(0.0, float(c) * alpha[h] * pooled[:, xs[h]].astype(np.float64))
              for h in range(HI))
    assert np.allclose(s, ref, rtol=4 * EPS32, atol=1e-12)
    assert (s >= 0).all()


def pin_scores_random(o):
    """Random inputs: scores equal the float64 formula within fp32 error."""
    rng = np.random.default_rng(14)
    HI, dI, nb = 4, 64, 300
    pooled = (rng.standard_normal((nb, dI)) / 8).astype(np.float32)
    qI = (rng.standard_normal((HI, dI)) / 8).astype(np.float32)
    w = rng.random(HI).astype(np.float32)
    c = float(np.float32(1 / math.sqrt(dI)))
    s = o.scores(qI, w, pooled, c)
    dots = pooled.astype(np.float64) @ qI.astype(np.float64).T          # [nb, HI]
    ref = (np.maximum(0.0, c * dots) * w.astype(np.float64)).sum(axis=1)
    mag = (np.abs(pooled.astype(np.float64)) @ np.abs(qI.astype(np.float64)).T * c
           * w.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(s - ref) <= (dI + 4) * EPS32 * mag + 1e-30)


def pin_value_gate(o):
    """Scores are positively homogeneous in the indexer query and in the
    softmax scale (so a selection cannot see either), while the values move
    exactly by the factor (the value gate of the LocalAI QSA-block commit)."""
    rng = np.random.default_rng(15)
    HI, dI, nb = 4, 32, 120
    pooled = (rng.standard_normal((nb, dI)) / 8).astype(np.float32)
    qI = (rng.standard_normal((HI, dI)) / 8).astype(np.float32)
    w = rng.random(HI).astype(np.float32)
    c = float(np.float32(1 / math.sqrt(dI)))
    s1 = o.scores(qI, w, pooled, c)
    s2 = o.scores(2 * qI, w, pooled, c)
    s3 = o.scores(qI, w, pooled, 2 * c)
    assert np.array_equal(s2, 2 * s1) and np.array_equal(s3, 2 * s1)
    assert np.array_equal(o.topk(s1, 16), o.topk(s2, 16))
    assert not np.array_equal(s1, s2)


# ---------------------------------------------------------------- top-k
def pin_topk_bruteforce(o):
    """Top-k against brute force on tiny inputs, with many exact ties."""
    rng = np.random.default_rng(16)
    for trial in range(400):
        nb = int(rng.integers(0, 13))
        k = int(rng.integers(1, 15))
        if trial % 2:
            s = rng.integers(0, 4, nb).astype(np.float32)
        else:
            s = rng.standard_normal(nb).astype(np.float32)
        got = o.topk(s, k)
        assert np.array_equal(got, brute_topk(s, k)), (s, k, got)
    assert np.array_equal(o.topk(np.ones(6, np.float32), 2), [0, 1])
    assert np.array_equal(o.topk(np.array([0, 3, 1, 3, 2], np.float32), 3), [1, 3, 4])


def pin_worked_count(o):
    """kv_len 3002, ratio 4, budget 2048: 512 of 750 blocks selected plus a
    2-token tail = 2050 keys; 8 x 2050 = 16400 against a dense 8 x 3002 =
    24016 (LocalAI QSA-block commit, section on the context length; numbers
    in tests/golden/qsa_worked_count.json)."""
    g = json.load(open(os.path.join(GOLDEN, "qsa_worked_count.json")))
    n, r, budget = g["kv_len"], g["compress_ratio"], g["budget"]
    rng = np.random.default_rng(17)
    nb = n // r
    assert nb == g["candidate_blocks"]
    s = rng.standard_normal(nb).astype(np.float32)
    sel = o.topk(s, budget // r)
    assert sel.size == g["selected_blocks"]
    toks = o.token_set(sel, r, n - 1)
    f = g["keys_visited_factor"]
    assert f * toks.size == g["keys_visited_qsa"] and f * n == g["keys_visited_dense"]
    assert toks.size <= min(n, g["visible_width_bound"]) == budget + r - 1
    # the same through the whole per-query path
    Hq, Hkv, D, HI, dI = 2, 1, 8, 1, 8
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    res = o.sequence(_dims(Hq, Hkv, D, HI, dI, r, budget), K, V, kI, np.array([n - 1]),
                     q[:1], qI[:1], w[:1], gate[:1])
    assert res["n_blocks"][0] == g["selected_blocks"]
    assert f * res["n_tokens"][0] == g["keys_visited_qsa"]


def pin_width_bound(o):
    """|U| = r*min(k, nb) + tail and |U| <= min(n, budget + r - 1) (porting
    article, width bound)."""
    rng = np.random.default_rng(18)
    for r in (4, 16, 64):
        for budget in (r, 4 * r, 32 * r):
            k = budget // r
            for p in list(range(0, 3 * r)) + list(rng.integers(0, 60 * r, 30)):
                n = p + 1
                nb = n // r
                sel = o.topk(rng.standard_normal(nb).astype(np.float32), k)
                toks = o.token_set(sel, r, int(p))
                assert toks.size == r * min(k, nb) + (n - r * nb)
                assert toks.size <= min(n, budget + r - 1)


def pin_token_set(o):
    """Token set = selected blocks + tail, ascending, unique, never above p."""
    rng = np.random.default_rng(19)
    for r in (4, 16):
        for p in range(0, 10 * r):
            n = p + 1
            nb = n // r
            sel = o.topk(rng.standard_normal(nb).astype(np.float32), 3)
            toks = o.token_set(sel, r, p)
            assert np.array_equal(toks, manual_token_set(sel, r, p))
            assert toks.size == 0 or toks.max() <= p
            assert p in toks if (n % r) else True


# ---------------------------------------------------------------- attention
def pin_dense_equivalence(o):
    """Budget >= context: every candidate is selected and QSA equals dense
    causal gated GQA (porting article, dense-equality bring-up); the dense
    layer mode (ratio 0) equals it too."""
    rng = np.random.default_rng(20)
    Hq, Hkv, D, HI, dI, r, n = 4, 2, 16, 2, 8, 8, 45
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    mask = np.tril(np.ones((n, n), bool))
    ref = sdpa_gated(q, K, V, gate, mask)
    for rr, budget in ((r, 64), (r, 48), (0, 0)):
        res = o.sequence(_dims(Hq, Hkv, D, HI, dI, rr, budget), K, V, kI, np.arange(n),
                         q, qI, w, gate)
        assert np.abs(res["out"] - ref).max() < 2e-6, (rr, budget)


def pin_sparse_vs_masked_sdpa(o):
    """Above the budget: brute-force selection on the oracle's scores plus a
    hand-built token set, fed as a mask to textbook attention, reproduces the
    oracle output; the scores match the float64 formula."""
    rng = np.random.default_rng(21)
    Hq, Hkv, D, HI, dI, r, budget, n = 4, 2, 16, 3, 8, 8, 32, 160
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    res = o.sequence(_dims(Hq, Hkv, D, HI, dI, r, budget), K, V, kI, np.arange(n),
                     q, qI, w, gate, want_scores=True)
    k = budget // r
    c = float(np.float32(1 / math.sqrt(dI)))
    nbf = n // r
    pooled64 = kI[:nbf * r].astype(np.float64).reshape(nbf, r, dI).mean(axis=1)
    mask = np.zeros((n, n), bool)
    for p in range(n):
        nb = (p + 1) // r
        s = res["scores"][p, :nb]
        ref_s = (np.maximum(0.0, c * (pooled64[:nb] @ qI[p].astype(np.float64).T))
                 * w[p].astype(np.float64)).sum(axis=1)
        assert np.allclose(s, ref_s, rtol=1e-5, atol=1e-7)
        assert np.all(np.isneginf(res["scores"][p, nb:]))
        sel = brute_topk(s, k)
        assert np.array_equal(res["sel"][p, :sel.size], sel)
        assert np.all(res["sel"][p, sel.size:] == -1)
        assert res["n_blocks"][p] == sel.size
        mask[p, manual_token_set(sel, r, p)] = True
    assert mask.sum(axis=1).min() > 0 and (mask.sum(axis=1) < np.arange(1, n + 1)).any()
    ref = sdpa_gated(q, K, V, gate, mask)
    assert np.abs(res["out"] - ref).max() < 2e-6


def pin_zero_query_probe(o):
    """q = 0 makes the softmax uniform: out = sigmoid(g) * mean of V over U.
    Probe columns of V reveal |tail|/|U| exactly and that no future row is
    read."""
    rng = np.random.default_rng(22)
    Hq, Hkv, D, HI, dI, r, budget, n = 2, 1, 8, 2, 8, 4, 12, 64
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    q[:] = 0
    for p in (22, 37, 38, 41, 50):
        nb = (p + 1) // r
        tau = p + 1 - r * nb
        V2 = V.copy()
        V2[:, :, 0] = 0
        V2[r * nb:p + 1, :, 0] = 1          # the tail rows
        V2[:, :, 1] = 0
        V2[p + 1:, :, 1] = 1                # every future row
        res = o.sequence(_dims(Hq, Hkv, D, HI, dI, r, budget), K, V2, kI, np.array([p]),
                         q[p:p + 1], qI[p:p + 1], w[p:p + 1], gate[p:p + 1])
        nU = r * min(budget // r, nb) + tau
        g0 = _sig(gate[p, :, 0])
        assert np.allclose(res["out"][0, :, 0], g0 * tau / nU, rtol=1e-6, atol=1e-9)
        assert np.all(res["out"][0, :, 1] == 0)


def pin_single_token(o):
    """Position 0: the only visible token is itself, out = sigmoid(g) V[0]."""
    rng = np.random.default_rng(23)
    Hq, Hkv, D, HI, dI = 4, 2, 16, 2, 8
    K, V, kI, q, qI, w, gate = _rand_seq(rng, 9, Hq, Hkv, D, HI, dI)
    res = o.sequence(_dims(Hq, Hkv, D, HI, dI, 4, 8), K, V, kI, np.array([0]),
                     q[:1], qI[:1], w[:1], gate[:1])
    ref = V[0][np.arange(Hq) // (Hq // Hkv)].astype(np.float64) * _sig(gate[0])
    assert np.allclose(res["out"][0], ref, rtol=1e-6, atol=1e-9)


def pin_gqa_equals_mha(o):
    """Query head h reads KV head h // (Hq/Hkv): GQA equals MHA over KV heads
    duplicated in contiguous groups."""
    rng = np.random.default_rng(24)
    Hq, Hkv, D, HI, dI, r, budget, n = 4, 2, 8, 2, 8, 4, 8, 40
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    dup = np.arange(Hq) // (Hq // Hkv)
    pos = np.arange(n)
    a = o.sequence(_dims(Hq, Hkv, D, HI, dI, r, budget), K, V, kI, pos, q, qI, w, gate)
    b = o.sequence(_dims(Hq, Hq, D, HI, dI, r, budget), K[:, dup], V[:, dup], kI, pos,
                   q, qI, w, gate)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["sel"], b["sel"])


def pin_nan_poison(o):
    """NaN in every row outside a query's token set (future rows and
    unselected blocks) leaves its output unchanged: the consumer gathers, it
    does not mask (LocalAI QSA-block commit, NaN-poison probe)."""
    rng = np.random.default_rng(25)
    Hq, Hkv, D, HI, dI, r, budget, n = 2, 1, 8, 2, 8, 4, 8, 60
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    dims = _dims(Hq, Hkv, D, HI, dI, r, budget)
    for p in (17, 30, 45):
        args = (np.array([p]), q[p:p + 1], qI[p:p + 1], w[p:p + 1], gate[p:p + 1])
        base = o.sequence(dims, K, V, kI, *args)
        U = manual_token_set(base["sel"][0, :base["n_blocks"][0]], r, p)
        K2, V2 = K.copy(), V.copy()
        off = np.setdiff1d(np.arange(n), U)
        K2[off] = np.nan
        V2[off] = np.nan
        pois = o.sequence(dims, K2, V2, kI, *args)
        assert np.array_equal(pois["out"], base["out"])


def pin_planted_selected(o):
    """Blocks whose indexer keys carry a large shared offset along a direction
    the query favours are selected (the relevance the indexer exists for)."""
    rng = np.random.default_rng(26)
    Hq, Hkv, D, HI, dI, r, budget, n = 2, 1, 8, 2, 16, 8, 32, 400
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    u = rng.standard_normal(dI)
    u /= np.linalg.norm(u)
    planted = [3, 17, 29, 41]
    for b in planted:
        kI[b * r:(b + 1) * r] += (1.5 * u).astype(np.float32)
    qI[:] = np.abs(qI) * np.sign(u)[None, None, :]
    res = o.sequence(_dims(Hq, Hkv, D, HI, dI, r, budget), K, V, kI, np.array([n - 1]),
                     q[-1:], qI[-1:], w[-1:], gate[-1:])
    assert set(planted) <= set(res["sel"][0].tolist())

# ------------------------------------------------ 8-bit K/V storage contract
def pin_e4m3_decode_matches_torch(o):
    """Every one of the 256 codes decodes to torch's float8_e4m3fn value (the
    OCP E4M3 format), NaN codes included."""
    codes = np.arange(256, dtype=np.uint8)
    got = o.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all((got == ref) | both_nan)
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


def pin_e4m3_encode_rounding(o):
    """Encoding is round-to-nearest-even to the finite codes: it inverts the
    decoding on every finite code, agrees with torch's float8_e4m3fn
    conversion on random values and on every midpoint between neighbouring
    codes (ties to the even code), and saturates at +-448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = o.e4m3_decode(codes)
    assert np.array_equal(o.e4m3_encode(vals), codes)
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.standard_normal(3000) * 30, rng.standard_normal(1000) * 0.01,
                        rng.uniform(-440, 440, 500)]).astype(np.float32)
    pos = np.sort(np.unique(o.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1].astype(np.float64) + pos[1:]) / 2)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3_encode(x), ref)
    big = np.array([448.0, 449.0, 470.0, 1e6, -500.0], np.float32)
    assert np.array_equal(o.e4m3_encode(big), np.array([0x7E, 0x7E, 0x7E, 0x7E, 0xFE], np.uint8))


def pin_fwht_is_sylvester_hadamard(o):
    """The transform is multiplication by the Sylvester Hadamard matrix
    (H_1 = [1], H_2n = [[H, H], [H, -H]]): exact on small integers, and
    applying it twice multiplies by n."""
    for n in (2, 8, 128):
        H = np.array([[1.0]])
        while H.shape[0] < n:
            H = np.block([[H, H], [H, -H]])
        rng = np.random.default_rng(n)
        x = rng.integers(-8, 9, size=(5, n)).astype(np.float32)
        assert np.array_equal(o.fwht(x), (x.astype(np.float64) @ H.T).astype(np.float32))
        assert np.array_equal(o.fwht(o.fwht(x)), x * n)


def pin_kv8_storage_is_transparent_when_exact(o):
    """With K/V whose stored form is exact (values on the 8-bit grid; with
    rotation, K = H e / D and V = H f / D for small integers e, f, so the
    rotated rows are the integers themselves), QSA over the 8-bit storage
    equals QSA over the plain K/V: the rotation of the query, the 1/D on the
    scores and the un-rotation of the output cancel exactly as the storage
    contract says."""
    rng = np.random.default_rng(41)
    Hq, Hkv, D, HI, dI, r, budget, n = 4, 2, 32, 2, 16, 8, 48, 200
    _, _, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    dims = _dims(Hq, Hkv, D, HI, dI, r, budget)
    pos = np.array([37, 120, n - 1])
    # no rotation: values on the grid (multiples of 1/8 times a power of two scale)
    scale = 0.25
    Kg = (rng.integers(-15, 16, size=(n, Hkv, D)) / 8.0 * scale).astype(np.float32)
    Vg = (rng.integers(-15, 16, size=(n, Hkv, D)) / 8.0 * scale).astype(np.float32)
    Kc = o.kv8_encode(Kg, False, 1.0 / scale)
    Vc = o.kv8_encode(Vg, False, 1.0 / scale)
    assert np.array_equal(o.e4m3_decode(Kc) * np.float32(scale), Kg)
    a = o.sequence_kv8(dims, Kc, Vc, False, scale, scale, kI, pos, q[pos], qI[pos], w[pos],
                       gate[pos])
    b = o.sequence(dims, Kg, Vg, kI, pos, q[pos], qI[pos], w[pos], gate[pos])
    assert np.array_equal(a["sel"], b["sel"])
    assert np.allclose(a["out"], b["out"], rtol=1e-5, atol=1e-6)
    # different scales for K and V
    Vh = (Vg * np.float32(2.0)).astype(np.float32)
    a = o.sequence_kv8(dims, Kc, o.kv8_encode(Vh, False, 1.0 / (2 * scale)), False, scale,
                       2 * scale, kI, pos, q[pos], qI[pos], w[pos], gate[pos])
    b = o.sequence(dims, Kg, Vh, kI, pos, q[pos], qI[pos], w[pos], gate[pos])
    assert np.allclose(a["out"], b["out"], rtol=1e-5, atol=1e-6)
    # rotation: the rotated rows are small integers
    e = rng.integers(-6, 7, size=(n, Hkv, D)).astype(np.float32)
    f = rng.integers(-6, 7, size=(n, Hkv, D)).astype(np.float32)
    Kr = o.fwht(e) / np.float32(D)
    Vr = o.fwht(f) / np.float32(D)
    Kc = o.kv8_encode(Kr, True, 1.0)
    Vc = o.kv8_encode(Vr, True, 1.0)
    assert np.array_equal(o.e4m3_decode(Kc), e) and np.array_equal(o.e4m3_decode(Vc), f)
    a = o.sequence_kv8(dims, Kc, Vc, True, 1.0, 1.0, kI, pos, q[pos], qI[pos], w[pos],
                       gate[pos])
    b = o.sequence(dims, Kr, Vr, kI, pos, q[pos], qI[pos], w[pos], gate[pos])
    assert np.array_equal(a["sel"], b["sel"])
    assert np.allclose(a["out"], b["out"], rtol=1e-4, atol=1e-6)
    # and the storage is not an identity: unrotated storage of the same rows differs
    c = o.sequence_kv8(dims, o.kv8_encode(Kr, False, 64.0), o.kv8_encode(Vr, False, 64.0), False,
                       1 / 64.0, 1 / 64.0, kI, pos, q[pos], qI[pos], w[pos], gate[pos])
    assert not np.allclose(c["out"], b["out"], rtol=1e-4, atol=1e-6)



# ------------------------------------------------------------- block front end
def _complex_rope(x, R, theta, pos):
    """Rotate-half RoPE written as complex multiplication in float64: the
    pair (x_i, x_{i+R/2}) is the complex number x_i + j x_{i+R/2}, turned by
    exp(j pos theta^(-2i/R))."""
    x = np.asarray(x, np.float64).copy()
    h = R // 2
    if h == 0:
        return x
    i = np.arange(h, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * np.power(float(theta), -2.0 * i / R)
    z = (x[..., :h] + 1j * x[..., h:R]) * np.exp(1j * ang)
    x[..., :h], x[..., h:R] = z.real, z.imag
    return x


def pin_rope_against_complex_rotation(o):
    """RoPE equals the complex-number rotation of each rotate-half pair; at
    position 0 it is the identity bit for bit; values past the rotary dims
    are untouched bit for bit."""
    rng = np.random.default_rng(40)
    for n, R, theta in ((16, 16, 10000.0), (64, 32, 1e6), (12, 8, 500.0)):
        x = rng.standard_normal((7, n)).astype(np.float32)
        pos = np.array([0, 1, 2, 17, 1000, 65535, 262143])
        got = o.rope(x, R, theta, pos)
        ref = _complex_rope(x, R, theta, pos)
        assert np.abs(got - ref).max() < 4 * EPS32 * np.abs(x).max() * 2, (n, R)
        assert np.array_equal(got[0], x[0])
        assert np.array_equal(got[:, R:], x[:, R:])


def pin_rope_relative_position(o):
    """<rope(q, p), rope(k, s)> depends on p - s only (shift both by m)."""
    rng = np.random.default_rng(41)
    q = rng.standard_normal((5, 32)).astype(np.float32)
    k = rng.standard_normal((5, 32)).astype(np.float32)
    p, s = np.array([3, 50, 700, 9, 1]), np.array([0, 49, 100, 9, 300])
    for m in (1, 37, 4096):
        a = np.sum(o.rope(q, 32, 10000.0, p).astype(np.float64) *
                   o.rope(k, 32, 10000.0, s), axis=1)
        b = np.sum(o.rope(q, 32, 10000.0, p + m).astype(np.float64) *
                   o.rope(k, 32, 10000.0, s + m), axis=1)
        assert np.abs(a - b).max() < 1e-4, m


def pin_rms_norm_closed_forms(o):
    """RMSNorm with the (1 + w) weight: a constant row c gives
    sign(c) (1 + w) / sqrt(1 + eps/c^2); a row with mean square 1 and eps 0
    gives x (1 + w); the result does not change when the row is scaled."""
    from oracle import block as ob
    w = np.linspace(-0.5, 0.5, 8).astype(np.float32)
    for c in (2.0, -0.25):
        got = ob.rms_norm(np.full((1, 8), c, np.float32), w, 1e-6)
        ref = np.sign(c) * (1.0 + w.astype(np.float64)) / math.sqrt(1.0 + 1e-6 / c ** 2)
        assert np.abs(got[0] - ref).max() < 2 * EPS32
    x = np.array([[1, -1, 1, 1, -1, -1, 1, -1]], np.float32)
    assert np.array_equal(ob.rms_norm(x, w, 0.0), (x * (1.0 + w)).astype(np.float32))
    y = np.random.default_rng(42).standard_normal((3, 8)).astype(np.float32)
    assert np.abs(ob.rms_norm(y, w, 0.0) - ob.rms_norm(4 * y, w, 0.0)).max() < 4 * EPS32


def pin_pooled_key_rotation(o):
    """With rotary indexer keys each pooled key is rotated at its block's
    first position: scores equal the float64 formula on means rotated by
    complex multiplication at j*r."""
    rng = np.random.default_rng(43)
    Hq, Hkv, D, HI, dI, r, n = 2, 1, 8, 2, 16, 4, 37
    K, V, kI, q, qI, w, gate = _rand_seq(rng, n, Hq, Hkv, D, HI, dI)
    dims = _dims(Hq, Hkv, D, HI, dI, r, 8)
    dims.update(idx_rope_dim=12, idx_rope_theta=100.0)
    pos = np.array([n - 1, 20])
    res = o.sequence(dims, K, V, kI, pos, q[pos], qI[pos], w[pos], gate[pos], want_scores=True)
    nb = n // r
    pooled = kI[:nb * r].astype(np.float64).reshape(nb, r, dI).mean(axis=1)
    pooled = _complex_rope(pooled, 12, 100.0, np.arange(nb) * r)
    c = 1.0 / math.sqrt(dI)
    for t, p in enumerate(pos):
        nbt = (p + 1) // r
        ref = (w[p][:, None] * np.maximum(c * qI[p].astype(np.float64) @ pooled[:nbt].T, 0)).sum(0)
        assert np.abs(res["scores"][t, :nbt] - ref).max() < 1e-5 * max(1.0, np.abs(ref).max())


def _block_dims(**kw):
    bd = dict(n_q_heads=4, n_kv_heads=2, head_dim=16, n_idx_heads=2, idx_dim=8, block_size=4,
              budget=8, attn_scale=0.0, idx_scale=0.0, idx_rope_dim=8, idx_rope_theta=1000.0,
              rotary_dim=8, rope_theta=10000.0, norm_eps=1e-6)
    bd.update(kw)
    return bd


def pin_block_reduces_to_core(o):
    """Stacked identity projections, rows of mean square 1 with eps 0 and
    zero norm weights, no rotation, o_proj = [I; 0]: the block is the core
    QSA on the slices of x, and y its attention output."""
    from oracle import block as ob
    rng = np.random.default_rng(44)
    bd = _block_dims(rotary_dim=0, idx_rope_dim=0, norm_eps=0.0)
    Hq, Hkv, D, HI, dI = 4, 2, 16, 2, 8
    rows = ob.split_rows(bd)
    dm = rows["total"]
    n = 23
    x = (rng.standard_normal((n, dm)) * 0.5).astype(np.float32)
    a, b = rows["q"]
    x[:, a:b] = np.where(rng.random((n, b - a)) < 0.5, -1.0, 1.0)
    a, b = rows["k"]
    x[:, a:b] = np.where(rng.random((n, b - a)) < 0.5, -1.0, 1.0)
    x = ob.bf16_round(x)
    Wo = np.zeros((dm, Hq * D), np.float32)
    Wo[:Hq * D] = np.eye(Hq * D, dtype=np.float32)
    pos = np.array([n - 1, 13, 5])
    res = ob.block(o, bd, x, np.eye(dm, dtype=np.float32), np.zeros(D, np.float32),
                   np.zeros(D, np.float32), Wo, pos)
    sl = lambda name, shape: x[:, slice(*rows[name])].reshape(n, *shape)  # noqa: E731
    ref = o.sequence(ob.core_dims(bd), sl("k", (Hkv, D)), sl("v", (Hkv, D)), sl("kI", (dI,)),
                     pos, sl("q", (Hq, D))[pos], sl("qI", (HI, dI))[pos],
                     np.ones((3, HI), np.float32), sl("gate", (Hq, D))[pos])
    assert np.array_equal(res["sel"], ref["sel"])
    assert np.array_equal(res["y"][:, :Hq * D], ob.bf16_round(ref["out"]).reshape(3, -1))
    assert not res["y"][:, Hq * D:].any()


def _torch_block(bd, x, W_in, qn, kn, W_o):
    """The dense QSA block (budget >= context) from torch library routines in
    float64: linear, rms_norm, complex-number RoPE, scaled_dot_product_attention
    (causal, GQA by repetition), sigmoid gate, linear; rounded to bf16 where
    the path stores bf16 (torch's own bfloat16 conversion)."""
    F = torch.nn.functional
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    bf = lambda t: t.to(torch.bfloat16).to(torch.float64)  # noqa: E731
    Hq, Hkv, D = bd["n_q_heads"], bd["n_kv_heads"], bd["head_dim"]
    n = x.shape[0]
    P = F.linear(T(x), T(W_in)).to(torch.float32).to(torch.float64)
    o = 0
    def take(m):
        nonlocal o
        t = P[:, o:o + m]
        o += m
        return t
    q, g, k, v = take(Hq * D), take(Hq * D), take(Hkv * D), take(Hkv * D)
    q = F.rms_norm(q.reshape(n, Hq, D), (D,), eps=bd["norm_eps"]) * (1 + T(qn))
    k = F.rms_norm(k.reshape(n, Hkv, D), (D,), eps=bd["norm_eps"]) * (1 + T(kn))
    pos = np.arange(n)[:, None]
    q = bf(T(_complex_rope(q.numpy(), bd["rotary_dim"], bd["rope_theta"], pos)))
    k = bf(T(_complex_rope(k.numpy(), bd["rotary_dim"], bd["rope_theta"], pos)))
    v, g = bf(v.reshape(n, Hkv, D)), bf(g.reshape(n, Hq, D))
    rep = Hq // Hkv
    att = F.scaled_dot_product_attention(
        q.permute(1, 0, 2)[None], k.permute(1, 0, 2).repeat_interleave(rep, 0)[None].contiguous(),
        v.permute(1, 0, 2).repeat_interleave(rep, 0)[None].contiguous(), is_causal=True)
    att = att[0].permute(1, 0, 2) * torch.sigmoid(g)
    return F.linear(bf(att.reshape(n, Hq * D)), T(W_o)).numpy()


def pin_block_dense_matches_torch(o):
    """Budget above the context (every block selected) and the dense layer:
    the oracle's block equals the block built from torch routines."""
    from oracle import block as ob
    rng = np.random.default_rng(45)
    n, dm = 29, 24
    for r, budget in ((4, 64), (0, 0)):
        bd = _block_dims(block_size=r, budget=budget)
        if r == 0:
            bd.update(n_idx_heads=0, idx_dim=0, idx_rope_dim=0)
        rows = ob.split_rows(bd)
        x = ob.bf16_round(rng.standard_normal((n, dm)).astype(np.float32))
        W_in = ob.bf16_round((rng.standard_normal((rows["total"], dm)) / math.sqrt(dm)).astype(np.float32))
        qn = ob.bf16_round((0.3 * rng.standard_normal(16)).astype(np.float32))
        kn = ob.bf16_round((0.3 * rng.standard_normal(16)).astype(np.float32))
        W_o = ob.bf16_round((rng.standard_normal((dm, 64)) / 8).astype(np.float32))
        got = ob.block(o, bd, x, W_in, qn, kn, W_o, np.arange(n))["y"]
        ref = _torch_block(bd, x, W_in, qn, kn, W_o)
        err = np.abs(got - ref).max()
        assert err < 2e-4 * np.abs(ref).max(), (r, err)


def pin_block_index_scores(o):
    """The block's pre-top-k scores above the budget equal the indexer built
    from float64 numpy: rotated indexer query at the token's position, raw
    indexer keys mean-pooled, each mean rotated at its block's first
    position (complex-number RoPE), relu-weighted with all-ones weights."""
    from oracle import block as ob
    rng = np.random.default_rng(46)
    n, dm = 41, 24
    bd = _block_dims(block_size=4, budget=8)
    rows = ob.split_rows(bd)
    x = ob.bf16_round(rng.standard_normal((n, dm)).astype(np.float32))
    W_in = ob.bf16_round((rng.standard_normal((rows["total"], dm)) / math.sqrt(dm)).astype(np.float32))
    z16 = np.zeros(16, np.float32)
    W_o = np.zeros((dm, 64), np.float32)
    pos = np.array([n - 1, 30, 17])
    res = ob.block(o, bd, x, W_in, z16, z16, W_o, pos, want_scores=True)
    P = x.astype(np.float64) @ W_in.astype(np.float64).T
    qI = P[:, slice(*rows["qI"])].reshape(n, 2, 8)
    kI = ob.bf16_round(P[:, slice(*rows["kI"])].astype(np.float32)).astype(np.float64)
    nb = n // 4
    pooled = _complex_rope(kI[:nb * 4].reshape(nb, 4, 8).mean(axis=1), 8, 1000.0,
                           np.arange(nb) * 4)
    for t, p in enumerate(pos):
        qr = _complex_rope(qI[p], 8, 1000.0, np.full(2, p))
        nbt = (p + 1) // 4
        ref = np.maximum(qr @ pooled[:nbt].T / math.sqrt(8), 0).sum(0)
        assert np.abs(res["scores"][t, :nbt] - ref).max() < 5e-3 * np.abs(ref).max(), p


ALL_PINS = [pin_pool_exact, pin_pool_random, pin_scores_onehot, pin_scores_random,
            pin_value_gate, pin_topk_bruteforce, pin_worked_count, pin_width_bound,
            pin_token_set, pin_dense_equivalence, pin_sparse_vs_masked_sdpa,
            pin_zero_query_probe, pin_single_token, pin_gqa_equals_mha, pin_nan_poison,
            pin_planted_selected, pin_e4m3_decode_matches_torch, pin_e4m3_encode_rounding,
            pin_fwht_is_sylvester_hadamard, pin_kv8_storage_is_transparent_when_exact,
            pin_rope_against_complex_rotation, pin_rope_relative_position,
            pin_rms_norm_closed_forms, pin_pooled_key_rotation, pin_block_reduces_to_core,
            pin_block_dense_matches_torch, pin_block_index_scores]
