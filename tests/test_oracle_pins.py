"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
library routines and brute force.  Each test names what it pins and the page
passage (page title + section) it comes from."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import TINY, WORKLOADS, ModelShape
from tests.helpers import make_case, run_blend, run_full, rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY_W = WORKLOADS["tiny"]


def _read_cases(name):
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {}
            cases.append(cur)
        else:
            cur[key] = [float(v) for v in vals]
    return cases


# ---------------------------------------------------------------- RoPE
def test_rope_worked_example_golden():
    """CacheBlend explainer (0h-n0), RoPE section: R(m) and theta_i, hand-worked
    examples (catches sign, pairing-convention and frequency mistakes)."""
    for c in _read_cases("rope_worked_example.txt"):
        dh = int(c["head_dim"][0])
        x = np.array(c["x"]).reshape(1, 1, dh)
        y = oracle.rope_rotate(x, c["pos"][0], c["base"][0]).ravel()
        np.testing.assert_allclose(y, c["y"], rtol=0, atol=2e-16)


def test_rope_rerotate_closed_form():
    """Prompt Cache explainer, RoPE position adjustment: a key encoded at p'
    and rotated by p - p' equals the key encoded at p directly."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 4, 64))
    j = rng.integers(0, 3000, size=50)
    for delta in (0, 1, 640, 3840, 8191):
        a = oracle.rope_rotate(oracle.rope_rotate(x, j, 1e4), delta, 1e4)
        b = oracle.rope_rotate(x, j + delta, 1e4)
        assert rel_err(a, b) < 1e-12
        xf = x.astype(np.float32)
        a32 = oracle.rope_rotate(oracle.rope_rotate(xf, j, 1e4), delta, 1e4)
        assert rel_err(a32, b) < 1e-5


def test_rope_relative_position_identity():
    """CacheBlend explainer (0h-n0), RoPE section: the score between a query at
    m+l and a key at m depends on l only; for q = k it is
    sum_i (q_2i^2 + q_2i+1^2) cos(l theta_i)."""
    rng = np.random.default_rng(2)
    dh = 128
    q = rng.standard_normal((1, 1, dh))
    k = rng.standard_normal((1, 1, dh))
    th = 1e4 ** (-2.0 * np.arange(dh // 2) / dh)
    for l in (0, 1, 7, 300):
        scores = []
        for m in (0, 5, 1000, 4000):
            qa = oracle.rope_rotate(q, m + l, 1e4).ravel()
            ka = oracle.rope_rotate(k, m, 1e4).ravel()
            scores.append(qa @ ka)
        assert max(scores) - min(scores) < 1e-10 * max(1.0, abs(scores[0]))
        qq = oracle.rope_rotate(q, 17 + l, 1e4).ravel() @ oracle.rope_rotate(q, 17, 1e4).ravel()
        qv = q.ravel()
        closed = np.sum((qv[0::2] ** 2 + qv[1::2] ** 2) * np.cos(l * th))
        assert abs(qq - closed) < 1e-10 * abs(closed)


# ---------------------------------------------------------------- block pieces
def test_rmsnorm_and_silu_vs_library():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 33))
    g = rng.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g),
                                       eps=1e-5).numpy()
    assert rel_err(oracle.rmsnorm(x, g, 1e-5), ref) < 1e-14
    # closed form: a constant row c maps to c / sqrt(c^2 + eps)
    c = np.full((1, 8), 3.0)
    np.testing.assert_allclose(oracle.rmsnorm(c, np.ones(8), 1e-5), 3.0 / math.sqrt(9 + 1e-5),
                               rtol=1e-15)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert rel_err(oracle.silu(x), ref) < 1e-14


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 1)])
def test_attention_vs_sdpa(hq, hkv):
    """Causal attention by real position (scattered, sorted query positions)
    equals torch's scaled_dot_product_attention with a boolean mask; GQA head
    map equals SDPA's grouped-query semantics."""
    rng = np.random.default_rng(4)
    nk, dh = 90, 16
    qpos = np.sort(rng.choice(nk, size=23, replace=False))
    q = rng.standard_normal((23, hq, dh))
    k = rng.standard_normal((nk, hkv, dh))
    v = rng.standard_normal((nk, hkv, dh))
    got = oracle.attention(q, qpos, k, v, np.arange(nk))
    mask = torch.from_numpy(np.arange(nk)[None, :] <= qpos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
        torch.from_numpy(v).transpose(0, 1), attn_mask=mask,
        enable_gqa=(hq != hkv)).transpose(0, 1).numpy()
    assert rel_err(got, ref) < 1e-13


def test_projection_orientation_brute_force():
    """Weights are row-major [out][in]: y_i = sum_j W[i][j] x_j (loop form)."""
    shape = ModelShape(1, 8, 2, 1, 4, 12, vocab=16)
    rng = np.random.default_rng(5)
    w = {"attn_norm": np.ones(8), "wq": rng.standard_normal((8, 8)),
         "wk": rng.standard_normal((4, 8)), "wv": rng.standard_normal((4, 8))}
    x = rng.standard_normal((1, 8))
    q, k, v = oracle.qkv_rows(w, shape, x, np.array([0]))
    hn = x[0] / math.sqrt(np.mean(x[0] ** 2) + shape.rms_eps)
    for i in range(4):
        assert abs(v.ravel()[i] - sum(w["wv"][i][j] * hn[j] for j in range(8))) < 1e-12
    for i in range(8):   # position 0: no rotation
        assert abs(q.ravel()[i] - sum(w["wq"][i][j] * hn[j] for j in range(8))) < 1e-12


# ---------------------------------------------------------------- prefill invariants
def test_prefill_causal_prefix():
    """A token's K/V and output depend only on the tokens before it: the
    prefill of a prefix equals the leading rows of the longer prefill."""
    case = make_case(TINY, (40,), 0, seed=0)
    k, v, outs = run_full(case)
    k2, v2, outs2 = oracle.prefill(case.weights, case.shape, case.x0[:17])
    assert rel_err(k2, k[:, :17]) < 1e-12 and rel_err(v2, v[:, :17]) < 1e-12
    assert rel_err(outs2[-1], outs[-1][:17]) < 1e-12


def test_prefill_position_shift():
    """Shifting every position by p rotates K by p at every layer and leaves V
    and the outputs unchanged (scores depend on relative distance only)."""
    case = make_case(TINY, (48,), 0, seed=1)
    k0, v0, o0 = run_full(case)
    kp, vp, op = oracle.prefill(case.weights, case.shape, case.x0, pos0=1000)
    for l in range(TINY.n_layers):
        assert rel_err(kp[l], oracle.rope_rotate(k0[l], 1000, TINY.rope_base)) < 1e-10
        assert rel_err(vp[l], v0[l]) < 1e-10
    assert rel_err(op[-1], o0[-1]) < 1e-10


# ---------------------------------------------------------------- deviation / top-k
def test_deviation_definition():
    """CacheBlend explainer (0h-n0) eq. 1 squared (L2 over the token's KV) and
    the selection code's sum of squared K differences."""
    rng = np.random.default_rng(6)
    kn, kc, vn, vc = (rng.standard_normal((9, 3, 8)) for _ in range(4))
    d = oracle.kv_deviation(kn, vn, kc, vc, "KV")
    for j in range(9):
        ref = np.linalg.norm(np.concatenate([(kn[j] - kc[j]).ravel(), (vn[j] - vc[j]).ravel()]))
        assert abs(d[j] - ref ** 2) < 1e-12 * ref ** 2
    dk = torch.sum((torch.from_numpy(kn - kc).reshape(9, -1)) ** 2, dim=-1).numpy()
    assert rel_err(oracle.kv_deviation(kn, vn, kc, vc, "K"), dk) < 1e-15


def _brute_topk(dev, k):
    """The unique k-subset whose every member precedes every non-member under
    (NaN first, larger value first, smaller index first)."""
    n = len(dev)

    def before(a, b):
        da, db = dev[a], dev[b]
        na, nb = math.isnan(da), math.isnan(db)
        if na != nb:
            return na
        if not na and da != db:
            return da > db
        return a < b

    found = [s for s in itertools.combinations(range(n), k)
             if all(before(a, b) for a in s for b in range(n) if b not in s)]
    assert len(found) == 1
    return list(found[0])


def test_topk_brute_force_with_ties_and_nan():
    rng = np.random.default_rng(7)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        vals = rng.choice([0.0, -0.0, 1.0, 2.5, np.inf, np.nan, -1.0, 3.0], size=n)
        for k in range(1, n + 1):
            assert list(oracle.topk_select(vals, k)) == _brute_topk(list(vals), k)


def test_topk_vs_torch_distinct():
    """On distinct values the kept set equals torch.topk's, then sorted by
    position as in the CacheBlend explainer's selection code."""
    rng = np.random.default_rng(8)
    for n, k in [(1, 1), (10, 1), (10, 10), (384, 57), (3840, 691), (8192, 1228)]:
        d = rng.permutation(n).astype(np.float64) + rng.random(n) * 0.5
        ref = torch.topk(torch.from_numpy(d), k).indices.sort().values.numpy()
        np.testing.assert_array_equal(oracle.topk_select(d, k), ref)


# ---------------------------------------------------------------- schedule
def test_schedule_shape_and_endpoints():
    """k = max(floor(n r), 1) (selection code); r = 100% recomputes all, r = 0
    recomputes none (full KV reuse); non-increasing."""
    assert oracle.schedule(384, 1500, "fixed", 2) == [384, 384, 57]
    assert oracle.schedule(3840, 1500, "fixed", 4) == [3840, 3840, 576, 576, 576]
    assert oracle.schedule(10, 1, "fixed", 3) == [10, 10, 1, 1]
    assert oracle.schedule(384, 0, "gradual", 2) == [0, 0, 0]
    for L in (1, 2, 32, 60):
        for r in (1, 500, 1000, 1500, 1800, 5000, 10000):
            for kind in ("fixed", "gradual"):
                s = oracle.schedule(3840, r, kind, L)
                assert len(s) == L + 1 and s[0] == 3840 and s[1] == 3840
                assert all(b <= a for a, b in zip(s, s[1:]))
                if r == 10000:
                    assert s == [3840] * (L + 1)
    # gradual proposal (parity unpinned): regression values
    assert oracle.schedule(384, 1500, "gradual", 2) == [384, 384, 69]
    s = oracle.schedule(3840, 1500, "gradual", 32)
    assert s[:10] == [3840, 3840, 691, 633, 604, 590, 583, 579, 577, 576]
    assert s[-1] == 576


def test_kv_size_formula_vs_printed_examples():
    for line in open(os.path.join(GOLDEN, "kv_size_examples.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, L, H, dh, S, b, approx, tol = line.split()
        got = oracle.kv_size_bytes(int(L), int(H), int(dh), int(S), int(b))
        assert abs(got - float(approx)) <= float(tol) * float(approx), name
    assert oracle.kv_size_bytes(80, 64, 128, 4000, 2) / 32e9 == pytest.approx(0.33, abs=0.01)


# ---------------------------------------------------------------- blend invariants
@pytest.fixture(scope="module")
def tiny_case():
    return make_case(TINY, TINY_W.chunk_lens, TINY_W.n_suffix, seed=0)


@pytest.fixture(scope="module")
def tiny_full(tiny_case):
    return run_full(tiny_case)


def test_full_recompute_equals_prefill(tiny_case, tiny_full):
    """P-a: r = 100% (every chunk row kept at every layer) is an ordinary full
    prefill of the fused prompt."""
    L, nc = TINY.n_layers, tiny_case.n_chunk_tokens
    res = run_blend(tiny_case, [nc] * (L + 1))
    k, v, outs = tiny_full
    assert rel_err(res["fused_k"], k) < 1e-10
    assert rel_err(res["fused_v"], v) < 1e-10
    assert rel_err(res["hidden"], outs[-1]) < 1e-10
    # min_tokens above N forces the same full prefill
    res2 = oracle.blend(tiny_case.weights, TINY, tiny_case.x0, tiny_case.chunks,
                        tiny_case.offsets, tiny_case.n_suffix, [0] * (L + 1),
                        min_tokens=10 ** 6)
    assert rel_err(res2["fused_k"], k) < 1e-10


def test_single_chunk_r0_is_cache():
    """P-b: one chunk at offset 0 with no recompute leaves the cache as is."""
    case = make_case(TINY, (96,), 0, seed=2)
    res = run_blend(case, [0] * (TINY.n_layers + 1))
    np.testing.assert_array_equal(res["fused_k"], case.chunks[0][0])
    np.testing.assert_array_equal(res["fused_v"], case.chunks[0][1])


def test_layer0_deviation_vanishes(tiny_case):
    """P-f: layer-0 K/V depend on the token and its position only, so the
    recomputed rows equal the re-rotated cache up to rounding."""
    res = run_blend(tiny_case, oracle.schedule(tiny_case.n_chunk_tokens, 1500, "gradual", 2))
    scale = np.max(np.sum(tiny_case.chunks[0][0][0].reshape(128, -1) ** 2, axis=1))
    assert np.nanmax(res["dev"][0]) < 1e-24 * scale


def test_first_chunk_matches_full_prefill(tiny_case, tiny_full):
    """P-g: the chunk at offset 0 has no preceding context, so its rows equal
    full prefill at every layer whatever is selected."""
    res = run_blend(tiny_case, oracle.schedule(tiny_case.n_chunk_tokens, 1500, "gradual", 2))
    k, v, _ = tiny_full
    n0 = tiny_case.chunks[0][0].shape[1]
    assert rel_err(res["fused_k"][:, :n0], k[:, :n0]) < 1e-10
    assert rel_err(res["fused_v"][:, :n0], v[:, :n0]) < 1e-10
    assert np.max(res["dev"][1][:n0]) < 1e-20 * np.max(res["dev"][1][n0:])


def test_check_layer_identity(tiny_case, tiny_full):
    """P-h: at the check layer the recomputed K/V are exact, so dev_1 is the
    true deviation of the cache from full prefill (eq. 1 squared) and the
    fused-vs-full error equals the deviation of the rows not kept."""
    nc = tiny_case.n_chunk_tokens
    k, v, _ = tiny_full
    fk0, fv0 = oracle.rerotate_chunks(TINY, tiny_case.chunks, tiny_case.offsets,
                                      tiny_case.n_tokens)
    true_dev = oracle.kv_deviation(k[1][:nc], v[1][:nc], fk0[1][:nc], fv0[1][:nc])
    for r in (500, 1500, 5000):
        res = run_blend(tiny_case, oracle.schedule(nc, r, "fixed", 2))
        assert rel_err(res["dev"][1], true_dev) < 1e-10
        kept = set(res["sel"][1].tolist())
        err = np.sum((res["fused_k"][1][:nc] - k[1][:nc]) ** 2, axis=(1, 2)) + \
            np.sum((res["fused_v"][1][:nc] - v[1][:nc]) ** 2, axis=(1, 2))
        dropped = [j for j in range(nc) if j not in kept]
        assert abs(err.sum() - true_dev[dropped].sum()) < 1e-9 * true_dev.sum()
        # the kept rows are exactly the largest deviations
        assert min(true_dev[list(kept)]) >= max(true_dev[dropped])


def test_forced_selection_replay(tiny_case, tiny_full):
    """Teacher forcing (the parity rule for selections that differ by
    rounding at the threshold): forcing the sets the oracle picks itself
    reproduces the run bit for bit; forcing any other valid set at the check
    layer keeps the check-layer identity (fused-vs-full error = deviation of
    the rows not kept, CacheBlend explainer (0h-n0), eq. 1 with the K/V merge
    equations) and moves only the rows it changes; invalid sets raise."""
    case = tiny_case
    nc = case.n_chunk_tokens
    sched = oracle.schedule(nc, 1500, "gradual", TINY.n_layers)
    nat = run_blend(case, sched)
    same = oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                        sched, forced_sel=nat["sel"])
    for key in ("fused_k", "fused_v", "hidden"):
        assert np.array_equal(same[key], nat[key])
    rng = np.random.default_rng(5)
    forced = np.sort(rng.choice(nc, size=sched[2], replace=False))
    alt = oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                       sched, forced_sel=[None, forced])
    assert np.array_equal(alt["sel"][1], forced)
    assert np.array_equal(alt["fused_k"][0], nat["fused_k"][0])
    assert np.array_equal(alt["dev"][1], nat["dev"][1])
    k, v, _ = tiny_full
    err = np.sum((alt["fused_k"][1][:nc] - k[1][:nc]) ** 2, axis=(1, 2)) + \
        np.sum((alt["fused_v"][1][:nc] - v[1][:nc]) ** 2, axis=(1, 2))
    dropped = np.setdiff1d(np.arange(nc), forced)
    assert abs(err.sum() - alt["dev"][1][dropped].sum()) < 1e-9 * alt["dev"][1].sum()
    for bad in (forced[:-1], np.concatenate([forced[:-1], forced[:1]]), forced + nc):
        with pytest.raises(ValueError):
            oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                         sched, forced_sel=[None, bad])


def test_deviation_falls_as_r_grows():
    """North-star check: total KV deviation of the fused cache from full
    prefill does not grow as r grows, and is zero at r = 100% (tiny config,
    seeds 0-4, gradual schedule)."""
    rs = [0, 500, 1000, 1500, 1800, 5000, 10000]
    for seed in range(5):
        case = make_case(TINY, TINY_W.chunk_lens, TINY_W.n_suffix, seed=seed)
        k, v, _ = run_full(case)
        tot = []
        for r in rs:
            res = run_blend(case, oracle.schedule(case.n_chunk_tokens, r, "gradual", 2))
            tot.append(float(np.sum((res["fused_k"] - k) ** 2) + np.sum((res["fused_v"] - v) ** 2)))
        assert all(b <= a * (1 + 1e-12) for a, b in zip(tot, tot[1:])), (seed, tot)
        assert tot[-1] < 1e-20 * tot[0]


def test_gqa_blend_full_recompute():
    """P-a again with grouped-query attention (Yi-style 56/8 ratio scaled down)."""
    shape = ModelShape(2, 128, 7, 1, 16, 256, vocab=512)
    case = make_case(shape, (40, 24), 8, seed=3)
    nc = case.n_chunk_tokens
    res = run_blend(case, [nc] * 3)
    k, v, outs = run_full(case)
    assert rel_err(res["fused_k"], k) < 1e-10 and rel_err(res["hidden"], outs[-1]) < 1e-10


# ------------------------------------------------------------ quantized chunk KV
# CacheGen explainer, "ステップ1: チャネル別量子化" and "圧縮率と品質のトレードオフ".

@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_exact_grid_roundtrip(bits):
    """Values on a per-channel grid z + q*s (s a power of two, both extreme
    codes present) come back as exactly q and exactly x: pins the zero point
    (the minimum), the denominator 2^b - 1 and the orientation of the map."""
    rng = np.random.default_rng(11)
    L, n, H, dh = 2, 9, 2, 8
    C = H * dh
    top = 2 ** bits - 1
    q = rng.integers(0, top + 1, size=(L, n, C))
    q[:, 0, :] = 0
    q[:, 1, :] = top
    e = rng.integers(-12, -2, size=(L, 1, C)).astype(np.float64)
    s = 2.0 ** e
    z = rng.integers(-500, 500, size=(L, 1, C)) * s
    x = (z + q * s).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), z + q * s)       # exact in float32
    codes, scale, zero = oracle.quantize_channels(x.reshape(L, n, H, dh), bits)
    assert np.array_equal(codes, q)
    assert np.array_equal(scale, s[:, 0, :].astype(np.float32))
    assert np.array_equal(zero, z[:, 0, :].astype(np.float32))
    back = oracle.dequantize_channels(codes, scale, zero, H, dh)
    assert np.array_equal(back.reshape(L, n, C), x.astype(np.float64))


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_error_bound_and_extremes(bits):
    """|x' - x| <= s_c / 2 (nearest level), min -> 0 and max -> 2^b - 1."""
    rng = np.random.default_rng(12)
    L, n, H, dh = 3, 40, 2, 16
    x = (rng.standard_normal((L, n, H, dh)) * rng.uniform(0.01, 3, size=(L, 1, H, dh))
         ).astype(np.float32)
    codes, scale, zero = oracle.quantize_channels(x, bits)
    back = oracle.dequantize_channels(codes, scale, zero, H, dh).reshape(L, n, -1)
    flat = x.reshape(L, n, -1).astype(np.float64)
    err = np.abs(back - flat)
    bound = scale.astype(np.float64)[:, None, :] * 0.5 * (1 + 1e-5) + 1e-6 * np.abs(flat)
    assert np.all(err <= bound)
    lo, hi = flat.argmin(axis=1), flat.argmax(axis=1)
    li = np.arange(L)[:, None]
    ci = np.arange(flat.shape[2])[None, :]
    assert np.all(codes[li, lo, ci] == 0)
    assert np.all(codes[li, hi, ci] == 2 ** bits - 1)


def test_quantize_nearest_level_brute_force():
    """Each code is the level z + q*s nearest to x among all 2^b levels
    (checked away from ties)."""
    rng = np.random.default_rng(13)
    for bits in (4, 8):
        x = rng.standard_normal((1, 7, 1, 6)).astype(np.float32)
        codes, scale, zero = oracle.quantize_channels(x, bits)
        flat = x.reshape(7, 6).astype(np.float64)
        levels = zero[0].astype(np.float64)[None, :] + \
            np.arange(2 ** bits)[:, None] * scale[0].astype(np.float64)[None, :]
        for t in range(7):
            for c in range(6):
                d = np.abs(levels[:, c] - flat[t, c])
                order = np.argsort(d)
                if d[order[1]] - d[order[0]] < 1e-6 * scale[0, c]:
                    continue
                assert codes[0, t, c] == order[0]


def test_quantize_constant_channel():
    x = np.ones((1, 5, 1, 4), dtype=np.float32) * np.float32(0.375)
    x[0, :, 0, 1] = np.arange(5)
    codes, scale, zero = oracle.quantize_channels(x, 8)
    assert scale[0, 0] == 0 and np.all(codes[0, :, 0] == 0)
    back = oracle.dequantize_channels(codes, scale, zero, 1, 4)
    assert np.all(back[0, :, 0, 0] == 0.375)
    assert codes[0, 0, 1] == 0 and codes[0, 4, 1] == 255


def test_code_packing():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    assert oracle.pack_codes(codes, 4).tolist() == [[0x21, 0x43, 0x0F]]
    rng = np.random.default_rng(14)
    c = rng.integers(0, 16, size=(3, 5, 8)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(c, 4), 4), c)
    assert np.array_equal(oracle.pack_codes(c, 8), c)


@pytest.mark.parametrize("bits,ratio", [(8, 2), (4, 4)])
def test_code_bytes_vs_printed_ratio(bits, ratio):
    """Code bytes against FP16 storage: about 2x for 8 bits and 4x for 4
    bits, as the CacheGen explainer's trade-off table prints (the per-channel
    scale and zero are 8 bytes per channel per layer on top)."""
    L, n, H, dh = 2, 64, 2, 8
    codes = np.zeros((L, n, H * dh), dtype=np.uint8)
    fp16_bytes = oracle.kv_size_bytes(L, H, dh, n, 2) // 2      # K alone
    assert fp16_bytes / oracle.pack_codes(codes, bits).nbytes == ratio


# ------------------------------------------------------------ load controller
# CacheBlend explainer, "パイプライン実行とロードコントローラ".

def test_controller_worked_example_golden():
    for line in open(os.path.join(GOLDEN, "load_controller_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        rec_ms, r, load_ms, tok_bytes, n, r_min, want = line.split()
        t_prefill = float(rec_ms) / 1e3 / float(r)
        thr = int(tok_bytes) * int(n) / (float(load_ms) / 1e3)
        assert oracle.load_time(int(tok_bytes), int(n), thr) == pytest.approx(float(load_ms) / 1e3)
        assert oracle.controller_ratio(t_prefill, int(tok_bytes), int(n), thr,
                                       int(r_min)) == int(want)


def test_load_time_vs_printed_transfer():
    """CachedAttention explainer, cost analysis: about 10.5 GB of 70B KV for
    4000 tokens takes about 330 ms over 32 GB/s."""
    per_token = oracle.kv_size_bytes(80, 64, 128, 1, 2)
    assert oracle.load_time(per_token, 4000, 32e9) == pytest.approx(0.33, abs=0.01)


def test_controller_properties():
    rng = np.random.default_rng(31)
    for _ in range(200):
        tp = float(rng.uniform(1e-3, 1.0))
        thr = float(rng.uniform(1e9, 64e9))
        tok = int(rng.integers(1024, 1 << 16))
        n = int(rng.integers(1, 1 << 17))
        rmin = int(rng.integers(0, 10001))
        r = oracle.controller_ratio(tp, tok, n, thr, rmin)
        tl = oracle.load_time(tok, n, thr)
        assert rmin <= r <= 10000 or (r == 10000 and rmin <= 10000)
        if r < 10000:
            # the chosen recompute time covers the load to within half a basis point
            assert r / 10000 * tp >= tl - 0.5e-4 * tp
            assert r == rmin or abs(r / 10000 - tl / tp) <= 0.5e-4 + 1e-12
        else:
            assert tl >= 0.99995 * tp or rmin == 10000
    # load hidden under r_min: r_min wins; instant storage: r_min
    assert oracle.controller_ratio(1.0, 1, 1, 1e12, 1500) == 1500
    # load slower than a full prefill: recompute everything
    assert oracle.controller_ratio(0.001, 1 << 20, 1 << 20, 1e9, 1500) == 10000


# ------------------------------------------------------------ LRU chunk tier
# CachedAttention explainer, "エビクションポリシー"; Prompt Cache explainer,
# "キャッシュヒット率とエビクション".

def test_lru_replay_hand_example():
    """Budget 3 units, unit-size entries.  Batch [1,2,3]: all miss, stored.
    Batch [1,4]: 1 hits (now most recent: order 2,3,1), 4 evicts 2.
    Batch [2,3]: 2 misses, 3 hits (order 1,4,3); 2 evicts 1.
    Batch [1,4,1]: 1 misses twice in the lookup, 4 hits (order 3,2,4);
    inserting 1 evicts 3, the repeated 1 is already resident."""
    b = lambda *ks: [(k, 1) for k in ks]
    out = oracle.lru_replay(3, [b(1, 2, 3), b(1, 4), b(2, 3), b(1, 4, 1)])
    assert out == [([False] * 3, []), ([True, False], [2]), ([False, True], [1]),
                   ([False, True, False], [3])]


def test_lru_replay_sizes_and_oversize():
    """Byte budgets: a large entry evicts several least-recent ones; an
    entry above the budget is never stored and evicts nothing."""
    out = oracle.lru_replay(10, [[("a", 4), ("b", 3), ("c", 3)], [("d", 6)], [("e", 11)],
                                 [("c", 3), ("b", 3)]])
    assert out[1] == ([False], ["a", "b"])
    assert out[2] == ([False], [])
    assert out[3] == ([True, False], ["d"])       # c was refreshed by its hit


def test_lru_replay_protects_the_batch():
    """Entries a batch uses are not released to make room for its own
    misses: budget 3, batch [1,2,3] stored; batch [1,2,5,6]: 1, 2 hit, 5
    evicts 3, and 6 finds only entries of this batch to release, so it is
    not stored."""
    b = lambda *ks: [(k, 1) for k in ks]
    out = oracle.lru_replay(3, [b(1, 2, 3), b(1, 2, 5, 6), b(6)])
    assert out[1] == ([True, True, False, False], [3])
    assert out[2] == ([False], [1])


def test_lru_hit_rate_matches_brute_force():
    """With a budget holding every key, the hit flags are 'seen before in an
    earlier batch' exactly; with budget 0 nothing ever hits."""
    rng = np.random.default_rng(32)
    batches = [[(int(k), 5) for k in rng.integers(0, 20, size=8)] for _ in range(12)]
    out = oracle.lru_replay(10 ** 9, batches)
    seen = set()
    for batch, (hits, ev) in zip(batches, out):
        assert hits == [k in seen for k, _ in batch] and ev == []
        seen |= {k for k, _ in batch}
    assert all(not any(h) for h, _ in oracle.lru_replay(0, batches))


# ------------------------------------------------------------ first token, decode step
# CacheBlend explainer (abeam.tech), "用語解説" (KV cache reuse in generation, TTFT).

def test_decode_step_equals_longer_prefill():
    """Decoding token N on the full-prefill cache of tokens 0..N-1 equals
    the last row of a full prefill of tokens 0..N (the cache is exactly what
    incremental decoding needs), and its K/V rows equal that prefill's row N.
    GQA and MHA shapes."""
    for shape in (TINY, ModelShape(2, 256, 14, 2, 128, 512, vocab=512)):
        case = make_case(shape, (50, 31), 9, seed=5)
        x = case.x0
        n = x.shape[0] - 1
        k_ctx, v_ctx, _ = oracle.prefill(case.weights, shape, x[:n])
        k_all, v_all, outs = oracle.prefill(case.weights, shape, x)
        h, kn, vn = oracle.decode_step(case.weights, shape, x[n], k_ctx, v_ctx, n)
        assert np.max(np.abs(h - outs[-1][n])) <= 1e-10 * np.max(np.abs(outs[-1][n]))
        assert np.max(np.abs(kn - k_all[:, n])) <= 1e-10 * np.max(np.abs(k_all[:, n]))
        assert np.max(np.abs(vn - v_all[:, n])) <= 1e-10 * np.max(np.abs(v_all[:, n]))
    # no context at all: the token attends to itself only (a one-token prefill)
    h0, _, _ = oracle.decode_step(case.weights, shape, x[0], k_ctx[:, :0], v_ctx[:, :0], 0)
    _, _, o1 = oracle.prefill(case.weights, shape, x[:1])
    assert np.allclose(h0, o1[-1][0], rtol=0, atol=1e-12 * np.max(np.abs(o1[-1][0])))


def test_lm_head_vs_library():
    rng = np.random.default_rng(51)
    x = rng.standard_normal((3, 64))
    g = rng.uniform(0.5, 1.5, 64)
    w = rng.standard_normal((100, 64)) * 0.02
    xt = torch.from_numpy(x)
    want = torch.nn.functional.rms_norm(xt, (64,), torch.from_numpy(g), eps=1e-5) @ \
        torch.from_numpy(w).T.contiguous()
    assert np.allclose(oracle.lm_head(x, g, w, 1e-5), want.numpy(), rtol=1e-12, atol=1e-14)


def test_argmax_first_brute_force():
    rng = np.random.default_rng(52)
    for _ in range(300):
        v = rng.integers(-3, 4, size=int(rng.integers(1, 9))).astype(np.float64)
        if rng.random() < 0.2:
            v[rng.integers(0, v.size)] = np.nan
        best = None
        for i, x in enumerate(v):       # NaN first, then larger, then earlier
            key = (0 if np.isnan(x) else 1, 0.0 if np.isnan(x) else -x, i)
            best = key if best is None or key < best else best
        assert oracle.argmax_first(v) == best[2]
    assert oracle.argmax_first(np.array([1.0, 3.0, 3.0])) == 1
    assert oracle.argmax_first(np.array([-np.inf, -np.inf])) == 0


# ------------------------------------------------------------ selection variants
# CacheBlend explainer (0h-n0), "HKVD（High KV Deviation）トークン選定".

def test_spearman_vs_library():
    import scipy.stats
    rng = np.random.default_rng(71)
    for _ in range(50):
        n = int(rng.integers(3, 40))
        a = rng.integers(0, 6, size=n).astype(float)       # with ties
        b = a + rng.standard_normal(n)
        assert oracle.spearman(a, b) == pytest.approx(scipy.stats.spearmanr(a, b)[0], abs=1e-12)
    x = np.arange(10.0)
    assert oracle.spearman(x, x ** 3) == pytest.approx(1.0)
    assert oracle.spearman(x, -x) == pytest.approx(-1.0)


def test_given_scores_closed_forms(tiny_case):
    """Constant scores tie everywhere: the position rule keeps the first
    s[l+1] positions.  Scores = -position keep the same set; scores =
    position keep the last ones, narrowing gradually."""
    case = tiny_case
    nc = case.n_chunk_tokens
    sched = oracle.schedule(nc, 1500, "gradual", TINY.n_layers)
    for scores, want in ((np.zeros(nc), lambda k, prev: prev[:k]),
                         (-np.arange(nc, dtype=float), lambda k, prev: prev[:k]),
                         (np.arange(nc, dtype=float), lambda k, prev: prev[len(prev) - k:])):
        ref = oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                           case.n_suffix, sched, dev_mode="GIVEN", given_scores=scores)
        prev = np.arange(nc)
        for l in range(TINY.n_layers):
            prev = want(sched[l + 1], prev) if sched[l + 1] < len(prev) else prev
            assert np.array_equal(ref["sel"][l], prev), l


def test_given_scores_equal_to_deviation_reproduce_hkvd(tiny_case):
    """Feeding the check layer's measured deviation back as given scores
    (fixed schedule, one narrowing step) reproduces the HKVD selection."""
    case = tiny_case
    nc = case.n_chunk_tokens
    sched = oracle.schedule(nc, 1500, "fixed", TINY.n_layers)
    ref = run_blend(case, sched)
    g = oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                     case.n_suffix, sched, dev_mode="GIVEN", given_scores=ref["dev"][1])
    assert np.array_equal(g["sel"][1], ref["sel"][1])


# ------------------------------------------------------ attention deviation
# CacheBlend explainer (0h-n0), "KVキャッシュの定義と偏差メトリクス" eq. 2 and
# the first-layer rule of "HKVD（High KV Deviation）トークン選定".

def test_attention_deviation_brute_force():
    """Probabilities and their squared differences by explicit loops."""
    rng = np.random.default_rng(81)
    for hq, hkv in ((2, 2), (3, 1), (4, 2)):
        nq, nk, dh = 5, 7, 4
        q = rng.standard_normal((nq, hq, dh))
        k1 = rng.standard_normal((nk, hkv, dh))
        k0 = rng.standard_normal((nk, hkv, dh))
        qpos = np.sort(rng.choice(nk, size=nq, replace=False))
        got = oracle.attention_deviation(q, qpos, k1, k0, np.arange(nk))
        for i in range(nq):
            tot = 0.0
            for h in range(hq):
                g = h * hkv // hq
                rows = []
                for kk in (k1, k0):
                    sc = [sum(q[i, h, e] * kk[j, g, e] for e in range(dh)) / math.sqrt(dh)
                          for j in range(qpos[i] + 1)]
                    mx = max(sc)
                    ex = [math.exp(x - mx) for x in sc]
                    rows.append([x / sum(ex) for x in ex])
                tot += sum((a - b) ** 2 for a, b in zip(*rows))
            assert abs(got[i] - tot) < 1e-12 * max(1.0, tot), (hq, i)


def test_attention_deviation_vs_library_and_closed_forms():
    rng = np.random.default_rng(82)
    nq, nk, hq, hkv, dh = 11, 40, 4, 2, 16
    q = rng.standard_normal((nq, hq, dh))
    k1 = rng.standard_normal((nk, hkv, dh))
    k0 = k1 + 0.3 * rng.standard_normal((nk, hkv, dh))
    qpos = np.sort(rng.choice(nk, size=nq, replace=False))
    got = oracle.attention_deviation(q, qpos, k1, k0, np.arange(nk))
    mask = torch.from_numpy(np.arange(nk)[None, :] > qpos[:, None])

    def probs(k):
        qt = torch.from_numpy(q).transpose(0, 1)                       # [hq, nq, dh]
        kt = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).transpose(0, 1)
        s = qt @ kt.transpose(1, 2) / math.sqrt(dh)
        return torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1)
    ref = ((probs(k1) - probs(k0)) ** 2).sum(dim=(0, 2)).numpy()
    assert rel_err(got, ref) < 1e-12
    # identical keys: exactly zero; any keys: 0 <= dev <= 2 per query head
    assert np.array_equal(oracle.attention_deviation(q, qpos, k1, k1, np.arange(nk)),
                          np.zeros(nq))
    far = 50.0 * rng.standard_normal((nk, hkv, dh))
    d = oracle.attention_deviation(q, qpos, k1, far, np.arange(nk))
    assert np.all(d >= 0) and np.all(d <= 2 * hq + 1e-12)
    # a query that sees one key has the same (one-hot) row under both
    assert oracle.attention_deviation(q[:1], np.array([0]), k1, k0, np.arange(nk))[0] == 0.0


def test_attention_deviation_blend(tiny_case, tiny_full):
    """'ATTN' mode: at the check layer every chunk row is recomputed, so the
    deviation is eq. 2 row by row between the full-prefill attention (its
    queries and keys) and the attention over the re-rotated cache; the
    first chunk (no preceding context) deviates by rounding only; later
    layers narrow by KV deviation (the same as a KV-mode run forced onto the
    same sets); r = 100% is the full prefill."""
    case = tiny_case
    nc, L = case.n_chunk_tokens, TINY.n_layers
    sched = oracle.schedule(nc, 1500, "gradual", L)
    res = oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                       sched, dev_mode="ATTN")
    # eq. 2 row-wise against the actual full prefill at layer 1
    k, v, outs = tiny_full
    q1, k1, _ = oracle.qkv_rows(case.weights[1], TINY, outs[0], np.arange(case.n_tokens))
    fk0, _ = oracle.rerotate_chunks(TINY, case.chunks, case.offsets, case.n_tokens)
    want = oracle.attention_deviation(q1[:nc], np.arange(nc), k1[:nc], fk0[1][:nc], np.arange(nc))
    assert rel_err(res["dev"][1], want) < 1e-9
    n0 = case.chunks[0][0].shape[1]
    assert np.max(res["dev"][1][:n0]) < 1e-20 * np.max(res["dev"][1][n0:])
    assert np.array_equal(res["sel"][1], np.sort(oracle.topk_select(res["dev"][1], sched[2])))
    # layer 0 (all candidates) by attention deviation too: context-free keys, ~0
    assert np.max(res["dev"][0]) < 1e-20
    kv = oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                      sched, dev_mode="KV", forced_sel=res["sel"])
    for l in range(2, L):
        assert np.array_equal(res["dev"][l], kv["dev"][l], equal_nan=True)
    full = oracle.blend(case.weights, TINY, case.x0, case.chunks, case.offsets, case.n_suffix,
                        [nc] * (L + 1), dev_mode="ATTN")
    assert rel_err(full["fused_k"], k) < 1e-10 and rel_err(full["hidden"], outs[-1]) < 1e-10
