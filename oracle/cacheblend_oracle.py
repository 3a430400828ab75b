"""CPU oracle for CacheBlend-style fusion of independently precomputed chunk KV caches.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
reference that the HIP library is checked against.  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.  It
imports nothing from the product package, and the product never imports it.

Arithmetic is NumPy in float64 by default (`dtype=np.float32` exists only to
time a CPU baseline); no blocking, fusion or reordering beyond what the
definitions below state.

Pages followed (cited by page title and section):
  [CB1] "論文解説: CacheBlend — RAGシステム向けKV Cache融合による高速LLMサービング"
        (0h-n0.github.io): sections "KVキャッシュの定義と偏差メトリクス"
        (KV deviation, eq. 1), "選択的再計算" (Steps 1-4, K/V merge eqs.),
        "HKVD（High KV Deviation）トークン選定" (gradual filtering and the
        top-k selection code), "RoPE（Rotary Position Embedding）との整合性"
        (rotation matrix R(m), theta_i), "設定パラメータ" (check layer,
        ratio, min tokens), "パイプライン実行とロードコントローラ" (load
        and recompute delays, the optimal ratio r*).
  [CB2] "CacheBlend: Fast Large Language Model Serving for RAG with Cached
        Knowledge Fusion" explainer (abeam.tech): sections "チャンク単位でKVを
        保存する" (positions corrected to the real input positions) and
        "高いずれを持つトークンだけを再計算する" (Q/K/V from selected tokens
        only; selected tokens attend over the whole input).
  [PC]  "論文解説: Prompt Cache — モジュラーAttention再利用による低レイテンシ推論"
        (0h-n0.github.io): section "RoPEにおける位置調整" (k(p) = R(p-p')k(p')).
  [CA]  "論文解説: CachedAttention — マルチターン会話のKVキャッシュ階層管理によるコスト50%削減"
        (0h-n0.github.io):
        "エビクションポリシー" (LRU from GPU HBM to CPU DRAM).
  [CG]  "論文解説: CacheGen — KVキャッシュ圧縮とストリーミングで長文コンテキストの
        LLM推論を高速化" (0h-n0.github.io): "技術的詳細", step 1 "チャネル別
        量子化" (per-channel scale and zero point) and "圧縮率と品質のトレード
        オフ" (bit widths).

Readings taken where the pages are silent or disagree (each is listed with
its reason in the design notes):
  * Q, K and V are computed for the selected chunk rows plus the suffix only.
  * Chunks are precomputed at chunk-local positions 0..n_c-1; at fusion the
    cached K of chunk c is rotated by its offset o_c; V is not rotated.
  * Deviation = sum of squared differences over the concatenated K and V of
    all KV heads (mode 'KV'); 'K' and 'V' restrict it to one of the two.
    It compares the recomputed row against the re-rotated cached row.
  * Layer indices are 0-based; layer 0 recomputes every chunk row, the check
    layer is layer 1.
  * Rows recomputed but not kept keep their cached K/V in the fused cache.
  * Top-k ties: order by (deviation descending, position ascending), NaN
    above +inf, -0.0 equal to +0.0; the kept set is returned in ascending
    position order.
  * Quantized chunk KV: statistics per chunk, layer and channel over the
    chunk's tokens; K is quantized as stored (chunk-local positions, before
    rotation); round() is round half to even; codes decided in float32.
  * Pre-norm Llama block: RMSNorm, RoPE on interleaved pairs (2i, 2i+1) with
    theta_i = base^(-2i/d_head), causal softmax attention with GQA head map
    h -> floor(h * H_kv / H_q), SwiGLU MLP, no biases.

  * Per-token attention deviation (first-layer rule of HKVD selection): for
    a chunk row, the sum over query heads and keys of the squared difference
    between its attention probabilities over the recomputed keys and over
    the cached keys, at layers where every chunk row is recomputed (so the
    first equal the full prefill's); later layers narrow by KV deviation.

Pin status: every function here is pinned by tests/test_oracle_pins.py and
tests/test_oracle_block_pins.py (the transformer block against transformers'
Llama layer) except the constants of the gradual schedule (`schedule`, kind
'gradual'), which are a proposal the pages do not fix: parity unpinned (both
sides consume the same integer schedule).
"""
import math
import time

import numpy as np


# --------------------------------------------------------------------------
# RoPE  [CB1 "RoPE（Rotary Position Embedding）との整合性": R(m) acts on each
# pair (2i, 2i+1) with angle m*theta_i, theta_i = 10000^(-2i/d);
# PC "RoPEにおける位置調整": moving a key from p' to p is R(p - p').]
# --------------------------------------------------------------------------
def rope_theta(head_dim: int, base: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / head_dim)


def rope_rotate(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Apply R(pos * theta_i) to every pair (x[..., 2i], x[..., 2i+1]).

    x: [n, H, d_head]; pos: [n] (or a scalar) rotation amount per row.  Used both
    to encode a row at absolute position pos and to move a cached key by a
    position delta (the rotation composes additively).
    """
    x = np.asarray(x)
    n, _, dh = x.shape
    pos = np.broadcast_to(np.asarray(pos, dtype=np.float64), (n,))
    ang = pos[:, None] * rope_theta(dh, base)[None, :]          # [n, dh/2]
    c = np.cos(ang)[:, None, :].astype(x.dtype)
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# --------------------------------------------------------------------------
# Transformer block pieces (pre-norm Llama block)
# --------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q, qpos, k, v, kpos):
    """Causal softmax attention by real position [CB1 "選択的再計算" Step 4;
    CB2: the selected tokens attend over the whole fused input].

    q: [nq, Hq, dh] at positions qpos; k, v: [nk, Hkv, dh] at positions kpos.
    Key j is visible to query i iff kpos[j] <= qpos[i].  Query head h reads KV
    head floor(h * Hkv / Hq).
    """
    nq, hq, dh = q.shape
    hkv = k.shape[1]
    qpos = np.asarray(qpos)
    kpos = np.asarray(kpos)
    out = np.zeros_like(q)
    hidden = kpos[None, :] > qpos[:, None]                     # [nq, nk]
    scale = 1.0 / math.sqrt(dh)
    for h in range(hq):
        g = (h * hkv) // hq
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(hidden, -np.inf, s)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def qkv_rows(w, shape, x, pos):
    """Step 2 of selective recompute for the rows x at positions pos."""
    n = x.shape[0]
    hn = rmsnorm(x, w["attn_norm"].astype(x.dtype), shape.rms_eps)
    q = (hn @ w["wq"].T).reshape(n, shape.n_q_heads, shape.head_dim)
    k = (hn @ w["wk"].T).reshape(n, shape.n_kv_heads, shape.head_dim)
    v = (hn @ w["wv"].T).reshape(n, shape.n_kv_heads, shape.head_dim)
    return rope_rotate(q, pos, shape.rope_base), rope_rotate(k, pos, shape.rope_base), v


def finish_rows(w, shape, x, att):
    """O projection + residual, then RMSNorm + SwiGLU MLP + residual."""
    n = x.shape[0]
    h = x + att.reshape(n, shape.q_dim) @ w["wo"].T
    hn = rmsnorm(h, w["mlp_norm"].astype(x.dtype), shape.rms_eps)
    return h + (silu(hn @ w["w_gate"].T) * (hn @ w["w_up"].T)) @ w["w_down"].T


def _cast_weights(weights, dtype):
    return [None if w is None else {k: np.asarray(a, dtype=dtype) for k, a in w.items()}
            for w in weights]


def prefill(weights, shape, x, pos0: int = 0, n_layers=None, dtype=np.float64):
    """Ordinary full prefill of n tokens at positions pos0..pos0+n-1.

    Returns (K [L][n][Hkv][dh], V [L][n][Hkv][dh], per-layer outputs [L][n][d]).
    Also used to precompute a chunk's KV alone at chunk-local positions
    (pos0 = 0) [CB2 "チャンク単位でKVを保存する"].
    """
    L = shape.n_layers if n_layers is None else n_layers
    W = _cast_weights(weights[:L], dtype)
    x = np.asarray(x, dtype=dtype)
    n = x.shape[0]
    pos = np.arange(pos0, pos0 + n)
    ks = np.zeros((L, n, shape.n_kv_heads, shape.head_dim), dtype=dtype)
    vs = np.zeros_like(ks)
    outs = []
    for l in range(L):
        q, k, v = qkv_rows(W[l], shape, x, pos)
        ks[l], vs[l] = k, v
        x = finish_rows(W[l], shape, x, attention(q, pos, k, v, pos))
        outs.append(x)
    return ks, vs, outs


# --------------------------------------------------------------------------
# Recompute schedule  [CB1 "HKVD（High KV Deviation）トークン選定" gradual
# filtering; "設定パラメータ" check layer [1], ratio [0.15]]
# --------------------------------------------------------------------------
def schedule(n_chunk_tokens: int, r_bp: int, kind: str, n_layers: int):
    """Integer schedule s[0..L]: s[0] = chunk rows recomputed at layer 0,
    s[l+1] = chunk rows kept after layer l.

    r_bp is the ratio in basis points.  k = max(floor(n*r), 1) as in the
    selection code of CB1.  'fixed': ratio r from the check layer (1) on.
    'gradual' (constants are a proposal, parity unpinned): the check layer
    keeps r1 = min(1, 1.2 r) and the excess over r halves at every later layer.
    """
    L, n = n_layers, n_chunk_tokens
    if r_bp < 0 or r_bp > 10000:
        raise ValueError("ratio out of range")
    if r_bp == 0 or n == 0:
        return [0] * (L + 1)
    s = [n, n]
    if kind == "fixed":
        kk = max(1, (n * r_bp) // 10000)
        s += [kk] * (L - 1)
    elif kind == "gradual":
        r1 = min(10000, (12 * r_bp) // 10)
        for l in range(1, L):
            e = min(l - 1, 30)
            kk = max(1, (n * (r_bp * 2 ** e + r1 - r_bp)) // (10000 * 2 ** e))
            s.append(min(kk, s[-1]))
    else:
        raise ValueError(kind)
    return s[:L + 1]


# --------------------------------------------------------------------------
# KV deviation and HKVD selection  [CB1 eq. 1 (token KV deviation, L2 norm)
# and the selection code (sum of squared differences, k = max(int(n r), 1),
# top-k, indices re-sorted by position)]
# --------------------------------------------------------------------------
def kv_deviation(k_new, v_new, k_cached, v_cached, mode: str = "KV"):
    """Per-row squared L2 distance between recomputed and cached KV rows."""
    n = k_new.shape[0]
    dk = np.sum(((k_new - k_cached) ** 2).reshape(n, -1), axis=1)
    dv = np.sum(((v_new - v_cached) ** 2).reshape(n, -1), axis=1)
    if mode == "KV":
        return dk + dv
    if mode == "K":
        return dk
    if mode == "V":
        return dv
    raise ValueError(mode)


def attention_probs(q, qpos, k, kpos):
    """Causal softmax probability rows: [nq, Hq, nk], row (i, h) over the keys
    with kpos <= qpos[i], query head h reading KV head floor(h * Hkv / Hq)."""
    nq, hq, dh = q.shape
    hkv = k.shape[1]
    hidden = np.asarray(kpos)[None, :] > np.asarray(qpos)[:, None]
    out = np.zeros((nq, hq, k.shape[0]), dtype=q.dtype)
    for h in range(hq):
        g = (h * hkv) // hq
        s = (q[:, h, :] @ k[:, g, :].T) / math.sqrt(dh)
        s = np.where(hidden, -np.inf, s)
        p = np.exp(s - np.max(s, axis=1, keepdims=True))
        out[:, h, :] = p / np.sum(p, axis=1, keepdims=True)
    return out


def attention_deviation(q, qpos, k_new, k_cached, kpos):
    """Per-token attention deviation [CB1 "KVキャッシュの定義と偏差メトリクス"
    eq. 2 (attention deviation, L2 norm over the attention matrix) taken row
    by row, as the first-layer rule of "HKVD（High KV Deviation）トークン選定"
    ranks tokens by it]: for query row i, the sum over query heads and keys
    of the squared difference between its causal attention probabilities
    over the recomputed keys k_new and over the cached keys k_cached (same
    positions kpos).  At a layer where every chunk row is recomputed the
    first are the full-prefill probabilities and the second what full KV
    reuse would attend with."""
    d = attention_probs(q, qpos, k_new, kpos) - attention_probs(q, qpos, k_cached, kpos)
    return np.sum((d * d).reshape(d.shape[0], -1), axis=1)


def topk_select(dev, k: int) -> np.ndarray:
    """Indices of the k largest deviations, returned in ascending order.

    Total order: NaN first, then larger value first, then smaller index first
    (so equal values, including -0.0 vs +0.0, keep position order).
    """
    dev = [float(x) for x in np.asarray(dev).ravel()]
    order = sorted(range(len(dev)),
                   key=lambda j: (0 if math.isnan(dev[j]) else 1,
                                  0.0 if math.isnan(dev[j]) else -dev[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


# --------------------------------------------------------------------------
# Fusion (blend)  [CB1 "選択的再計算" Steps 1-4 and K/V merge eqs.;
# "HKVD トークン選定" gradual filtering; CB2 sections on position correction
# and selective recompute]
# --------------------------------------------------------------------------
def rerotate_chunks(shape, chunks, offsets, n_tokens, dtype=np.float64):
    """Fused cache before recompute: chunk c's cached K rotated by its offset,
    V copied, both placed at positions o_c..o_c+n_c-1."""
    L = chunks[0][0].shape[0] if chunks else shape.n_layers
    fk = np.zeros((L, n_tokens, shape.n_kv_heads, shape.head_dim), dtype=dtype)
    fv = np.zeros_like(fk)
    for (kc, vc), o in zip(chunks, offsets):
        nc = kc.shape[1]
        for l in range(L):
            fk[l, o:o + nc] = rope_rotate(np.asarray(kc[l], dtype=dtype), o, shape.rope_base)
            fv[l, o:o + nc] = np.asarray(vc[l], dtype=dtype)
    return fk, fv


def check_offsets(chunks, offsets):
    o = 0
    for (kc, _), oc in zip(chunks, offsets):
        if oc != o:
            raise ValueError("chunk offsets must start at 0 and be contiguous")
        o += kc.shape[1]
    return o


def blend(weights, shape, x0, chunks, offsets, n_suffix, sched, dev_mode="KV",
          min_tokens=0, dtype=np.float64, n_layers=None, timings=None, given_scores=None,
          forced_sel=None):
    """Fuse independently precomputed chunk KVs with selective recompute.

    weights: per-layer dicts; x0: [N][d] embeddings of all prompt tokens in
    fused order; chunks: list of (K [L][n_c][Hkv][dh], V) precomputed at
    chunk-local positions; offsets: contiguous chunk starts; the last n_suffix
    tokens are the query suffix; sched: integer schedule s[0..L].

    Returns a dict with fused_k/fused_v [L][N][Hkv][dh], sel (list of kept
    chunk positions per layer, ascending), dev [L][N_c] (NaN where not
    measured), layer_pos/layer_out (rows and outputs of every layer), hidden
    (final rows).  When `timings` is a list, the wall time of every layer is
    appended to it (seconds); the arithmetic is unaffected.  dev_mode 'GIVEN'
    ranks chunk tokens by given_scores [N_c] (by position) instead of the
    measured deviation, with the same top-k rule and schedule.  dev_mode
    'ATTN' ranks by attention deviation (attention_deviation) at every layer
    whose candidates are all the chunk rows (up to and including the check
    layer), and by the KV deviation over K and V at later layers.

    forced_sel (teacher forcing): a list with one entry per layer, None or
    the kept positions to use at that layer instead of the top-k of the
    measured deviations.  A forced set must be s[l+1] distinct positions of
    the layer's candidates.  Everything else is computed as usual, so a
    checker can replay a run whose selection differed from this one's by
    rounding at the threshold and keep comparing the layers after it.
    """
    L = shape.n_layers if n_layers is None else n_layers
    W = _cast_weights(weights[:L], dtype)
    nc_tot = check_offsets(chunks, offsets)
    N = nc_tot + n_suffix
    x0 = np.asarray(x0, dtype=dtype)
    assert x0.shape[0] == N
    sched = list(sched)
    if len(sched) != L + 1:
        raise ValueError("schedule needs L+1 entries")
    if N < min_tokens:                      # short prompt: plain full prefill
        sched = [nc_tot] * (L + 1)
    if sched[0] not in (0, nc_tot) or any(b > a for a, b in zip(sched, sched[1:])):
        raise ValueError("schedule must start at 0 or N_c and be non-increasing")

    fk, fv = rerotate_chunks(shape, chunks, offsets, N, dtype)
    dev = np.full((L, nc_tot), np.nan)
    suffix = np.arange(nc_tot, N)
    C = np.arange(nc_tot) if sched[0] == nc_tot else np.arange(0)
    x = x0[np.concatenate([C, suffix])]
    sel, layer_pos, layer_out = [], [], []
    for l in range(L):
        t_start = time.perf_counter()
        R = np.concatenate([C, suffix])            # Step 1: rows recomputed here
        q, k, v = qkv_rows(W[l], shape, x, R)      # Step 2
        nC = len(C)
        if nC:
            if dev_mode == "GIVEN":
                d = np.asarray(given_scores, dtype=np.float64)[C]
            elif dev_mode == "ATTN" and nC == nc_tot:
                # every chunk row recomputed: their new keys against the
                # cached keys of the same positions (chunk rows 0..N_c-1)
                d = attention_deviation(q[:nC], C, k[:nC], fk[l][:nc_tot], np.arange(nc_tot))
            else:
                d = kv_deviation(k[:nC], v[:nC], fk[l][C], fv[l][C],
                                 "KV" if dev_mode == "ATTN" else dev_mode)
            dev[l, C] = d
            keep = (np.arange(nC) if sched[l + 1] == nC
                    else topk_select(d, sched[l + 1]))
            if forced_sel is not None and forced_sel[l] is not None:
                want = np.asarray(forced_sel[l], dtype=np.int64)
                keep = np.searchsorted(C, want)
                if (len(want) != sched[l + 1] or len(np.unique(want)) != len(want)
                        or np.any(keep >= nC) or np.any(C[np.minimum(keep, nC - 1)] != want)):
                    raise ValueError(f"forced selection of layer {l} is not {sched[l + 1]} "
                                     "distinct candidate positions")
                keep = np.sort(keep)
        else:
            keep = np.arange(0)
        rows = np.concatenate([keep, nC + np.arange(n_suffix)]).astype(np.int64)
        P = R[rows]
        fk[l][P] = k[rows]                         # Step 3: K/V merge
        fv[l][P] = v[rows]
        att = attention(q[rows], P, fk[l], fv[l], np.arange(N))   # Step 4
        x = finish_rows(W[l], shape, x[rows], att)
        C = C[keep]
        sel.append(C.copy())
        layer_pos.append(P)
        layer_out.append(x)
        if timings is not None:
            timings.append(time.perf_counter() - t_start)
    return {"fused_k": fk, "fused_v": fv, "sel": sel, "dev": dev,
            "layer_pos": layer_pos, "layer_out": layer_out, "hidden": x,
            "schedule": sched}


# --------------------------------------------------------------------------
# Per-channel quantized chunk KV  [CG "技術的詳細", "ステップ1: チャネル別量子化":
# per channel c of the H*d_h channels, zero point z_c = min over tokens,
# scale s_c = (max - min) / (2^b - 1), code = round((x - z_c) / s_c);
# restored as code * s_c + z_c ("デコード"); b = 8 by default, 4 and 2 also
# listed in "圧縮率と品質のトレードオフ"]
# --------------------------------------------------------------------------
def quantize_channels(x, bits: int):
    """Codes of x [L][n][H_kv][d_h] per layer and channel.

    The code is an integer decided in float32, as the kernel decides it:
    z = min_t x, s = (max_t x - z) / (2^b - 1), code = rint((x - z) / s)
    (round half to even), clamped to [0, 2^b - 1]; a channel with s = 0
    (all tokens equal) gets code 0.  Inputs must be finite.

    Returns codes [L][n][H_kv*d_h] (uint8, one code per element), scale and
    zero [L][H_kv*d_h] (float32).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    x = np.asarray(x, dtype=np.float32)
    L, n = x.shape[0], x.shape[1]
    flat = x.reshape(L, n, -1)
    levels = np.float32(2 ** bits - 1)
    zero = flat.min(axis=1)
    scale = (flat.max(axis=1) - zero) / levels
    codes = np.zeros(flat.shape, dtype=np.uint8)
    for l in range(L):
        live = scale[l] > 0
        q = np.rint((flat[l][:, live] - zero[l][live]) / scale[l][live])
        codes[l][:, live] = np.clip(q, 0, levels).astype(np.uint8)
    return codes, scale.astype(np.float32), zero.astype(np.float32)


def dequantize_channels(codes, scale, zero, n_kv_heads, head_dim):
    """x' = code * s_c + z_c in float64, shaped [L][n][H_kv][d_h]."""
    codes = np.asarray(codes, dtype=np.float64)
    y = codes * np.asarray(scale, np.float64)[:, None, :] + np.asarray(zero, np.float64)[:, None, :]
    return y.reshape(codes.shape[0], codes.shape[1], n_kv_heads, head_dim)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Storage bytes of the codes along the channel axis: 8-bit codes as
    they are; 4-bit codes two per byte, channel 2i in the low nibble and
    channel 2i+1 in the high nibble (a storage layout of this library; the
    pages fix none)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return codes.copy()
    if codes.shape[-1] % 2:
        raise ValueError("4-bit packing needs an even channel count")
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed, bits: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return packed.copy()
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# Cross-layer consistency of HKVD tokens  [CB1 "HKVD（High KV Deviation）
# トークン選定", insight 2: tokens of high KV deviation stay highly correlated
# between consecutive layers, checked with Spearman's rank correlation]
# --------------------------------------------------------------------------
def spearman(a, b):
    """Spearman's rho: the Pearson correlation of the ranks (ties share the
    mean of their ranks)."""
    def ranks(x):
        x = np.asarray(x, dtype=np.float64)
        order = np.argsort(x, kind="stable")
        r = np.empty(x.size)
        r[order] = np.arange(1, x.size + 1)
        for v in np.unique(x):                     # average ranks of ties
            m = x == v
            if m.sum() > 1:
                r[m] = r[m].mean()
        return r
    ra, rb = ranks(a), ranks(b)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / np.sqrt((ra * ra).sum() * (rb * rb).sum()))


def layer_rank_correlation(dev):
    """rho between the deviations of consecutive layers over the tokens
    measured at both ([L][N_c] with NaN where not measured): list of L-1
    values (NaN where fewer than 3 tokens are shared)."""
    out = []
    for l in range(len(dev) - 1):
        m = ~np.isnan(dev[l]) & ~np.isnan(dev[l + 1])
        out.append(spearman(dev[l][m], dev[l + 1][m]) if m.sum() >= 3 else float("nan"))
    return out


# --------------------------------------------------------------------------
# First token and one decode step on the fused cache  [CB2 "用語解説": the KV
# cache lets generation skip recomputing past tokens; TTFT is the time to
# the first output token]
# --------------------------------------------------------------------------
def lm_head(x, final_norm, w_lm, eps):
    """Logits of rows x [rows][d]: W_lm rmsnorm(x; final_norm)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return rmsnorm(x, np.asarray(final_norm, np.float64), eps) @ np.asarray(w_lm, np.float64).T


def argmax_first(v):
    """Index of the largest entry: NaN above everything, smallest index among
    equal values."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.flatnonzero(np.isnan(v))
    if nan.size:
        return int(nan[0])
    return int(np.flatnonzero(v == v.max())[0])


def decode_step(weights, shape, x_new, fused_k, fused_v, n_ctx, dtype=np.float64):
    """One token (input row x_new [d]) at position n_ctx through every layer,
    attending over the first n_ctx rows of fused_k / fused_v [L][>=n_ctx]
    [Hkv][dh] and its own key and value.  Returns (hidden [d], k_new
    [L][Hkv][dh], v_new)."""
    L = shape.n_layers
    W = _cast_weights(weights[:L], dtype)
    x = np.asarray(x_new, dtype=dtype)[None, :]
    pos = np.array([n_ctx])
    ks, vs = [], []
    for l in range(L):
        q, k, v = qkv_rows(W[l], shape, x, pos)
        K = np.concatenate([np.asarray(fused_k[l][:n_ctx], dtype=dtype), k], axis=0)
        V = np.concatenate([np.asarray(fused_v[l][:n_ctx], dtype=dtype), v], axis=0)
        att = attention(q, pos, K, V, np.arange(n_ctx + 1))
        x = finish_rows(W[l], shape, x, att)
        ks.append(k[0])
        vs.append(v[0])
    return x[0], np.stack(ks), np.stack(vs)


# --------------------------------------------------------------------------
# Load controller  [CB1 "パイプライン実行とロードコントローラ": T_recompute =
# r T_prefill; T_load = PerTokenKVSize * L / Throughput(D) with L the input
# tokens; r* = max(r_min, T_load / T_prefill)]
# --------------------------------------------------------------------------
def load_time(per_token_kv_bytes, n_tokens, throughput_bytes_per_s):
    """T_load in seconds."""
    return per_token_kv_bytes * n_tokens / throughput_bytes_per_s


def controller_ratio(t_prefill_s, per_token_kv_bytes, n_tokens, throughput_bytes_per_s,
                     r_min_bp):
    """r* in basis points: max(r_min, T_load / T_prefill), the ratio taken to
    the nearest basis point (halves up) and capped at 10000 (where the load
    takes longer than a full prefill, recomputing everything is quicker)."""
    t_load = load_time(per_token_kv_bytes, n_tokens, throughput_bytes_per_s)
    ratio = t_load / t_prefill_s
    bp = math.floor(ratio * 10000.0 + 0.5)
    return int(min(10000, max(r_min_bp, bp)))


# --------------------------------------------------------------------------
# HBM tier of the chunk store  [CA "エビクションポリシー": least recently used
# entries leave GPU HBM when it is full; PC "キャッシュヒット率とエビクション":
# hit rate H = sum_i p_i * [module i in cache], LRU eviction]
# --------------------------------------------------------------------------
def lru_replay(capacity_bytes, batches):
    """Replays batches of chunk uses against an LRU store of a byte budget.

    batches: list of batches, each a list of (key, bytes) uses in prompt
    order.  Per batch: every use is looked up first (a hit refreshes the
    entry to most recent); then, in order, every use whose key is not
    resident is inserted as most recent, evicting least recently used
    entries that this batch does not use until it fits; when that cannot
    make room (or the entry is larger than the budget) it is not inserted.
    Returns per batch the list of hit flags and the keys evicted, in
    eviction order."""
    from collections import OrderedDict
    store = OrderedDict()          # key -> bytes; last = most recent
    used = 0
    out = []
    for batch in batches:
        hits = []
        for key, _ in batch:
            hit = key in store
            if hit:
                store.move_to_end(key)
            hits.append(hit)
        in_batch = {key for key, _ in batch}
        evicted = []
        for key, size in batch:
            if key in store:
                continue
            evictable = [k for k in store if k not in in_batch]      # least recent first
            free = capacity_bytes - used
            if size > free + sum(store[k] for k in evictable):
                continue
            for k in evictable:
                if used + size <= capacity_bytes:
                    break
                used -= store.pop(k)
                evicted.append(k)
            store[key] = size
            used += size
        out.append((hits, evicted))
    return out


def kv_size_bytes(n_layers, n_kv_heads, head_dim, n_tokens, bytes_per_elem):
    """Bytes of a K and V cache: 2 * L * H_kv * d_head * S * b  [CacheGen
    explainer, KV cache structure section; CachedAttention explainer,
    cost analysis section]."""
    return 2 * n_layers * n_kv_heads * head_dim * n_tokens * bytes_per_elem
