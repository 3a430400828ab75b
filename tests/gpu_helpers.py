"""GPU-side helpers for the parity tests: move seeded numpy inputs to the
device in the run dtype and build library models.  Expected values always
come from the oracle, never from the library."""
import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a, dt="f32"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(TORCH_DT[dt]).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_model(npk, case, dt):
    s = case.shape
    layers = []
    for w in case.weights:
        layers.append({k: dev(v, dt).contiguous() for k, v in w.items()})
    return npk.Model(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn_dim,
                     layers, rope_base=s.rope_base, rms_eps=s.rms_eps)


def quant_chunk(codes, bits, on_host=False):
    """One chunk descriptor from oracle codes (K codes, V codes, qparams)."""
    kc, vc, qp = codes
    t = [torch.from_numpy(np.ascontiguousarray(a)) for a in (kc, vc, qp)]
    t = [x.pin_memory() if on_host else x.cuda() for x in t]
    L, n, width = kc.shape
    return {"k": t[0], "v": t[1], "qparams": t[2], "n_tokens": n, "on_host": int(on_host),
            "layer_stride": n * width * 8 // bits, "kv_format": 1 if bits == 8 else 2}


def chunk_inputs(case, dt, on_host=False, quant=None):
    """Chunk caches as [L][n_c][Hkv][dh] tensors (device, or pinned host);
    quant = (codes from helpers.quantize_case, bits) passes them as codes."""
    if quant is not None:
        codes, bits = quant
        return [quant_chunk(c, bits, on_host) for c in codes]
    chunks = []
    for k, v in case.chunks:
        kt, vt = dev(k, dt), dev(v, dt)
        if on_host:
            kt = kt.cpu().pin_memory()
            vt = vt.cpu().pin_memory()
        L, n = k.shape[0], k.shape[1]
        chunks.append({"k": kt, "v": vt, "n_tokens": n, "on_host": int(on_host),
                       "layer_stride": n * k.shape[2] * k.shape[3]})
    return chunks


def run_gpu_blend(npk, model, case, dt, schedule, dev_mode=0, on_host=False, plan=False,
                  quant=None, chunks=None, given_scores=None):
    s = case.shape
    N, Nc, L = case.n_tokens, case.n_chunk_tokens, s.n_layers
    tdt = TORCH_DT[dt]
    if chunks is None:
        chunks = chunk_inputs(case, dt, on_host, quant)
    x0 = dev(case.x0, dt)
    fk = torch.full((L, N, s.n_kv_heads, s.head_dim), float("nan"), dtype=tdt, device="cuda")
    fv = torch.full_like(fk, float("nan"))
    sel = torch.full((L, max(1, Nc)), -1, dtype=torch.int32, device="cuda")
    dev_out = torch.full((L, max(1, Nc)), float("nan"), dtype=torch.float32, device="cuda")
    n_last = case.n_suffix + schedule[-1]
    hid = torch.full((max(1, n_last), s.d_model), float("nan"), dtype=torch.float32,
                     device="cuda")
    kw = dict(sel_idx=sel, hidden_out=hid, deviation=dev_out, schedule=schedule,
              dev_mode=dev_mode, given_scores=given_scores)
    if plan:
        p = npk.Plan(model, chunks, case.offsets, case.n_suffix, x0, fk, fv, **kw)
        for l in range(L):
            if l + 1 < L:
                p.fetch_kv(l + 1)
            p.prefill_layer(l)
        p.synchronize()
        p.destroy()
        cnt = p.sel_count
    else:
        cnt = npk.cb_blend(model, chunks, case.offsets, case.n_suffix, x0, fk, fv, **kw)
    torch.cuda.synchronize()
    return {"fused_k": fk, "fused_v": fv, "sel": sel, "dev": dev_out, "hidden": hid[:n_last],
            "sel_count": cnt}


def pool_inputs(bcase, dt, on_host=False):
    """Pool chunk caches (device or pinned host); unused entries get the
    first used entry's buffers (they are never read)."""
    used = [c for c in bcase.pool if c is not None]
    filler = used[0] if used else None
    out = []
    for c in bcase.pool:
        k, v = c if c is not None else filler
        kt, vt = dev(k, dt), dev(v, dt)
        if on_host:
            kt = kt.cpu().pin_memory()
            vt = vt.cpu().pin_memory()
        n = k.shape[1]
        out.append({"k": kt, "v": vt, "n_tokens": n, "on_host": int(on_host),
                    "layer_stride": n * k.shape[2] * k.shape[3]})
    return out


def run_gpu_batch(npk, model, bcase, dt, schedules=None, recompute_bp=1500,
                  schedule_kind=0, dev_mode=0, on_host=False, dev_fill=float("nan"),
                  override=None, pool=None):
    """cb_blend_batch over the whole batch; returns the stacked outputs split
    per request (views) plus the raw stacked tensors.  override: {pool index:
    chunk descriptor} replacing the plain pool entries (e.g. quantized);
    pool: the whole pool (chunk dicts or a resolved descriptor array)."""
    s = bcase.shape
    L = s.n_layers
    tdt = TORCH_DT[dt]
    pool = pool_inputs(bcase, dt, on_host) if pool is None else pool
    for i, c in (override or {}).items():
        pool[i] = c
    reqs = []
    for i, r in enumerate(bcase.requests):
        d = {"chunk_ids": r["chunk_ids"], "n_suffix": r["n_suffix"]}
        if schedules is not None:
            d["schedule"] = schedules[i]
        reqs.append(d)
    Ns = [c.n_tokens for c in bcase.cases]
    Ncs = [c.n_chunk_tokens for c in bcase.cases]
    Ntot, Nctot = sum(Ns), sum(Ncs)
    x0 = dev(bcase.x0, dt)
    fk = torch.full((L, Ntot, s.n_kv_heads, s.head_dim), float("nan"), dtype=tdt, device="cuda")
    fv = torch.full_like(fk, float("nan"))
    sel = torch.full((L, max(1, Nctot)), -1, dtype=torch.int32, device="cuda")
    dev_out = torch.full((L, max(1, Nctot)), dev_fill, dtype=torch.float32, device="cuda")
    # hidden rows per request are s_b[L] + N_s,b; computed from the returned counts,
    # so allocate the upper bound N_b
    hid = torch.full((Ntot, s.d_model), float("nan"), dtype=torch.float32, device="cuda")
    cnt = npk.cb_blend_batch(model, pool, reqs, x0, fk, fv, sel_idx=sel, hidden_out=hid,
                             deviation=dev_out, recompute_bp=recompute_bp,
                             schedule_kind=schedule_kind, dev_mode=dev_mode)
    torch.cuda.synchronize()
    per = []
    G = C = H = 0
    for b, c in enumerate(bcase.cases):
        n_last = c.n_suffix + cnt[b][-1]
        per.append({"fused_k": fk[:, G:G + Ns[b]], "fused_v": fv[:, G:G + Ns[b]],
                    "sel": sel[:, C:C + Ncs[b]], "dev": dev_out[:, C:C + Ncs[b]],
                    "hidden": hid[H:H + n_last], "sel_count": cnt[b]})
        G += Ns[b]
        C += Ncs[b]
        H += n_last
    return per, {"fused_k": fk, "fused_v": fv, "sel": sel, "dev": dev_out, "hidden": hid[:H]}


TOL = {"f32": 1e-4, "bf16": 2e-2}
BAND = {"f32": 1e-3, "bf16": 5e-2}


def compare(case, gpu, sched, dt, dev_mode="KV", given_scores=None, check_hidden=True,
            allow_swaps=None, oracle_dtype=np.float64, dev_floor=None):
    """A GPU fusion against the oracle replayed with the GPU's kept sets
    (teacher forcing), layer by layer, to the end.

    At every layer the GPU's kept set must be the replay's own top-k of the
    same candidates (CacheBlend explainer (0h-n0), HKVD selection: the
    largest deviations, ties by position), or differ from it only in rows
    whose deviations lie within the rounding band of the k-th largest (GPU
    and oracle deviations differ by rounding).  Then every layer's fused K
    and V, the measured deviations of every narrowing layer and the
    last-layer rows are compared at the dtype's tolerance (normwise max
    relative error).  allow_swaps (default: bf16 only) permits such
    threshold swaps at all.  oracle_dtype: the replay's arithmetic (float32
    bounds the CPU time at full model width; its error is far below the bf16
    tolerance).  dev_floor: swaps are also accepted within dev_floor times
    the layer's largest candidate deviation (the rounding level of a
    measure whose values can be zero, such as the attention deviation of
    rows without preceding context; default 5e-3 for 'ATTN', else 0), plus,
    for 'ATTN', 2e-7 per query head (the float32 floor of the kernel's
    one-pass form of the measure).
    Returns (replay, swaps per layer, errors): errors holds the measured
    normwise errors of K, V per layer and of the last rows."""
    import oracle
    from tests.helpers import rel_err
    if allow_swaps is None:
        allow_swaps = dt != "f32"
    tol, band = TOL[dt], BAND[dt]
    if dev_floor is None:
        dev_floor = 5e-3 if dev_mode == "ATTN" else 0.0
    L = case.shape.n_layers
    Nc = case.n_chunk_tokens
    gsel = [gpu["sel"][l, :sched[l + 1]].cpu().numpy().astype(np.int64) for l in range(L)]
    ref = oracle.blend(case.weights, case.shape, case.x0, case.chunks, case.offsets,
                       case.n_suffix, sched, dev_mode=dev_mode, given_scores=given_scores,
                       forced_sel=gsel, dtype=oracle_dtype)
    cand = np.arange(Nc) if sched[0] == Nc else np.arange(0)
    swaps = []
    errs = {"K": [], "V": [], "hidden": None}
    for l in range(L):
        k = sched[l + 1]
        got = gsel[l]
        assert len(got) == k, (l, len(got), k)
        if k < len(cand):
            d = ref["dev"][l][cand]
            want = cand[oracle.topk_select(d, k)]
            diff = np.setxor1d(got, want)
            if diff.size:
                assert allow_swaps, ("kept set differs", l, diff)
                kth = np.sort(d)[::-1][k - 1]
                floor = dev_floor * np.max(np.abs(d))
                if dev_mode == "ATTN":
                    floor += 2e-7 * case.shape.n_q_heads
                for j in diff:
                    assert abs(ref["dev"][l][j] - kth) <= band * abs(kth) + floor, (l, j, kth)
            swaps.append(int(diff.size // 2))
        else:
            np.testing.assert_array_equal(got, cand)
            swaps.append(0)
        ek = rel_err(host(gpu["fused_k"][l]), ref["fused_k"][l])
        ev = rel_err(host(gpu["fused_v"][l]), ref["fused_v"][l])
        errs["K"].append(ek)
        errs["V"].append(ev)
        assert ek < tol, ("K", l, ek)
        assert ev < tol, ("V", l, ev)
        if len(cand) and k < len(cand):
            m = ~np.isnan(ref["dev"][l])
            d_gpu = host(gpu["dev"][l])
            assert np.all(~np.isnan(d_gpu[m])), ("dev NaN", l)
            d_ref = ref["dev"][l][m]
            if dev_mode == "ATTN":     # a measure that is zero for some rows: absolute floor
                err = np.max(np.abs(d_gpu[m] - d_ref))
                assert err <= band * np.max(np.abs(d_ref)) + 2e-7 * case.shape.n_q_heads, \
                    ("dev", l, err)
            else:
                assert rel_err(d_gpu[m], d_ref) < band, ("dev", l)
        cand = got
    if check_hidden:
        errs["hidden"] = rel_err(host(gpu["hidden"]), ref["hidden"])
        assert errs["hidden"] < tol, ("hidden", errs["hidden"])
    return ref, swaps, errs
