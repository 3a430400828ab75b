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


def chunk_inputs(case, dt, on_host=False):
    """Chunk caches as [L][n_c][Hkv][dh] tensors (device, or pinned host)."""
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


def run_gpu_blend(npk, model, case, dt, schedule, dev_mode=0, on_host=False, plan=False):
    s = case.shape
    N, Nc, L = case.n_tokens, case.n_chunk_tokens, s.n_layers
    tdt = TORCH_DT[dt]
    chunks = chunk_inputs(case, dt, on_host)
    x0 = dev(case.x0, dt)
    fk = torch.full((L, N, s.n_kv_heads, s.head_dim), float("nan"), dtype=tdt, device="cuda")
    fv = torch.full_like(fk, float("nan"))
    sel = torch.full((L, max(1, Nc)), -1, dtype=torch.int32, device="cuda")
    dev_out = torch.full((L, max(1, Nc)), float("nan"), dtype=torch.float32, device="cuda")
    n_last = case.n_suffix + schedule[-1]
    hid = torch.full((max(1, n_last), s.d_model), float("nan"), dtype=torch.float32,
                     device="cuda")
    kw = dict(sel_idx=sel, hidden_out=hid, deviation=dev_out, schedule=schedule,
              dev_mode=dev_mode)
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
