"""Shared helpers of the GPU parity tests (all comparisons are against the CPU oracle)."""
import numpy as np
import torch

import moe_synth as ms
import oracle
import routing_align_sort_amd as moe

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 6e-2, "e2m1": 6e-2}


def device():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    moe.load_library()              # fails loudly if the HIP library is not built
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns / values of a device tensor as the oracle takes them."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, moe.FP4, moe.E8M0):
        return t.view(torch.uint8).numpy()
    return t.numpy()


# the generator's MXFP4 weights are uint8 (code pairs); the binding views them
# as float4_e2m1fn_x2 with float8_e8m0fnu scales
ODT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3", torch.uint8: "e2m1"}
INTER = {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3", "e2m1": "e4m3"}


def as_library_weights(L):
    """(w13, w2, w13_scale, w2_scale) of a generated layer in the binding's dtypes."""
    w13, w2, s13, s2 = L["w13"], L["w2"], L.get("w13_scale"), L.get("w2_scale")
    if w13.dtype == torch.uint8:
        return w13.view(moe.FP4), w2.view(moe.FP4), s13.view(moe.E8M0), s2.view(moe.E8M0)
    return w13, w2, s13, s2


def oracle_tokens(x, w13, w2, ids, w, toks, w13_scale=None, w2_scale=None):
    """Oracle FFN + combine for the tokens ``toks`` only.

    Copies to the host just the expert slabs those tokens use (the inputs, as
    the generator made them) and renumbers their ids.  Returns (out [n,H] f64,
    y_slots [n*K,H] f32)."""
    toks = np.asarray(toks)
    E = w13.shape[0]
    sub_ids = ids[toks]
    used = sorted({int(e) for e in sub_ids.ravel() if 0 <= e < E})
    remap = {e: i for i, e in enumerate(used)}
    rid = np.array([[remap.get(int(e), -1) for e in row] for row in sub_ids], np.int32)
    sel = torch.tensor(used, dtype=torch.long, device=w13.device)
    w13h = host_bits(w13.index_select(0, sel)) if used else None
    w2h = host_bits(w2.index_select(0, sel)) if used else None
    s13 = s2 = None
    if w13_scale is not None and used:
        s13 = w13_scale.index_select(0, sel).cpu().numpy()
        s2 = w2_scale.index_select(0, sel).cpu().numpy()
    wdt = ODT[w13.dtype]
    xdt = ODT[x.dtype]
    xh = host_bits(x[torch.as_tensor(toks, device=x.device)])
    if not used:
        H = x.shape[1]
        return np.zeros((len(toks), H)), np.zeros((len(toks) * ids.shape[1], H), np.float32)
    out, y = oracle.moe_layer(xh, w13h, w2h, rid, w[toks], w_dtype=wdt, x_dtype=xdt,
                              inter=INTER[wdt], w13_scale=s13, w2_scale=s2, E=len(used))
    return out, y


# Oracle results of the full-size workloads, computed once per test session
# and shared by the test files that compare those workloads (keyed by the
# workload's name and the compared tokens; the generators are seeded, so the
# same name always means the same inputs).
_ORACLE_CACHE = {}


def oracle_layer_cached(name, cfg, L, toks=None):
    """(ids, w, toks, out_ref [n,H] f64, y_ref [n*K,H] f32) of workload ``name``.

    ``toks`` None compares every token; otherwise the given token indices."""
    ids, w = route_oracle(cfg, L)
    toks = np.arange(cfg["T"]) if toks is None else np.asarray(toks)
    key = (name, toks.tobytes())
    if key not in _ORACLE_CACHE:
        say(f"oracle: {name}, {len(toks)} tokens x {ids.shape[1]} slots (cached for this session)")
        ref, yref = oracle_tokens(L["x"], L["w13"], L["w2"], ids, w, toks, L.get("w13_scale"),
                                  L.get("w2_scale"))
        _ORACLE_CACHE[key] = (ref, yref)
    ref, yref = _ORACLE_CACHE[key]
    return ids, w, toks, ref, yref


def seeded_subset(T, n, seed=0):
    """A sorted seeded sample of n of T tokens (the compute-bound shapes' 256-token subsets)."""
    return np.sort(np.random.default_rng(seed).choice(T, size=n, replace=False))


def compare_out(out, toks, ref, dtype, label):
    """max|gpu - oracle| / max|oracle| over the compared tokens' output rows, asserted."""
    got = out[torch.as_tensor(toks, device=out.device)].float().cpu().numpy()
    err = rel_err(got, ref)
    say(f"{label}: out rel err {err:.3e} over {len(toks)} tokens (tol {TOL[dtype]})")
    assert err <= TOL[dtype], (label, err)
    return err


def compare_slots(y_rows, toks, ids, yref, dtype, label):
    """The same bar on the slot rows y_slots[t*K+k] of the compared tokens
    (rows of skipped slots are not written, so they are left out)."""
    K = ids.shape[1]
    slots = (np.asarray(toks)[:, None] * K + np.arange(K)[None]).ravel()
    valid = ids[toks].ravel() >= 0
    got = y_rows[torch.as_tensor(slots[valid], device=y_rows.device)].float().cpu().numpy()
    err = rel_err(got, yref[valid])
    say(f"{label}: y_slots rel err {err:.3e} over {int(valid.sum())} slots (tol {TOL[dtype]})")
    assert err <= TOL[dtype], (label, err)
    return err


def route_oracle(cfg, L, K=None):
    """The oracle's routing of a generated layer's logits."""
    ids, w = oracle.route_topk(L["logits"].cpu().numpy(), K or cfg["K"], score=cfg["score"],
                               bias=None if L["bias"] is None else L["bias"].cpu().numpy(),
                               n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                               renormalize=cfg["renormalize"], append_shared=bool(cfg.get("shared")))
    return ids, w


def make_gpu_layer(cfg, L, B=None, packed=None, top1="auto", slot_dtype=torch.float32, schedule="two_launch"):
    w13, w2, s13, s2 = as_library_weights(L)
    return moe.MoELayer(w13, w2, T=cfg["T"], K=cfg["K"], B=B or cfg["B"], packed=packed, top1=top1,
                        slot_dtype=slot_dtype, schedule=schedule,
                        score=cfg["score"], n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                        renormalize=cfg["renormalize"], shared=bool(cfg.get("shared")),
                        w13_scale=s13, w2_scale=s2,
                        x_dtype=L["x"].dtype,
                        out_dtype=torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16)
