"""Seeded synthetic inputs shaped like the ATMA paper's workloads (shared by tests and benchmark).

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and the benchmark) and
the fp64 oracle (through the tests) consume exactly the tensors drawn here.

Shapes follow the paper's 378M-class global layer (Section 3.1: head dimension 128
for the recurrent memory; 16 Polar heads of width 64 in the evaluated configs), its
2K training length (Section 4.2) and its evaluation lengths through 256K (Section
4.2 "Evaluation", Table 3).  The paper's datasets are not used: seeded Gaussian
inputs stand in for them, and planted repeated "needle" keys stand in for the
synthetic-haystack retrieval structure.

Recipe (one ``torch.Generator`` per workload, seeded; draw order fixed):
  1. gated-delta q, k, v ~ N(0, 1); gate logits a ~ N(3, 0.5), b ~ N(0, 1);
     alpha = sigmoid(a), beta = sigmoid(b) (fp32 gates); q and k are then scaled to
     unit L2 norm per token and head (a precondition of the memory, Appendix A.2);
  2. Polar q, k, v ~ N(0, 1);
  3. v_null ~ N(0, 1) (fp32, per head);
  then cast to the workload dtype (round-to-nearest-even).  Polar per-head
  parameters are fixed ramps over the heads: temp_raw in [-2, 1], null_slope_raw in
  [0, 2], null_bias in [0, 1], mag_beta in [0.1, 1.0], eps = 1e-12.
  Needle workloads overwrite round(0.1 T) distinct positions per (batch, head) with
  one shared N(0, 1) needle vector, in both the memory keys (before normalisation)
  and the Polar keys.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    gdn_H: int = 0          # 0 = no gated-delta part
    gdn_D: int = 128
    polar_Hq: int = 0       # 0 = no Polar part
    polar_Hkv: int = 0
    polar_D: int = 64
    dtype: str = "bf16"     # "bf16" or "f32" for q, k, v and outputs
    chunk: int = 64
    needle_frac: float = 0.0
    seed: int = 0
    note: str = ""


WORKLOADS = {
    "gdn_t256_d64_f32": Workload("gdn_t256_d64_f32", B=1, T=256, gdn_H=1, gdn_D=64, dtype="f32",
                                 note="memory only, fp32, one head, 4 chunks"),
    "layer_b8_t2k": Workload("layer_b8_t2k", B=8, T=2048, gdn_H=8, gdn_D=128, polar_Hq=16, polar_Hkv=16,
                             note="378M-class layer at the 2K training length"),
    "prefill_b2_t16k_needle": Workload("prefill_b2_t16k_needle", B=2, T=16384, gdn_H=8, gdn_D=128, polar_Hq=16,
                                       polar_Hkv=16, needle_frac=0.1, note="hybrid prefill with planted needles"),
    "prefill_b1_t64k": Workload("prefill_b1_t64k", B=1, T=65536, gdn_H=8, gdn_D=128, polar_Hq=16, polar_Hkv=16,
                                note="long-context prefill"),
    "prefill_b1_t256k": Workload("prefill_b1_t256k", B=1, T=262144, gdn_H=8, gdn_D=128, polar_Hq=16, polar_Hkv=16,
                                 note="evaluation-length prefill"),
}

DECODE_CONTEXT = 262144  # evaluation-length KV cache (Table 3 / Section 4.2 reach 256K)


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def polar_params(Hq: int, D: int, gen: torch.Generator | None = None, device="cpu") -> dict:
    """Per-head Polar parameters: fixed ramps plus a seeded fp32 v_null [Hq, D]."""
    def ramp(lo, hi):
        return torch.linspace(lo, hi, Hq, dtype=torch.float32) if Hq > 1 else torch.tensor([lo], dtype=torch.float32)
    v_null = torch.randn(Hq, D, generator=gen, dtype=torch.float32, device=gen.device if gen else "cpu")
    p = {
        "temp_raw": ramp(-2.0, 1.0),
        "null_slope_raw": ramp(0.0, 2.0),
        "null_bias": ramp(0.0, 1.0),
        "mag_beta": ramp(0.1, 1.0),
        "v_null": v_null,
        "eps": 1e-12,
    }
    return {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in p.items()}


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _plant_needles(x: torch.Tensor, frac: float, gen: torch.Generator) -> None:
    """x [B, T, H, D]: per (b, h) write one shared N(0,1) vector at round(frac*T) distinct positions."""
    B, T, H, D = x.shape
    n = int(round(frac * T))
    if n == 0:
        return
    for b in range(B):
        for h in range(H):
            pos = torch.randperm(T, generator=gen, device=gen.device)[:n]
            needle = torch.randn(D, generator=gen, device=gen.device, dtype=x.dtype)
            x[b, pos, h, :] = needle


def make_gdn_inputs(B, T, H, Dk, Dv=None, dtype="bf16", seed=0, device="cpu", needle_frac=0.0,
                    gen: torch.Generator | None = None) -> dict:
    """q, k, v [B,T,H,D] in ``dtype``; alpha, beta [B,T,H] fp32."""
    Dv = Dk if Dv is None else Dv
    if gen is None:
        gen = torch.Generator(device=device).manual_seed(seed)
    dev = gen.device
    q = torch.randn(B, T, H, Dk, generator=gen, device=dev)
    k = torch.randn(B, T, H, Dk, generator=gen, device=dev)
    v = torch.randn(B, T, H, Dv, generator=gen, device=dev)
    a = torch.randn(B, T, H, generator=gen, device=dev) * 0.5 + 3.0
    b = torch.randn(B, T, H, generator=gen, device=dev)
    if needle_frac > 0:
        _plant_needles(k, needle_frac, gen)
    td = torch_dtype(dtype)
    return {
        "q": _unit(q).to(td).contiguous(),
        "k": _unit(k).to(td).contiguous(),
        "v": v.to(td).contiguous(),
        "alpha": torch.sigmoid(a).contiguous(),
        "beta": torch.sigmoid(b).contiguous(),
    }


def make_polar_inputs(B, T, Hq, Hkv, D, dtype="bf16", seed=0, device="cpu", needle_frac=0.0,
                      gen: torch.Generator | None = None) -> dict:
    """q [B,T,Hq,D], k, v [B,T,Hkv,D] in ``dtype`` plus per-head params."""
    if gen is None:
        gen = torch.Generator(device=device).manual_seed(seed)
    dev = gen.device
    td = torch_dtype(dtype)
    q = torch.randn(B, T, Hq, D, generator=gen, device=dev)
    k = torch.randn(B, T, Hkv, D, generator=gen, device=dev)
    v = torch.randn(B, T, Hkv, D, generator=gen, device=dev)
    if needle_frac > 0:
        _plant_needles(k, needle_frac, gen)
    params = polar_params(Hq, D, gen, device=dev)
    return {"q": q.to(td).contiguous(), "k": k.to(td).contiguous(), "v": v.to(td).contiguous(), "params": params}


def make_workload(w: Workload | str, device="cpu") -> dict:
    """Draw every input of a workload in the fixed order: memory, then Polar (+ v_null)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    gen = torch.Generator(device=device).manual_seed(w.seed)
    out = {"workload": w}
    if w.gdn_H:
        out["gdn"] = make_gdn_inputs(w.B, w.T, w.gdn_H, w.gdn_D, dtype=w.dtype, needle_frac=w.needle_frac, gen=gen)
    if w.polar_Hq:
        out["polar"] = make_polar_inputs(w.B, w.T, w.polar_Hq, w.polar_Hkv, w.polar_D, dtype=w.dtype,
                                         needle_frac=w.needle_frac, gen=gen)
    return out


def make_decode_inputs(B, context, Hq=16, Hkv=16, D=64, gdn_H=8, gdn_D=128, Lmax=None, dtype="bf16", seed=0,
                       device="cpu") -> dict:
    """One decode step: a KV cache holding ``context`` tokens (the newest one included) in a
    [B, Lmax, Hkv, D] buffer, a new query [B, Hq, D], and a memory step (q, k, v [B, H, D],
    alpha, beta [B, H], state [B, H, D, D] fp32 drawn as a scaled Gaussian)."""
    Lmax = context if Lmax is None else Lmax
    gen = torch.Generator(device=device).manual_seed(seed)
    dev = gen.device
    td = torch_dtype(dtype)
    kc = torch.empty(B, Lmax, Hkv, D, device=dev, dtype=td)
    vc = torch.empty(B, Lmax, Hkv, D, device=dev, dtype=td)
    # fill in slices to bound fp32 temporaries on large caches
    step = max(1, (1 << 24) // (Hkv * D))
    for b in range(B):
        for t0 in range(0, Lmax, step):
            t1 = min(Lmax, t0 + step)
            kc[b, t0:t1] = torch.randn(t1 - t0, Hkv, D, generator=gen, device=dev).to(td)
            vc[b, t0:t1] = torch.randn(t1 - t0, Hkv, D, generator=gen, device=dev).to(td)
    q = torch.randn(B, Hq, D, generator=gen, device=dev).to(td)
    params = polar_params(Hq, D, gen, device=dev)
    gq = _unit(torch.randn(B, gdn_H, gdn_D, generator=gen, device=dev)).to(td)
    gk = _unit(torch.randn(B, gdn_H, gdn_D, generator=gen, device=dev)).to(td)
    gv = torch.randn(B, gdn_H, gdn_D, generator=gen, device=dev).to(td)
    ga = torch.sigmoid(torch.randn(B, gdn_H, generator=gen, device=dev) * 0.5 + 3.0)
    gb = torch.sigmoid(torch.randn(B, gdn_H, generator=gen, device=dev))
    state = torch.randn(B, gdn_H, gdn_D, gdn_D, generator=gen, device=dev) * 0.1
    return {"q": q, "k_cache": kc, "v_cache": vc, "cache_len": context, "Lmax": Lmax, "params": params,
            "gdn": {"q": gq, "k": gk, "v": gv, "alpha": ga, "beta": gb, "state": state}}
