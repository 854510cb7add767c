"""Helpers shared by the GPU parity tests: uploads of synthetic layers, the
library path of one MoE layer through the C ABI, and the comparison bars."""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth

# FP16 outputs: normalised L2 <= 5e-3 and max |err| <= 2e-2 against the oracle
L2_BAR = 5e-3
MAXABS_BAR = 2e-2
# routing weights (fp32 on the GPU, fp64 in the oracle)
W_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_fp16_close(gpu: np.ndarray, ref: np.ndarray, what: str,
                      l2: float = L2_BAR, maxabs: float = MAXABS_BAR) -> Dict[str, float]:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    den = np.linalg.norm(r)
    e2 = np.linalg.norm(g - r) / (den if den > 0 else 1.0)
    ea = float(np.max(np.abs(g - r))) if g.size else 0.0
    assert e2 <= l2, f"{what}: normalised L2 {e2:.3e} > {l2}"
    assert ea <= maxabs, f"{what}: max abs {ea:.3e} > {maxabs}"
    return dict(l2=e2, maxabs=ea)


def upload_int4(int4_list: Sequence) -> tuple:
    """(table, keep-alive list) for per-expert GPTQ dicts (None allowed)."""
    keep = []
    gpu = []
    for ex in int4_list:
        if ex is None:
            gpu.append(None)
            continue
        d = {key: tuple(dev(t) for t in ex[key]) for key in ("w13", "w2")}
        keep.append(d)
        gpu.append(d)
    return fve.w4_expert_table(gpu), keep


def upload_f16(f16_list: Sequence) -> tuple:
    keep = []
    gpu = []
    for ex in f16_list:
        if ex is None:
            gpu.append(None)
            continue
        d = (dev(ex[0]), dev(ex[1]))
        keep.append(d)
        gpu.append(d)
    return fve.f16_expert_table(gpu), keep


class Layer:
    """A synthetic MoE layer restricted to the experts a set of token
    batches touches (the others stay NULL in the device tables, which the
    kernels would report through err_word if they were ever routed to)."""

    def __init__(self, shape: synth.LayerShape, token_batches: Sequence[np.ndarray],
                 layer: int = 0, int4: bool = True, f16: bool = True):
        self.shape = shape
        self.router = synth.router(shape, layer)
        touched = set()
        for x in token_batches:
            r = oracle.route_topk(x, self.router, shape.k, shape.renormalize)
            touched.update(int(e) for e in r["ids"].ravel())
        self.touched = sorted(touched)
        data = synth.make_layer(shape, layer, experts=self.touched, int4=int4, f16=True)
        self.f16 = data["f16"]
        self.int4 = data["int4"]
        self.shared = data["shared"]
        self.d_router = dev(self.router)
        self.d_gate = None
        if self.shared is not None and self.shared.get("gate") is not None:
            self.d_gate = dev(self.shared["gate"])
        self.t4 = self.t16 = self.tsh = None
        if int4:
            self.t4, self._k4 = upload_int4(self.int4)
        if f16:
            self.t16, self._k16 = upload_f16(self.f16)
        if self.shared is not None:
            self.tsh, self._ksh = upload_f16([(self.shared["w13"], self.shared["w2"])])


def run_layer(L: Layer, x: torch.Tensor, kind: str, err: Optional[torch.Tensor] = None,
              counters: Optional[torch.Tensor] = None, layer_idx: int = 0,
              residual: bool = False) -> Dict[str, torch.Tensor]:
    """Route, count, gather, expert FFN (kind = 'int4' draft or 'f16'
    verify), shared expert, combine -- every step through the C ABI."""
    s = L.shape
    T = x.shape[0]
    ids, w, gate = fve.moe_route_topk(x, L.d_router, s.k, s.renormalize, L.d_gate)
    if counters is not None:
        fve.elb_count(ids, s.E, layer_idx, counters, err)
    maps = fve.moe_gather(ids, s.E, err)
    if kind == "int4":
        ws = fve.new_workspace(0, T, s.k, s.H, s.I, s.E)
        y = fve.w4a16_grouped_ffn(x, maps, L.t4, T, s.k, s.H, s.I, s.E, ws, err_word=err)
    else:
        ws = fve.new_workspace(1, T, s.k, s.H, s.I, s.E)
        y = fve.verify_grouped_gemm(x, maps["sorted_token"], maps["offsets"], L.t16, T, T * s.k,
                                    s.H, s.I, s.E, ws, active=maps["active"],
                                    n_active=maps["n_active"], err_word=err)
    sh = None
    if L.shared is not None:
        Is = s.shared_I
        iota = torch.arange(T, dtype=torch.int32, device=x.device)
        offs = torch.tensor([0, T], dtype=torch.int32, device=x.device)
        wsh = fve.new_workspace(1, T, 1, s.H, Is, 1)
        sh = fve.verify_grouped_gemm(x, iota, offs, L.tsh, T, T, s.H, Is, 1, wsh, err_word=err)
    out = fve.moe_combine(y, maps["pair_pos"], w, sh, gate, x if residual else None)
    return dict(ids=ids, w=w, gate=gate, maps=maps, y=y, shared=sh, out=out)


def qwen_chunk_layers(L: int, dev) -> tuple:
    """L Qwen-shaped chunk layers generated on the device (torch Philox
    streams of the input recipe): ChunkLayer list, each with its FP16 target
    experts in page-locked host memory as [E, 3HI] (w13 [2I, H] then
    w2 [H, I]), and the same experts in HBM as [L, E, 3HI]."""
    from fp16_verify_expert_amd.chunk import ChunkLayer
    s = synth.QWEN_CHUNK
    full = torch.empty((L, s.E, 3 * s.H * s.I), dtype=torch.float16, device=dev)
    layers = []
    for l in range(L):
        g = synth.torch_layer(s, l, dev)
        for e, (w13, w2) in enumerate(g["f16"]):
            full[l, e, :2 * s.I * s.H].copy_(w13.reshape(-1))
            full[l, e, 2 * s.I * s.H:].copy_(w2.reshape(-1))
        del g["f16"]
        host_f16 = torch.empty((s.E, 3 * s.H * s.I), dtype=torch.float16, pin_memory=True)
        host_f16.copy_(full[l])
        layers.append(ChunkLayer(router=g["router"], int4=g["int4"], host_f16=host_f16,
                                 shared=(g["shared"]["w13"], g["shared"]["w2"]),
                                 shared_gate=g["shared"]["gate"]))
        if l % 6 == 5:
            say(f"  generated {l + 1}/{L} layers")
    torch.cuda.synchronize()
    return layers, full


def chunk_layer_np(layer, experts: Sequence[int], kind: str, H: int, I: int) -> list:
    """numpy copies of a ChunkLayer's experts for the oracle (others None):
    kind "int4" the draft's GPTQ tensors, "f16" the target's (w13, w2) from
    the page-locked host copy."""
    E = layer.host_f16.shape[0]
    out = [None] * E
    for e in experts:
        if kind == "int4":
            out[e] = {key: tuple(host(t) for t in layer.int4[e][key]) for key in ("w13", "w2")}
        else:
            row = layer.host_f16[e].numpy()
            out[e] = (row[:2 * I * H].reshape(2 * I, H), row[2 * I * H:].reshape(H, I))
    return out


def chunk_shared_np(layer) -> dict:
    return dict(w13=host(layer.shared[0]), w2=host(layer.shared[1]),
                gate=host(layer.shared_gate))
