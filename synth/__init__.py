"""Seeded synthetic inputs for the routed-expert MoE FFN path.

This module is the only code shared by the CPU oracle side (tests, the
bench's CPU baseline) and the HIP side (binding tests, bench, smoke).  It
draws random tensors and prepares the draft's INT4 weights from the FP16
target weights; it computes none of the MoE layer itself (no routing, no
dequantisation, no products, no combine).

Workload shapes follow the MoE models named on the pages (DeepSeek-V2-Lite,
Qwen1.5-MoE-A2.7B, Phi-3.5-MoE; "Specter previews expert routing with an INT4
copy of the model itself", artifact paragraph) at batch one, with one decode
token per draft step and K+1 tokens per verification.  Trained checkpoints and
the prompt datasets are replaced by seeded Gaussian tensors:

* weights ~ N(0, 0.02) (0.02 read as the standard deviation), drawn in fp32
  and rounded to fp16 (round-to-nearest-even);
* token activations ~ N(0, 1), drawn in fp32 and rounded to fp16;
* the draft's routed experts are the round-to-nearest GPTQ INT4 (group 128)
  quantisation of the same FP16 target weights ("Specter previews expert
  routing ...": the draft is a GPTQ INT4 group-size-128 copy of the target's
  routed experts whose routers and shared experts reuse the target's tensors).

Every tensor comes from its own PCG64 stream keyed by
SeedSequence([base_seed, config_id, layer, expert, tensor_id, step]), so any
single expert can be regenerated on its own and generation parallelises.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

BASE_SEED = 0
GROUP = 128

# tensor ids inside the seed key
T_ROUTER, T_W13, T_W2, T_SH_W13, T_SH_W2, T_SH_GATE, T_TOKENS, T_AWQ13, T_AWQ2 = range(9)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE layer's shape (hidden H, routed experts E, top-k, expert
    intermediate I, shared-expert intermediate (0 = none), sigmoid gate on the
    shared expert)."""
    name: str
    config_id: int
    H: int
    E: int
    k: int
    I: int
    shared_I: int = 0
    shared_gate: bool = False
    renormalize: bool = False

    @property
    def int4_bytes_per_expert(self) -> int:
        """Packed nibbles + fp16 scales + packed 4-bit zeros of w13 and w2."""
        H, I = self.H, self.I
        w13 = H * 2 * I // 2 + (H // GROUP) * 2 * I * 2 + (H // GROUP) * (2 * I // 8) * 4
        w2 = I * H // 2 + (I // GROUP) * H * 2 + (I // GROUP) * (H // 8) * 4
        return w13 + w2

    @property
    def f16_bytes_per_expert(self) -> int:
        return 2 * 3 * self.H * self.I

    @property
    def shared_f16_bytes(self) -> int:
        return 2 * 3 * self.H * self.shared_I


# The five workloads.  Index = position of the workload in the list of
# measured configurations.
TINY = LayerShape("tiny", 0, H=256, E=8, k=2, I=512)
DS = LayerShape("ds_v2_lite", 1, H=2048, E=64, k=6, I=1408, shared_I=2 * 1408)
QWEN = LayerShape("qwen15_moe", 2, H=2048, E=60, k=4, I=1408, shared_I=5632, shared_gate=True)
PHI = LayerShape("phi35_moe", 3, H=4096, E=16, k=2, I=6400)
QWEN_CHUNK = LayerShape("qwen15_moe_chunk", 4, H=2048, E=60, k=4, I=1408, shared_I=5632,
                        shared_gate=True)

WORKLOADS = {
    "tiny": dict(shape=TINY, draft_T=(4,), verify_T=()),
    "ds_draft": dict(shape=DS, draft_T=(1, 4, 16), verify_T=()),
    "qwen_verify": dict(shape=QWEN, draft_T=(), verify_T=(9,)),
    "phi_layer": dict(shape=PHI, draft_T=(1,), verify_T=(17,)),
    "qwen_chunk": dict(shape=QWEN_CHUNK, draft_T=(1,), verify_T=(17,), layers=24, draft_steps=16,
                       resident=16),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def normal_f16(key: Sequence[int], shape, std: float) -> np.ndarray:
    """N(0, std) drawn in fp32 from the stream `key`, rounded to fp16 (RNE)."""
    a = _rng(*key).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.astype(np.float16).reshape(shape)


# ---------------------------------------------------------------------------
# Draft weight preparation: round-to-nearest into the GPTQ INT4 checkpoint
# layout.  This replaces GPTQ's calibration (which needs data); both the
# oracle and the kernels receive its output as input.
#   qweight int32 [K/8, N]   : nibble i (bits 4i..4i+3) of word [r, n] = row 8r+i
#   scales  fp16  [K/128, N]
#   qzeros  int32 [K/128, N/8]: nibble i of word [g, c] = zero of column 8c+i
# (zeros stored as-is, no "-1" offset; no act-order permutation.)
# ---------------------------------------------------------------------------

def rtn_quantize(w_kn: np.ndarray, bits: int = 4):
    """Quantise a fp16 [K, N] matrix per (group of 128 rows, column).

    Returns (q uint8 [K, N] in 0..2^bits-1, scales fp16 [K/128, N], zeros
    uint8 [K/128, N]) with W ~= (q - z) * s.
    """
    K, N = w_kn.shape
    assert K % GROUP == 0
    qmax = float((1 << bits) - 1)
    w = w_kn.astype(np.float32).reshape(K // GROUP, GROUP, N)
    lo = np.minimum(w.min(axis=1), np.float32(0))
    hi = np.maximum(w.max(axis=1), np.float32(0))
    s16 = ((hi - lo) / np.float32(qmax)).astype(np.float16)
    s16 = np.where(hi == lo, np.float16(1), s16)
    s16 = np.where(s16 == 0, np.float16(1), s16)  # spans below fp16's range
    s = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / s), 0, qmax).astype(np.float32)
    q = np.clip(np.rint(w / s[:, None, :]) + z[:, None, :], 0, qmax).astype(np.uint8)
    return q.reshape(K, N), s16, z.astype(np.uint8)


def pack_gptq(q: np.ndarray, s16: np.ndarray, z: np.ndarray, bits: int = 4):
    """Pack bits-bit codes and zeros into the GPTQ int32 layout (32/bits codes
    per word along K for the codes, along N for the zeros)."""
    per = 32 // bits
    K, N = q.shape
    q32 = q.astype(np.uint32).reshape(K // per, per, N)
    qweight = np.zeros((K // per, N), dtype=np.uint32)
    for i in range(per):
        qweight |= q32[:, i, :] << np.uint32(bits * i)
    G = z.shape[0]
    z32 = z.astype(np.uint32).reshape(G, N // per, per)
    qzeros = np.zeros((G, N // per), dtype=np.uint32)
    for i in range(per):
        qzeros |= z32[:, :, i] << np.uint32(bits * i)
    return qweight.view(np.int32), np.ascontiguousarray(s16), qzeros.view(np.int32)


def gptq_from_linear(w_nk: np.ndarray, bits: int = 4):
    """GPTQ tensors (bits-bit codes) for an nn.Linear-layout fp16 weight [N, K]."""
    q, s, z = rtn_quantize(np.ascontiguousarray(w_nk.T), bits)
    return pack_gptq(q, s, z, bits)


# ---------------------------------------------------------------------------
# Layer tensors
# ---------------------------------------------------------------------------

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def router(shape: LayerShape, layer: int = 0, seed: int = BASE_SEED) -> np.ndarray:
    """fp16 [E, H] router shared by draft and target."""
    return normal_f16((seed, shape.config_id, layer, 0, T_ROUTER, 0), (shape.E, shape.H), 0.02)


def expert_f16(shape: LayerShape, layer: int, expert: int, seed: int = BASE_SEED):
    """FP16 target expert: w13 [2I, H] (gate rows then up rows), w2 [H, I]."""
    w13 = normal_f16((seed, shape.config_id, layer, expert, T_W13, 0), (2 * shape.I, shape.H), 0.02)
    w2 = normal_f16((seed, shape.config_id, layer, expert, T_W2, 0), (shape.H, shape.I), 0.02)
    return w13, w2


def expert_int4(w13: np.ndarray, w2: np.ndarray, bits: int = 4):
    """Draft expert: GPTQ g128 (INT4 unless bits says 2 or 8) of the target's
    w13 and w2."""
    return dict(w13=gptq_from_linear(w13, bits), w2=gptq_from_linear(w2, bits))


def awq_factors(key: Sequence[int], n: int) -> np.ndarray:
    """Positive per-input-channel factors 2^u, u ~ U(-1, 1), rounded to fp16
    (stand-ins for the activation-statistics factors AWQ chooses, which need
    calibration data)."""
    u = _rng(*key).uniform(-1.0, 1.0, n).astype(np.float32)
    return np.exp2(u).astype(np.float16)


def expert_awq(shape: LayerShape, layer: int, expert: int, w13: np.ndarray, w2: np.ndarray,
               seed: int = BASE_SEED):
    """AWQ-style draft expert: input channel c of w13 (hidden) and of w2
    (intermediate) multiplied by its factor a[c] before the same RTN GPTQ
    INT4 g128 quantisation; returns the GPTQ tensors and the factors
    (a13 [H], a2 [I]), by which the kernels divide the activations."""
    a13 = awq_factors((seed, shape.config_id, layer, expert, T_AWQ13, 0), w13.shape[1])
    a2 = awq_factors((seed, shape.config_id, layer, expert, T_AWQ2, 0), w2.shape[1])
    s13 = (w13.astype(np.float32) * a13.astype(np.float32)[None, :]).astype(np.float16)
    s2 = (w2.astype(np.float32) * a2.astype(np.float32)[None, :]).astype(np.float16)
    return dict(w13=gptq_from_linear(s13), w2=gptq_from_linear(s2), a13=a13, a2=a2)


def quant_bytes_per_expert(shape: LayerShape, bits: int) -> int:
    """Packed codes + fp16 scales + packed zeros of w13 and w2 at `bits`."""
    H, I = shape.H, shape.I
    mats = ((H, 2 * I), (I, H))  # (K, N)
    return sum(K * N * bits // 8 + (K // GROUP) * N * 2 + (K // GROUP) * N * bits // 8
               for K, N in mats)


def shared_expert(shape: LayerShape, layer: int = 0, seed: int = BASE_SEED):
    """FP16 shared expert (w13 [2*Is, H], w2 [H, Is]) and the optional fp16
    sigmoid-gate vector [H]; None when the shape has no shared expert."""
    if shape.shared_I == 0:
        return None
    Is = shape.shared_I
    if shape.name == "ds_v2_lite":
        # two shared experts of intermediate I; concatenated they are one
        # expert of intermediate 2I (gate rows, then up rows; w2 columns).
        parts = []
        for j in range(2):
            w13 = normal_f16((seed, shape.config_id, layer, 1000 + j, T_SH_W13, 0),
                             (2 * shape.I, shape.H), 0.02)
            w2 = normal_f16((seed, shape.config_id, layer, 1000 + j, T_SH_W2, 0),
                            (shape.H, shape.I), 0.02)
            parts.append((w13, w2))
        I = shape.I
        w13 = np.concatenate([parts[0][0][:I], parts[1][0][:I], parts[0][0][I:], parts[1][0][I:]])
        w2 = np.concatenate([parts[0][1], parts[1][1]], axis=1)
        return dict(w13=w13, w2=w2, parts=parts, gate=None)
    w13 = normal_f16((seed, shape.config_id, layer, 1000, T_SH_W13, 0), (2 * Is, shape.H), 0.02)
    w2 = normal_f16((seed, shape.config_id, layer, 1000, T_SH_W2, 0), (shape.H, Is), 0.02)
    gate = None
    if shape.shared_gate:
        gate = normal_f16((seed, shape.config_id, layer, 1000, T_SH_GATE, 0), (shape.H,), 0.02)
    return dict(w13=w13, w2=w2, parts=None, gate=gate)


def tokens(shape: LayerShape, T: int, step: int = 0, layer: int = 0, seed: int = BASE_SEED):
    """fp16 [T, H] token activations ~ N(0, 1)."""
    return normal_f16((seed, shape.config_id, layer, 0, T_TOKENS, step), (T, shape.H), 1.0)


def token_stream(shape: LayerShape, n: int, rho: float, step: int = 0,
                 seed: int = BASE_SEED) -> np.ndarray:
    """fp16 [n, H] token rows with N(0, 1) marginals and lag-one correlation
    rho between consecutive rows (an AR(1) stream): consecutive tokens then
    tend to route alike, a knob for the routing locality of real text.
    rho = 0 gives independent rows."""
    g = _rng(seed, shape.config_id, 0, 0, T_TOKENS, 1_000_000 + step)
    eps = g.standard_normal((n, shape.H), dtype=np.float32)
    out = np.empty_like(eps)
    c = np.float32(np.sqrt(1.0 - rho * rho))
    out[0] = eps[0]
    for t in range(1, n):
        out[t] = np.float32(rho) * out[t - 1] + c * eps[t]
    return out.astype(np.float16)


def make_layer(shape: LayerShape, layer: int = 0, seed: int = BASE_SEED,
               experts: Optional[Sequence[int]] = None, int4: bool = True,
               f16: bool = True, threads: Optional[int] = None) -> Dict:
    """All tensors of one MoE layer.

    Returns dict(router, shared, f16=[(w13, w2)] * E, int4=[dict] * E).
    `experts` restricts generation to a subset (others are None).
    """
    idx = list(range(shape.E)) if experts is None else list(experts)

    def one(e):
        w13, w2 = expert_f16(shape, layer, e, seed)
        q = expert_int4(w13, w2) if int4 else None
        return e, ((w13, w2) if f16 else None), q

    f16_list: List = [None] * shape.E
    q_list: List = [None] * shape.E
    with ThreadPoolExecutor(threads or _threads()) as ex:
        for e, f, q in ex.map(one, idx):
            f16_list[e] = f
            q_list[e] = q
    return dict(shape=shape, layer=layer, router=router(shape, layer, seed),
                shared=shared_expert(shape, layer, seed), f16=f16_list, int4=q_list)


# ---------------------------------------------------------------------------
# Device-side generation for the large multi-layer workload (24 layers x 60
# experts = 12.5 G parameters would take tens of minutes in NumPy).  Same
# recipe -- N(0, 0.02) fp32 draws rounded to fp16, RTN into the GPTQ layout
# -- from torch's Philox generator seeded per tensor; the values differ from
# the NumPy streams above, so a comparison always hands the same generated
# tensors to the oracle and to the kernels.
# ---------------------------------------------------------------------------

def _torch_seed(*key: int) -> int:
    ss = np.random.SeedSequence([int(v) for v in key])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def torch_normal_f16(key, shape, std, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*key))
    a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        a.mul_(std)
    return a.to(torch.float16)


def torch_gptq_from_linear(w_nk):
    """GPTQ INT4 (qweight int32 [K/8, N], scales fp16 [K/128, N], qzeros int32
    [K/128, N/8]) of an fp16 nn.Linear weight [N, K] on its device; same RTN
    rule as `rtn_quantize`."""
    import torch
    w = w_nk.t().float()
    K, N = w.shape
    wg = w.reshape(K // GROUP, GROUP, N)
    lo = torch.clamp(wg.amin(dim=1), max=0.0)
    hi = torch.clamp(wg.amax(dim=1), min=0.0)
    s16 = ((hi - lo) / 15.0).to(torch.float16)
    one = torch.ones_like(s16)
    s16 = torch.where(hi == lo, one, s16)
    s16 = torch.where(s16 == 0, one, s16)
    s = s16.float()
    z = torch.clamp(torch.round(-lo / s), 0, 15)
    q = torch.clamp(torch.round(wg / s[:, None, :]) + z[:, None, :], 0, 15).to(torch.int32)
    q = q.reshape(K // 8, 8, N)
    qweight = torch.zeros((K // 8, N), dtype=torch.int32, device=w.device)
    for i in range(8):
        qweight |= q[:, i, :] << (4 * i)
    zi = z.to(torch.int32).reshape(K // GROUP, N // 8, 8)
    qzeros = torch.zeros((K // GROUP, N // 8), dtype=torch.int32, device=w.device)
    for i in range(8):
        qzeros |= zi[:, :, i] << (4 * i)
    return qweight.contiguous(), s16.contiguous(), qzeros.contiguous()


def torch_layer(shape: LayerShape, layer: int, device, seed: int = BASE_SEED, int4: bool = True):
    """One layer generated on `device`: router, shared expert (+gate), and per
    expert the FP16 target weights (w13 [2I, H], w2 [H, I]) and, optionally,
    their GPTQ INT4 draft copies."""
    c = shape.config_id
    out = dict(router=torch_normal_f16((seed, c, layer, 0, T_ROUTER, 0), (shape.E, shape.H), 0.02,
                                       device), f16=[], int4=[])
    for e in range(shape.E):
        w13 = torch_normal_f16((seed, c, layer, e, T_W13, 0), (2 * shape.I, shape.H), 0.02, device)
        w2 = torch_normal_f16((seed, c, layer, e, T_W2, 0), (shape.H, shape.I), 0.02, device)
        out["f16"].append((w13, w2))
        if int4:
            out["int4"].append(dict(w13=torch_gptq_from_linear(w13), w2=torch_gptq_from_linear(w2)))
    out["shared"] = None
    if shape.shared_I:
        Is = shape.shared_I
        out["shared"] = dict(
            w13=torch_normal_f16((seed, c, layer, 1000, T_SH_W13, 0), (2 * Is, shape.H), 0.02, device),
            w2=torch_normal_f16((seed, c, layer, 1000, T_SH_W2, 0), (shape.H, Is), 0.02, device),
            gate=(torch_normal_f16((seed, c, layer, 1000, T_SH_GATE, 0), (shape.H,), 0.02, device)
                  if shape.shared_gate else None))
    return out
