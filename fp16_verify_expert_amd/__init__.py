"""Python binding of libsmoe.so (the routed-expert MoE FFN path for gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the stream; outputs not passed in are
allocated with torch.  Functions carry the C entry points' names.  There is no
CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "smoe.h")
ABI_VERSION = 7

SMOE_DERR_BAD_ID = 1
SMOE_DERR_NULL_EXPERT = 2

_STATUS = {0: "SMOE_OK", 1: "SMOE_ERR_NULL", 2: "SMOE_ERR_SHAPE", 3: "SMOE_ERR_UNSUPPORTED",
           4: "SMOE_ERR_HIP", 5: "SMOE_ERR_NOT_PINNED", 6: "SMOE_ERR_WORKSPACE"}


class SmoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "smoe_abi_version": (_i, []),
    "smoe_last_error": (ctypes.c_char_p, []),
    "smoe_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_route_topk": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "elb_count": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "moe_gather": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_plan": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp,
                            _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "w4a16_grouped_ffn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp,
                               _sz, _vp, _vp]),
    "w4a16_grouped_ffn_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                       _vp, _vp, _vp]),
    "w4a16_grouped_ffn_shared": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                      _vp, _vp, _vp, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "awq_grouped_ffn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp,
                             _vp, _sz, _vp, _vp]),
    "wq_grouped_ffn": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                            _sz, _vp, _vp]),
    "moe_draft_route_ffn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _i, _vp, _vp,
                                 _vp, _vp, _sz, _vp, _vp]),
    "moe_combine_route_logits": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                      ctypes.c_float, _vp, _vp, _i, _vp, _vp]),
    # x, w_router, w_shared_gate, logits, H, I, E, k, renorm, layer, L, counters, experts,
    # group_size, ids, w, gate, off, sorted_token, sorted_pair, pair_pos, active, n_active,
    # y_sorted, shared_w13, shared_w2, shared_I, shared_h, shared_out, residual, out,
    # norm_out, eps, next_router, next_shared_gate, next_E, next_logits, ws, ws_bytes, err,
    # stream
    "moe_draft_layer": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                             _vp, _vp, _i, _vp, _vp, _sz, _vp, _vp]),
    "smoe_draft_layer_supported": (_i, [_i, _i, _i, _i, _i]),
    "verify_grouped_gemm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                 _vp, _sz, _vp, _vp]),
    "verify_grouped_gemm_shared": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                        _vp, _vp, _vp, _i, _vp, _vp, _vp, _sz, _vp, _vp]),
    "moe_combine": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, ctypes.c_float,
                         _vp]),
    "expert_stage_async": (_i, [_vp, _vp, _sz, _vp, _vp]),
    "smoe_stream_read": (_i, [_vp, _sz, _vp, _i, _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        v = L.smoe_abi_version()
        if v != ABI_VERSION:
            raise ImportError(f"libsmoe ABI {v} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


def header_functions() -> Sequence[str]:
    """Names of the functions declared in include/smoe.h."""
    txt = open(HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:smoe_status|int|const char\*|size_t)\s+(\w+)\s*\(", txt, re.M)
    return names


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise SmoeError(name, st, lib().smoe_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _s(stream) -> _vp:
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name}: expected a contiguous {dtype} CUDA tensor, got "
                         f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")


def workspace_bytes(which: int, T: int, k: int, H: int, I: int, E: int) -> int:
    return int(lib().smoe_workspace_bytes(which, T, k, H, I, E))


def new_workspace(which: int, T: int, k: int, H: int, I: int, E: int,
                  device="cuda") -> torch.Tensor:
    """Zero-filled workspace (the kernels need no initialisation; zeroed so
    unused bytes are deterministic)."""
    n = max(256, workspace_bytes(which, T, k, H, I, E))
    return torch.zeros(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- calls ----

def moe_route_topk(x, w_router, k: int, renormalize: bool = False, w_shared_gate=None, *,
                   topk_ids=None, topk_w=None, shared_gate=None, stream=None):
    _check(x, torch.float16, "x")
    _check(w_router, torch.float16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if w_shared_gate is not None:
        _check(w_shared_gate, torch.float16, "w_shared_gate")
        if shared_gate is None:
            shared_gate = torch.empty((T,), dtype=torch.float32, device=dev)
    _call("moe_route_topk", _p(x), _p(w_router), _p(w_shared_gate), T, H, E, k,
          1 if renormalize else 0, _p(topk_ids), _p(topk_w),
          _p(shared_gate) if w_shared_gate is not None else None, _s(stream))
    return topk_ids, topk_w, shared_gate


def elb_count(topk_ids, E: int, layer: int, counters, err_word=None, stream=None):
    _check(topk_ids, torch.int32, "topk_ids")
    _check(counters, torch.int32, "counters")
    T, k = topk_ids.shape
    L = counters.shape[0]
    _call("elb_count", _p(topk_ids), T, k, E, layer, L, _p(counters), _p(err_word), _s(stream))
    return counters


def moe_gather(topk_ids, E: int, err_word=None, *, out=None, stream=None):
    """Returns dict(offsets, sorted_token, sorted_pair, pair_pos, active, n_active)."""
    _check(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    if out is None:
        out = _new_maps(T, k, E, topk_ids.device)
    _call("moe_gather", _p(topk_ids), T, k, E, _p(out["offsets"]), _p(out["sorted_token"]),
          _p(out["sorted_pair"]), _p(out["pair_pos"]), _p(out["active"]), _p(out["n_active"]),
          _p(err_word), _s(stream))
    return out


def _new_maps(T: int, k: int, E: int, dev) -> dict:
    n = max(T * k, 1)
    return dict(offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                sorted_token=torch.empty(n, dtype=torch.int32, device=dev),
                sorted_pair=torch.empty(n, dtype=torch.int32, device=dev),
                pair_pos=torch.empty(n, dtype=torch.int32, device=dev),
                active=torch.empty(E, dtype=torch.int32, device=dev),
                n_active=torch.empty(1, dtype=torch.int32, device=dev))


def moe_route_plan(x, w_router, k: int, renormalize: bool = False, w_shared_gate=None, *,
                   counters=None, layer: int = 0, err_word=None, topk_ids=None, topk_w=None,
                   shared_gate=None, maps=None, logits_ws=None, spread: bool = True,
                   stream=None):
    """Routing, ELB update (when counters is given) and gather maps.  With
    spread (the default) the call passes the library a logits workspace
    (logits_ws, a device tensor of at least T*(E+1) fp32, allocated here when
    None), so large steps spread the router dot products over the chip;
    spread=False passes none.  Returns (topk_ids, topk_w, shared_gate, maps)
    with maps as from moe_gather."""
    _check(x, torch.float16, "x")
    _check(w_router, torch.float16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if w_shared_gate is not None:
        _check(w_shared_gate, torch.float16, "w_shared_gate")
        if shared_gate is None:
            shared_gate = torch.empty((T,), dtype=torch.float32, device=dev)
    L = 0
    if counters is not None:
        _check(counters, torch.int32, "counters")
        L = counters.shape[0]
    if maps is None:
        maps = _new_maps(T, k, E, dev)
    if not spread:
        logits_ws = None
    elif logits_ws is None:
        logits_ws = torch.empty(max(1, T * (E + 1)), dtype=torch.float32, device=dev)
    else:
        _check(logits_ws, torch.float32, "logits_ws")
    ws_bytes = logits_ws.numel() * logits_ws.element_size() if logits_ws is not None else 0
    _call("moe_route_plan", _p(x), _p(w_router), _p(w_shared_gate), T, H, E, k,
          1 if renormalize else 0, layer, L, _p(counters), _p(topk_ids), _p(topk_w),
          _p(shared_gate) if w_shared_gate is not None else None, _p(maps["offsets"]),
          _p(maps["sorted_token"]), _p(maps["sorted_pair"]), _p(maps["pair_pos"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(logits_ws), ws_bytes, _p(err_word),
          _s(stream))
    return topk_ids, topk_w, shared_gate, maps


def w4_expert_table(experts: Sequence, device="cuda") -> torch.Tensor:
    """Device array of smoe_w4_expert from per-expert dicts
    {w13: (qweight, scales, qzeros), w2: (...)} of CUDA tensors (None = absent)."""
    rows = []
    for ex in experts:
        if ex is None:
            rows.append([0] * 6)
            continue
        r = []
        for key in ("w13", "w2"):
            for t in ex[key]:
                r.append(0 if t is None else t.data_ptr())
        rows.append(r)
    return torch.tensor(rows, dtype=torch.int64).to(device)


def f16_expert_table(experts: Sequence, device="cuda") -> torch.Tensor:
    """Device array of smoe_f16_expert from (w13, w2) CUDA tensor pairs."""
    rows = [[0, 0] if ex is None else [0 if t is None else t.data_ptr() for t in ex]
            for ex in experts]
    return torch.tensor(rows, dtype=torch.int64).to(device)


def w4a16_grouped_ffn(x, maps, table, T: int, k: int, H: int, I: int, E: int, workspace,
                      *, y_sorted=None, err_word=None, stream=None):
    _check(x, torch.float16, "x")
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), H), dtype=torch.float16, device=x.device)
    _call("w4a16_grouped_ffn", _p(x), _p(maps["sorted_token"]), _p(maps["offsets"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(table), T, k, H, I, E, 128,
          _p(y_sorted), _p(workspace), workspace.numel() * workspace.element_size(),
          _p(err_word), _s(stream))
    return y_sorted


def w4a16_grouped_ffn_shared(x, maps, table, T: int, k: int, H: int, I: int, E: int, workspace,
                             shared, *, y_sorted=None, shared_h=None, shared_out=None,
                             err_word=None, stream=None):
    """w4a16_grouped_ffn plus the dense FP16 shared expert shared = (w13
    [2 Is, H], w2 [H, Is]) over all T rows of x.  Returns (y_sorted,
    shared_out [T, H])."""
    _check(x, torch.float16, "x")
    sw13, sw2 = shared
    _check(sw13, torch.float16, "shared w13")
    _check(sw2, torch.float16, "shared w2")
    Is = sw2.shape[1]
    dev = x.device
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), H), dtype=torch.float16, device=dev)
    if shared_h is None:
        shared_h = torch.empty((T, Is), dtype=torch.float16, device=dev)
    if shared_out is None:
        shared_out = torch.empty((T, H), dtype=torch.float16, device=dev)
    _call("w4a16_grouped_ffn_shared", _p(x), _p(maps["sorted_token"]), _p(maps["offsets"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(table), T, k, H, I, E, 128,
          _p(y_sorted), _p(sw13), _p(sw2), Is, _p(shared_h), _p(shared_out), _p(workspace),
          workspace.numel() * workspace.element_size(), _p(err_word), _s(stream))
    return y_sorted, shared_out


def w4a16_grouped_ffn_noalloc(x, maps, table, T: int, k: int, H: int, I: int, E: int, *,
                              y_sorted=None, err_word=None, stream=None):
    """w4a16_grouped_ffn with the library's own scratch in place of a
    workspace (allocates nothing inside the library; y_sorted is allocated
    here only when not passed)."""
    _check(x, torch.float16, "x")
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), H), dtype=torch.float16, device=x.device)
    _call("w4a16_grouped_ffn_noalloc", _p(x), _p(maps["sorted_token"]), _p(maps["offsets"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(table), T, k, H, I, E, 128,
          _p(y_sorted), _p(err_word), _s(stream))
    return y_sorted


NOALLOC_SCRATCH_BYTES = 4 << 20


def awq_scale_table(scales: Sequence, device="cuda") -> torch.Tensor:
    """Device array of 2E fp16 pointers from per-expert (a13 [H], a2 [I])
    CUDA tensors (None = absent)."""
    rows = []
    for sc in scales:
        rows += [0, 0] if sc is None else [sc[0].data_ptr(), sc[1].data_ptr()]
    return torch.tensor(rows, dtype=torch.int64).to(device)


def awq_grouped_ffn(x, maps, table, scale_table, T: int, k: int, H: int, I: int, E: int,
                    workspace, *, y_sorted=None, err_word=None, stream=None):
    """w4a16_grouped_ffn for AWQ-style experts: per-input-channel divisors
    (scale_table from awq_scale_table) applied to each projection's input."""
    _check(x, torch.float16, "x")
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), H), dtype=torch.float16, device=x.device)
    _call("awq_grouped_ffn", _p(x), _p(maps["sorted_token"]), _p(maps["offsets"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(table), _p(scale_table), T, k, H, I, E,
          128, _p(y_sorted), _p(workspace), workspace.numel() * workspace.element_size(),
          _p(err_word), _s(stream))
    return y_sorted


def wq_grouped_ffn(x, maps, table, T: int, k: int, H: int, I: int, E: int, workspace,
                   bits: int, *, y_sorted=None, err_word=None, stream=None):
    """w4a16_grouped_ffn for 2-, 4- or 8-bit GPTQ-layout experts."""
    _check(x, torch.float16, "x")
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), H), dtype=torch.float16, device=x.device)
    _call("wq_grouped_ffn", _p(x), _p(maps["sorted_token"]), _p(maps["offsets"]),
          _p(maps["active"]), _p(maps["n_active"]), _p(table), T, k, H, I, E, bits, 128,
          _p(y_sorted), _p(workspace), workspace.numel() * workspace.element_size(),
          _p(err_word), _s(stream))
    return y_sorted


def moe_draft_route_ffn(x, w_router, k: int, table, I: int, workspace,
                        renormalize: bool = False, w_shared_gate=None, *, counters=None,
                        layer: int = 0, err_word=None, topk_ids=None, topk_w=None,
                        shared_gate=None, maps=None, y_sorted=None, shared=None, shared_h=None,
                        shared_out=None, logits=None, stream=None):
    """One-token draft step: moe_route_plan and w4a16_grouped_ffn in three
    launches.  With shared = (w13 [2 Is, H], w2 [H, Is]) fp16, a dense shared
    expert computed in the same launches (shared_h: [Is] fp16 scratch,
    shared_out: [1, H] fp16 out).  Returns (topk_ids, topk_w, shared_gate,
    maps, y_sorted), plus shared_out when a shared expert is given.  logits
    (fp32 [E (+1)], optional): the router logits of x from
    moe_combine_route_logits, taken instead of a logits launch."""
    _check(x, torch.float16, "x")
    _check(w_router, torch.float16, "w_router")
    T, H = x.shape
    if T != 1:
        raise ValueError(f"moe_draft_route_ffn takes one token, got T={T}")
    E = w_router.shape[0]
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((1, k), dtype=torch.float32, device=dev)
    if w_shared_gate is not None:
        _check(w_shared_gate, torch.float16, "w_shared_gate")
        if shared_gate is None:
            shared_gate = torch.empty((1,), dtype=torch.float32, device=dev)
    L = 0
    if counters is not None:
        _check(counters, torch.int32, "counters")
        L = counters.shape[0]
    if maps is None:
        maps = _new_maps(1, k, E, dev)
    if y_sorted is None:
        y_sorted = torch.empty((k, H), dtype=torch.float16, device=dev)
    sw13 = sw2 = None
    Is = 0
    if shared is not None:
        sw13, sw2 = shared
        _check(sw13, torch.float16, "shared w13")
        _check(sw2, torch.float16, "shared w2")
        Is = sw2.shape[1]
        if shared_h is None:
            shared_h = torch.empty((Is,), dtype=torch.float16, device=dev)
        if shared_out is None:
            shared_out = torch.empty((1, H), dtype=torch.float16, device=dev)
    _call("moe_draft_route_ffn", _p(x), _p(w_router), _p(w_shared_gate), H, I, E, k,
          1 if renormalize else 0, layer, L, _p(counters), _p(table), 128, _p(topk_ids),
          _p(topk_w), _p(shared_gate) if w_shared_gate is not None else None,
          _p(maps["offsets"]), _p(maps["sorted_token"]), _p(maps["sorted_pair"]),
          _p(maps["pair_pos"]), _p(maps["active"]), _p(maps["n_active"]), _p(y_sorted),
          _p(sw13), _p(sw2), Is, _p(shared_h) if shared is not None else None,
          _p(shared_out) if shared is not None else None, _p(logits),
          _p(workspace), workspace.numel() * workspace.element_size(), _p(err_word), _s(stream))
    if shared is not None:
        return topk_ids, topk_w, shared_gate, maps, y_sorted, shared_out
    return topk_ids, topk_w, shared_gate, maps, y_sorted


def draft_layer_supported(H: int, I: int, E: int, k: int, shared_I: int = 0) -> bool:
    """True when moe_draft_layer has a one-launch geometry for this layer
    shape on the current device."""
    return bool(lib().smoe_draft_layer_supported(H, I, E, k, shared_I))


def new_layer_workspace(k: int, H: int, I: int, E: int, device="cuda") -> torch.Tensor:
    """Zero-filled moe_draft_layer workspace (its barrier counters start at
    zero; every completed call leaves them zero)."""
    n = max(256, workspace_bytes(2, 1, k, H, I, E))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_draft_layer(x, w_router, k: int, table, I: int, workspace, renormalize: bool = False,
                    w_shared_gate=None, *, logits=None, counters=None, layer: int = 0,
                    err_word=None, topk_ids=None, topk_w=None, shared_gate=None, maps=None,
                    y_sorted=None, shared=None, shared_h=None, shared_out=None, residual=None,
                    out=None, norm_out=None, norm_eps: float = 1e-6, next_router=None,
                    next_shared_gate=None, next_logits=None, stream=None):
    """One-token draft step of a whole MoE layer in one launch:
    moe_draft_route_ffn followed by moe_combine (norm_out None) or
    moe_combine_route_logits (next_router given), with bit-identical
    outputs.  logits: the router logits of x from the launch before (None:
    computed in the launch).  norm_out: a tensor, True to allocate one, or
    None.  Returns a dict with topk_ids, topk_w, shared_gate, maps, y_sorted,
    shared_out, out, norm_out and next_logits (None where not computed)."""
    _check(x, torch.float16, "x")
    _check(w_router, torch.float16, "w_router")
    T, H = x.shape
    if T != 1:
        raise ValueError(f"moe_draft_layer takes one token, got T={T}")
    E = w_router.shape[0]
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((1, k), dtype=torch.float32, device=dev)
    if w_shared_gate is not None:
        _check(w_shared_gate, torch.float16, "w_shared_gate")
        if shared_gate is None:
            shared_gate = torch.empty((1,), dtype=torch.float32, device=dev)
    L = 0
    if counters is not None:
        _check(counters, torch.int32, "counters")
        L = counters.shape[0]
    if maps is None:
        maps = _new_maps(1, k, E, dev)
    if y_sorted is None:
        y_sorted = torch.empty((k, H), dtype=torch.float16, device=dev)
    sw13 = sw2 = None
    Is = 0
    if shared is not None:
        sw13, sw2 = shared
        _check(sw13, torch.float16, "shared w13")
        _check(sw2, torch.float16, "shared w2")
        Is = sw2.shape[1]
        if shared_h is None:
            shared_h = torch.empty((Is,), dtype=torch.float16, device=dev)
        if shared_out is None:
            shared_out = torch.empty((1, H), dtype=torch.float16, device=dev)
    if residual is not None:
        _check(residual, torch.float16, "residual")
    if out is None:
        out = torch.empty((1, H), dtype=torch.float16, device=dev)
    if norm_out is True or (norm_out is None and next_router is not None):
        norm_out = torch.empty((1, H), dtype=torch.float16, device=dev)
    nE = 0
    if next_router is not None:
        _check(next_router, torch.float16, "next_router")
        nE = next_router.shape[0]
        if next_shared_gate is not None:
            _check(next_shared_gate, torch.float16, "next_shared_gate")
        if next_logits is None:
            next_logits = torch.empty(nE + (1 if next_shared_gate is not None else 0),
                                      dtype=torch.float32, device=dev)
    _call("moe_draft_layer", _p(x), _p(w_router), _p(w_shared_gate), _p(logits), H, I, E, k,
          1 if renormalize else 0, layer, L, _p(counters), _p(table), 128, _p(topk_ids),
          _p(topk_w), _p(shared_gate) if w_shared_gate is not None else None,
          _p(maps["offsets"]), _p(maps["sorted_token"]), _p(maps["sorted_pair"]),
          _p(maps["pair_pos"]), _p(maps["active"]), _p(maps["n_active"]), _p(y_sorted),
          _p(sw13), _p(sw2), Is, _p(shared_h) if shared is not None else None,
          _p(shared_out) if shared is not None else None, _p(residual), _p(out),
          _p(norm_out), float(norm_eps), _p(next_router), _p(next_shared_gate), nE,
          _p(next_logits) if next_router is not None else None,
          _p(workspace), workspace.numel() * workspace.element_size(), _p(err_word), _s(stream))
    return dict(topk_ids=topk_ids, topk_w=topk_w, shared_gate=shared_gate, maps=maps,
                y_sorted=y_sorted, shared_out=shared_out if shared is not None else None,
                out=out, norm_out=norm_out,
                next_logits=next_logits if next_router is not None else None)


def verify_grouped_gemm(x, sorted_token, offsets, table, T: int, rows: int, H: int, I: int,
                        E: int, workspace, *, active=None, n_active=None, expert_mask=None,
                        y_sorted=None, err_word=None, stream=None):
    _check(x, torch.float16, "x")
    if y_sorted is None:
        y_sorted = torch.empty((max(rows, 1), H), dtype=torch.float16, device=x.device)
    _call("verify_grouped_gemm", _p(x), _p(sorted_token), _p(offsets), _p(active),
          _p(n_active), _p(table), _p(expert_mask), T, rows, H, I, E, _p(y_sorted),
          _p(workspace), workspace.numel() * workspace.element_size(), _p(err_word), _s(stream))
    return y_sorted


def verify_grouped_gemm_shared(x, sorted_token, offsets, table, T: int, rows: int, H: int,
                               I: int, E: int, workspace, shared, *, active=None, n_active=None,
                               expert_mask=None, y_sorted=None, shared_h=None, shared_out=None,
                               err_word=None, stream=None):
    """verify_grouped_gemm over the routed experts and the dense shared
    expert shared = (w13 [2 Is, H], w2 [H, Is]) over all T rows of x in the
    same launches.  Returns (y_sorted, shared_out [T, H])."""
    _check(x, torch.float16, "x")
    sw13, sw2 = shared
    _check(sw13, torch.float16, "shared w13")
    _check(sw2, torch.float16, "shared w2")
    Is = sw2.shape[1]
    dev = x.device
    if y_sorted is None:
        y_sorted = torch.empty((max(rows, 1), H), dtype=torch.float16, device=dev)
    if shared_h is None:
        shared_h = torch.empty((T, Is), dtype=torch.float16, device=dev)
    if shared_out is None:
        shared_out = torch.empty((T, H), dtype=torch.float16, device=dev)
    _call("verify_grouped_gemm_shared", _p(x), _p(sorted_token), _p(offsets), _p(active),
          _p(n_active), _p(table), _p(expert_mask), T, rows, H, I, E, _p(y_sorted), _p(sw13),
          _p(sw2), Is, _p(shared_h), _p(shared_out), _p(workspace),
          workspace.numel() * workspace.element_size(), _p(err_word), _s(stream))
    return y_sorted, shared_out


def moe_combine(y_sorted, pair_pos, topk_w, shared_out=None, shared_scale=None, residual=None,
                *, out=None, norm_out=None, norm_eps: float = 1e-6, stream=None):
    """Returns out, or (out, norm_out) when norm_out is given (a tensor, or
    True to allocate one)."""
    T, k = topk_w.shape
    H = y_sorted.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.float16, device=y_sorted.device)
    want_norm = norm_out is not None and norm_out is not False
    if norm_out is True:
        norm_out = torch.empty((T, H), dtype=torch.float16, device=y_sorted.device)
    _call("moe_combine", _p(y_sorted), _p(pair_pos), _p(topk_w), _p(shared_out),
          _p(shared_scale), _p(residual), T, k, H, _p(out),
          _p(norm_out) if want_norm else None, float(norm_eps), _s(stream))
    return (out, norm_out) if want_norm else out


def moe_combine_route_logits(y_sorted, pair_pos, topk_w, w_router, shared_out=None,
                             shared_scale=None, residual=None, w_shared_gate=None, *, out=None,
                             norm_out=None, logits=None, norm_eps: float = 1e-6, stream=None):
    """One token: moe_combine (with the norm epilogue) and the next layer's
    router logits of the normalised row.  Returns (out, norm_out, logits)."""
    _check(y_sorted, torch.float16, "y_sorted")
    _check(w_router, torch.float16, "w_router")
    T, k = topk_w.shape
    if T != 1:
        raise ValueError(f"moe_combine_route_logits takes one token, got T={T}")
    H = y_sorted.shape[1]
    E = w_router.shape[0]
    dev = y_sorted.device
    if out is None:
        out = torch.empty((1, H), dtype=torch.float16, device=dev)
    if norm_out is None:
        norm_out = torch.empty((1, H), dtype=torch.float16, device=dev)
    if logits is None:
        logits = torch.empty(E + (1 if w_shared_gate is not None else 0), dtype=torch.float32,
                             device=dev)
    _call("moe_combine_route_logits", _p(y_sorted), _p(pair_pos), _p(topk_w), _p(shared_out),
          _p(shared_scale), _p(residual), k, H, _p(out), _p(norm_out), float(norm_eps),
          _p(w_router), _p(w_shared_gate), E, _p(logits), _s(stream))
    return out, norm_out, logits


def expert_stage_async(dst: torch.Tensor, src_pinned: torch.Tensor, side_stream=None,
                       done_event=None) -> None:
    nbytes = src_pinned.numel() * src_pinned.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("expert_stage_async: destination smaller than source")
    ev = None
    if done_event is not None:
        if not done_event.cuda_event:      # torch creates the event lazily
            done_event.record(side_stream if side_stream is not None else None)
        ev = _vp(done_event.cuda_event)
    _call("expert_stage_async", _p(dst), _vp(src_pinned.data_ptr()), nbytes, _s(side_stream), ev)


def smoe_stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int = 2048,
                     stream=None) -> torch.Tensor:
    """Measurement aid: one streaming read of `src` (XOR per workgroup into
    sink, uint32/int32 [blocks])."""
    _check(sink, torch.int32, "sink")
    if sink.numel() < blocks:
        raise ValueError("smoe_stream_read: sink holds fewer words than blocks")
    _call("smoe_stream_read", _p(src), src.numel() * src.element_size(), _p(sink), blocks,
          _s(stream))
    return sink
