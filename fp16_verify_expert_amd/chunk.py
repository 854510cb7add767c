"""Draft chunk + verify over several MoE layers with offloaded target experts.

Cited: "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
Speculative Offloading" (AI summary), Key Contributions 3-4 and Methodology in
Plain English; "Specter previews expert routing with an INT4 copy of the model
itself", What shipped.  The INT4 draft lives wholly in device memory.  Each
draft step adds its expert choices to a per-layer counter table on the GPU; a
copy of that table taken when the chunk ends picks the FP16 target experts to
place in HBM.  The verify then runs a layer's on-device experts first, while
the others are copied from page-locked host memory on a separate stream, and
the layer's remaining work waits on the copy's event.

This module only sequences calls of the C ABI (routing, ELB counters, gather,
W4A16 draft FFN, FP16 verify FFN with an expert mask, combine, expert staging)
and does the host-side bookkeeping the copies need (which experts are resident,
which are missing, where each expert's weights live).  Layers are pre-norm
residual blocks: x <- x + MoE(rms(x)), the normalised input of the next layer
being written by the combine epilogue; the first layer takes the incoming
token rows (unit RMS in expectation) as its normalised input.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import (expert_stage_async, f16_expert_table, moe_combine, moe_draft_route_ffn,
               moe_gather, moe_route_plan,
               moe_route_topk, new_workspace, verify_grouped_gemm, w4_expert_table,
               w4a16_grouped_ffn)


@dataclass
class ChunkLayer:
    """One layer's weights.  `host_f16` is a page-locked CPU tensor
    [E, 3*H*I] fp16 holding each target expert as w13 [2I, H] followed by
    w2 [H, I]; the INT4 draft experts and the shared expert live in HBM."""
    router: torch.Tensor                 # fp16 [E, H] (cuda)
    int4: Sequence[Dict]                 # per expert {w13: (qw, s, qz), w2: (...)} (cuda)
    host_f16: torch.Tensor               # pinned fp16 [E, 3*H*I]
    shared: Optional[tuple] = None       # (w13 [2Is, H], w2 [H, Is]) fp16 cuda
    shared_gate: Optional[torch.Tensor] = None   # fp16 [H] cuda


def top_resident(counts: np.ndarray, n: int) -> List[int]:
    """The n experts with the largest ELB counts, ties to the lower id."""
    order = np.lexsort((np.arange(counts.shape[0]), -counts.astype(np.int64)))
    return sorted(int(e) for e in order[:n])


class ChunkEngine:
    def __init__(self, layers: Sequence[ChunkLayer], H: int, E: int, k: int, I: int,
                 shared_I: int, n_resident: int, verify_T: int, device="cuda"):
        self.layers = list(layers)
        self.L = len(self.layers)
        self.H, self.E, self.k, self.I, self.Is = H, E, k, I, shared_I
        self.nres = n_resident
        self.Tv = verify_T
        self.dev = torch.device(device)
        self.ebytes = 3 * H * I * 2
        self.w13_bytes = 2 * I * H * 2
        dev = self.dev
        self.counters = torch.zeros((self.L, E), dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.pool = torch.empty((self.L, n_resident, 3 * H * I), dtype=torch.float16, device=dev)
        self.stage = torch.empty((2, E, 3 * H * I), dtype=torch.float16, device=dev)
        # per layer: the expert held by each pool slot (-1 = empty)
        self.resident: List[List[int]] = [[-1] * n_resident for _ in range(self.L)]
        self.t4 = [w4_expert_table(l.int4, device=dev) for l in self.layers]
        self.tsh = [None if l.shared is None else f16_expert_table([l.shared], device=dev)
                    for l in self.layers]
        self.side = torch.cuda.Stream(device=dev)    # staging of misses; default priority
        self.copy = torch.cuda.Stream(device=dev)    # prefetch into the pools; default priority
        self.ev_layer = [torch.cuda.Event() for _ in range(self.L)]  # prefetches of layer l landed
        self.ev_round_done = torch.cuda.Event()      # the last verify read the pools
        self.snap_host = [torch.zeros((self.L, E), dtype=torch.int32).pin_memory()
                          for _ in range(2)]
        self.snap_ev = [torch.cuda.Event() for _ in range(2)]
        self.ev_staged = [torch.cuda.Event() for _ in range(2)]
        self.ev_free = [torch.cuda.Event() for _ in range(2)]
        # per-layer pinned upload buffers (an async upload must not see its
        # source rewritten before it ran)
        self.h_table = torch.zeros((self.L, E, 2), dtype=torch.int64).pin_memory()
        self.h_mask = torch.zeros((self.L, 2, E), dtype=torch.uint8).pin_memory()
        self.d_table = torch.zeros((self.L, E, 2), dtype=torch.int64, device=dev)
        self.d_mask = torch.zeros((self.L, 2, E), dtype=torch.uint8, device=dev)
        self.ws_d = new_workspace(0, 1, k, H, I, E, device=dev)
        self.ws_v = new_workspace(1, verify_T, k, H, I, E, device=dev)
        self.ws_sh = {T: new_workspace(1, T, 1, H, shared_I, 1, device=dev)
                      for T in (1, verify_T)} if shared_I else {}
        self.sh_out = {T: torch.empty((T, H), dtype=torch.float16, device=dev)
                       for T in (1, verify_T)} if shared_I else {}
        # the draft step's shared expert rides in the routed launches: its h
        # between the projections
        self.sh_h = torch.empty((max(shared_I, 1),), dtype=torch.float16, device=dev)
        self.iota = torch.arange(max(verify_T, 1), dtype=torch.int32, device=dev)
        self.offs = {T: torch.tensor([0, T], dtype=torch.int32, device=dev) for T in (1, verify_T)}
        self.stats = dict(staged_experts=0, staged_bytes=0, hit_experts=0, miss_experts=0)

    # ------------------------------------------------------------- draft ----
    def _shared(self, l: int, x: torch.Tensor):
        if self.tsh[l] is None:
            return None
        T = x.shape[0]
        return verify_grouped_gemm(x, self.iota[:T], self.offs[T], self.tsh[l], T, T, self.H,
                                   self.Is, 1, self.ws_sh[T], y_sorted=self.sh_out[T],
                                   err_word=self.err)

    def draft_step(self, x: torch.Tensor, record: Optional[list] = None) -> torch.Tensor:
        """One INT4 draft decode step (T = 1) through all layers, counting each
        layer's expert choices in the ELB table."""
        xn = x
        for l, ly in enumerate(self.layers):
            # routing, ELB update and gather maps folded into the gate/up
            # launch, then the down projection; the FP16 shared expert's
            # columns in the same two launches (measured: as two launches of
            # its own on a side stream it overlapped nothing, 15.6 us of a
            # 39.5 us layer-step)
            res = moe_draft_route_ffn(xn, ly.router, self.k, self.t4[l], self.I, self.ws_d, False,
                                      ly.shared_gate, counters=self.counters, layer=l,
                                      err_word=self.err, shared=ly.shared, shared_h=self.sh_h,
                                      shared_out=self.sh_out[1] if ly.shared is not None else None)
            ids, w, gate, maps, y = res[:5]
            sh = res[5] if ly.shared is not None else None
            out, xn_next = moe_combine(y, maps["pair_pos"], w, sh, gate, x, norm_out=True)
            if record is not None:
                record.append(dict(layer=l, x=x, xn=xn, ids=ids, out=out, xn_next=xn_next))
            x, xn = out, xn_next
        return x

    # ------------------------------------------------------ draft graph ----
    def capture_draft(self) -> None:
        """Record one draft step (all layers, T = 1) as a HIP graph reading a
        fixed input row; draft_step_graph then costs one launch per step.
        Every buffer the step touches is allocated here, before capture, or
        from the graph's private pool during it; the library's kernels write
        no memsets."""
        self.x_static = torch.zeros((1, self.H), dtype=torch.float16, device=self.dev)
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream())
        # a first eager pass on the capture stream (one-time library set-up),
        # then the counters are restored
        saved = self.counters.clone()
        with torch.cuda.stream(side):
            self.draft_step(self.x_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.counters.copy_(saved)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out_static = self.draft_step(self.x_static)
        torch.cuda.synchronize()

    def draft_step_graph(self, x: torch.Tensor) -> torch.Tensor:
        """draft_step(x) through the captured graph; returns the graph's
        output buffer (overwritten by the next replay)."""
        self.x_static.copy_(x)
        self.graph.replay()
        return self.out_static

    # ------------------------------------------------------ any-T forward ----
    def forward(self, x: torch.Tensor, kind: str, full: Optional[torch.Tensor] = None,
                record: Optional[list] = None) -> torch.Tensor:
        """All layers over T rows with every expert in HBM: kind "int4" runs
        the draft's W4A16 experts, kind "f16" the target's FP16 experts read
        from `full` ([L, E, 3HI]).  No ELB update, no staging.  Each layer's
        ids are appended to `record` ([T, k] int32 tensors)."""
        T = x.shape[0]
        ws = new_workspace(0 if kind == "int4" else 1, T, self.k, self.H, self.I, self.E,
                           device=self.dev)
        xn = x
        for l, ly in enumerate(self.layers):
            ids, w, gate = moe_route_topk(xn, ly.router, self.k, False, ly.shared_gate)
            maps = moe_gather(ids, self.E, self.err)
            sh = None
            if self.tsh[l] is not None:
                wsh = new_workspace(1, T, 1, self.H, self.Is, 1, device=self.dev)
                sh = verify_grouped_gemm(xn, self.iota_n(T), self.offs_n(T), self.tsh[l], T, T,
                                         self.H, self.Is, 1, wsh, err_word=self.err)
            if kind == "int4":
                y = w4a16_grouped_ffn(xn, maps, self.t4[l], T, self.k, self.H, self.I, self.E, ws,
                                      err_word=self.err)
            else:
                y = verify_grouped_gemm(xn, maps["sorted_token"], maps["offsets"],
                                        self._resident_table(full, l), T, T * self.k, self.H,
                                        self.I, self.E, ws, active=maps["active"],
                                        n_active=maps["n_active"], err_word=self.err)
            out, xn_next = moe_combine(y, maps["pair_pos"], w, sh, gate, x, norm_out=True)
            if record is not None:
                record.append(ids)
            x, xn = out, xn_next
        return x

    def iota_n(self, T: int) -> torch.Tensor:
        return torch.arange(T, dtype=torch.int32, device=self.dev)

    def offs_n(self, T: int) -> torch.Tensor:
        return torch.tensor([0, T], dtype=torch.int32, device=self.dev)

    def snapshot(self) -> np.ndarray:
        """Copy of the ELB table (synchronises)."""
        return self.counters.cpu().numpy()

    def clear_counters(self) -> None:
        self.counters.zero_()

    # ---------------------------------------------------------- residency ----
    def place_residents(self, counts: np.ndarray) -> None:
        """Chunk boundary: the top experts of each layer by ELB count become
        resident (copied from pinned host memory into the layer's pool)."""
        for l in range(self.L):
            res = top_resident(counts[l], self.nres)
            self.resident[l] = list(res)
            for j, e in enumerate(res):
                self.pool[l, j].copy_(self.layers[l].host_f16[e], non_blocking=True)

    # ----------------------------------------------------------- planner ----
    def prefetch(self, counts: np.ndarray) -> int:
        """Layer-aware prefetch from an ELB snapshot: in every layer the
        experts with the largest counts (count > 0, at most the pool size)
        should be resident; the missing ones are copied from pinned host
        memory into pool slots on the copy stream, highest count first,
        reusing the slots of residents that fell out of that set (empty slots
        first, then the lowest count).  Layer l's event is recorded after its
        copies, so it marks that every prefetch into its pool issued so far
        has landed (the copy stream runs them in order).  Returns the number
        of experts copied."""
        n = 0
        for l in range(self.L):
            c = counts[l]
            want = [e for e in sorted(top_resident(c, self.nres), key=lambda e: (-int(c[e]), e))
                    if c[e] > 0]
            res = self.resident[l]
            have = set(e for e in res if e >= 0)
            load = [e for e in want if e not in have]
            if load:
                wset = set(want)
                free = [j for j, e in enumerate(res) if e < 0 or e not in wset]
                free.sort(key=lambda j: (res[j] >= 0, int(c[res[j]]) if res[j] >= 0 else -1))
                for e, j in zip(load, free):
                    expert_stage_async(self.pool[l, j], self.layers[l].host_f16[e], self.copy)
                    res[j] = e
                    n += 1
            self.ev_layer[l].record(self.copy)
        self.stats["prefetched_experts"] = self.stats.get("prefetched_experts", 0) + n
        return n

    def _snapshot_async(self, i: int) -> None:
        """Enqueue a copy of the ELB table into page-locked buffer i."""
        self.snap_host[i].copy_(self.counters, non_blocking=True)
        self.snap_ev[i].record()

    def _snapshot_read(self, i: int) -> np.ndarray:
        self.snap_ev[i].synchronize()
        return self.snap_host[i].numpy().copy()

    def run_round(self, xs: Sequence[torch.Tensor], xv: torch.Tensor, planner: bool = True,
                  chunk0: int = 2, step_s: float = 1.3e-3, h2d_gbps: float = 55.0,
                  timing: Optional[dict] = None) -> torch.Tensor:
        """One speculation round: len(xs) INT4 draft steps (graph-replayed;
        capture_draft first), then the FP16 verify of xv.

        planner=True: Cold Start -- the first chunk of chunk0 steps is drafted
        with no prediction; Prefetch Overlap -- while each next chunk drafts,
        the snapshot of the chunk before it drives prefetches on the copy
        stream, and the next chunk is sized so that its drafting roughly
        covers the transfer just issued (step_s per step, h2d_gbps per
        copy); Final Cleanup -- the last snapshot's prefetches, then the
        verify, where each layer's hits wait only for that layer's
        prefetches and misses are staged behind them.  Residency carries over
        from round to round.  planner=False: draft every step, snapshot,
        place the top experts of every layer, then verify (all copies exposed).
        `timing` (dict) receives HIP events: start, drafted, end."""
        main = torch.cuda.current_stream()
        ev = {k: torch.cuda.Event(enable_timing=True) for k in ("start", "drafted", "end")}
        self.clear_counters()
        ev["start"].record(main)
        steps = len(xs)
        if not planner:
            for x in xs:
                self.draft_step_graph(x)
            ev["drafted"].record(main)
            self.place_residents(self.snapshot())
        else:
            # pools may be rewritten only once the previous round's verify read them
            self.copy.wait_event(self.ev_round_done)
            done, c, pending, k = 0, max(1, chunk0), None, 0
            while done < steps:
                n = min(c, steps - done)
                for st in range(done, done + n):
                    self.draft_step_graph(xs[st])
                done += n
                self._snapshot_async(k % 2)
                if pending is not None:
                    nload = self.prefetch(self._snapshot_read(pending))
                    t_copy = nload * self.ebytes / (h2d_gbps * 1e9)
                    c = max(1, int(round(t_copy / step_s)))
                pending = k % 2
                k += 1
            ev["drafted"].record(main)
            self.prefetch(self._snapshot_read(pending))
        out = self.verify(xv)
        self.ev_round_done.record(main)
        ev["end"].record(main)
        if timing is not None:
            timing.update(ev)
        return out

    # ------------------------------------------------------------ verify ----
    def verify(self, x: torch.Tensor, record: Optional[list] = None,
               all_resident: Optional[torch.Tensor] = None) -> torch.Tensor:
        """FP16 verification of T = K+1 rows through all layers.  Hits run
        first; misses are staged on the side stream and run after the copy
        event.  With `all_resident` ([L, E, 3HI] in HBM) every expert is read
        from there instead (the reference for residency invariance)."""
        main = torch.cuda.current_stream()
        T = x.shape[0]
        xn = x
        # routing and maps in one plan (no ELB update: verification does not
        # tally draft choices) while it fits one workgroup's limits
        plan = T * self.k <= 1024 and T * (self.E + 1) <= 4096
        lg = torch.empty(max(1, T * (self.E + 1)), dtype=torch.float32, device=self.dev)
        for l, ly in enumerate(self.layers):
            if plan:
                ids, w, gate, maps = moe_route_plan(xn, ly.router, self.k, False, ly.shared_gate,
                                                    err_word=self.err, logits_ws=lg)
            else:
                ids, w, gate = moe_route_topk(xn, ly.router, self.k, False, ly.shared_gate)
                maps = moe_gather(ids, self.E, self.err)
            # the shared expert in line on the caller's stream: on a side
            # stream beside the routed experts the 17-token verify was slower
            # (4.25 against 4.17 ms over 24 layers; a cross-stream join costs
            # about 6 us and the concurrent launches slow each other)
            sh = self._shared(l, xn)
            rows = T * self.k
            y = torch.empty((rows, self.H), dtype=torch.float16, device=self.dev)
            if all_resident is not None:
                verify_grouped_gemm(xn, maps["sorted_token"], maps["offsets"],
                                    self._resident_table(all_resident, l),
                                    T, rows, self.H, self.I, self.E, self.ws_v,
                                    active=maps["active"], n_active=maps["n_active"],
                                    y_sorted=y, err_word=self.err)
            else:
                self._verify_staged(l, xn, maps, y, main)
            out, xn_next = moe_combine(y, maps["pair_pos"], w, sh, gate, x, norm_out=True)
            if record is not None:
                record.append(dict(layer=l, x=x, xn=xn, ids=ids, out=out, xn_next=xn_next))
            x, xn = out, xn_next
        return x

    def _resident_table(self, full: torch.Tensor, l: int) -> torch.Tensor:
        """Device descriptor table of layer l pointing into `full` ([L, E,
        3HI] in HBM), built once per buffer."""
        key = (full.data_ptr(), full.shape[0])
        if getattr(self, "_full_key", None) != key:
            base = full.data_ptr()
            step = full.stride(1) * full.element_size()
            lay = full.stride(0) * full.element_size()
            tab = torch.empty((self.L, self.E, 2), dtype=torch.int64)
            for li in range(self.L):
                for e in range(self.E):
                    p = base + li * lay + e * step
                    tab[li, e, 0], tab[li, e, 1] = p, p + self.w13_bytes
            self._full_tab = tab.to(self.dev)
            self._full_key = key
        return self._full_tab[l]

    def _verify_staged(self, l, x, maps, y, main) -> None:
        T = x.shape[0]
        rows = T * self.k
        act = maps["active"].cpu().numpy()          # the target router's decisions
        needed = [int(e) for e in act if e >= 0]
        res = self.resident[l]
        slot = {e: j for j, e in enumerate(res) if e >= 0}
        hits = [e for e in needed if e in slot]
        misses = [e for e in needed if e not in slot]
        b = l % 2
        tab = self.h_table[l]
        tab.zero_()
        mask = self.h_mask[l]
        mask.zero_()
        for e in hits:
            p = self.pool[l, slot[e]].data_ptr()
            tab[e, 0], tab[e, 1] = p, p + self.w13_bytes
            mask[0, e] = 1
        for j, e in enumerate(misses):
            p = self.stage[b, j].data_ptr()
            tab[e, 0], tab[e, 1] = p, p + self.w13_bytes
            mask[1, e] = 1
        self.d_table[l].copy_(tab, non_blocking=True)
        self.d_mask[l].copy_(mask, non_blocking=True)
        if misses:
            # the staging buffer is free once the misses two layers back ran
            self.side.wait_event(self.ev_free[b])
            for j, e in enumerate(misses):
                last = j == len(misses) - 1
                expert_stage_async(self.stage[b, j], self.layers[l].host_f16[e], self.side,
                                   self.ev_staged[b] if last else None)
        kw = dict(active=maps["active"], n_active=maps["n_active"], y_sorted=y, err_word=self.err)
        if hits:
            main.wait_event(self.ev_layer[l])  # this layer's prefetches (if any) have landed
            verify_grouped_gemm(x, maps["sorted_token"], maps["offsets"], self.d_table[l], T, rows,
                                self.H, self.I, self.E, self.ws_v, expert_mask=self.d_mask[l, 0],
                                **kw)
        if misses:
            main.wait_event(self.ev_staged[b])
            verify_grouped_gemm(x, maps["sorted_token"], maps["offsets"], self.d_table[l], T, rows,
                                self.H, self.I, self.E, self.ws_v, expert_mask=self.d_mask[l, 1],
                                **kw)
            self.ev_free[b].record(main)
        self.stats["hit_experts"] += len(hits)
        self.stats["miss_experts"] += len(misses)
        self.stats["staged_experts"] += len(misses)
        self.stats["staged_bytes"] += len(misses) * self.ebytes
