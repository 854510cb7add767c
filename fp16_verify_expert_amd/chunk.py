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

from . import (expert_stage_async, f16_expert_table, moe_combine, moe_combine_route_logits,
               moe_draft_route_ffn, moe_gather, moe_route_plan,
               moe_route_topk, new_workspace, verify_grouped_gemm, verify_grouped_gemm_shared,
               w4_expert_table,
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


class _StepBuffers:
    """Device buffers of one row count T, allocated once and reused by every
    layer and call: routing outputs, gather maps, expert outputs, the logits
    workspace of the routing plan, both FFN workspaces, the shared expert's
    output and workspace, and two ping-pong pairs for a layer's output and
    its normalised copy (the next layer's input)."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, Is: int, dev):
        i32, f32, f16 = torch.int32, torch.float32, torch.float16
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.gate = torch.empty((T,), dtype=f32, device=dev)
        n = max(T * k, 1)
        self.maps = dict(offsets=torch.empty(E + 1, dtype=i32, device=dev),
                         sorted_token=torch.empty(n, dtype=i32, device=dev),
                         sorted_pair=torch.empty(n, dtype=i32, device=dev),
                         pair_pos=torch.empty(n, dtype=i32, device=dev),
                         active=torch.empty(E, dtype=i32, device=dev),
                         n_active=torch.empty(1, dtype=i32, device=dev))
        self.y = torch.empty((n, H), dtype=f16, device=dev)
        self.lg = torch.empty(max(1, T * (E + 1)), dtype=f32, device=dev)
        self.ws_w4 = new_workspace(0, T, k, H, I, E, device=dev)
        self.ws_f16 = new_workspace(1, T, k, H, I, E, device=dev)
        self.sh_out = torch.empty((T, H), dtype=f16, device=dev) if Is else None
        self.sh_h = torch.empty((T, Is), dtype=f16, device=dev) if Is else None
        self.ws_sh = new_workspace(1, T, 1, H, Is, 1, device=dev) if Is else None
        self.iota = torch.arange(T, dtype=i32, device=dev)
        self.offs = torch.tensor([0, T], dtype=i32, device=dev)
        self.out = [torch.empty((T, H), dtype=f16, device=dev) for _ in range(2)]
        self.xn = [torch.empty((T, H), dtype=f16, device=dev) for _ in range(2)]
        # router logits of the next layer (draft chain, one token)
        self.next_lg = torch.empty(E + 1, dtype=f32, device=dev)


def top_resident(counts: np.ndarray, n: int) -> List[int]:
    """The n experts with the largest ELB counts, ties to the lower id."""
    order = np.lexsort((np.arange(counts.shape[0]), -counts.astype(np.int64)))
    return sorted(int(e) for e in order[:n])


def topk_agreement(draft_ids: np.ndarray, target_ids: np.ndarray) -> np.ndarray:
    """|draft ids & target ids| / k for every (layer, token) of two [L, N, k]
    id arrays: the draft/target routing agreement of [S1] Key Contributions
    1 and Main Findings (an INT4 copy keeps the experts its target chooses)."""
    L, N, k = target_ids.shape
    out = np.empty((L, N))
    for l in range(L):
        for t in range(N):
            out[l, t] = len(set(draft_ids[l, t].tolist()) & set(target_ids[l, t].tolist())) / k
    return out


def distinct_experts(ids: np.ndarray, depths: Sequence[int]) -> Dict[int, float]:
    """For each depth K, the mean over layers and non-overlapping windows of
    K consecutive tokens of the number of distinct experts a window routes
    to, from [L, N, k] ids: the demand a K-token speculation puts on one
    layer ([S1] Main Findings: distinct experts per layer grow with the
    depth)."""
    L, N, _ = ids.shape
    out = {}
    for K in depths:
        counts = [len(np.unique(ids[l, w * K:(w + 1) * K])) for l in range(L)
                  for w in range(N // K)]
        out[K] = float(np.mean(counts))
    return out


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
        # per row count, buffers reused by every layer and call (the draft
        # step's T = 1 and the verify's T are made here, others on first use)
        self._buf: Dict[int, _StepBuffers] = {}
        for T in (1, verify_T):
            self.bufs(T)
        # the draft step's shared expert rides in the routed launches: its h
        # between the projections
        self.sh_h = torch.empty((max(shared_I, 1),), dtype=torch.float16, device=dev)
        self.stats = dict(staged_experts=0, staged_bytes=0, hit_experts=0, miss_experts=0)

    def bufs(self, T: int) -> _StepBuffers:
        """The reusable buffers of row count T (allocated on first use)."""
        b = self._buf.get(T)
        if b is None:
            b = _StepBuffers(T, self.H, self.E, self.k, self.I, self.Is, self.dev)
            self._buf[T] = b
        return b

    def _combine(self, l: int, b: _StepBuffers, y, sh, gate, x, fresh: bool):
        """moe_combine of layer l with the residual x and the next layer's
        normalised input.  The outputs go to b's ping-pong buffers, or to new
        tensors when `fresh` (recorded layers, and the last layer, whose
        output the caller keeps)."""
        last = l == self.L - 1
        out = None if (fresh or last) else b.out[l % 2]
        xn = True if fresh else b.xn[l % 2]
        return moe_combine(y, b.maps["pair_pos"], b.w, sh, gate, x, out=out, norm_out=xn)

    # ------------------------------------------------------------- draft ----
    def _shared(self, l: int, x: torch.Tensor):
        if self.tsh[l] is None:
            return None
        T = x.shape[0]
        b = self.bufs(T)
        return verify_grouped_gemm(x, b.iota, b.offs, self.tsh[l], T, T, self.H, self.Is, 1,
                                   b.ws_sh, y_sorted=b.sh_out, err_word=self.err)

    @staticmethod
    def _record(record, l, x, xn, ids, out, xn_next) -> None:
        if record is not None:
            record.append(dict(layer=l, x=x, xn=xn, ids=ids.clone(), out=out, xn_next=xn_next))

    def draft_step(self, x: torch.Tensor, record: Optional[list] = None,
                   fuse_combine: bool = True) -> torch.Tensor:
        """One INT4 draft decode step (T = 1) through all layers, counting each
        layer's expert choices in the ELB table.  With fuse_combine, the
        combine of layer l and the router logits of layer l+1 run as one
        launch (moe_combine_route_logits), so a layer takes three launches
        instead of four; outputs are bit-identical either way."""
        b = self.bufs(1)
        fresh = record is not None
        xn = x
        lg = None
        for l, ly in enumerate(self.layers):
            # routing, ELB update and gather maps folded into the gate/up
            # launch, then the down projection; the FP16 shared expert's
            # columns in the same two launches (measured: as two launches of
            # its own on a side stream it overlapped nothing, 15.6 us of a
            # 39.5 us layer-step)
            has_sh = ly.shared is not None
            res = moe_draft_route_ffn(xn, ly.router, self.k, self.t4[l], self.I, b.ws_w4, False,
                                      ly.shared_gate, counters=self.counters, layer=l,
                                      err_word=self.err, topk_ids=b.ids, topk_w=b.w,
                                      shared_gate=b.gate if ly.shared_gate is not None else None,
                                      maps=b.maps, y_sorted=b.y, shared=ly.shared,
                                      shared_h=self.sh_h, shared_out=b.sh_out if has_sh else None,
                                      logits=lg)
            gate = res[2]
            sh = res[5] if has_sh else None
            if fuse_combine and l < self.L - 1:
                nxt = self.layers[l + 1]
                out = None if fresh else b.out[l % 2]
                xnn = None if fresh else b.xn[l % 2]
                out, xn_next, lg = moe_combine_route_logits(
                    b.y, b.maps["pair_pos"], b.w, nxt.router, sh, gate, x, nxt.shared_gate,
                    out=out, norm_out=xnn, logits=b.next_lg)
            else:
                out, xn_next = self._combine(l, b, b.y, sh, gate, x, fresh)
            self._record(record, l, x, xn, b.ids, out, xn_next)
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
        from `full` ([L, E, 3HI]).  No ELB update, no staging.  `record`
        receives one dict per layer (layer, x, xn, ids [T, k], out,
        xn_next)."""
        T = x.shape[0]
        b = self.bufs(T)
        fresh = record is not None
        xn = x
        for l, ly in enumerate(self.layers):
            _, _, gate = moe_route_topk(xn, ly.router, self.k, False, ly.shared_gate,
                                        topk_ids=b.ids, topk_w=b.w,
                                        shared_gate=b.gate if ly.shared_gate is not None else None)
            moe_gather(b.ids, self.E, self.err, out=b.maps)
            if kind == "int4":
                sh = self._shared(l, xn)
                w4a16_grouped_ffn(xn, b.maps, self.t4[l], T, self.k, self.H, self.I, self.E,
                                  b.ws_w4, y_sorted=b.y, err_word=self.err)
            else:
                sh = self._verify_f16(l, xn, b, self._resident_table(full, l))
            out, xn_next = self._combine(l, b, b.y, sh, gate, x, fresh)
            self._record(record, l, x, xn, b.ids, out, xn_next)
            x, xn = out, xn_next
        return x

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
                  timing: Optional[dict] = None, record: Optional[dict] = None) -> torch.Tensor:
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
        `timing` (dict) receives HIP events: start, drafted, end.
        `record` (dict) receives the draft steps' per-layer records under
        "draft" (the steps then run eagerly, which is bit-identical to the
        graph replays), every ELB snapshot the round acted on under
        "snapshots" as (draft steps done, [L, E] counts), and the verify's
        per-layer records under "verify"."""
        main = torch.cuda.current_stream()
        ev = {k: torch.cuda.Event(enable_timing=True) for k in ("start", "drafted", "end")}
        self.clear_counters()
        ev["start"].record(main)
        steps = len(xs)
        draft = self.draft_step_graph
        snaps = None
        if record is not None:
            rec_d = record.setdefault("draft", [])
            snaps = record.setdefault("snapshots", [])
            draft = lambda x: self.draft_step(x, rec_d)
        if not planner:
            for x in xs:
                draft(x)
            ev["drafted"].record(main)
            counts = self.snapshot()
            if snaps is not None:
                snaps.append((steps, counts))
            self.place_residents(counts)
        else:
            # pools may be rewritten only once the previous round's verify read them
            self.copy.wait_event(self.ev_round_done)
            done, c, pending, k = 0, max(1, chunk0), None, 0
            pending_done = 0

            def read(i, n_done):
                counts = self._snapshot_read(i)
                if snaps is not None:
                    snaps.append((n_done, counts))
                return counts

            while done < steps:
                n = min(c, steps - done)
                for st in range(done, done + n):
                    draft(xs[st])
                done += n
                self._snapshot_async(k % 2)
                if pending is not None:
                    nload = self.prefetch(read(pending, pending_done))
                    t_copy = nload * self.ebytes / (h2d_gbps * 1e9)
                    c = max(1, int(round(t_copy / step_s)))
                pending, pending_done = k % 2, done
                k += 1
            ev["drafted"].record(main)
            self.prefetch(read(pending, pending_done))
        out = self.verify(xv, None if record is None else record.setdefault("verify", []))
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
        b = self.bufs(T)
        fresh = record is not None
        xn = x
        # routing and maps in one plan (no ELB update: verification does not
        # count draft choices) while it fits one workgroup's limits
        plan = T * self.k <= 1024 and T * (self.E + 1) <= 4096
        for l, ly in enumerate(self.layers):
            g_out = b.gate if ly.shared_gate is not None else None
            if plan:
                _, _, gate, _ = moe_route_plan(xn, ly.router, self.k, False, ly.shared_gate,
                                               err_word=self.err, topk_ids=b.ids, topk_w=b.w,
                                               shared_gate=g_out, maps=b.maps, logits_ws=b.lg)
            else:
                _, _, gate = moe_route_topk(xn, ly.router, self.k, False, ly.shared_gate,
                                            topk_ids=b.ids, topk_w=b.w, shared_gate=g_out)
                moe_gather(b.ids, self.E, self.err, out=b.maps)
            maps = b.maps
            # the shared expert's items ride in the routed experts' launches
            # (verify_grouped_gemm_shared): as launches of their own after
            # them, or on a side stream beside them, the layer was slower
            if all_resident is not None:
                sh = self._verify_f16(l, xn, b, self._resident_table(all_resident, l))
            else:
                sh = self._verify_staged(l, xn, maps, b, main)
            out, xn_next = self._combine(l, b, b.y, sh, gate, x, fresh)
            self._record(record, l, x, xn, b.ids, out, xn_next)
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

    def _verify_f16(self, l, x, b, table, mask=None):
        """The FP16 routed experts of layer l from `table` (optionally only
        those with mask 1) and its shared expert in the same launches; returns
        the shared output (None without one)."""
        T = x.shape[0]
        kw = dict(active=b.maps["active"], n_active=b.maps["n_active"], expert_mask=mask,
                  y_sorted=b.y, err_word=self.err)
        sh = self.layers[l].shared
        if sh is None:
            verify_grouped_gemm(x, b.maps["sorted_token"], b.maps["offsets"], table, T,
                                T * self.k, self.H, self.I, self.E, b.ws_f16, **kw)
            return None
        verify_grouped_gemm_shared(x, b.maps["sorted_token"], b.maps["offsets"], table, T,
                                   T * self.k, self.H, self.I, self.E, b.ws_f16, sh,
                                   shared_h=b.sh_h, shared_out=b.sh_out, **kw)
        return b.sh_out

    def _verify_staged(self, l, x, maps, bufs, main):
        T = x.shape[0]
        rows = T * self.k
        y, ws = bufs.y, bufs.ws_f16
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
        # the shared expert rides in the first of the two launches
        sh = None
        if hits:
            main.wait_event(self.ev_layer[l])  # this layer's prefetches (if any) have landed
            sh = self._verify_f16(l, x, bufs, self.d_table[l], self.d_mask[l, 0])
        if misses:
            main.wait_event(self.ev_staged[b])
            if hits:
                verify_grouped_gemm(x, maps["sorted_token"], maps["offsets"], self.d_table[l], T,
                                    rows, self.H, self.I, self.E, ws, active=maps["active"],
                                    n_active=maps["n_active"], expert_mask=self.d_mask[l, 1],
                                    y_sorted=y, err_word=self.err)
            else:
                sh = self._verify_f16(l, x, bufs, self.d_table[l], self.d_mask[l, 1])
            self.ev_free[b].record(main)
        self.stats["hit_experts"] += len(hits)
        self.stats["miss_experts"] += len(misses)
        self.stats["staged_experts"] += len(misses)
        self.stats["staged_bytes"] += len(misses) * self.ebytes
        return sh
