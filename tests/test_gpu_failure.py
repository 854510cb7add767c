"""Failure handling of the staging path on the GPU, forced from the host so
that every kernel still exits normally.

* A pageable (not page-locked) host source is refused by
  expert_stage_async with SMOE_ERR_NOT_PINNED and nothing is copied.
* A late stage: a bounded spin kernel queued on the side stream ahead of the
  staging copies delays them well past the hit GEMMs; the verify's miss
  GEMMs wait on the copy events, so the output still equals the all-resident
  run bit for bit, and the main stream's verify takes at least the delay.
"""
import time

import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import synth
from fp16_verify_expert_amd.chunk import ChunkEngine
from gpu_util import host, qwen_chunk_layers, say

pytestmark = pytest.mark.gpu


def test_stage_from_pageable_memory_is_refused():
    dst = torch.full((4096,), 7, dtype=torch.float16, device="cuda")
    src = torch.ones(4096, dtype=torch.float16)              # pageable
    assert not src.is_pinned()
    with pytest.raises(fve.SmoeError) as ei:
        fve.expert_stage_async(dst, src, torch.cuda.current_stream())
    assert ei.value.status == 5 and "page-locked" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(dst == 7)                               # nothing was copied
    # the same copy from page-locked memory goes through
    pinned = torch.ones(4096, dtype=torch.float16).pin_memory()
    ev = torch.cuda.Event()
    side = torch.cuda.Stream()
    fve.expert_stage_async(dst, pinned, side, ev)
    torch.cuda.current_stream().wait_event(ev)
    torch.cuda.synchronize()
    assert torch.all(dst == 1)


def test_late_stage_still_matches_all_resident():
    s = synth.QWEN_CHUNK
    dev = torch.device("cuda")
    L = 3
    layers, full = qwen_chunk_layers(L, dev)
    eng = ChunkEngine(layers, s.H, s.E, s.k, s.I, s.shared_I, 16, 17, device=dev)
    xs = [torch.from_numpy(synth.tokens(s, 1, step=st)).to(dev) for st in range(16)]
    for x in xs:
        eng.draft_step(x)
    eng.place_residents(eng.snapshot())
    xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=16)).to(dev)])
    ref = eng.verify(xv, all_resident=full).clone()
    torch.cuda.synchronize()
    # measure the spin kernel's duration, then queue it ahead of the copies
    spin = 200_000_000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(spin)
    b.record()
    torch.cuda.synchronize()
    delay_ms = a.elapsed_time(b)
    say(f"late stage: side stream held for {delay_ms:.1f} ms")
    assert delay_ms > 5.0
    before = eng.stats["staged_experts"]
    with torch.cuda.stream(eng.side):
        torch.cuda._sleep(spin)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    out = eng.verify(xv)
    t1.record()
    torch.cuda.synchronize()
    assert eng.stats["staged_experts"] > before            # misses were staged
    assert torch.equal(out, ref)
    assert t0.elapsed_time(t1) >= 0.9 * delay_ms
    assert int(host(eng.err)[0]) == 0
