"""GPU parity of the 24-layer draft chunk + verify with offloaded experts, at
the configuration's stated size: 24 Qwen-shaped layers (H 2048, 60 experts,
top-4, I 1408, shared expert 5632 with a sigmoid gate), 16 INT4 draft steps
with an ELB table [24, 60], 16 of 60 FP16 experts resident per layer, the
rest staged from pinned host memory, then a 17-token FP16 verify.

Layers are pre-norm residual blocks x <- x + MoE(rms(x)).  Parity is
teacher-forced per layer: the oracle recomputes layer l from the GPU's own
layer-l input (normalised input and residual).  Routing ids and the ELB table
must equal the oracle's exactly over all 384 layer-steps; FP16 outputs meet
the normalised-L2 / max-abs bars on sampled layers; the verify output must be
bit-identical to a run with every expert resident.  The prefetch planner's
snapshots and the route-fidelity probe's routing are held to the oracle too.
"""
import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth
from fp16_verify_expert_amd.chunk import (ChunkEngine, distinct_experts, top_resident,
                                          topk_agreement)
from gpu_util import (assert_fp16_close, chunk_layer_np, chunk_shared_np, host,
                      qwen_chunk_layers, say)

pytestmark = pytest.mark.gpu

LAYERS = 24
STEPS = 16
RESIDENT = 16
TV = 17
SAMPLED = (0, 11, 23)           # layers held to the full oracle layer


@pytest.fixture(scope="module")
def chunk():
    fve.lib()
    s = synth.QWEN_CHUNK
    dev = torch.device("cuda")
    say(f"chunk: generating {LAYERS} layers")
    layers, full = qwen_chunk_layers(LAYERS, dev)
    eng = ChunkEngine(layers, s.H, s.E, s.k, s.I, s.shared_I, RESIDENT, TV, device=dev)
    xs = [torch.from_numpy(synth.tokens(s, 1, step=st)).to(dev) for st in range(STEPS)]
    rec_d = []
    eng.clear_counters()
    for st in range(STEPS):
        eng.draft_step(xs[st], rec_d)
    torch.cuda.synchronize()
    counts = eng.snapshot()
    eng.place_residents(counts)
    xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=STEPS)).to(dev)])
    rec_v = []
    out = eng.verify(xv, rec_v)
    torch.cuda.synchronize()
    say(f"chunk: staged {eng.stats['staged_experts']} experts, hits {eng.stats['hit_experts']}")
    yield dict(shape=s, eng=eng, layers=layers, full=full, counts=counts, rec_d=rec_d,
               rec_v=rec_v, xv=xv, out=out)
    del eng, layers, full
    torch.cuda.empty_cache()


def _oracle_ids(s, layer, xn):
    return oracle.route_topk(host(xn), host(layer.router), s.k, False,
                             host(layer.shared_gate))["ids"]


def _check_layer(s, layer, r, kind, what):
    """Teacher-forced oracle layer on the GPU's own inputs of record r."""
    xn = host(r["xn"])
    ids = host(r["ids"])
    experts = chunk_layer_np(layer, sorted(set(ids.ravel().tolist())), kind, s.H, s.I)
    ref = oracle.moe_layer(xn, host(layer.router), s.k, experts, kind, chunk_shared_np(layer),
                           residual=host(r["x"]))
    assert np.array_equal(ids, ref["route"]["ids"]), what
    st = assert_fp16_close(host(r["out"]), ref["out"], what)
    assert_fp16_close(host(r["xn_next"]), oracle.rms_norm(host(r["out"])), what + " norm")
    return st


def _oracle_counts(s, layers, rec, steps):
    """ELB tables from the oracle's routing of the recorded draft inputs
    (records are step-major, layer-minor): {n: table after the first n
    steps} for every n in `steps`; every recorded id must equal the
    oracle's."""
    ref = np.zeros((LAYERS, s.E), np.int32)
    out = {0: ref.copy()} if 0 in steps else {}
    for i, r in enumerate(rec[:max(steps) * LAYERS]):
        l = r["layer"]
        ids = _oracle_ids(s, layers[l], r["xn"])
        assert np.array_equal(host(r["ids"]), ids), f"step {i // LAYERS} layer {l} ids"
        ref = oracle.elb_update(ref, ids, l)
        if (i + 1) % LAYERS == 0 and (i + 1) // LAYERS in steps:
            out[(i + 1) // LAYERS] = ref.copy()
    return out


def test_chunk_error_word_clear(chunk):
    assert int(host(chunk["eng"].err)[0]) == 0
    assert len(chunk["rec_d"]) == STEPS * LAYERS and len(chunk["rec_v"]) == LAYERS
    for r in chunk["rec_d"] + chunk["rec_v"]:
        assert torch.isfinite(r["out"]).all()


def test_chunk_elb_counters_exact(chunk):
    """All 384 layer-steps: ids exact, and the [24, 60] table equal to the
    oracle's counts; every layer's row sums to 16 steps x top-4."""
    s = chunk["shape"]
    ref = _oracle_counts(s, chunk["layers"], chunk["rec_d"], [STEPS])[STEPS]
    assert chunk["counts"].shape == (LAYERS, s.E)
    assert np.array_equal(chunk["counts"], ref)
    assert np.all(ref.sum(axis=1) == STEPS * s.k)


@pytest.mark.parametrize("step", [0, 7, 15])
def test_chunk_draft_layers_teacher_forced(chunk, step):
    s = chunk["shape"]
    for l in SAMPLED:
        r = chunk["rec_d"][step * LAYERS + l]
        assert r["layer"] == l
        st = _check_layer(s, chunk["layers"][l], r, "int4", f"draft step {step} layer {l}")
        say(f"draft step {step} layer {l}: l2={st['l2']:.2e}")


def test_chunk_residency_from_snapshot(chunk):
    eng = chunk["eng"]
    for l in range(LAYERS):
        c = chunk["counts"][l]
        res = eng.resident[l]
        assert res == top_resident(c, RESIDENT) and len(res) == RESIDENT
        # no non-resident expert has a larger count than a resident one
        assert min(c[res]) >= max(np.delete(c, res))


def test_chunk_verify_teacher_forced(chunk):
    s = chunk["shape"]
    for r in chunk["rec_v"]:
        l = r["layer"]
        assert np.array_equal(host(r["ids"]), _oracle_ids(s, chunk["layers"][l], r["xn"]))
    for l in SAMPLED:
        st = _check_layer(s, chunk["layers"][l], chunk["rec_v"][l], "f16", f"verify layer {l}")
        say(f"verify layer {l}: l2={st['l2']:.2e}")
    assert chunk["eng"].stats["staged_experts"] > 0


def test_chunk_verify_residency_invariant(chunk):
    eng = chunk["eng"]
    rec = []
    out = eng.verify(chunk["xv"], rec, all_resident=chunk["full"])
    torch.cuda.synchronize()
    assert torch.equal(out, chunk["out"])
    for a, b in zip(rec, chunk["rec_v"]):
        assert torch.equal(a["out"], b["out"])
    # and a second staged run reproduces the first bit for bit
    out2 = eng.verify(chunk["xv"])
    torch.cuda.synchronize()
    assert torch.equal(out2, chunk["out"])


def test_chunk_draft_graph_matches_eager(chunk):
    """The draft step captured as one HIP graph reproduces the eager step bit
    for bit on every replay (replays interleaved with eager work and
    synchronisations), and counts the same ELB choices."""
    s = chunk["shape"]
    eng = chunk["eng"]
    saved = eng.counters.clone()
    xs = [torch.from_numpy(synth.tokens(s, 1, step=50 + j)).cuda() for j in range(3)]
    eng.clear_counters()
    ref = [eng.draft_step(x).clone() for x in xs]
    c_ref = eng.counters.clone()
    eng.capture_draft()
    eng.clear_counters()
    for rep in range(3):
        for j, x in enumerate(xs):
            out = eng.draft_step_graph(x)
            torch.cuda.synchronize()
            assert torch.equal(out, ref[j]), (rep, j)
            eng.snapshot()                       # eager work + a sync between replays
    assert torch.equal(eng.counters, 3 * c_ref)
    assert int(host(eng.err)[0]) == 0
    eng.counters.copy_(saved)


def test_chunk_draft_fused_combine_matches_four_launch_chain(chunk):
    """The draft step with each layer's combine fused with the next layer's
    router logits (three launches per layer) equals the four-launch chain bit
    for bit: every layer's input, ids, output and normalised output, and the
    ELB counts."""
    s = chunk["shape"]
    eng = chunk["eng"]
    saved = eng.counters.clone()
    for j in range(2):
        x = torch.from_numpy(synth.tokens(s, 1, step=80 + j)).cuda()
        eng.clear_counters()
        ra = []
        oa = eng.draft_step(x, ra, fuse_combine=False).clone()
        ca = eng.counters.clone()
        eng.clear_counters()
        rb = []
        ob = eng.draft_step(x, rb, fuse_combine=True).clone()
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(ca, eng.counters)
        for a, b in zip(ra, rb):
            for key in ("x", "xn", "ids", "out", "xn_next"):
                assert torch.equal(a[key], b[key]), (j, a["layer"], key)
    assert int(host(eng.err)[0]) == 0
    eng.counters.copy_(saved)


def test_chunk_forward_matches_draft_and_verify(chunk):
    """The any-T forward used by the route-fidelity probe runs the very same
    kernels: FP16 over 17 rows equals the all-resident verify bit for bit, and
    INT4 over one row equals the draft step."""
    s = chunk["shape"]
    eng = chunk["eng"]
    ref = eng.verify(chunk["xv"], all_resident=chunk["full"]).clone()
    rec = []
    out = eng.forward(chunk["xv"], "f16", chunk["full"], rec)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert len(rec) == LAYERS and all(r["ids"].shape == (17, s.k) for r in rec)
    saved = eng.counters.clone()
    x1 = chunk["xv"][:1].contiguous()
    d = eng.draft_step(x1).clone()
    f = eng.forward(x1, "int4")
    torch.cuda.synchronize()
    assert torch.equal(f, d)
    eng.counters.copy_(saved)
    assert int(host(eng.err)[0]) == 0


def test_chunk_route_fidelity_probe_against_oracle(chunk):
    """The route-fidelity probe on a short correlated token stream: every
    layer's draft and target ids equal the oracle's routing of the recorded
    layer inputs, and the agreement and distinct-expert figures computed from
    the GPU ids equal those recomputed here, by plain loops, from the
    oracle's ids."""
    s = chunk["shape"]
    eng = chunk["eng"]
    N = 32
    x = torch.from_numpy(synth.token_stream(s, N, 0.8, step=7)).cuda()
    rd, rt = [], []
    eng.forward(x, "int4", record=rd)
    eng.forward(x, "f16", chunk["full"], record=rt)
    torch.cuda.synchronize()
    assert int(host(eng.err)[0]) == 0
    o_d = np.stack([_oracle_ids(s, chunk["layers"][r["layer"]], r["xn"]) for r in rd])
    o_t = np.stack([_oracle_ids(s, chunk["layers"][r["layer"]], r["xn"]) for r in rt])
    g_d = np.stack([host(r["ids"]) for r in rd])
    g_t = np.stack([host(r["ids"]) for r in rt])
    assert np.array_equal(g_d, o_d) and np.array_equal(g_t, o_t)
    # the probe's statistics from the GPU ids ...
    agree = topk_agreement(g_d, g_t)
    depths = [1, 2, 4, 8, 16, 32]
    dist = distinct_experts(g_t, depths)
    # ... against plain recomputations from the oracle's ids
    for l in range(LAYERS):
        for t in range(N):
            same = sum(1 for e in o_d[l, t] if e in set(o_t[l, t].tolist()))
            assert agree[l, t] == same / s.k
    for K in depths:
        total, n = 0, 0
        for l in range(LAYERS):
            for w in range(N // K):
                total += len(set(o_t[l, w * K:(w + 1) * K].ravel().tolist()))
                n += 1
        assert abs(dist[K] - total / n) <= 1e-12 * dist[K]
    assert dist[1] == s.k and dist[32] > dist[1]
    say(f"route fidelity: agreement {agree.mean():.3f}, distinct K=1/16/32 "
        f"{dist[1]:.1f}/{dist[16]:.1f}/{dist[32]:.1f}")


def test_chunk_planner_rounds_residency_invariant(chunk):
    """Speculation rounds with the prefetch planner (chunked drafting, ELB
    snapshots driving prefetches on the copy stream, per-layer events, misses
    staged at verify) and with boundary placement: every round's output is
    bit-identical to the all-resident verify of the same rows."""
    s = chunk["shape"]
    eng = chunk["eng"]
    if not hasattr(eng, "graph"):
        eng.capture_draft()
    before = eng.stats.get("prefetched_experts", 0)
    for r, planner in enumerate((True, True, False, True)):
        xs = [torch.from_numpy(synth.tokens(s, 1, step=300 + 20 * r + st)).cuda()
              for st in range(STEPS)]
        xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=300 + 20 * r + STEPS)).cuda()])
        say(f"round {r} planner={planner}")
        out = eng.run_round(xs, xv, planner=planner).clone()
        ref = eng.verify(xv, all_resident=chunk["full"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        for l in range(LAYERS):
            held = [e for e in eng.resident[l] if e >= 0]
            assert len(set(held)) == len(held)
    assert eng.stats["prefetched_experts"] > before
    assert int(host(eng.err)[0]) == 0


def test_chunk_planner_round_against_oracle(chunk):
    """One planner round (residency carried over from earlier rounds) held to
    the oracle: every ELB snapshot the planner acted on equals the oracle's
    counts over the draft steps done by then, sampled verify layers match the
    teacher-forced oracle layer, and the output is bit-identical to the
    all-resident verify."""
    s = chunk["shape"]
    eng = chunk["eng"]
    xs = [torch.from_numpy(synth.tokens(s, 1, step=700 + st)).cuda() for st in range(STEPS)]
    xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=700 + STEPS)).cuda()])
    rec = {}
    out = eng.run_round(xs, xv, planner=True, record=rec).clone()
    ref = eng.verify(xv, all_resident=chunk["full"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert int(host(eng.err)[0]) == 0
    snaps = rec["snapshots"]
    assert len(snaps) >= 2 and snaps[-1][0] == STEPS
    assert [n for n, _ in snaps] == sorted(n for n, _ in snaps)
    ref = _oracle_counts(s, chunk["layers"], rec["draft"], [n for n, _ in snaps])
    for n_done, counts in snaps:
        assert np.array_equal(counts, ref[n_done]), n_done
    say(f"planner round: snapshots after {[n for n, _ in snaps]} draft steps")
    for l in SAMPLED:
        _check_layer(s, chunk["layers"][l], rec["verify"][l], "f16", f"planner verify layer {l}")
