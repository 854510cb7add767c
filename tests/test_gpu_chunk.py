"""GPU parity of the multi-layer draft chunk + verify with offloaded experts
(Qwen-shaped layers: H 2048, 60 experts, top-4, I 1408, shared expert 5632
with a sigmoid gate; 16 resident experts per layer, the rest staged from
pinned host memory).

Layers are pre-norm residual blocks x <- x + MoE(rms(x)).  Parity is
teacher-forced per layer: the oracle recomputes layer l from the GPU's own
layer-l input (normalised input and residual), and the fused normalisation
of each layer's output against the oracle's rms_norm.  The ELB table must equal the oracle's counts of the
same inputs exactly; the verify output must be bit-identical to a run with
every expert resident (staging changes where weights come from, never what is
computed)."""
import numpy as np
import pytest
import torch

import fp16_verify_expert_amd as fve
import oracle
import synth
from fp16_verify_expert_amd.chunk import ChunkEngine, ChunkLayer, top_resident
from gpu_util import assert_fp16_close, host, say

pytestmark = pytest.mark.gpu

LAYERS = 3
STEPS = 16
RESIDENT = 16
TV = 17


@pytest.fixture(scope="module")
def chunk():
    fve.lib()
    s = synth.QWEN_CHUNK
    dev = torch.device("cuda")
    layers, gen = [], []
    for l in range(LAYERS):
        g = synth.torch_layer(s, l, dev)
        host_f16 = torch.empty((s.E, 3 * s.H * s.I), dtype=torch.float16, pin_memory=True)
        for e, (w13, w2) in enumerate(g["f16"]):
            host_f16[e, :2 * s.I * s.H].copy_(w13.reshape(-1))
            host_f16[e, 2 * s.I * s.H:].copy_(w2.reshape(-1))
        layers.append(ChunkLayer(router=g["router"], int4=g["int4"], host_f16=host_f16,
                                 shared=(g["shared"]["w13"], g["shared"]["w2"]),
                                 shared_gate=g["shared"]["gate"]))
        gen.append(g)
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
    return dict(shape=s, eng=eng, gen=gen, counts=counts, rec_d=rec_d, rec_v=rec_v, xv=xv,
                out=out)


def _np_layer(g, experts, kind):
    """numpy copies of the given experts (others None) for the oracle."""
    E = len(g["f16"])
    out = [None] * E
    for e in experts:
        if kind == "int4":
            out[e] = {key: tuple(host(t) for t in g["int4"][e][key]) for key in ("w13", "w2")}
        else:
            out[e] = tuple(host(t) for t in g["f16"][e])
    return out


def _shared_np(g):
    sh = g["shared"]
    return dict(w13=host(sh["w13"]), w2=host(sh["w2"]), gate=host(sh["gate"]))


def test_chunk_error_word_clear(chunk):
    assert int(host(chunk["eng"].err)[0]) == 0
    for r in chunk["rec_d"] + chunk["rec_v"]:
        assert torch.isfinite(r["out"]).all()


def test_chunk_elb_counters_exact(chunk):
    s = chunk["shape"]
    ref = np.zeros((LAYERS, s.E), np.int32)
    for r in chunk["rec_d"]:
        g = chunk["gen"][r["layer"]]
        x = host(r["xn"])
        ro = oracle.route_topk(x, host(g["router"]), s.k, False, host(g["shared"]["gate"]))
        assert np.array_equal(host(r["ids"]), ro["ids"])
        ref = oracle.elb_update(ref, ro["ids"], r["layer"])
    assert np.array_equal(chunk["counts"], ref)
    assert np.all(ref.sum(axis=1) == STEPS * s.k)


@pytest.mark.parametrize("step", [0, 7, 15])
def test_chunk_draft_layers_teacher_forced(chunk, step):
    s = chunk["shape"]
    for l in range(LAYERS):
        r = chunk["rec_d"][step * LAYERS + l]
        g = chunk["gen"][l]
        xn = host(r["xn"])
        ids = host(r["ids"])
        experts = _np_layer(g, sorted(set(ids.ravel().tolist())), "int4")
        ref = oracle.moe_layer(xn, host(g["router"]), s.k, experts, "int4", _shared_np(g),
                               residual=host(r["x"]))
        assert np.array_equal(ids, ref["route"]["ids"])
        assert_fp16_close(host(r["out"]), ref["out"], f"draft step {step} layer {l}")
        assert_fp16_close(host(r["xn_next"]), oracle.rms_norm(host(r["out"])),
                          f"draft step {step} layer {l} norm")


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
        g = chunk["gen"][l]
        xn = host(r["xn"])
        ids = host(r["ids"])
        experts = _np_layer(g, sorted(set(ids.ravel().tolist())), "f16")
        ref = oracle.moe_layer(xn, host(g["router"]), s.k, experts, "f16", _shared_np(g),
                               residual=host(r["x"]))
        assert np.array_equal(ids, ref["route"]["ids"])
        st = assert_fp16_close(host(r["out"]), ref["out"], f"verify layer {l}")
        assert_fp16_close(host(r["xn_next"]), oracle.rms_norm(host(r["out"])),
                          f"verify layer {l} norm")
        say(f"verify layer {l}: l2={st['l2']:.2e}")
    assert chunk["eng"].stats["staged_experts"] > 0


def test_chunk_verify_residency_invariant(chunk):
    s = chunk["shape"]
    eng = chunk["eng"]
    full = torch.empty((LAYERS, s.E, 3 * s.H * s.I), dtype=torch.float16, device="cuda")
    for l in range(LAYERS):
        full[l].copy_(eng.layers[l].host_f16)
    rec = []
    out = eng.verify(chunk["xv"], rec, all_resident=full)
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


def test_chunk_forward_matches_draft_and_verify(chunk):
    """The any-T forward used by the route-fidelity probe runs the very same
    kernels: FP16 over 17 rows equals the all-resident verify bit for bit, and
    INT4 over one row equals the draft step."""
    s = chunk["shape"]
    eng = chunk["eng"]
    full = torch.empty((LAYERS, s.E, 3 * s.H * s.I), dtype=torch.float16, device="cuda")
    for l in range(LAYERS):
        full[l].copy_(eng.layers[l].host_f16)
    ref = eng.verify(chunk["xv"], all_resident=full).clone()
    rec = []
    out = eng.forward(chunk["xv"], "f16", full, rec)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert len(rec) == LAYERS and all(r.shape == (17, s.k) for r in rec)
    saved = eng.counters.clone()
    x1 = chunk["xv"][:1].contiguous()
    d = eng.draft_step(x1).clone()
    f = eng.forward(x1, "int4")
    torch.cuda.synchronize()
    assert torch.equal(f, d)
    eng.counters.copy_(saved)
    assert int(host(eng.err)[0]) == 0


def test_chunk_planner_rounds_residency_invariant(chunk):
    """Speculation rounds with the prefetch planner (chunked drafting, ELB
    snapshots driving prefetches on the copy stream, per-layer events, misses
    staged at verify) and with boundary placement: every round's output is
    bit-identical to the all-resident verify of the same rows."""
    s = chunk["shape"]
    eng = chunk["eng"]
    full = torch.empty((LAYERS, s.E, 3 * s.H * s.I), dtype=torch.float16, device="cuda")
    for l in range(LAYERS):
        full[l].copy_(eng.layers[l].host_f16)
    if not hasattr(eng, "graph"):
        eng.capture_draft()
    before = eng.stats.get("prefetched_experts", 0)
    for r, planner in enumerate((True, True, False, True)):
        xs = [torch.from_numpy(synth.tokens(s, 1, step=300 + 20 * r + st)).cuda()
              for st in range(STEPS)]
        xv = torch.cat(xs + [torch.from_numpy(synth.tokens(s, 1, step=300 + 20 * r + STEPS)).cuda()])
        say(f"round {r} planner={planner}")
        out = eng.run_round(xs, xv, planner=planner).clone()
        ref = eng.verify(xv, all_resident=full)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        for l in range(LAYERS):
            held = [e for e in eng.resident[l] if e >= 0]
            assert len(set(held)) == len(held)
    assert eng.stats["prefetched_experts"] > before
    assert int(host(eng.err)[0]) == 0
