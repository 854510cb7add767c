"""The C ABI library loads, exports every entry point declared in
include/smoe.h, and rejects bad arguments on the host (no GPU needed: these
calls return before anything touches a device)."""
import ctypes
import os

import pytest

import fp16_verify_expert_amd as fve

pytestmark = pytest.mark.skipif(not os.path.exists(fve.LIB_PATH),
                                reason="libsmoe.so not built")

V = ctypes.c_void_p
FAKE = V(0x1000)  # never dereferenced: the checks below fail before any use


def test_exports_every_header_function():
    names = fve.header_functions()
    expected = {"smoe_abi_version", "smoe_last_error", "moe_route_topk", "elb_count",
                "moe_gather", "moe_route_plan", "w4a16_grouped_ffn", "wq_grouped_ffn",
                "moe_draft_route_ffn", "w4a16_grouped_ffn_noalloc", "moe_combine_route_logits",
                "awq_grouped_ffn", "moe_draft_layer", "smoe_draft_layer_supported",
                "verify_grouped_gemm_shared", "w4a16_grouped_ffn_shared",
                "verify_grouped_gemm", "moe_combine",
                "expert_stage_async", "smoe_workspace_bytes", "smoe_stream_read"}
    assert set(names) == expected
    L = ctypes.CDLL(fve.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert fve.lib().smoe_abi_version() == fve.ABI_VERSION


def _header_param_counts():
    """Parameter count of every function declared in include/smoe.h."""
    import re
    txt = open(fve.HEADER_PATH).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:smoe_status|int|const char\*|size_t)\s+(\w+)\s*\(([^)]*)\)\s*;",
                         txt, re.M | re.S):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else len(params.split(","))
    return out


def test_binding_signatures_match_header():
    """The binding's ctypes argument lists have the header's parameter counts
    (a drifted declaration would pass arguments in the wrong slots)."""
    counts = _header_param_counts()
    assert set(counts) == set(fve.header_functions())
    for name, (_, args) in fve._SIGS.items():
        assert name in counts, name
        assert len(args) == counts[name], (name, len(args), counts[name])


def _err():
    return fve.lib().smoe_last_error().decode()


def test_route_validation():
    L = fve.lib()
    assert L.moe_route_topk(None, FAKE, None, 1, 256, 8, 2, 0, FAKE, FAKE, None, None) == 1
    assert "required" in _err()
    assert L.moe_route_topk(FAKE, FAKE, None, 1, 200, 8, 2, 0, FAKE, FAKE, None, None) == 2
    assert "H=200" in _err()
    assert L.moe_route_topk(FAKE, FAKE, None, 1, 256, 8, 9, 0, FAKE, FAKE, None, None) == 2
    assert L.moe_route_topk(FAKE, FAKE, None, 1, 256, 300, 2, 0, FAKE, FAKE, None, None) == 2
    assert L.moe_route_topk(FAKE, FAKE, FAKE, 1, 256, 8, 2, 0, FAKE, FAKE, None, None) == 1
    assert L.moe_route_topk(V(0x1002), FAKE, None, 1, 256, 8, 2, 0, FAKE, FAKE, None, None) == 2
    assert "aligned" in _err()
    # T == 0 is a no-op and succeeds without a device
    assert L.moe_route_topk(FAKE, FAKE, None, 0, 256, 8, 2, 0, FAKE, FAKE, None, None) == 0
    assert _err() == ""


def test_elb_validation():
    L = fve.lib()
    assert L.elb_count(None, 1, 2, 8, 0, 1, FAKE, None, None) == 1
    assert L.elb_count(FAKE, 1, 2, 8, 1, 1, FAKE, None, None) == 2      # layer >= L
    assert L.elb_count(FAKE, 1, 9, 8, 0, 1, FAKE, None, None) == 2      # k > E
    assert L.elb_count(FAKE, 0, 2, 8, 0, 1, FAKE, None, None) == 0


def test_gather_validation():
    L = fve.lib()
    assert L.moe_gather(FAKE, 1, 2, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert L.moe_gather(FAKE, 1 << 20, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert L.moe_gather(FAKE, 1, 3, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 2


def test_route_plan_validation():
    L = fve.lib()
    outs = [FAKE] * 3   # ids, w, gate
    maps = [FAKE] * 6   # offsets, sorted_token, sorted_pair, pair_pos, active, n_active

    def call(x=FAKE, wr=FAKE, wsg=None, T=1, H=256, E=8, k=2, layer=0, Lc=1, counters=FAKE,
             gate=None, mp=None, ws=None, wsb=0):
        m = maps if mp is None else mp
        return L.moe_route_plan(x, wr, wsg, T, H, E, k, 0, layer, Lc, counters, outs[0], outs[1],
                                gate, *m, ws, wsb, None, None)
    assert call(x=None) == 1
    assert call(wsg=FAKE) == 1                      # gate output missing
    assert call(mp=[None] + maps[1:]) == 1          # offsets missing
    assert call(H=200) == 2
    assert call(k=9) == 2
    assert call(T=513, k=2) == 2 and "1024" in _err()        # T*k > 1024
    assert call(T=100, E=64, k=2) == 2 and "4096" in _err()  # T*(E+1) > 4096
    assert call(layer=1, Lc=1) == 2                 # layer outside [0, L)
    assert call(x=V(0x1002)) == 2 and "aligned" in _err()
    assert call(T=-1) == 2
    # the logits workspace: T*E fp32 (T*(E+1) with a shared gate), 16-byte aligned
    assert call(T=4, E=8, ws=FAKE, wsb=4 * 4 * 8 - 1) == 6 and "128 needed" in _err()
    assert call(T=4, E=8, wsg=FAKE, gate=FAKE, ws=FAKE, wsb=4 * 4 * 8) == 6 and "144" in _err()
    assert call(T=4, E=8, ws=V(0x1004), wsb=1 << 10) == 6 and "aligned" in _err()


def test_wq_validation():
    L = fve.lib()
    args = [FAKE] * 6
    need = L.smoe_workspace_bytes(0, 4, 2, 256, 512, 8)

    def call(bits=8, gs=128, I=512, ws=FAKE, wsb=None, T=4):
        return L.wq_grouped_ffn(*args, T, 2, 256, I, 8, bits, gs, FAKE, ws,
                                need if wsb is None else wsb, None, None)
    assert call(bits=3) == 3 and "bits=3" in _err()
    assert call(bits=16) == 3
    assert call(gs=64) == 3
    assert call(I=500) == 2
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6
    assert L.wq_grouped_ffn(*args[:5], None, 4, 2, 256, 512, 8, 2, 128, FAKE, FAKE, need, None,
                            None) == 1
    # w4a16_grouped_ffn reports its own name
    assert L.w4a16_grouped_ffn(*args, 1, 2, 256, 500, 8, 128, FAKE, FAKE, 1 << 20, None,
                               None) == 2
    assert _err().startswith("w4a16_grouped_ffn")


def test_draft_route_ffn_validation():
    L = fve.lib()
    maps = [FAKE] * 6   # offsets, sorted_token, sorted_pair, pair_pos, active, n_active
    need = L.smoe_workspace_bytes(0, 1, 2, 256, 512, 8)
    assert need > 0

    def call(x=FAKE, wr=FAKE, wsg=None, H=256, I=512, E=8, k=2, layer=0, Lc=1, counters=FAKE,
             table=FAKE, gs=128, gate=None, mp=None, y=FAKE, ws=FAKE, wsb=None,
             sh=(None, None, 0, None, None), lg=None):
        m = maps if mp is None else mp
        return L.moe_draft_route_ffn(x, wr, wsg, H, I, E, k, 0, layer, Lc, counters, table, gs,
                                     FAKE, FAKE, gate, *m, y, *sh, lg, ws,
                                     need if wsb is None else wsb, None, None)
    assert call(x=None) == 1
    assert call(table=None) == 1
    assert call(y=None) == 1
    assert call(wsg=FAKE) == 1                      # gate output missing
    assert call(mp=maps[:4] + [None, FAKE]) == 1    # active missing
    assert call(H=200) == 2
    assert call(I=500) == 2
    assert call(k=9) == 2
    assert call(E=64, k=33) == 2 and "32" in _err()
    assert call(gs=64) == 3
    assert call(layer=1, Lc=1) == 2                 # layer outside [0, L)
    assert call(x=V(0x1002)) == 2 and "aligned" in _err()
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6
    # the optional dense shared expert
    assert call(sh=(FAKE, FAKE, 1024, FAKE, None)) == 1 and "shared_out" in _err()
    assert call(sh=(FAKE, None, 1024, FAKE, FAKE)) == 1
    assert call(sh=(FAKE, FAKE, 1000, FAKE, FAKE)) == 2 and "shared_I" in _err()
    assert call(sh=(FAKE, FAKE, 0, FAKE, FAKE)) == 2
    assert call(sh=(FAKE, FAKE, 8320, FAKE, FAKE)) == 2 and "8192" in _err()
    assert call(sh=(FAKE, FAKE, 1024, V(0x1002), FAKE)) == 2 and "aligned" in _err()
    assert call(sh=(None, FAKE, 1000, None, None), wsb=need - 1) == 6  # ignored without shared_w13
    # precomputed logits: checked like the other inputs (alignment), no device use here
    assert call(lg=V(0x1002)) == 2 and "aligned" in _err()
    assert call(lg=FAKE, ws=None) == 6


def test_draft_layer_validation():
    L = fve.lib()
    maps = [FAKE] * 6   # offsets, sorted_token, sorted_pair, pair_pos, active, n_active
    need = L.smoe_workspace_bytes(2, 1, 2, 256, 512, 8)
    assert need > 0

    def call(x=FAKE, wr=FAKE, wsg=None, lg=None, H=256, I=512, E=8, k=2, layer=0, Lc=1,
             counters=FAKE, table=FAKE, gs=128, gate=None, y=FAKE, sh=(None, None, 0, None, None),
             res=None, out=V(0x3000), nrm=None, eps=1e-6, nxt=(None, None, 0, None), ws=FAKE,
             wsb=None):
        return L.moe_draft_layer(x, wr, wsg, lg, H, I, E, k, 0, layer, Lc, counters, table, gs,
                                 FAKE, FAKE, gate, *maps, y, *sh, res, out, nrm, eps, *nxt, ws,
                                 need if wsb is None else wsb, None, None)
    assert call(x=None) == 1
    assert call(table=None) == 1
    assert call(y=None) == 1
    assert call(out=None) == 1 and "required" in _err()
    assert call(wsg=FAKE) == 1                      # gate output missing
    assert call(sh=(FAKE, FAKE, 1024, FAKE, None)) == 1 and "shared_out" in _err()
    assert call(nxt=(FAKE, None, 8, V(0x4000))) == 1 and "norm_out" in _err()
    assert call(nxt=(FAKE, None, 8, None), nrm=V(0x5000)) == 1
    assert call(H=200) == 2
    assert call(I=500) == 2
    assert call(k=9) == 2
    assert call(sh=(FAKE, FAKE, 1000, FAKE, FAKE)) == 2 and "shared_I" in _err()
    assert call(nxt=(FAKE, None, 0, V(0x4000)), nrm=V(0x5000)) == 2 and "next_E" in _err()
    assert call(gs=64) == 3
    assert call(layer=1, Lc=1) == 2                 # layer outside [0, L)
    assert call(nrm=V(0x3000)) == 2                 # norm_out aliases out
    assert call(eps=-1.0) == 2
    assert call(x=V(0x1002)) == 2 and "aligned" in _err()
    assert call(lg=V(0x1002)) == 2 and "aligned" in _err()
    assert call(res=V(0x1002)) == 2 and "aligned" in _err()
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6
    # no device here: the shape query answers no
    assert L.smoe_draft_layer_supported(4096, 6400, 16, 2, 0) == 0


def test_combine_route_logits_validation():
    L = fve.lib()

    def call(y=FAKE, pp=FAKE, w=FAKE, sh=None, sc=None, res=None, k=2, H=256, out=FAKE,
             nrm=V(0x2000), eps=1e-6, wr=FAKE, wsg=None, E=8, lg=FAKE):
        return L.moe_combine_route_logits(y, pp, w, sh, sc, res, k, H, out, nrm, eps, wr, wsg, E,
                                          lg, None)
    assert call(y=None) == 1
    assert call(nrm=None) == 1
    assert call(wr=None) == 1 and "w_router" in _err()
    assert call(lg=None) == 1
    assert call(k=0) == 2
    assert call(E=257) == 2
    assert call(H=200) == 2
    assert call(H=8320) == 2 and "8192" in _err()
    assert call(y=V(0x1002)) == 2 and "aligned" in _err()
    assert call(nrm=FAKE) == 2                      # norm_out aliases out
    assert call(eps=-1.0) == 2


def test_w4a16_validation():
    L = fve.lib()
    args = [FAKE] * 6
    assert L.w4a16_grouped_ffn(*args, 1, 2, 256, 512, 8, 64, FAKE, FAKE, 1 << 20, None, None) == 3
    assert "group_size" in _err()
    assert L.w4a16_grouped_ffn(*args, 1, 2, 256, 500, 8, 128, FAKE, FAKE, 1 << 20, None, None) == 2
    need = L.smoe_workspace_bytes(0, 4, 2, 256, 512, 8)
    assert need > 0
    assert L.w4a16_grouped_ffn(*args, 4, 2, 256, 512, 8, 128, FAKE, FAKE, need - 1, None,
                               None) == 6
    assert L.w4a16_grouped_ffn(*args, 4, 2, 256, 512, 8, 128, FAKE, None, need, None, None) == 6
    assert L.w4a16_grouped_ffn(*args[:5], None, 4, 2, 256, 512, 8, 128, FAKE, FAKE, need, None,
                               None) == 1
    assert L.w4a16_grouped_ffn(*args, 0, 2, 256, 512, 8, 128, FAKE, None, 0, None, None) == 0


def test_w4a16_noalloc_validation():
    """Host checks of the allocation-free variant; none reaches a device."""
    L = fve.lib()
    args = [FAKE] * 6
    # h alone needs T*k*I*2 bytes: 600 rows at I = 6400 exceed the 4 MiB scratch
    assert L.w4a16_grouped_ffn_noalloc(*args, 300, 2, 4096, 6400, 16, 128, FAKE, None,
                                       None) == 2
    msg = _err()
    assert msg.startswith("w4a16_grouped_ffn_noalloc") and "scratch" in msg
    assert fve.NOALLOC_SCRATCH_BYTES == 4 << 20
    # 256 rows at I = 6400 fit (the limit the header names); 330 rows do not
    assert L.smoe_workspace_bytes(0, 256, 1, 4096, 6400, 16) <= fve.NOALLOC_SCRATCH_BYTES
    assert L.smoe_workspace_bytes(0, 330, 1, 4096, 6400, 16) > fve.NOALLOC_SCRATCH_BYTES
    # the checks of w4a16_grouped_ffn, reported under this entry point's name
    assert L.w4a16_grouped_ffn_noalloc(*args, 1, 2, 256, 512, 8, 64, FAKE, None, None) == 3
    assert _err().startswith("w4a16_grouped_ffn_noalloc") and "group_size" in _err()
    assert L.w4a16_grouped_ffn_noalloc(*args, 1, 2, 256, 500, 8, 128, FAKE, None, None) == 2
    assert L.w4a16_grouped_ffn_noalloc(*args[:5], None, 4, 2, 256, 512, 8, 128, FAKE, None,
                                       None) == 1
    assert L.w4a16_grouped_ffn_noalloc(*args, 4, 2, 256, 512, 8, 128, None, None, None) == 1
    assert L.w4a16_grouped_ffn_noalloc(*args, -1, 2, 256, 512, 8, 128, FAKE, None, None) == 2
    assert L.w4a16_grouped_ffn_noalloc(*args, 0, 2, 256, 512, 8, 128, FAKE, None, None) == 0


def test_awq_validation():
    L = fve.lib()
    args = [FAKE] * 6
    need = L.smoe_workspace_bytes(0, 4, 2, 256, 512, 8)
    assert L.awq_grouped_ffn(*args, None, 4, 2, 256, 512, 8, 128, FAKE, FAKE, need, None,
                             None) == 1 and "act_scales" in _err()
    assert L.awq_grouped_ffn(*args, FAKE, 4, 2, 256, 512, 8, 64, FAKE, FAKE, need, None,
                             None) == 3
    assert _err().startswith("awq_grouped_ffn")
    assert L.awq_grouped_ffn(*args, FAKE, 4, 2, 256, 500, 8, 128, FAKE, FAKE, need, None,
                             None) == 2
    assert L.awq_grouped_ffn(*args, FAKE, 4, 2, 256, 512, 8, 128, FAKE, FAKE, need - 1, None,
                             None) == 6
    assert L.awq_grouped_ffn(*args, FAKE, 0, 2, 256, 512, 8, 128, FAKE, None, 0, None,
                             None) == 0


def test_stream_read_validation():
    L = fve.lib()
    assert L.smoe_stream_read(None, 16, FAKE, 1, None) == 1
    assert L.smoe_stream_read(FAKE, 16, None, 1, None) == 1
    assert L.smoe_stream_read(FAKE, 20, FAKE, 1, None) == 2
    assert L.smoe_stream_read(V(0x1008), 16, FAKE, 1, None) == 2
    assert L.smoe_stream_read(FAKE, 16, FAKE, 0, None) == 2
    assert L.smoe_stream_read(FAKE, 16, FAKE, 65536, None) == 2
    assert L.smoe_stream_read(FAKE, 0, FAKE, 4, None) == 0


def test_verify_validation():
    L = fve.lib()
    a = [FAKE, FAKE, FAKE]
    assert L.verify_grouped_gemm(*a, FAKE, None, FAKE, None, 9, 36, 2048, 1408, 60, FAKE, FAKE,
                                 1 << 30, None, None) == 1
    assert L.verify_grouped_gemm(*a, None, None, FAKE, None, 9, 36, 2048, 1400, 60, FAKE, FAKE,
                                 1 << 30, None, None) == 2
    need = L.smoe_workspace_bytes(1, 9, 4, 2048, 1408, 60)
    assert need >= 36 * 1408 * 2
    assert L.verify_grouped_gemm(*a, None, None, FAKE, None, 9, 36, 2048, 1408, 60, FAKE, FAKE,
                                 need - 1, None, None) == 6
    assert L.verify_grouped_gemm(*a, None, None, FAKE, None, 9, 0, 2048, 1408, 60, FAKE, None, 0,
                                 None, None) == 0


def test_verify_shared_validation():
    L = fve.lib()
    need = L.smoe_workspace_bytes(1, 4, 2, 256, 512, 8)

    def call(x=FAKE, st=FAKE, off=FAKE, act=None, na=None, tab=FAKE, T=4, rows=8, H=256, I=512,
             E=8, y=FAKE, w13=FAKE, w2=FAKE, Is=1024, sh=FAKE, so=FAKE, ws=FAKE, wsb=None):
        return L.verify_grouped_gemm_shared(x, st, off, act, na, tab, None, T, rows, H, I, E, y,
                                            w13, w2, Is, sh, so, ws,
                                            need if wsb is None else wsb, None, None)
    assert call(x=None) == 1
    assert call(w13=None) == 1 and "shared" in _err()
    assert call(so=None) == 1
    assert call(act=FAKE) == 1                      # active without n_active
    assert call(Is=1000) == 2 and "shared_I" in _err()
    assert call(H=200) == 2
    assert call(E=0) == 2
    assert call(sh=V(0x1002)) == 2 and "aligned" in _err()
    assert call(T=0) == 0                           # nothing to do
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6


def test_w4_shared_validation():
    L = fve.lib()
    need = L.smoe_workspace_bytes(0, 4, 2, 256, 512, 8)

    def call(x=FAKE, act=FAKE, T=4, H=256, gs=128, y=FAKE, w13=FAKE, w2=FAKE, Is=1024, sh=FAKE,
             so=FAKE, ws=FAKE, wsb=None):
        return L.w4a16_grouped_ffn_shared(x, FAKE, FAKE, act, FAKE, FAKE, T, 2, H, 512, 8, gs, y,
                                          w13, w2, Is, sh, so, ws,
                                          need if wsb is None else wsb, None, None)
    assert call(x=None) == 1
    assert call(act=None) == 1                      # the maps' active list is required
    assert call(w13=None) == 1 and "shared" in _err()
    assert call(so=None) == 1
    assert call(Is=1000) == 2 and "shared_I" in _err()
    assert call(H=200) == 2
    assert call(gs=64) == 3
    assert call(sh=V(0x1002)) == 2 and "aligned" in _err()
    assert call(T=0) == 0                           # nothing to do
    assert call(wsb=need - 1) == 6
    assert call(ws=None) == 6
    assert _err().startswith("w4a16_grouped_ffn_shared")


def test_combine_validation():
    L = fve.lib()
    assert L.moe_combine(FAKE, FAKE, None, None, None, None, 1, 2, 256, FAKE, None, 0.0, None) == 1
    assert L.moe_combine(FAKE, FAKE, FAKE, None, None, None, 70000, 2, 256, FAKE, None, 0.0,
                         None) == 2
    assert L.moe_combine(FAKE, FAKE, FAKE, V(0x1008), None, None, 1, 2, 256, FAKE, None, 0.0,
                         None) == 2
    assert L.moe_combine(FAKE, FAKE, FAKE, None, None, None, 1, 2, 256, FAKE, FAKE, 1e-6,
                         None) == 2                                   # norm_out aliases out
    assert L.moe_combine(FAKE, FAKE, FAKE, None, None, None, 1, 2, 256, FAKE, V(0x2000), -1.0,
                         None) == 2
    assert L.moe_combine(FAKE, FAKE, FAKE, None, None, None, 0, 2, 256, FAKE, None, 0.0, None) == 0


def test_stage_validation():
    L = fve.lib()
    assert L.expert_stage_async(None, FAKE, 16, None, None) == 1
    assert L.expert_stage_async(FAKE, FAKE, 0, None, None) == 0


def test_workspace_sizes():
    L = fve.lib()
    assert L.smoe_workspace_bytes(0, 1, 6, 2048, 1408, 64) > 0
    assert L.smoe_workspace_bytes(0, 1, 6, 2000, 1408, 64) == 0
    # moe_draft_layer (T = 1 only): barrier words, the logits, h [k, I]
    assert L.smoe_workspace_bytes(2, 1, 6, 2048, 1408, 64) == 256 + 512 + 6 * 1408 * 2
    assert L.smoe_workspace_bytes(2, 2, 6, 2048, 1408, 64) == 0
    assert L.smoe_workspace_bytes(3, 1, 6, 2048, 1408, 64) == 0
    assert L.smoe_workspace_bytes(1, 17, 2, 4096, 6400, 16) >= 34 * 6400 * 2
