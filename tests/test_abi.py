"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every entry point that include/kda.h
declares, and argument validation must turn every bad call into a status code
before anything reaches the HIP runtime.  Only calls that fail validation (or
that have nothing to enqueue) are made here.
"""
import ctypes
import os
import re

import pytest

import kda_gated_delta_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("kda.h", "kda_profile.h")]

OK, INVALID, UNSUPPORTED, LAUNCH, WORKSPACE, SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5


def _declared():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert set(declared) == set(kda.EXPORTED), declared
    L = kda.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    assert kda.status_string(OK) == "KDA_OK"
    assert kda.status_string(INVALID) == "KDA_ERR_INVALID_ARGUMENT"
    assert kda.status_string(UNSUPPORTED) == "KDA_ERR_UNSUPPORTED"
    assert kda.status_string(LAUNCH) == "KDA_ERR_LAUNCH"
    assert kda.status_string(WORKSPACE) == "KDA_ERR_WORKSPACE"
    assert kda.status_string(SCRATCH_LIMIT) == "KDA_ERR_SCRATCH_LIMIT"
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


P = ctypes.c_void_p(4096)  # aligned, never dereferenced: calls below fail validation
P_MIS = ctypes.c_void_p(4096 + 4)


def test_gate_prep_validation():
    L = kda.lib()
    # T = 0: nothing to enqueue
    assert L.kda_gate_prep(None, None, None, None, 0, 2, 16, 0.0, None, None, None) == OK
    assert L.kda_gate_prep(P, P, P, None, 4, 2, 16, 0.0, None, P, None) == INVALID
    assert L.kda_gate_prep(P, P, P, None, 4, 2, 24, 0.0, P, P, None) == UNSUPPORTED
    assert L.kda_gate_prep(P, P, P, None, -1, 2, 16, 0.0, P, P, None) == INVALID
    assert L.kda_gate_prep(P, P, P, None, 4, 0, 16, 0.0, P, P, None) == INVALID
    assert L.kda_gate_prep(P, P, P, None, 4, 2, 16, 0.5, P, P, None) == INVALID
    assert L.kda_gate_prep(P_MIS, P, P, None, 4, 2, 16, 0.0, P, P, None) == INVALID


def test_decode_validation():
    L = kda.lib()
    args = lambda **kw: [kw.get("io", 1), P, P, P, P, P, 1.0, kw.get("pool", P),
                         kw.get("n_slots", 8), P, kw.get("B", 2), 4, kw.get("K", 128),
                         kw.get("V", 128), kw.get("o", P), None]
    assert L.kda_recurrent_decode(*args(io=7)) == UNSUPPORTED
    assert L.kda_recurrent_decode(*args(B=0)) == INVALID
    assert L.kda_recurrent_decode(*args(n_slots=0)) == INVALID
    assert L.kda_recurrent_decode(*args(K=48)) == UNSUPPORTED
    assert L.kda_recurrent_decode(*args(V=256)) == UNSUPPORTED
    assert L.kda_recurrent_decode(*args(o=None)) == INVALID
    assert L.kda_recurrent_decode(*args(pool=P_MIS)) == INVALID


def test_verify_validation():
    L = kda.lib()
    args = lambda **kw: [kw.get("io", 1), P, P, P, P, P, 1.0, P, 8, P, 2,
                         kw.get("Tv", 4), 4, 128, 128, kw.get("inter", P), P, None]
    assert L.kda_verify(*args(Tv=0)) == INVALID
    assert L.kda_verify(*args(inter=None)) == INVALID
    assert L.kda_verify(*args(inter=P_MIS)) == INVALID
    assert L.kda_verify(*args(io=2)) == UNSUPPORTED


def test_prefill_validation_and_workspace():
    L = kda.lib()
    ws = kda.kda_chunk_prefill_workspace_size(7680, 4, 32, 128, 128, 64)
    assert ws > 0 and ws % 256 == 0
    # monotone in T and N
    assert kda.kda_chunk_prefill_workspace_size(7681, 4, 32, 128, 128, 64) >= ws
    assert kda.kda_chunk_prefill_workspace_size(7680, 5, 32, 128, 128, 64) >= ws
    n = ctypes.c_size_t(12345)
    assert L.kda_chunk_prefill_workspace_size(64, 1, 2, 16, 16, 48, ctypes.byref(n)) == UNSUPPORTED
    assert L.kda_chunk_prefill_workspace_size(64, 1, 2, 16, 32, 16, ctypes.byref(n)) == UNSUPPORTED
    assert L.kda_chunk_prefill_workspace_size(64, 1, 2, 24, 24, 16, ctypes.byref(n)) == UNSUPPORTED
    assert L.kda_chunk_prefill_workspace_size(-1, 1, 2, 16, 16, 16, ctypes.byref(n)) == INVALID
    assert L.kda_chunk_prefill_workspace_size(64, 0, 2, 16, 16, 16, ctypes.byref(n)) == INVALID
    assert L.kda_chunk_prefill_workspace_size(64, 1, 2, 16, 16, 16, None) == INVALID
    assert n.value == 12345  # untouched on error
    with pytest.raises(kda.KdaError):
        kda.kda_chunk_prefill_workspace_size(64, 1, 2, 16, 32, 16)

    def call(**kw):
        return L.kda_chunk_prefill(
            kw.get("io", 1), P, P, P, P, P, kw.get("cu", P), kw.get("N", 4),
            kw.get("T", 7680), 32, kw.get("K", 128), kw.get("V", 128),
            kw.get("chunk", 64), 1.0, None, P, P, kw.get("ws", P),
            kw.get("ws_bytes", ws), None)
    assert call(chunk=48) == UNSUPPORTED
    assert call(K=64, V=128) == UNSUPPORTED
    assert call(N=0) == INVALID
    assert call(cu=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=ws - 1) == WORKSPACE
    assert call(ws=ctypes.c_void_p(4096 + 64)) == WORKSPACE  # not 256-aligned

    # the marked variant (of the gated call) validates the same way, and
    # needs four events
    marks = (ctypes.c_void_p * 4)(P, P, P, P)
    no_mark = (ctypes.c_void_p * 4)(P, P, None, P)
    base = [1, P, P, P, P, P, P, None, 0.0, P, 4, 7680, 32, 128, 128, 64, 1.0, None, P, P, P,
            ws, None]
    assert L.kda_chunk_prefill_marked(*base, None) == INVALID
    assert L.kda_chunk_prefill_marked(*base, no_mark) == INVALID
    bad = list(base)
    bad[15] = 48
    assert L.kda_chunk_prefill_marked(*bad, marks) == UNSUPPORTED
    bad = list(base)
    bad[21] = ws - 1
    assert L.kda_chunk_prefill_marked(*bad, marks) == WORKSPACE
    bad = list(base)
    bad[8] = 0.5
    assert L.kda_chunk_prefill_marked(*bad, marks) == INVALID

    # the gated variant: a positive lower bound, a missing A_log
    def gated(**kw):
        return L.kda_chunk_prefill_gated(
            1, P, P, P, P, P, kw.get("A_log", P), None, kw.get("lb", 0.0), P, 4,
            kw.get("T", 7680), 32, 128, 128, kw.get("chunk", 64), 1.0, None, P, P,
            kw.get("ws", P), ws, None)
    assert gated(lb=0.5) == INVALID
    assert gated(A_log=None) == INVALID
    assert gated(chunk=48) == UNSUPPORTED
    assert gated(ws=None) == WORKSPACE


def test_binding_rejects_cpu_and_wrong_dtypes():
    import torch
    q = torch.zeros(2, 4, 16)
    with pytest.raises(TypeError):
        kda.kda_recurrent_decode(q.to(torch.float16), q, q, q, q[..., 0], 1.0,
                                 torch.zeros(4, 4, 16, 16), torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        kda.kda_gate_prep(torch.zeros(3, 2, 16), torch.zeros(3, 3), torch.zeros(2))


def test_replay_decode_validation():
    L = kda.lib()
    W, N, F = ctypes.c_void_p(8192), ctypes.c_void_p(8192 + 64), ctypes.c_void_p(8192 + 128)

    def args(**kw):
        return [kw.get("io", 1), P, P, P, P, P, 1.0, kw.get("pool", P), kw.get("n_slots", 8),
                P, kw.get("wp", W), kw.get("ff", F), kw.get("L", 16), kw.get("rd", P), P, P,
                kw.get("B", 4), 2, kw.get("K", 128), 128, kw.get("o", P), kw.get("nx", N), None]
    assert L.kda_replay_decode(*args(io=5)) == UNSUPPORTED
    assert L.kda_replay_decode(*args(B=0)) == INVALID
    assert L.kda_replay_decode(*args(n_slots=0)) == INVALID
    assert L.kda_replay_decode(*args(L=0)) == INVALID
    assert L.kda_replay_decode(*args(L=33)) == INVALID
    assert L.kda_replay_decode(*args(K=24)) == UNSUPPORTED
    assert L.kda_replay_decode(*args(wp=None)) == INVALID
    assert L.kda_replay_decode(*args(rd=None)) == INVALID
    assert L.kda_replay_decode(*args(o=None)) == INVALID
    assert L.kda_replay_decode(*args(pool=P_MIS)) == INVALID
    assert L.kda_replay_decode(*args(rd=P_MIS)) == INVALID
    # the cursor output may not overlap the cursors or the flush flags
    assert L.kda_replay_decode(*args(nx=W)) == INVALID
    assert L.kda_replay_decode(*args(nx=ctypes.c_void_p(8192 + 12))) == INVALID
    assert L.kda_replay_decode(*args(nx=ctypes.c_void_p(8192 + 120))) == INVALID


def test_prefill_snapshots_validation():
    L = kda.lib()
    WS = ctypes.c_void_p(1 << 20)

    def args(**kw):
        return [1, P, P, P, P, P, P, 2, kw.get("T", 256), 2, 64, 64, kw.get("chunk", 64), 1.0,
                None, None, P, kw.get("snap", P), kw.get("rows", 4), kw.get("iv", 64), WS,
                1 << 30, None]
    assert L.kda_chunk_prefill_snapshots(*args(iv=0)) == INVALID
    assert L.kda_chunk_prefill_snapshots(*args(iv=96)) == INVALID  # not a multiple of 64
    assert L.kda_chunk_prefill_snapshots(*args(snap=None)) == INVALID
    assert L.kda_chunk_prefill_snapshots(*args(snap=P_MIS)) == INVALID
    assert L.kda_chunk_prefill_snapshots(*args(rows=3)) == INVALID  # 256 / 64 = 4 rows needed
    assert L.kda_chunk_prefill_snapshots(*args(chunk=48, iv=96)) == UNSUPPORTED


def test_step_options_validation():
    L = kda.lib()
    op = kda.StepOpts()

    def dec(o=op, H=4):
        return L.kda_recurrent_decode_ex(1, P, P, P, P, P, 1.0, P, 8, P, 2, H, 64, 64, P,
                                         ctypes.byref(o), None)
    op.gate_mode = 3
    assert dec() == INVALID
    op.gate_mode = 1  # raw gate without A_log
    assert dec() == INVALID
    op.A_log = 4096
    op.gate_mode = 2  # safe gate needs a negative bound
    assert dec() == INVALID
    op.gate_mode, op.qk_heads = 0, 3  # 4 value heads are not a multiple of 3
    assert dec() == INVALID
    op.qk_heads, op.o_gate = 2, 4096  # output gate without a norm weight
    assert dec() == INVALID
    op.o_norm_w, op.o_gate_act = 4096, 2
    assert dec() == INVALID
    op.o_gate_act, op.o_norm_eps = 0, -1.0
    assert dec() == INVALID
    v = L.kda_verify_ex(1, P, P, P, P, P, 1.0, P, 8, P, 2, 0, 4, 64, 64, P, P,
                        ctypes.byref(kda.StepOpts()), None)
    assert v == INVALID  # Tv = 0


def test_prefill_options_validation():
    L = kda.lib()
    WS = ctypes.c_void_p(1 << 20)

    def call(op, H=4):
        return L.kda_chunk_prefill_ex(1, P, P, P, P, P, P, 2, 256, H, 64, 64, 64, 1.0, None,
                                      None, P, WS, 1 << 30, ctypes.byref(op), None)
    op = kda.PrefillOpts()
    op.per_head_gate = 1
    assert call(op, H=6) == UNSUPPORTED  # per-head gates need H a multiple of 4
    op = kda.PrefillOpts()
    op.qk_heads = 3
    assert call(op) == INVALID
    op = kda.PrefillOpts()
    op.gate_mode = 2  # safe gate without a negative bound
    assert call(op) == INVALID
    op = kda.PrefillOpts()
    op.snapshots, op.snapshot_interval, op.snapshot_rows = 4096, 96, 8
    assert call(op) == INVALID  # interval not a multiple of the chunk


def test_replay_options_validation():
    L = kda.lib()
    W, N, F = ctypes.c_void_p(8192), ctypes.c_void_p(8192 + 64), ctypes.c_void_p(8192 + 128)

    def call(o):
        return L.kda_replay_decode_ex(1, P, P, P, P, P, 1.0, P, 8, P, W, F, 16, P, P, P, 4, 2,
                                      128, 128, P, N, ctypes.byref(o), None)
    # the output norm's arguments are checked as for decode and verify
    op = kda.StepOpts()
    op.qk_l2norm = 1
    op.o_gate = 4096  # no weight
    assert call(op) == INVALID
    op.o_norm_w = 4096 + 4  # misaligned weight
    assert call(op) == INVALID
    op.o_norm_w, op.o_gate_act = 4096, 2  # unknown activation
    assert call(op) == INVALID
    op.o_gate_act, op.o_norm_eps = 0, -1.0
    assert call(op) == INVALID
    op = kda.StepOpts()
    op.gate_mode = 1  # no A_log
    assert call(op) == INVALID


def test_noalloc_prefill_validation():
    """kda_chunk_prefill_noalloc refuses on the host: the prefill's own
    argument errors, and a batch whose workspace exceeds the static scratch
    (KDA_ERR_SCRATCH_LIMIT), both before any HIP call."""
    L = kda.lib()

    def call(**kw):
        return L.kda_chunk_prefill_noalloc(
            kw.get("io", 1), P, P, P, P, P, P, kw.get("N", 1), kw.get("T", 64), kw.get("H", 2),
            kw.get("K", 128), kw.get("V", 128), kw.get("chunk", 64), 1.0, None, P, P, None, None)
    assert call(chunk=48) == UNSUPPORTED
    assert call(K=64, V=128) == UNSUPPORTED
    assert call(N=0) == INVALID
    assert call(T=-1) == INVALID
    assert call(T=1 << 20, H=32) == SCRATCH_LIMIT
    ws = kda.kda_chunk_prefill_workspace_size(8192, 1, 32, 128, 128, 64)
    assert ws > kda.NOALLOC_SCRATCH_BYTES and call(T=8192, H=32) == SCRATCH_LIMIT


def test_prefill_schedule():
    L = kda.lib()
    out = kda.PrefillSchedule()
    assert L.kda_chunk_prefill_schedule(4096, 1, 4, 128, 128, 64, None) == INVALID
    assert L.kda_chunk_prefill_schedule(4096, 1, 4, 128, 64, 64, ctypes.byref(out)) == UNSUPPORTED
    assert L.kda_chunk_prefill_schedule(4096, 0, 4, 128, 128, 64, ctypes.byref(out)) == INVALID
    # a short batch: one launch of each kernel, chain not cut
    s = kda.kda_chunk_prefill_schedule(7680, 4, 32, 128, 128, 64)
    assert s == dict(n_waves=1, segment_chunks=0, uses_maps=0, intra_launches=1,
                     state_launches=1, other_launches=1)
    # empty input: the chunk table and state pass still run (ht = h0)
    s = kda.kda_chunk_prefill_schedule(0, 1, 4, 128, 128, 64)
    assert s["intra_launches"] == 0 and s["state_launches"] == 1
    # a long chain is cut: waves or maps, with launch counts to match
    for H in (4, 32):
        s = kda.kda_chunk_prefill_schedule(65536, 1, H, 128, 128, 64)
        assert s["segment_chunks"] > 0
        if s["uses_maps"]:
            assert s["n_waves"] == 1 and s["state_launches"] == 2 and s["other_launches"] == 2
        else:
            assert s["n_waves"] > 1
            assert s["intra_launches"] == s["state_launches"] == s["n_waves"]
            assert s["n_waves"] * s["segment_chunks"] >= 1024
