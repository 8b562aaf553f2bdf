"""CPU checks of bench.py's host logic: the counter summaries it reads parse,
and the byte accounting of the packet share matches its definition."""
from __future__ import annotations

import pathlib
import re

import bench

PROFILES = pathlib.Path(__file__).resolve().parents[1] / "profiles"


def test_counter_summaries_parse():
    for name in ("write_bcast_440x5120_p8_counters.md", "packet_fused_512x7168_p8_counters.md"):
        text = (PROFILES / name).read_text()
        assert re.search(r"[Kk]ernel source hash[^`]*`([0-9a-f]{16})`", text), name
        m = re.search(r"scaled HBM bytes per launch:\s*([0-9.]+)", text)
        assert m and float(m.group(1)) > 0, name


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    got = bench.traffic_from_profiles("write_bcast_440x5120_p8", 72089600)
    text = (PROFILES / "write_bcast_440x5120_p8_counters.md").read_text()
    recorded = re.search(r"[Kk]ernel source hash[^`]*`([0-9a-f]{16})`", text).group(1)
    if recorded == bench.kernel_source_hash():
        assert got is not None and 0.99 < got / 72089600 < 1.05
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles("write_bcast_440x5120_p8", 72089600) is None


def test_source_hash_ignores_comments_but_not_code():
    src = "int f(int a) {  // the answer\n    return a + 1; /* one more */\n}\n"
    reworded = "// a new header line\nint f(int a) {\n  return a + 1;  // still one more\n}\n"
    changed = "int f(int a) {  // the answer\n    return a + 2; /* one more */\n}\n"
    assert bench.code_of(src) == bench.code_of(reworded)
    assert bench.code_of(src) != bench.code_of(changed)
    assert "answer" not in bench.code_of(src) and "return a + 1;" in bench.code_of(src)


def test_packet_byte_accounting():
    n = 512 * 7168
    # P = 8: read 2n + 2 * 3.5n, write 10n  ->  19n per rank
    assert bench.packet_fused_bytes(8, n) == 19 * n
    # P = 2: read 2n + 2 * 2n, write 10n -> 16n
    assert bench.packet_fused_bytes(2, 1000) == 16 * 1000


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    import sys
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    else:
        raise AssertionError("bench.py --gpus 2 did not exit")
    assert "ONE GPU" in capsys.readouterr().err


def test_cpu_rows_leg_covers_every_workload():
    """Every workload row gets an oracle timing; inputs here are small
    stand-ins of the rows' shapes so the check runs in a second."""
    import types

    from allreduce_reduction_way_amd import inputs as I, workloads as W

    rows = {}
    for w in W.ALL:
        P = w.P
        n = 1024 * P
        rows[w.name] = types.SimpleNamespace(name=w.name, alg_bytes=4 * n,
                                             host=I.make_inputs("uniform", P, n, seed=1))
    got = bench.cpu_rows_leg(rows, W, budget_s=0.01)
    assert set(got) == {w.name for w in W.ALL}
    for name, v in got.items():
        assert v["oracle_ms_per_step"] > 0 and v["oracle_gbs"] > 0, name


def test_cpu_rows_leg_rechecks_outputs_against_the_oracle():
    """The parity recheck on bench inputs: outputs equal to the oracle's pass,
    a single flipped element fails (CPU tensors stand in for device ones)."""
    import types

    import numpy as np
    import torch

    from allreduce_reduction_way_amd import inputs as I, workloads as W
    from oracle import oracle as O

    def t16(a):
        return torch.from_numpy(np.array(a, dtype=np.uint16).view(np.int16))   # a copy

    P, n = 8, 8 * 1024 + 8
    xs = I.make_inputs("uniform", P, n, seed=3)
    y = O.oneshot_sum(xs)
    nb = O.packet_scratch_bytes(P, n)
    pk_outs, _ = O.packet_fused(xs, 1, [np.zeros(nb, np.uint8) for _ in range(P)])
    b, e = O.slice_range(P, n, 3)
    rows = {
        W.WRITE_BCAST_440x5120.name: types.SimpleNamespace(outs=[t16(y) for _ in range(P)]),
        W.PACKET_512x7168.name: types.SimpleNamespace(outs=[t16(o) for o in pk_outs]),
        W.TWOSHOT_680x5120_R3.name: types.SimpleNamespace(outs=[t16(y) for _ in range(P)],
                                                          slice=(b, e)),
        W.LL_ENCODE_512x7168.name: types.SimpleNamespace(
            outs=[torch.from_numpy(O.ll_encode(xs[0], 1).view(np.uint8))]),
        W.LL_DECODE_512x7168.name: types.SimpleNamespace(outs=[t16(xs[0])]),
    }
    for name, r in rows.items():
        r.name, r.host, r.alg_bytes = name, xs, 4 * n
    got = bench.cpu_rows_leg(rows, W, budget_s=0.0)
    assert all(v["gpu_output_matches"] is True for v in got.values()), got
    rows[W.PACKET_512x7168.name].outs[5][100] += 1
    rows[W.TWOSHOT_680x5120_R3.name].outs[2][b + 7] += 1
    got = bench.cpu_rows_leg(rows, W, budget_s=0.0)
    assert got[W.PACKET_512x7168.name]["gpu_output_matches"] is False
    assert got[W.TWOSHOT_680x5120_R3.name]["gpu_output_matches"] is False
    assert got[W.WRITE_BCAST_440x5120.name]["gpu_output_matches"] is True


# ------------------------------------------------------------------------------
# Every device buffer a bench row addresses is held by the row.
#
# A row's launches, and any HIP graph it captured, address tensors by raw
# pointer.  If the row does not hold such a tensor, it goes back to torch's
# cache, and a graph replayed later reads freed memory.  Here stand-ins for
# torch and for the C library hand out fake device addresses and record every
# address a launch or a captured graph uses; each must lie inside a tensor the
# row keeps.

class _FakeTensor:
    _next = [0x10_0000_0000]

    def __init__(self, nbytes, elem=2):
        self.nbytes, self.elem = max(int(nbytes), 1), elem
        self.addr = _FakeTensor._next[0]
        _FakeTensor._next[0] += (self.nbytes + 0xFFFF) // 0x10000 * 0x10000 + 0x10000
        self.is_cuda = True

    def data_ptr(self):
        return self.addr

    def to(self, dev):
        return self

    def clone(self):
        return _FakeTensor(self.nbytes, self.elem)

    def view(self, *a):
        return self


def _fake_torch():
    import types

    def alloc(n, dtype=None, device=None):
        elem = 1 if dtype == "uint8" else 2
        return _FakeTensor(n * elem, elem)

    class Graph:
        def replay(self):
            pass

    class Capture:
        def __init__(self, g, stream=None):
            pass

        def __enter__(self):
            return self

        def __exit__(self, *a):
            return False

    cuda = types.SimpleNamespace(synchronize=lambda: None, CUDAGraph=Graph, graph=Capture)
    return types.SimpleNamespace(device=lambda s: s, int16="int16", uint8="uint8", int32="int32",
                                 from_numpy=lambda a: _FakeTensor(a.nbytes), empty=alloc,
                                 zeros=alloc, cuda=cuda)


def _fake_ar(touched):
    import types

    from allreduce_reduction_way_amd import ar as real

    def note(v):
        if isinstance(v, _FakeTensor):
            touched.append(v.addr)
        elif isinstance(v, int) and v >= 0x10_0000_0000:
            touched.append(v)
        elif isinstance(v, (list, tuple)):
            for x in v:
                note(x)

    def recorder(*args, **kw):
        note(list(args) + list(kw.values()))
        return 0

    class Lib:
        def __getattr__(self, name):
            return recorder

    lib = Lib()
    return types.SimpleNamespace(
        _ptrs=lambda bufs: tuple(b.addr if isinstance(b, _FakeTensor) else b for b in bufs),
        lib=lambda: lib, ArError=real.ArError, AR_CTRL_BYTES=real.AR_CTRL_BYTES,
        ar_packet_scratch_bytes=real.ar_packet_scratch_bytes, ar_slice_range=real.ar_slice_range,
        ar_ll_packets=real.ar_ll_packets, ar_packet_fused_epoch=recorder,
        ar_packet_fused=recorder, ar_ll_encode=recorder)


def test_every_buffer_a_row_addresses_is_kept_by_the_row():
    import types

    import numpy as np

    from allreduce_reduction_way_amd import workloads as W

    stub_inputs = types.SimpleNamespace(
        make_inputs=lambda dist, P, n, seed=0: [np.zeros(8, np.uint16) for _ in range(P)])
    for w in W.ALL:
        touched = []
        rows = bench.make_rows([w.name], _fake_torch(), _fake_ar(touched), stub_inputs, W)
        assert w.name in rows
        for row in rows.values():
            step = row.factory(0)
            for i in range(3):
                step(i)
        kept = [t for row in rows.values() for t in row.keep]
        assert touched, w.name
        for a in touched:
            assert any(t.addr <= a < t.addr + t.nbytes for t in kept), (w.name, hex(a))


def test_cpu_baseline_parallel_leg_is_bit_identical():
    import concurrent.futures

    import numpy as np

    from allreduce_reduction_way_amd import inputs as I
    from oracle import oracle as O

    xs = I.make_inputs("uniform", 8, 10_007, seed=4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=3) as pool:
        parts = bench.oracle_write_bcast_parallel(O, xs, pool, 3)
    assert len(parts) == 3
    for k in range(8):
        assert np.array_equal(np.concatenate([p[k] for p in parts]), O.oneshot_sum(xs))
    cb = bench.cpu_baseline(xs, budget_s=0.02)
    assert cb["cores"] == bench.host_cores() >= 1
    assert cb["parallel_equals_single_thread"] is True
    assert cb["value"] > 0 and cb["single_thread"]["value"] > 0 and cb["cpu_model"]
