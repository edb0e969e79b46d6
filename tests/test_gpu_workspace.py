"""The per-stream workspace of the GEMM entry points.

Calls that need device workspace (FP32 B split once into planes, split-K
partial sums) reuse one block per stream.  These tests make such calls on
several streams without host synchronisation in between, on more streams than
the library's table holds, with growing and shrinking sizes on one stream, and
from two host threads on one stream.  Every result must equal, bit for bit,
the same call made alone with the device idle (the kernels are deterministic),
and the references themselves are checked against the FP64 bound.
"""
import sys
import threading

import numpy as np
import pytest
import torch

from gpu_util import check_against_fp64, dev, host

pytestmark = pytest.mark.gpu

# (M, N, K, entry): "ws" = sgemm_emu_ex on FP32 B with SGEMM_EMU_PRESPLIT_B (B split
# into workspace planes); "fused" = sgemm_bf16x9's own choice; "nk" = caller-split planes
CASES = [
    (1024, 130, 64, "ws"),         # B planes in the workspace
    (6144, 256, 1024, "fused"),    # planes and split-K partials in one block (its own choice)
    (2048, 1000, 512, "ws"),       # a larger plane set
    (129, 130, 1024, "nk"),        # split-K partials only
    (1100, 257, 100, "ws"),        # ragged K: zero-padded planes
]


@pytest.fixture(scope="module")
def fe():
    import fp32_emulated_gemm_amd as fe
    return fe


class Problem:
    def __init__(self, fe, case, seed):
        M, N, K, entry = case
        self.case = case
        g = np.random.Generator(np.random.Philox(key=seed))
        self.A_h = g.standard_normal((M, K)).astype(np.float32)
        self.B_h = g.standard_normal((K, N)).astype(np.float32)
        self.A = dev(self.A_h)
        self.B = dev(self.B_h)
        self.planes = None
        if entry == "nk":
            Bt = dev(np.ascontiguousarray(self.B_h.T))
            self.planes = [torch.empty(N * K, dtype=torch.int16, device="cuda") for _ in range(3)]
            fe.split_f32_bf16x3(N, K, Bt, K, *self.planes, K)

    def launch(self, fe, C, stream):
        M, N, K, entry = self.case
        if entry == "fused":
            fe.sgemm_bf16x9(M, N, K, self.A, K, self.B, N, C, N, stream)
        elif entry == "ws":
            fe.sgemm_emu_ex(M, N, K, self.A, K, self.B, N, C, N, 5, fe.SGEMM_EMU_PRESPLIT_B, stream)
        else:
            fe.sgemm_emu_presplit_b(M, N, K, self.A, K, *self.planes, K, fe.SGEMM_EMU_B_NK, C, N, 5, stream)

    def out(self):
        M, N = self.case[0], self.case[1]
        return torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")

    def result(self, C):
        M, N = self.case[0], self.case[1]
        return host(C).reshape(M, N)


@pytest.fixture(scope="module")
def problems(fe):
    probs = [Problem(fe, c, 7000 + i) for i, c in enumerate(CASES)]
    refs = []
    for p in probs:
        print(f"workspace reference {p.case}", flush=True, file=sys.stderr)
        C = p.out()
        torch.cuda.synchronize()
        p.launch(fe, C, None)
        torch.cuda.synchronize()
        R = p.result(C)
        check_against_fp64(R, p.A_h, p.B_h, label=f"workspace reference {p.case}")
        refs.append(R)
    return probs, refs


def _same(R, C, what):
    assert np.array_equal(R.view(np.uint32), C.view(np.uint32)), what


def _run_schedule(fe, problems, schedule):
    """schedule: list of (problem index, stream).  Launch all, synchronise once,
    compare each output with its reference."""
    probs, refs = problems
    outs = [probs[i].out() for i, _ in schedule]
    torch.cuda.synchronize()
    for (i, s), C in zip(schedule, outs):
        probs[i].launch(fe, C, s)
    torch.cuda.synchronize()
    for n, ((i, s), C) in enumerate(zip(schedule, outs)):
        _same(refs[i], probs[i].result(C), f"call {n}: case {probs[i].case}")


def test_interleaved_streams(fe, problems):
    streams = [torch.cuda.Stream() for _ in range(3)]
    n = len(problems[0])
    schedule = [(i, streams[(i + rep) % 3]) for rep in range(3) for i in range(n)]
    print("workspace: interleaved on 3 streams", flush=True, file=sys.stderr)
    _run_schedule(fe, problems, schedule)


def test_more_streams_than_slots(fe, problems):
    """Eleven streams cycle through the table (eight slots): blocks of streams
    that dropped out are handed over after their last use."""
    streams = [torch.cuda.Stream() for _ in range(11)]
    n = len(problems[0])
    schedule = [(k % n, streams[k % 11]) for k in range(33)]
    print("workspace: 11 streams", flush=True, file=sys.stderr)
    _run_schedule(fe, problems, schedule)


def test_grow_and_shrink_on_one_stream(fe, problems):
    s = torch.cuda.Stream()
    order = [0, 2, 0, 1, 4, 2, 3, 0]   # small, large, small, planes + partials, ragged, large, partials, small
    print("workspace: one stream, changing sizes", flush=True, file=sys.stderr)
    _run_schedule(fe, problems, [(i, s) for i in order])


def test_default_stream_between_others(fe, problems):
    s = torch.cuda.Stream()
    schedule = [(1, None), (1, s), (2, None), (0, s), (1, None)]
    print("workspace: default stream and one other", flush=True, file=sys.stderr)
    _run_schedule(fe, problems, schedule)


def test_two_host_threads_on_one_stream(fe, problems):
    """Two threads enqueue on the same stream at once; each call holds the
    table's lock until its last launch, so their kernels never interleave."""
    probs, refs = problems
    s = torch.cuda.Stream()
    plan = {0: [1, 0, 2, 1, 4, 1], 1: [2, 1, 1, 0, 1, 4]}
    outs = {t: [probs[i].out() for i in plan[t]] for t in plan}
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            for i, C in zip(plan[t], outs[t]):
                probs[i].launch(fe, C, s)
        except Exception as e:  # reported below
            errors.append(e)

    print("workspace: two threads, one stream", flush=True, file=sys.stderr)
    threads = [threading.Thread(target=worker, args=(t,)) for t in plan]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in plan:
        for n, (i, C) in enumerate(zip(plan[t], outs[t])):
            _same(refs[i], probs[i].result(C), f"thread {t} call {n}: case {probs[i].case}")


def test_release_workspace_gives_memory_back(fe, problems):
    """sgemm_emu_release_workspace frees every retained block of the device and
    trims the library's pool: the driver's free memory rises by at least the
    planes of a 4096^3 call (A and B split into workspace planes, 2 x 96 MiB),
    and later calls allocate afresh and give the same bits."""
    n = 4096
    g = torch.Generator(device="cuda").manual_seed(11)
    A = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    B = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    C = torch.empty((n, n), device="cuda")
    print("workspace: 4096^3 then release", flush=True, file=sys.stderr)
    fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n)
    torch.cuda.synchronize()
    first = C.clone()
    free_before = torch.cuda.mem_get_info()[0]
    fe.sgemm_emu_release_workspace()
    free_after = torch.cuda.mem_get_info()[0]
    assert free_after - free_before >= 150 << 20, (free_before, free_after)
    fe.sgemm_emu_release_workspace()          # nothing left: still fine
    fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), C.view(torch.int32))
    del A, B, C, first
    print("workspace: the small cases after a release", flush=True, file=sys.stderr)
    s = torch.cuda.Stream()
    _run_schedule(fe, problems, [(i, s) for i in range(len(problems[0]))])


def test_graph_capture_allocates_nothing(fe):
    """On a stream being captured into a graph the library allocates nothing.
    Calls that need no workspace capture as usual (a forced pre-split of B falls
    back to the kernel that splits B itself: the same bits as the eager call,
    which used workspace planes); a K-split shape reports SGEMM_EMU_ECAPTURE
    with nothing enqueued, and runs with SGEMM_EMU_NO_WORKSPACE (one pass per
    tile).  Three replays, with eager calls and synchronisation between them,
    each equal the eager results bit for bit."""
    g = np.random.Generator(np.random.Philox(key=4242))

    def mat(r, c):
        return dev(g.standard_normal((r, c)).astype(np.float32))

    # (a) N x K planes, a grid with no K split (192 tiles) and N < 4096 (no A planes)
    M1, N1, K1 = 4096, 768, 256
    A1, Bt1 = mat(M1, K1), mat(N1, K1)
    P1 = [torch.empty((N1, K1), dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3(N1, K1, Bt1, K1, *P1, K1)
    # (b) FP32 B with the pre-split forced (workspace planes when eager)
    M2, N2, K2 = 4096, 1024, 256
    A2, B2 = mat(M2, K2), mat(K2, N2)
    assert fe.sgemm_emu_split_k(M1, N1, K1) == 1 and fe.sgemm_emu_split_k(M2, N2, K2) == 1
    ref1 = torch.empty((M1, N1), device="cuda")
    ref2 = torch.empty((M2, N2), device="cuda")
    fe.sgemm_emu_presplit_b(M1, N1, K1, A1, K1, *P1, K1, fe.SGEMM_EMU_B_NK, ref1, N1, 5)
    fe.sgemm_emu_ex(M2, N2, K2, A2, K2, B2, N2, ref2, N2, 5, fe.SGEMM_EMU_PRESPLIT_B)
    # (c) a K-split shape (N x K planes: the kernel that splits K)
    M3, N3, K3 = 129, 130, 1024
    A3, Bt3 = mat(M3, K3), mat(N3, K3)
    P3 = [torch.empty((N3, K3), dtype=torch.int16, device="cuda") for _ in range(3)]
    fe.split_f32_bf16x3(N3, K3, Bt3, K3, *P3, K3)
    assert fe.sgemm_emu_split_k(M3, N3, K3) > 1
    out1 = torch.empty_like(ref1)
    out2 = torch.empty_like(ref2)
    out3 = torch.zeros((M3, N3), device="cuda")
    # (d) the same small grid from FP32 B without workspace
    B4 = mat(K3, N3)
    ref4 = torch.empty((M3, N3), device="cuda")
    fe.sgemm_emu_ex(M3, N3, K3, A3, K3, B4, N3, ref4, N3, 5, fe.SGEMM_EMU_NO_WORKSPACE)
    out4 = torch.empty_like(ref4)
    torch.cuda.synchronize()
    print("graph capture: two calls without workspace, one K-split call", flush=True, file=sys.stderr)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        fe.sgemm_emu_presplit_b(M1, N1, K1, A1, K1, *P1, K1, fe.SGEMM_EMU_B_NK, out1, N1, 5, s)
        fe.sgemm_emu_ex(M2, N2, K2, A2, K2, B2, N2, out2, N2, 5, fe.SGEMM_EMU_PRESPLIT_B, s)
        with pytest.raises(fe.SgemmEmuError) as err:
            fe.sgemm_emu_presplit_b(M3, N3, K3, A3, K3, *P3, K3, fe.SGEMM_EMU_B_NK, out3, N3, 5, s)
        assert err.value.status == fe.SGEMM_EMU_ECAPTURE
        fe.sgemm_emu_ex(M3, N3, K3, A3, K3, B4, N3, out4, N3, 5, fe.SGEMM_EMU_NO_WORKSPACE, s)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"graph capture: replay {rep}", flush=True, file=sys.stderr)
        out1.fill_(float("nan"))
        out2.fill_(float("nan"))
        out4.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ref1.view(torch.int32), out1.view(torch.int32)), f"replay {rep}: N x K planes"
        assert torch.equal(ref2.view(torch.int32), out2.view(torch.int32)), f"replay {rep}: forced pre-split"
        assert bool((out3 == 0).all()), "the refused call enqueued work"
        assert torch.equal(ref4.view(torch.int32), out4.view(torch.int32)), f"replay {rep}: no workspace"
        # eager work between replays, on the default stream, with its workspace
        fe.sgemm_emu_ex(M2, N2, K2, A2, K2, B2, N2, out2, N2, 5, fe.SGEMM_EMU_PRESPLIT_B)
        torch.cuda.synchronize()
        assert torch.equal(ref2.view(torch.int32), out2.view(torch.int32)), f"eager after replay {rep}"
    del graph


def test_graph_capture_of_64_tiles(fe):
    """Small grids that run on 64 x 64 tiles need no workspace, so the default
    entry points capture into a graph on them: FP32 B on 1024^3 (where 128 x 128
    tiles would split B and take stream-K), the caller's N x K and K x N planes
    on 1024 x 1024 x 512.  Three replays, with eager calls and synchronisation
    between them, each equal the eager results bit for bit."""
    g = np.random.Generator(np.random.Philox(key=6464))

    def mat(r, c):
        return dev(g.standard_normal((r, c)).astype(np.float32))

    M1 = N1 = K1 = 1024
    assert fe.sgemm_emu_split_k_fp32_b(M1, N1, K1) == 1 and fe.sgemm_emu_split_k(M1, N1, K1) > 1
    A1, B1 = mat(M1, K1), mat(K1, N1)
    M2, N2, K2 = 1024, 1024, 512
    assert fe.sgemm_emu_split_k(M2, N2, K2) == 1 and fe.sgemm_emu_split_k_fp32_b(M2, N2, K2) == 1
    A2, B2 = mat(M2, K2), mat(K2, N2)
    Pnk = fe.split(B2.t().contiguous())
    Pkn = fe.split(B2)
    refs = [torch.empty((M1, N1), device="cuda"), torch.empty((M2, N2), device="cuda"),
            torch.empty((M2, N2), device="cuda")]
    outs = [torch.empty_like(r) for r in refs]

    def calls(o, stream=None):
        fe.sgemm_bf16x9(M1, N1, K1, A1, K1, B1, N1, o[0], N1, stream)
        fe.sgemm_emu_presplit_b(M2, N2, K2, A2, K2, *Pnk, K2, fe.SGEMM_EMU_B_NK, o[1], N2, 5, stream)
        fe.sgemm_emu_presplit_b(M2, N2, K2, A2, K2, *Pkn, N2, fe.SGEMM_EMU_B_KN, o[2], N2, 5, stream)

    calls(refs)
    torch.cuda.synchronize()
    assert torch.equal(refs[1].view(torch.int32), refs[2].view(torch.int32))
    print("graph capture: three calls on 64 x 64 tiles", flush=True, file=sys.stderr)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        calls(outs, s)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"graph capture of 64 x 64 tiles: replay {rep}", flush=True, file=sys.stderr)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (r, o) in enumerate(zip(refs, outs)):
            assert torch.equal(r.view(torch.int32), o.view(torch.int32)), f"replay {rep}: call {i}"
        # eager work between replays, on the default stream
        fe.sgemm_bf16x9(M1, N1, K1, A1, K1, B1, N1, outs[0], N1)
        torch.cuda.synchronize()
        assert torch.equal(refs[0].view(torch.int32), outs[0].view(torch.int32)), f"eager after replay {rep}"
    del graph
