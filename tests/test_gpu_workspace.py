"""GPU tests of the caller-owned split-K scratch (dg_fp8_gemm_nt_ws,
dg_get_workspace_size): the library allocates nothing and synchronises
nothing, so split-K decode GEMMs can be captured into graphs (the masked and
decode paths exist for graph-captured decoding: "DeepGEMM" README summary,
GeekNews, section "Dense and Grouped GEMM", masked paragraph).

Every result is held to the GEMM bar against the CPU oracle:
|D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg

from helpers import SENTINEL, Guarded, check_close, dense_problem, dev

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


class Case:
    """One dense problem on the device, its oracle result and a guarded output."""

    def __init__(self, M, N, K, seed):
        self.p = dense_problem(M, N, K, seed=seed, with_c=False)
        p = self.p
        self.a, self.sfa, self.b, self.sfb = dev(p["a"]), dev(p["sfa"]), dev(p["b"]), dev(p["sfb"])
        self.out = Guarded((M, N))
        self.ref = oracle.gemm_nt(p["a"], p["sfa"], p["b"], p["sfb"], None)
        self.shape = (M, N, K)

    def run(self, workspace):
        dg.fp8_gemm_nt(self.a, self.sfa, self.b, self.sfb, self.out.t, workspace=workspace)

    def reset(self):
        self.out.t.view(torch.int16).fill_(SENTINEL)

    def check(self, where):
        assert self.out.guards_intact(), where
        bits = self.out.bits()
        assert not np.any(bits == SENTINEL), f"{where}: output not written"
        check_close(bits, self.ref, f"{where} {self.shape}")


def test_workspace_size_rules():
    """Decode shapes split K and need scratch; prefill shapes do not; bad shapes
    are rejected."""
    for M, N, K in [(64, 2112, 7168), (128, 7168, 16384), (128, 2112, 7168)]:
        assert dg.get_workspace_size(M, N, K) > 0, (M, N, K)
    assert dg.get_workspace_size(4096, 4096, 7168) == 0
    with pytest.raises(dg.DGError):
        dg.get_workspace_size(64, 2112, 100)
    with pytest.raises(dg.DGError):
        dg.get_workspace_size(0, 2112, 1024)


def test_workspace_errors_and_no_split():
    """A workspace smaller than the configuration needs is an argument error
    (nothing launched, output untouched); a misaligned one an alignment error;
    none at all runs the unsplit kernel, to the same bar."""
    c = Case(64, 2112, 4096, seed=71)
    need = dg.get_workspace_size(*c.shape)      # the larger need of the two scale forms
    assert need > 4096
    small = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.DGError) as e:
        c.run(small)
    assert e.value.status == -4
    big = torch.zeros(need + 32, dtype=torch.uint8, device="cuda")
    with pytest.raises(dg.DGError) as e:
        c.run(big[8:8 + need])
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert np.all(c.out.bits() == SENTINEL)
    c.run(None)
    torch.cuda.synchronize()
    assert "splits=1 " in dg.last_config(), dg.last_config()
    c.check("no workspace")
    c.reset()
    c.run(big[:need])
    torch.cuda.synchronize()
    c.check("workspace")


def test_one_workspace_serves_calls_of_different_shapes():
    """One zeroed workspace, sized for the largest problem, reused in stream
    order by split-K calls of different shapes: every call finds the arrival
    counters back at zero."""
    cases = [Case(64, 700, 4096, 81), Case(128, 2112, 7168, 82), Case(40, 1500, 1024, 83), Case(128, 300, 2048, 84)]
    ws = torch.zeros(max(dg.get_workspace_size(*c.shape) for c in cases), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for c in cases:
            c.reset()
            c.run(ws)
            torch.cuda.synchronize()
            c.check(f"shared workspace rep {rep} ({dg.last_config()})")


def test_graph_capture_replay_and_concurrent_graphs():
    """The regression the caller-owned scratch exists for:
    1. a split-K decode GEMM is captured into a graph with its workspace;
    2. a larger split-K GEMM then runs eagerly on the same stream;
    3. the graph is replayed; then two captured graphs, each with its own
       workspace, are replayed at the same time on two streams;
    4. every replay, and the eager call, matches the oracle.  Outputs are
       refilled with the sentinel before each replay, so a replay that wrote
       nothing would fail."""
    small = Case(64, 2112, 4096, seed=91)
    large = Case(128, 7168, 8192, seed=92)
    other = Case(128, 2112, 7168, seed=93)
    for c in (small, large, other):
        assert dg.get_workspace_size(*c.shape) > 0
    ws_small, ws_large, ws_other = (dg.get_workspace(*c.shape) for c in (small, large, other))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()

    announce("capture split-K decode GEMMs")
    g_small = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_small, stream=s):
        small.run(ws_small)
    g_other = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_other, stream=s):
        other.run(ws_other)
    torch.cuda.synchronize()

    announce("eager larger split-K GEMM on the capture stream")
    with torch.cuda.stream(s):
        large.run(ws_large)
    torch.cuda.synchronize()
    large.check("eager after capture")

    for rep in range(3):
        announce(f"replay rep {rep}")
        small.reset()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g_small.replay()
        torch.cuda.synchronize()
        small.check(f"replay {rep}")
        # eager work between replays, on the same stream, sharing nothing
        large.reset()
        with torch.cuda.stream(s):
            large.run(ws_large)
        torch.cuda.synchronize()
        large.check(f"eager between replays {rep}")

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        announce(f"concurrent replays rep {rep}")
        small.reset()
        other.reset()
        torch.cuda.synchronize()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            g_small.replay()
        with torch.cuda.stream(s2):
            g_other.replay()
        torch.cuda.synchronize()
        small.check(f"concurrent replay {rep} (stream 1)")
        other.check(f"concurrent replay {rep} (stream 2)")
    del g_small, g_other
