"""The entry points allocate nothing and never synchronise, so a caller can
capture them into a HIP graph.  Each case captures one call, replays the
graph several times with the program's own eager work and synchronisations
between the replays, and checks every replay bit for bit against the eager
call on the same buffers.
"""
import pytest
import torch

import hyena_long_conv_amd as H
from tests.gpu_helpers import DEV, params_to_device
from tests.test_block import _bp_device
from workloads import (Config, GridConfig, make_activations, make_block_input, make_block_params,
                       make_filter_params, make_grid_activations, make_grid_kernel)

pytestmark = pytest.mark.gpu


def _replays_match(call, out, eager_ref):
    """Capture call() into a graph, then replay it three times; out must equal
    eager_ref after each replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                     # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        out.fill_(float("nan"))                    # eager work between replays
        scratch = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(out, eager_ref), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("N,B,D,L,io", [
    (2, 2, 8, 2048, "fp32"),      # single pass
    (3, 2, 3, 20000, "fp32"),     # four-step, channel-major pass groups
    (2, 1, 2, 65536, "bf16"),     # four-step, bf16 I/O
])
def test_forward_graph_replays(N, B, D, L, io):
    cfg = Config("g", N, B, D, L, io, 32, 17)
    h = H.filter_gen(params_to_device(make_filter_params(cfg)), L)
    spec = H.filter_spectrum(h)
    v, xs = make_activations(cfg, DEV)
    y = H._empty_like(v)
    ws = H._empty(max(1, H.forward_workspace_bytes(B, D, N, L, io)), dtype=torch.uint8, device=DEV)
    H.forward(v, xs, spec, out=y, workspace=ws)
    torch.cuda.synchronize()
    ref = y.clone()
    _replays_match(lambda: H.forward(v, xs, spec, out=y, workspace=ws), y, ref)


def test_nd_forward_graph_replays():
    cfg = GridConfig("g", 2, 2, 2, (150, 150), False, "fp32", 19)     # multi-pass 2-D grid
    v, xs = make_grid_activations(cfg, DEV)
    K = torch.from_numpy(make_grid_kernel(cfg)).to(DEV)
    spec = H.nd_filter_spectrum(K, cfg.dims)
    y = H._empty_like(v)
    ws = H._empty(H.nd_workspace_bytes(cfg.B * cfg.D, cfg.dims), dtype=torch.uint8, device=DEV)
    H.nd_forward(v, xs, spec, out=y, workspace=ws)
    torch.cuda.synchronize()
    ref = y.clone()
    _replays_match(lambda: H.nd_forward(v, xs, spec, out=y, workspace=ws), y, ref)


def test_block_forward_graph_replays():
    cfg = Config("g", 2, 2, 64, 3000, "bf16", 32, 23)
    bpd = _bp_device(make_block_params(cfg), cfg.io)
    u = make_block_input(cfg, DEV)
    spec = H.filter_spectrum(H.filter_gen(params_to_device(make_filter_params(cfg)), cfg.L))
    out = H._empty_like(u)
    ws = H._empty(H.block_workspace_bytes(cfg.B, cfg.D, cfg.N, cfg.L, cfg.io), dtype=torch.uint8, device=DEV)
    H.block_forward(u, bpd, spec, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = out.clone()
    _replays_match(lambda: H.block_forward(u, bpd, spec, out=out, workspace=ws), out, ref)
