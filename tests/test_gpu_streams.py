"""Streams and graph capture: the entry points enqueue kernels only (no
memset, copy or host wait), so they run on any stream and can be captured
into a HIP graph and replayed. Every replay is checked against the eager
result, with eager work and synchronisations between the replays."""
import numpy as np
import pytest

from nearest_centroid_assignment_amd import datagen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(n, k, d):
    import torch

    dev = "cuda:0"
    return (torch.empty(n, dtype=torch.int64, device=dev),
            torch.empty(n, dtype=torch.float32, device=dev),
            torch.empty(k, d, dtype=torch.float32, device=dev),
            torch.empty(k, dtype=torch.int64, device=dev))


def _same(a, b):
    import torch

    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def test_side_stream_matches_default_stream():
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce("lloyd step on a side stream")
    X, C = datagen.make("probe")
    Xg, Cg = gu.to_gpu(X), gu.to_gpu(C)
    n, d = X.shape
    k = C.shape[0]
    ref = _outputs(n, k, d)
    binding.kmeans_lloyd_step(Xg, Cg, *ref)
    torch.cuda.synchronize()
    out = _outputs(n, k, d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.kmeans_lloyd_step(Xg, Cg, *out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(ref, out):
        assert _same(a, b)


GRAPH_SHAPES = [
    ("probe", None),                       # 64 x 64 tiles, the one-launch counting path
    ("blobs", (2048, 512, 256)),           # full 256 x 256 tiles (the DMA kernel)
    ("blobs", (3000, 1500, 96)),           # k > 1024: the four-launch counting path
    ("blobs", (3000, 20, 64)),             # the small-k kernel (keys stored, no identity fill)
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name,shape", GRAPH_SHAPES,
                         ids=["probe", "2048x512x256", "3000x1500x96", "3000x20x64"])
def test_lloyd_step_graph_replays(name, shape, noalloc):
    """kmeans_lloyd_step (with a workspace) or kmeans_lloyd_step_noalloc (the
    static scratch) captured once; four replays alternate two centre sets,
    with the outputs (and the workspace) overwritten eagerly between them, and
    each must equal the eager step on its centres bit for bit."""
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce(f"lloyd step captured in a graph: {name} {shape} noalloc={noalloc}")
    if shape is None:
        X, C = datagen.make(name)
    else:
        X, C = datagen.make_blobs(*shape, kb=shape[1], sigma_c=1.0, sigma=0.5, seed=11)
    n, d = X.shape
    k = C.shape[0]
    Xg, Cg = gu.to_gpu(X), gu.to_gpu(C)
    C2 = gu.to_gpu(X[np.random.default_rng(7).choice(n, k, replace=False)])
    out = _outputs(n, k, d)
    ws = torch.empty(binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_LLOYD),
                     dtype=torch.uint8, device="cuda:0")

    def step(Cin, outs):
        if noalloc:
            binding.kmeans_lloyd_step_noalloc(Xg, Cin, *outs)
        else:
            binding.kmeans_lloyd_step(Xg, Cin, *outs, workspace=ws)

    # Eager references for both centre sets (a separate workspace each call).
    refs = []
    for Cin in (Cg, C2):
        r = _outputs(n, k, d)
        binding.kmeans_lloyd_step(Xg, Cin.clone(), *r)
        refs.append(r)
    torch.cuda.synchronize()

    Cin = Cg.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up (and one-time set-up) outside the capture
        step(Cin, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(Cin, out)
    torch.cuda.synchronize()

    for replay in range(4):
        which = replay % 2
        # Eager work between replays: clobber the outputs and the workspace,
        # and load the centres this replay must use.
        for t in out:
            t.fill_(-7)
        ws.fill_(0xA5)
        Cin.copy_(Cg if which == 0 else C2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(refs[which], out):
            assert _same(a, b), f"replay {replay}"
