"""The Lloyd step captured in a HIP graph (through torch.cuda.graph) and
replayed: nothing in it allocates, waits on the host or clears memory with a
memset, so the captured kernels replay on the same buffers. Every replay,
with eager work between replays that overwrites the outputs, must give the
eager step's bits."""
import numpy as np
import pytest

from nearest_centroid_assignment_amd import binding, datagen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SHAPES = [
    ("probe", None),                       # 64 x 64 tiles, fused counting launch
    ("blobs", (2048, 512, 256)),           # full 256 x 256 tiles (DMA kernel)
    ("blobs", (3000, 1500, 96)),           # k > 1024: the four counting launches
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name,shape", SHAPES, ids=["probe", "2048x512x256", "3000x1500x96"])
def test_lloyd_step_graph_replays(name, shape, noalloc):
    import torch

    gu.announce(f"graph replay {name} {shape} noalloc={noalloc}")
    if shape is None:
        X, C = datagen.make(name)
    else:
        n, k, d = shape
        X, C = datagen.make_blobs(n, k, d, kb=k, sigma_c=1.0, sigma=0.5, seed=11)
    n, d = X.shape
    k = C.shape[0]
    dev = torch.device("cuda:0")
    Xg, Cg = gu.to_gpu(X), gu.to_gpu(C)
    labels = torch.empty(n, dtype=torch.int64, device=dev)
    md = torch.empty(n, dtype=torch.float32, device=dev)
    C_new = torch.empty((k, d), dtype=torch.float32, device=dev)
    counts = torch.empty(k, dtype=torch.int64, device=dev)
    ws = torch.empty(binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_LLOYD),
                     dtype=torch.uint8, device=dev)

    def step():
        if noalloc:
            binding.kmeans_lloyd_step_noalloc(Xg, Cg, labels, md, C_new, counts)
        else:
            binding.kmeans_lloyd_step(Xg, Cg, labels, md, C_new, counts, workspace=ws)

    step()  # eager: the reference (and the library's one-time device set-up)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (labels, md, C_new, counts)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        # Eager work between replays: overwrite every output.
        labels.fill_(-3)
        md.fill_(-3.0)
        C_new.fill_(float("nan"))
        counts.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm, a, b in zip(("labels", "min_dist", "C_new", "counts"), ref,
                            (labels, md, C_new, counts)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {nm} differs"
    gu.announce(f"graph replay {name}: 3 replays equal the eager step")
