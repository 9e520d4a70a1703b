"""The allocation-free MoE entry point (qgemv_moe_noalloc) through the C ABI:
the same bits as qgemv_moe with a workspace, on two calls in a row (the
second smaller), and within the oracle's bound; oversize calls rejected."""
import numpy as np
import pytest

from gpu_helpers import check_tol, dev, moe_case
from oracle import gemv as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_weight_amd as qg
    qg.load()
    yield


def qg():
    import bit_quantized_weight_amd as m
    return m


@pytest.mark.parametrize("fmt", ["int4", "nvfp4"])
def test_moe_noalloc_equals_workspace_entry_point(fmt):
    # two calls in a row on the same static scratch, the second with fewer
    # tokens, fewer experts and smaller H / I
    for (E, H, I, N, k, seed) in [(24, 1024, 256, 8, 8, 1), (6, 256, 64, 2, 3, 2)]:
        print("noalloc", fmt, E, H, I, N, k, flush=True)
        bufs, Wgu, Wdn, xb, ids, gates, r = moe_case(fmt, E, H, I, N, k, seed=seed)
        d = [dev(b, torch) for b in bufs]
        args = (E, H, I, dev(xb, torch), dev(ids, torch), dev(gates, torch), k)
        nbytes = qg().moe_workspace_bytes(E, H, I, N, k)
        assert nbytes <= qg().moe_noalloc_max_bytes()
        wsp = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        y_ws = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
        y_na = torch.full((N, H), float("nan"), dtype=torch.float32, device="cuda")
        rd = dev(r, torch)
        qg().qgemv_moe(fmt, *d, *args, y_ws, N, wsp, nbytes, residual=rd)
        qg().qgemv_moe_noalloc(fmt, *d, *args, y_na, N, residual=rd)
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        y_ref, T = G.moe(G.x_from_bits(xb), ids, gates, Wgu, Wdn, r)
        check_tol(b, y_ref, T, f"noalloc {fmt} N={N}")


def test_moe_noalloc_rejects_oversize():
    big_H = 1 << 16
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(qg().QgemvError) as e:
        qg().qgemv_moe_noalloc("int4", t, t, t, t, 4, big_H, 4096, t, t, t, 8, t, 8)
    assert e.value.status == -5      # QGEMV_EWORKSPACE
