"""The allocation-free argmax entry point (mk_argmax_noalloc) against the
plan-based mk_argmax, through the C ABI: two calls in a row on one GPU, the
second with a smaller batch and vocabulary (the fixed scratch array still
holds the first call's slice winners), with ties and NaN in the rows."""
import numpy as np
import pytest

import synth
from persistent_task_graph_amd import harness, mk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _logits(B, V, seed):
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((B, V), generator=g, device="cuda", dtype=torch.float32)
    x[0, V // 3] = 50.0  # a tie: the lower index wins
    x[0, V - 1] = 50.0
    if B > 1:
        x[1] = 0.25  # all equal: index 0
    if B > 2:
        x[2, 5] = float("nan")  # NaN is never chosen
        x[2, V // 2] = 40.0
    return x


def _plan(B, V):
    shape = synth.ModelShape(n_layers=1, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=256, vocab=V,
                             qk_norm=False)
    return harness.build_plan(shape, B, 16)


def test_noalloc_argmax_equals_plan_argmax_on_two_calls():
    import torch

    for B, V, seed in ((16, 151936, 1), (3, 1000, 2)):
        print("argmax_noalloc: batch %d, vocab %d" % (B, V), flush=True)
        lg = _logits(B, V, seed)
        plan = _plan(B, V)
        want = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        got = torch.full((B,), -2, dtype=torch.int32, device="cuda")
        plan.argmax(lg, want)
        mk.argmax_noalloc(lg, got, B, V)
        torch.cuda.synchronize()
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert np.array_equal(w, g), (w, g)
        host = lg.cpu().numpy()
        assert g[0] == V // 3 and (B < 2 or g[1] == 0) and (B < 3 or g[2] == V // 2)
        for b in range(3, B):
            assert g[b] == int(np.argmax(host[b]))
        plan.close()


def test_noalloc_argmax_rejects_sizes_beyond_its_scratch():
    import torch

    lg = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
    out = torch.zeros((1,), dtype=torch.int32, device="cuda")
    for B, V in ((0, 8), (257, 8), (1, 0)):
        with pytest.raises(mk.MKError, match="mk_argmax_noalloc"):
            mk.argmax_noalloc(lg, out, B, V)
