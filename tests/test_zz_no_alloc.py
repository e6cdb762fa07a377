"""moe_forward_noalloc, the whole layer with the library's static scratch array as
its workspace, for callers that cannot allocate device memory: through the C ABI
against moe_forward (the same kernels with a caller-given workspace) on the same
inputs, bit for bit, over two calls in a row whose second is smaller (the array
keeps the first call's contents), and against the CPU oracle's bar."""
import ctypes

import numpy as np
import pytest

import moe_inputs as mi
from tests import parity

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    import sparse_mixture_experts_wg_amd as m

    return m


def test_noalloc_rejects_problems_beyond_the_scratch_array(moe):
    """Host-side check, before anything touches a GPU: the 8x7B prefill batch needs
    far more workspace than the 64 MiB array."""
    from sparse_mixture_experts_wg_amd import binding

    p = moe.problem(4096, 4096, 14336, 8, 2, "bf16", "f32")
    assert moe.forward_workspace_bytes(p) > moe.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    st = moe.lib.moe_forward_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None,
                                     None, None)
    assert st == binding.ERR_WORKSPACE
    assert "scratch" in moe.last_error()
    bad = moe.problem(0, 4096, 14336)
    st = moe.lib.moe_forward_noalloc(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None,
                                     None, None)
    assert st == binding.ERR_SHAPE


def _both(moe, p, dev, T, d):
    K = int(p.K)
    outs = []
    for fn in (moe.forward, moe.forward_noalloc):
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        y = fn(p, dev["x"], dev["w_g"], dev["w1"], dev["w3"], dev["w2"], topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        outs.append((parity.host_array(y), parity.host_array(idx), parity.host_array(w)))
    return outs


CASES = [
    # (name, config of the first call, T of the second, smaller call)
    ("tiled_then_stream", mi.Config("na1", T=600, d=256, h=512, wg_std="fan_in_d"), 24),
    ("decode_8x7b_shape", mi.Config("na2", T=32, d=4096, h=14336, x_kind="rmsnorm", wg_std=0.02), 5),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,cfg,T2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_forward(moe, oracle, name, cfg, T2):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"noalloc {name}: T={cfg.T} then T={T2}, d={cfg.d} h={cfg.h}", flush=True)
    inp = mi.make_inputs(cfg, seed=7)
    for T in (cfg.T, T2):
        p = moe.problem(T, cfg.d, cfg.h, cfg.E, cfg.K, cfg.dtype, "f32")
        assert moe.forward_workspace_bytes(p) <= moe.NOALLOC_SCRATCH_BYTES
        sub = dict(inp, x=np.ascontiguousarray(inp["x"][:T]))
        dev = parity.upload_inputs(sub, cfg.dtype)
        (y0, i0, w0), (y1, i1, w1) = _both(moe, p, dev, T, cfg.d)
        assert np.array_equal(i1, i0) and np.array_equal(w1, w0), f"T={T}: routing differs"
        assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32)), f"T={T}: y differs"
        # and the layer's own bar against the oracle (rule R, max|err| <= tol * RMS)
        toks = np.arange(T) if T <= 64 else parity.sample_tokens(T, 64, seed=0)
        l, idx_r, w_r, margin = oracle.route(sub["x"], sub["w_g"], cfg.K, cfg.dtype)
        idx_eval, _ = parity.check_routing(i1, w1, l, idx_r, margin, cfg.K, oracle)
        y_ref = oracle.forward_tokens(toks, sub["x"], sub["w1"], sub["w3"], sub["w2"], idx_eval,
                                      oracle.set_weights(l, idx_eval), cfg.dtype)
        rel = parity.check_output(y1[toks].astype(np.float64), y_ref, cfg.dtype, f"noalloc T={T}")
        print(f"  T={T}: bitwise equal to moe_forward, max|err|/RMS = {rel:.3e}", flush=True)
