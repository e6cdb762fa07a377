"""The C-ABI library without a GPU: it loads, exports what include/moe.h
declares, and rejects invalid arguments on the host before enqueuing anything.

Every call below fails validation, so no HIP call is made."""
import ctypes

import pytest

import sparse_mixture_experts_wg_amd as moe
from sparse_mixture_experts_wg_amd import binding

lib = moe.lib
FAKE = 1 << 20  # aligned, never dereferenced (validation fails first)


def _p(**kw):
    base = dict(T=64, d=256, h=384, E=8, K=2, dtype="bf16", out_dtype="f32", path="auto")
    base.update(kw)
    return moe.problem(**base)


def test_exports_every_declared_function():
    names = moe.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    for required in ("moe_route", "moe_permute", "moe_expert_swiglu", "moe_combine", "moe_forward"):
        assert required in names


def test_status_strings():
    assert moe.status_string(0) == "MOE_OK"
    assert moe.status_string(5) == "MOE_ERR_WORKSPACE"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), binding.ERR_SHAPE),
    (dict(d=0), binding.ERR_SHAPE),
    (dict(E=2, K=3), binding.ERR_SHAPE),
    (dict(E=9), binding.ERR_UNSUPPORTED),
    (dict(E=8, K=3), binding.ERR_UNSUPPORTED),
    (dict(d=192), binding.ERR_UNSUPPORTED),
    (dict(h=200), binding.ERR_UNSUPPORTED),
    (dict(dtype="f32", path="stream"), binding.ERR_UNSUPPORTED),
    (dict(T=1 << 31), binding.ERR_UNSUPPORTED),
    # the streaming path takes at most 2^21 routed rows (row groups in the grid's z)
    (dict(T=1 << 20, path="stream"), binding.ERR_UNSUPPORTED),
    # 32-bit work-item counts of the combine grid: T * ceil(d / 1024) < 2^24
    (dict(T=1 << 24, d=128), binding.ERR_UNSUPPORTED),
    (dict(T=1 << 22, d=4096), binding.ERR_UNSUPPORTED),
    # the tiled grid: h / 128 column blocks x token blocks of 256
    (dict(T=1 << 23, d=128, h=1 << 17), binding.ERR_UNSUPPORTED),
])
def test_problem_validation(kw, code):
    p = _p(**kw)
    assert moe.resolve_path(p) == -code
    assert moe.forward_workspace_bytes(p) == 0
    st = lib.moe_route(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == code, moe.last_error()
    assert moe.last_error()


def test_grid_limits_accept_the_largest_fitting_batch():
    # the largest T whose combine grid fits: 2^24 - 1 workgroups of 256
    assert moe.resolve_path(_p(T=(1 << 24) - 1, d=128, h=128)) == binding.PATH_TILED
    assert moe.resolve_path(_p(T=(1 << 22) - 1, d=4096, h=128)) == binding.PATH_TILED
    assert moe.resolve_path(_p(T=1 << 20, d=4096, h=14336)) == binding.PATH_TILED


def test_bad_dtype_and_flags():
    p = _p()
    p.dtype = 7
    assert moe.resolve_path(p) == -binding.ERR_UNSUPPORTED
    p = _p()
    p.flags = 2  # unknown bit
    assert moe.resolve_path(p) == -binding.ERR_UNSUPPORTED
    p = _p()
    p.flags = binding.FLAG_DOWN_PARTIALS  # a known bit is accepted
    assert moe.resolve_path(p) == binding.PATH_STREAM
    p = _p()
    p.path = 5
    assert moe.resolve_path(p) == -binding.ERR_UNSUPPORTED
    # the gate-up through perm_token is bf16 only (checked before anything is enqueued)
    p = _p()
    p.dtype = binding.F32
    assert lib.moe_expert_gate_up_rows(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == binding.ERR_UNSUPPORTED
    assert b"bf16 only" in lib.moe_last_error()


def test_path_resolution():
    # the automatic switch point comes from a batch-size sweep on MI355X (bench.py --sweep)
    assert moe.resolve_path(_p(T=96)) == binding.PATH_STREAM
    assert moe.resolve_path(_p(T=97)) == binding.PATH_TILED
    assert moe.resolve_path(_p(T=96, d=4096)) == binding.PATH_STREAM
    # wider models switch earlier (the 8x22B shape, d = 6144)
    assert moe.resolve_path(_p(T=32, d=6144, h=16384)) == binding.PATH_STREAM
    assert moe.resolve_path(_p(T=33, d=6144, h=16384)) == binding.PATH_TILED
    assert moe.resolve_path(_p(T=4096, path="stream")) == binding.PATH_STREAM
    assert moe.resolve_path(_p(T=8, path="tiled")) == binding.PATH_TILED
    assert moe.resolve_path(_p(dtype="f32")) == binding.PATH_TILED


def test_capacity_field():
    assert moe.resolve_path(_p(capacity=5)) == binding.PATH_STREAM
    assert moe.resolve_path(_p(capacity=-1)) == -binding.ERR_SHAPE
    p = _p()
    p.reserved = 3
    assert moe.resolve_path(p) == -binding.ERR_UNSUPPORTED
    assert moe.capacity_rows(4096, 2, 8, 1.0) == 1024
    assert moe.capacity_rows(100, 2, 8, 1.25) == 32  # ceil(31.25)
    assert ctypes.sizeof(binding.Problem) == 56


def test_capacity_rows_exact():
    """C = ceil(cf * T * K / E) in exact arithmetic: a float product lands just above
    the integer for 1.1 x 400 x 2 / 8 = 110 (and 1.1 x 200 x 2 / 8 = 55) and would
    keep one row too many."""
    assert moe.capacity_rows(200, 2, 8, 1.1) == 55
    assert moe.capacity_rows(400, 2, 8, 1.1) == 110
    assert moe.capacity_rows(400, 2, 8, (11, 10)) == 110
    assert moe.capacity_rows(401, 2, 8, (11, 10)) == 111  # 110.275 rounds up
    assert moe.capacity_rows(7, 1, 3, 1.0) == 3           # ceil(7 / 3)
    assert moe.capacity_rows(4096, 2, 8, 0.0) == 0
    # every case with K = 2, E = 8 and T < 5000 against exact rational arithmetic
    from fractions import Fraction
    for cf in ("0.5", "0.9", "1.0", "1.1", "1.2", "1.25", "1.3", "1.5", "2.0", "3.3"):
        q = Fraction(cf)
        for T in range(1, 5000, 7):
            want = -(-(q.numerator * T * 2) // (q.denominator * 8))
            assert moe.capacity_rows(T, 2, 8, float(cf)) == want, (cf, T)
    for args in ((0, 2, 8, 1, 1), (10, 0, 8, 1, 1), (10, 3, 2, 1, 1), (10, 2, 8, -1, 1),
                 (10, 2, 8, 1, 0)):
        assert lib.moe_capacity_rows(*args) == -binding.ERR_SHAPE, args
    assert lib.moe_capacity_rows(1 << 26, 2, 2, 1 << 20, 1) == -binding.ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError):
        moe.capacity_rows(0, 2, 8, 1.0)


def test_down_parts():
    """Partial sums only when asked for, on the tiled bf16 path: 4 parts when they all fit
    one round of workgroups, 1 from 8 rounds on, else 2; a part needs an even count of
    64-wide k-blocks."""
    P = binding.FLAG_DOWN_PARTIALS
    assert moe.down_parts(_p(T=4096, d=4096, h=14336)) == 1
    assert moe.down_parts(_p(T=4096, d=4096, h=14336, flags=P)) == 2   # 640 tiles: 3 rounds
    assert moe.down_parts(_p(T=16384, d=4096, h=14336, flags=P)) == 1  # 2176 tiles: 9 rounds
    assert moe.down_parts(_p(T=2048, d=4096, h=14336, flags=P)) == 2
    assert moe.down_parts(_p(T=8192, d=6144, h=16384, flags=P)) == 2   # 1728 tiles: 7 rounds
    assert moe.down_parts(_p(T=1024, d=1024, h=14336, flags=P)) == 4   # 32 tiles
    assert moe.down_parts(_p(T=4096, d=4096, h=14336 + 128, flags=P)) == 1  # 226 k-blocks
    assert moe.down_parts(_p(T=32, d=4096, h=14336, flags=P)) == 1      # streaming path
    # 64-token tiles: two workgroups per compute unit, 4 x 128 tiles fit one round
    assert moe.down_parts(_p(T=32, d=4096, h=14336, flags=P, path="tiled")) == 4
    assert moe.down_parts(_p(T=64, d=128, h=256, dtype="f32", flags=P)) == 1
    # the layer's own workspace makes room for the partial sums it uses
    S, d, h = 4096 * 2, 4096, 14336
    acts = S * h * 2  # act, bf16 (no x_perm: the bf16 gate-up reads x through perm_token)
    assert moe.forward_workspace_bytes(_p(T=4096, d=d, h=h)) >= acts + 2 * S * d * 4
    with pytest.raises(moe.MoeError):
        moe.down_parts(_p(T=0))


def test_block_entry_points_validate():
    p = _p()
    eps = ctypes.c_float(1e-5)
    # eps must be finite and > 0; nothing is enqueued on failure
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        st = lib.moe_rmsnorm(ctypes.byref(p), FAKE, FAKE, ctypes.c_float(bad), FAKE, None)
        assert st == binding.ERR_UNSUPPORTED, bad
    assert lib.moe_rmsnorm(ctypes.byref(p), None, FAKE, eps, FAKE, None) == binding.ERR_NULL
    assert "h" in moe.last_error()
    assert lib.moe_combine_residual(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE,
                                    None) == binding.ERR_NULL
    assert "residual" in moe.last_error()
    need = moe.block_workspace_bytes(p)
    assert need >= moe.forward_workspace_bytes(p) + 64 * 256 * 2
    st = lib.moe_block_forward(ctypes.byref(p), FAKE, FAKE, eps, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None, FAKE, need - 1, None)
    assert st == binding.ERR_WORKSPACE
    st = lib.moe_block_forward(ctypes.byref(p), FAKE, None, eps, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None, FAKE, need, None)
    assert st == binding.ERR_NULL and "norm_w" in moe.last_error()


def test_null_and_alignment():
    p = _p()
    assert lib.moe_route(ctypes.byref(p), None, FAKE, FAKE, FAKE, None, None) == binding.ERR_NULL
    assert "x" in moe.last_error()
    assert lib.moe_route(None, FAKE, FAKE, FAKE, FAKE, None, None) == binding.ERR_NULL
    assert lib.moe_route(ctypes.byref(p), FAKE + 8, FAKE, FAKE, FAKE, None, None) == binding.ERR_ALIGN
    assert lib.moe_combine(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE + 4, None) == binding.ERR_ALIGN
    assert lib.moe_permute(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == binding.ERR_NULL
    assert lib.moe_expert_gate_up(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, None) == binding.ERR_NULL
    assert lib.moe_expert_gate_up_rows(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                       None) == binding.ERR_NULL
    # the index-only permute still needs its index arrays
    assert lib.moe_permute(ctypes.byref(p), None, FAKE, None, FAKE, FAKE, None, None) == binding.ERR_NULL
    assert lib.moe_expert_down(ctypes.byref(p), FAKE, FAKE, None, FAKE, None) == binding.ERR_NULL


def test_workspace_sizes_and_too_small():
    p = _p(T=100, d=256, h=512, E=8, K=2)
    S = 200
    need = moe.forward_workspace_bytes(p)

    def a256(n):
        return (n + 255) // 256 * 256
    # bf16: act (bf16) + o_perm (f32, with the partial sums the layer lets the down
    # projection leave) + 4 int/float index arrays + offsets, each piece 256-B aligned;
    # no x_perm (the gate-up reads the token rows through perm_token)
    parts = moe.down_parts(_p(T=100, d=256, h=512, flags=binding.FLAG_DOWN_PARTIALS))
    assert parts == 4
    assert need == (4 * a256(S * 4) + a256(9 * 4) + a256(S * 512 * 2) +
                    a256(parts * S * 256 * 4))
    # float32 gathers x_perm [S, d] as well (and never splits the down projection)
    f32p = _p(T=100, d=256, h=512, E=8, K=2, dtype="f32")
    assert moe.forward_workspace_bytes(f32p) == (4 * a256(S * 4) + a256(9 * 4) +
                                                 a256(S * 256 * 4) + a256(S * 512 * 4) +
                                                 a256(S * 256 * 4))
    assert need % 256 == 0
    assert moe.expert_workspace_bytes(p) == S * 512 * 2
    st = lib.moe_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                         need - 1, None)
    assert st == binding.ERR_WORKSPACE, moe.last_error()
    st = lib.moe_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                         FAKE + 16, need, None)
    assert st == binding.ERR_ALIGN  # ws must be 256-byte aligned
    st = lib.moe_expert_swiglu(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               moe.expert_workspace_bytes(p) - 1, None)
    assert st == binding.ERR_WORKSPACE
    f32 = _p(T=100, d=256, h=512, dtype="f32")
    assert moe.expert_workspace_bytes(f32) == S * 512 * 4


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    p = _p(T=4, d=128, h=128)
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.route(p, x, torch.zeros((128, 8), dtype=torch.bfloat16),
                  topk_idx=x, topk_w=x)
