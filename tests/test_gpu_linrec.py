"""Parity of the linear-recurrence pair scan (HIP, through the C ABI) with the
oracle: h[t] = a[t] h[t-1] + b[t] computed by scanning the pairs (a, b)
("Parallel Prefix Sum (Scan), in depth", section "What scan builds").  fp32
results within 1e-5 of the magnitude scan (the same scan over |a|, |b|) of
the fp64 oracle; exact where the arithmetic is exact."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import LINREC_TILE, assert_linrec_close, dev, host, require_gpu, say, ws_error_word
from pins import golden

pytestmark = pytest.mark.gpu

WT = LINREC_TILE


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


@pytest.fixture(autouse=True, scope="module")
def _single_pass_only(dw):
    """Every call of this module runs the single-pass chained form, whatever
    its size (the two-level form has its own tests)."""
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    yield
    dw.ps_small_n_config(old)


def _nan(n):
    import torch
    return torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")


def _run(dw, a, b, inclusive, with_a=True, workspace=None):
    da, db = dev(a), dev(b)
    ob = _nan(a.size)
    oa = _nan(a.size) if with_a else None
    tot = _nan(2)
    dw.ps_scan_linrec_f32(da, db, ob, out_a=oa, inclusive=inclusive, total=tot, workspace=workspace)
    return (host(oa) if with_a else None), host(ob), host(tot)


def _oracle(orc, a, b, inclusive):
    return orc.scan_linrec_f32(np.stack([a, b], axis=1), inclusive)


def _check_total(orc, a, b, tot):
    """The total is the fold of all pairs: the last inclusive pair."""
    if a.size == 0:
        assert tot.tolist() == [1.0, 0.0]
        return
    A, B, SA, SB, _ = _oracle(orc, a, b, True)
    assert_linrec_close(tot[:1], tot[1:], A[-1:], B[-1:], SA[-1:], SB[-1:], False, first=a.size - 1)


def _check(dw, orc, a, b, inclusive, with_a=True):
    ga, gb, gt = _run(dw, a, b, inclusive, with_a)
    A, B, SA, SB, _ = _oracle(orc, a, b, inclusive)
    worst = assert_linrec_close(ga, gb, A, B, SA, SB, not inclusive)
    _check_total(orc, a, b, gt)
    return worst


def test_tile_shape(dw):
    assert dw.ps_linrec_tile_elements() == WT


def test_page_example(dw, orc):
    g = golden("p2_recurrence_example.json")
    a = np.array(g["a"], np.float32)
    b = np.array(g["b"], np.float32)
    say("linrec page example")
    ga, gb, gt = _run(dw, a, b, True)
    # the page's decimals, up to the float32 rounding of 0.9 and 0.1
    assert np.allclose(gb, g["h"], rtol=1e-6, atol=0), gb
    assert gt[1] == gb[-1] and gt[0] == ga[-1]
    _check(dw, orc, a, b, True)
    _check(dw, orc, a, b, False)


EDGE = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, WT - 1, WT, WT + 1, 2 * WT - 1, 2 * WT,
        2 * WT + 1, 3 * WT + 7, 257 * WT, 513 * WT + 1, 1_000_003]


@pytest.mark.parametrize("n", EDGE)
@pytest.mark.parametrize("inclusive", [False, True])
def test_edge_sizes(dw, orc, n, inclusive):
    a, b = wl.linrec_pairs(n, seed=n + 21)
    say("linrec edge", n, inclusive)
    _check(dw, orc, a, b, inclusive)


@pytest.mark.parametrize("n", [WT + 3, 40 * WT + 777, 1 << 21])
@pytest.mark.parametrize("inclusive", [False, True])
def test_signed_multipliers(dw, orc, n, inclusive):
    """Multipliers of both signs and above 1 in magnitude: every grouping
    must compose the maps in index order (the operator is not commutative)."""
    a, b = wl.linrec_pairs(n, seed=n + 22, a_lo=-1.5, a_hi=1.5)
    say("linrec signed", n, inclusive)
    _check(dw, orc, a, b, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_b_plane_only(dw, orc, inclusive):
    """out_a = NULL: only B is written."""
    n = 100 * WT + 9
    a, b = wl.linrec_pairs(n, seed=23)
    say("linrec B only", inclusive)
    _check(dw, orc, a, b, inclusive, with_a=False)


def test_unit_multipliers_are_the_sum_scan(dw, orc):
    """a = 1: B is the fp32 sum scan of b and A stays exactly 1."""
    n = 300 * WT + 5
    b = wl.normal_f32(n, seed=24)
    a = np.ones(n, np.float32)
    say("linrec a = 1")
    ga, gb, _ = _run(dw, a, b, True)
    assert np.all(ga == 1.0)
    ref, absprefix, _ = orc.scan_f32_sum(b, inclusive=True)
    err = np.abs(gb.astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * absprefix)
    _check(dw, orc, a, b, False)


def test_zero_inputs_keep_zero_state(dw, orc):
    """b = 0: h stays exactly 0 whatever the decays; A is the running product."""
    n = 50 * WT + 1
    a, _ = wl.linrec_pairs(n, seed=25, a_lo=0.5, a_hi=1.0)
    b = np.zeros(n, np.float32)
    say("linrec b = 0")
    for inclusive in (False, True):
        ga, gb, _ = _run(dw, a, b, inclusive)
        assert np.all(gb == 0.0), inclusive
        _check(dw, orc, a, b, inclusive)


def test_zero_multipliers_forget(dw, orc):
    """a = 0: the state forgets at every step, so h[t] = b[t] exactly."""
    n = 20 * WT + 33
    b = wl.normal_f32(n, seed=26)
    a = np.zeros(n, np.float32)
    say("linrec a = 0")
    ga, gb, _ = _run(dw, a, b, True)
    assert np.array_equal(gb, b) and np.all(ga == 0.0)
    ga, gb, _ = _run(dw, a, b, False)
    assert gb[0] == 0.0 and ga[0] == 1.0
    assert np.array_equal(gb[1:], b[:-1]) and np.all(ga[1:] == 0.0)


def test_empty_writes_total(dw):
    import torch
    tot = _nan(2)
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    dw.ps_scan_linrec_f32(e, e, e.clone(), total=tot)
    assert host(tot).tolist() == [1.0, 0.0]


@pytest.mark.parametrize("inclusive", [False, True])
def test_unaligned_buffers(dw, orc, inclusive):
    """Every plane one float past a 16-byte boundary: the per-element path."""
    import torch
    n = 7 * WT + 13
    a, b = wl.linrec_pairs(n, seed=27)
    va = dev(np.concatenate(([0], a)).astype(np.float32))[1:]
    vb = dev(np.concatenate(([0], b)).astype(np.float32))[1:]
    oa = torch.full((n + 1,), float("nan"), dtype=torch.float32, device="cuda")[1:]
    ob = torch.full((n + 1,), float("nan"), dtype=torch.float32, device="cuda")[1:]
    assert all(t.data_ptr() % 16 != 0 for t in (va, vb, oa, ob))
    say("linrec unaligned", inclusive)
    dw.ps_scan_linrec_f32(va, vb, ob, out_a=oa, inclusive=inclusive)
    A, B, SA, SB, _ = _oracle(orc, a, b, inclusive)
    assert_linrec_close(host(oa), host(ob), A, B, SA, SB, not inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_in_place(dw, orc, inclusive):
    """out_a = a and out_b = b: each plane overwritten by its own scan."""
    n = 600 * WT + 17
    a, b = wl.linrec_pairs(n, seed=28)
    da, db = dev(a), dev(b)
    say("linrec in place", inclusive)
    dw.ps_scan_linrec_f32(da, db, db, out_a=da, inclusive=inclusive)
    A, B, SA, SB, _ = _oracle(orc, a, b, inclusive)
    assert_linrec_close(host(da), host(db), A, B, SA, SB, not inclusive)


def test_repeated_runs_reuse_workspace(dw, orc):
    import torch
    n = 1 << 24
    a, b = wl.linrec_pairs(n, seed=29)
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_linrec_f32", None, None, None, None, n, 1, None, None))
    A, B, SA, SB, _ = _oracle(orc, a, b, True)
    for it in range(5):
        say("linrec repeat", it)
        ga, gb, _ = _run(dw, a, b, True, workspace=ws)
        assert_linrec_close(ga, gb, A, B, SA, SB, False)
        assert ws_error_word(ws) == 0


def test_fallback_every_stall(dw, orc):
    """A fallback after every stalled poll reduces pairs from the input in
    tile order and installs both descriptor words; PARTIALs after every
    window."""
    import torch
    n = (1 << 24) + 5
    a, b = wl.linrec_pairs(n, seed=30, a_lo=-1.0, a_hi=1.0)
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_linrec_f32", None, None, None, None, n, 0, None, None))
    old = dw.ps_lookback_config_get()
    dw.ps_lookback_config(1, 1)
    try:
        for inclusive in (False, True):
            A, B, SA, SB, _ = _oracle(orc, a, b, inclusive)
            say("linrec fallback", inclusive)
            ga, gb, _ = _run(dw, a, b, inclusive, workspace=ws)
            assert_linrec_close(ga, gb, A, B, SA, SB, not inclusive)
            assert ws_error_word(ws) == 0
    finally:
        dw.ps_lookback_config(*old)


@pytest.mark.parametrize("inclusive", [True, False])
def test_large_config(dw, orc, inclusive):
    """2^27 pairs, decays in [0.9, 1), inputs N(0, 1): every element checked."""
    a, b = wl.linrec_pairs()
    say("linrec config 2^27", inclusive)
    worst = _check(dw, orc, a, b, inclusive)
    say("linrec config 2^27 worst error / tolerance", worst)


@pytest.mark.parametrize("inclusive", [False, True])
def test_decays_near_one_check_a_everywhere(dw, orc, inclusive):
    """Decays in [1 - 2^-22, 1) over 2^22 pairs: the running product A stays
    above 0.3 at every index, so the A plane is held to its rounding bound
    everywhere, never to the absolute floor."""
    n = 1 << 22
    a, b = wl.linrec_pairs(n, seed=26, a_lo=1.0 - 2.0 ** -22, a_hi=1.0)
    A, _, SA, _, _ = _oracle(orc, a, b, True)
    assert A[-1] > 0.3 and np.all(1e-5 * SA > 1e6 * 2.0 ** -100)
    say("linrec decays near one", inclusive)
    _check(dw, orc, a, b, inclusive)


def _power_of_two_decays(n, seed):
    """a[t] = 2^e[t] with e in {-1, 0, +1}, the running exponent kept within
    [-40, 40]: every product of consecutive factors is an exact power of two
    inside the fp32 range, whatever the grouping."""
    g = wl.rng(seed)
    step = g.choice(np.array([-1, 0, 1]), size=n, p=[0.1, 0.8, 0.1])
    e = np.empty(n, np.int64)
    s = 0
    for i in range(n):  # a bounded walk: steps that would leave [-40, 40] turn round
        d = int(step[i])
        if abs(s + d) > 40:
            d = -d
        e[i] = d
        s += d
    return np.ldexp(np.float32(1.0), e).astype(np.float32)


@pytest.mark.parametrize("inclusive", [False, True])
def test_power_of_two_decays_a_exact(dw, orc, inclusive):
    """Decays that are powers of two: A is exact in fp32 at every one of 2^22
    indices in any grouping, so it must equal the oracle bit for bit -- a
    dropped or doubled factor in any cross-tile carry x.a * y.a shows."""
    n = 1 << 22
    a = _power_of_two_decays(n, seed=28)
    b = wl.normal_f32(n, seed=29)
    ga, gb, _ = _run(dw, a, b, inclusive)
    A, B, SA, SB, _ = _oracle(orc, a, b, inclusive)
    say("linrec power-of-two decays", inclusive)
    assert np.all((np.abs(A) >= 2.0 ** -40) & (np.abs(A) <= 2.0 ** 40))
    assert np.array_equal(ga.astype(np.float64), A)
    assert_linrec_close(ga, gb, A, B, SA, SB, not inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_sign_multipliers_exact(dw, orc, inclusive):
    """a = +-1 and small integer b: every product and every partial sum is an
    exact fp32 integer in any grouping, so A (= +-1) and B must equal the
    oracle bit for bit at every index -- a wrong sign anywhere in a
    cross-tile carry shows."""
    n = 200 * WT + 33
    g = wl.rng(27)
    a = np.where(g.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    b = g.integers(-4, 5, size=n).astype(np.float32)
    ga, gb, _ = _run(dw, a, b, inclusive)
    A, B, _, _, _ = _oracle(orc, a, b, inclusive)
    say("linrec sign multipliers", inclusive)
    assert np.array_equal(ga.astype(np.float64), A)
    assert np.array_equal(gb.astype(np.float64), B)
    assert np.all(np.abs(A) == 1.0)
