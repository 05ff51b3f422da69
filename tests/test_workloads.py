"""The seeded input generators: determinism, encodings, shapes and the
load structure the workloads are meant to have."""
import numpy as np
import pytest

import moe_workloads as W
from oracle import moe_oracle as O


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.0e-3], np.float32)
    got = W.bf16_to_f32(W.bf16_bits(vals))
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2 ** -6 and got[3] == -2.5
    assert got[4] == 1.0
    assert abs(got[5] - 3.0e-3) <= 3.0e-3 * 2 ** -8
    # every bf16 value survives a round trip exactly
    allbits = np.arange(0, 0x7F80, dtype=np.uint16)
    assert (W.bf16_bits(W.bf16_to_f32(allbits)) == allbits).all()


def test_determinism_and_independence():
    wl = W.get("c4s")
    assert (W.gen_x(wl) == W.gen_x(wl)).all()
    a = W.gen_expert(wl, 3)
    b = W.gen_expert(wl, 3)
    c = W.gen_expert(wl, 4)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
    assert not (a[0] == c[0]).all()
    gu, dn = W.gen_all_experts(wl, threads=3)
    assert (gu[3] == a[0]).all() and (dn[4] == c[1]).all()
    assert gu.shape == (wl.E, 2 * wl.f, wl.d) and dn.shape == (wl.E, wl.d, wl.f)


def test_distributions():
    wl = W.get("c2s")
    x = W.values(W.gen_x(wl), wl.dtype)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    gu, dn = W.gen_expert(wl, 0)
    g = W.values(gu, wl.dtype)
    assert abs(g.std() - 0.02) < 0.001


def test_zipf_bias_is_log_prior():
    wl = W.get("c4")
    _, bias = W.gen_router(wl)
    p = np.exp(bias.astype(np.float64))
    assert abs(p.sum() - 1) < 1e-5
    ps = np.sort(p)[::-1]
    r = np.arange(1, wl.E + 1)
    np.testing.assert_allclose(ps / ps[0], r ** -1.1, rtol=1e-5)


def test_all_workloads_tileable():
    for wl in list(W.WORKLOADS.values()) + list(W.SMALL_WORKLOADS.values()):
        assert wl.d % 64 == 0 and wl.f % 64 == 0 and wl.f_shared % 64 == 0
        assert 1 <= wl.k <= wl.E <= 256 and wl.P < 2 ** 31


@pytest.mark.parametrize("name", ["c4", "c4s"])
def test_fine_grained_load_has_empty_experts(name):
    """Zipf(1.1) popularity: the realised load is skewed and leaves experts empty."""
    wl = W.get(name)
    x = W.values(W.gen_x(wl), wl.dtype)
    wr, bias = W.gen_router(wl)
    ids, _ = O.route(O.router_logits(x, W.values(wr, wl.dtype), bias), wl.k, wl.score)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    assert (counts == 0).sum() >= 1
    assert counts.max() > 10 * np.median(counts)


def test_mixtral_load_near_uniform():
    wl = W.get("c2")
    x = W.values(W.gen_x(wl), wl.dtype)
    wr, bias = W.gen_router(wl)
    ids, _ = O.route(O.router_logits(x, W.values(wr, wl.dtype), bias), wl.k, wl.score)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    assert counts.min() > 0.8 * wl.P / wl.E and counts.max() < 1.2 * wl.P / wl.E


def test_gen_ids_valid():
    ids = W.gen_ids(50, 16, 4, 1, 1.0)
    assert all(len(set(r)) == 4 for r in ids)
    assert ids.min() >= 0 and ids.max() < 16
