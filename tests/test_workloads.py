"""The seeded input generator: determinism, shapes, distributions, needles."""

import numpy as np
import torch

import workloads
from workloads import LayerShape, as_f64


def test_layer_inputs_are_deterministic_and_shaped():
    sh = LayerShape(n=300, d=256, Hq=4, Hkv=1, dh=64, f=512, r=16, P=8)
    a = workloads.make_layer(sh, seed=3)
    b = workloads.make_layer(sh, seed=3)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    assert a["x"].dtype == torch.bfloat16 and a["x"].shape == (300, 256)
    assert a["wq"].shape == (256, 256) and a["wk"].shape == (64, 256)
    assert a["wg"].shape == (512, 256) and a["wd"].shape == (256, 512)
    assert a["u_t"].shape == (16, 256) and a["v_t"].shape == (256, 16)
    assert abs(as_f64(a["wg"]).std() - 0.02) < 1e-3
    assert abs(as_f64(a["x"]).std() - 1.0) < 2e-2
    assert not torch.equal(a["x"], workloads.make_layer(sh, seed=4)["x"])


def test_projected_needles_align_with_probe_queries():
    sh = LayerShape(n=400, d=256, Hq=4, Hkv=2, dh=32, P=8)
    inp = workloads.make_layer(sh, seed=0, with_ffn=False, needles=6)
    pos = inp["needle_pos"].numpy()
    assert len(pos) == 6 and pos.max() < sh.n - sh.P
    x, wq, wk = as_f64(inp["x"]), as_f64(inp["wq"]), as_f64(inp["wk"])
    q = (x[-sh.P:] @ wq.T).reshape(sh.P, sh.Hkv, 2, sh.dh).sum(2)
    k = (x @ wk.T).reshape(sh.n, sh.Hkv, sh.dh)
    ordinary = np.sqrt((np.delete(k, pos, 0) ** 2).sum(-1).mean(0))
    for j, p in enumerate(pos):
        u = q[j % sh.P]
        cos = (k[p] * u).sum(-1) / np.linalg.norm(k[p], axis=-1) / np.linalg.norm(u, axis=-1)
        assert (cos > 0.99).all()
        assert np.allclose(np.linalg.norm(k[p], axis=-1) / ordinary, 4.0, rtol=0.05)


def test_clustered_keys_with_needles():
    sh = LayerShape(n=2048, d=256, Hq=4, Hkv=2, dh=32, f=256, r=8, P=16)
    inp = workloads.make_layer(sh, seed=0, needles=32, clustered_keys=(16, 0.3))
    assert "wk" not in inp and inp["k"].shape == (2048, 2, 32)
    k = as_f64(inp["k"])
    pos = inp["needle_pos"].numpy()
    rest = np.delete(k, pos, 0)
    # sixteen tight clusters per head: two keys of one cluster are about
    # sigma*sqrt(2*dh) = 2.4 apart, keys of different clusters about 8.4
    d = np.sqrt(((rest[:64, 0, None, :] - rest[None, :, 0, :]) ** 2).sum(-1))
    nearest = np.sort(d, axis=1)[:, 1]
    assert np.median(nearest) < 3.2 and np.median(d) > 6.0


def test_scores_generator():
    s = workloads.make_scores(1000, seed=1, ties=50).numpy()
    assert s.dtype == np.float32 and (s >= 0).all()
    assert len(np.unique(s)) < 1000
