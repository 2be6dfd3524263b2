"""The seeded input generator: reproducible bytes and the stated distributions."""
import numpy as np

import moegen
from oracle import formats as F
from oracle import moe as M


def test_reproducible_and_expert_independent():
    sp = moegen.spec("tiny")
    a = moegen.weights(sp)
    b = moegen.weights(sp)
    for key in a:
        assert np.array_equal(a[key], b[key])
    e3 = moegen.expert(sp, 3)
    assert np.array_equal(e3["w1_codes"], a["w1_codes"][3])
    assert np.array_equal(moegen.batch(sp, 16)["x"], moegen.batch(sp, 16)["x"])
    assert not np.array_equal(moegen.batch(sp, 16)["x"][:8], moegen.batch(sp, 8)["x"])


def test_shapes():
    sp = moegen.spec("tiny")
    w = moegen.weights(sp)
    E, H, I = 8, 256, 512
    assert w["w1_codes"].shape == (E, 2 * I, H // 16) and w["w1_codes"].dtype == np.uint32
    assert w["w1_scales"].shape == (E, 2 * I, H // 32) and w["w1_scales"].dtype == np.uint16
    assert w["w2_codes"].shape == (E, H, I // 16)
    assert w["w2_scales"].shape == (E, H, I // 32)
    sp3 = moegen.spec("w3", E=4)
    w3 = moegen.expert(sp3, 0)
    assert w3["w1_codes"].shape == (1024, 2048 // 32 * 3) and w3["w1_scales"].shape == (1024, 32)
    b = moegen.batch(sp, 5)
    assert b["logits"].shape == (5, E) and b["logits"].dtype == np.float32
    assert b["x"].shape == (5, H) and b["x"].dtype == np.uint16


def test_distributions():
    sp = moegen.spec("tiny")
    ex = moegen.expert(sp, 0)
    s = F.bf16_value(ex["w1_scales"])
    assert np.all((np.abs(s) >= 0.005 * (1 - 2**-8)) & (np.abs(s) <= 0.02 * (1 + 2**-8)))
    assert 0.4 < np.mean(s > 0) < 0.6
    codes = ((ex["w1_codes"][..., None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(-1)
    frac = np.bincount(codes, minlength=4) / codes.size
    assert np.all(np.abs(frac - 0.25) < 0.01)
    x = F.bf16_value(moegen.batch(sp, 64)["x"])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    sp3 = moegen.spec("w3", E=2)
    sb = moegen.expert(sp3, 1)["w1_scales"]
    assert set(np.unique((sb >> 3) & 15)) == {5, 6, 7}
    sm = moegen.spec("mixed", E=40, n_hot=4)
    hx = moegen.expert(sm, 0, "mxfp4")
    assert set(np.unique(hx["w1_scales"])) == {120, 121}


def test_zipf_routing_group_sizes_span_zero_to_thousands():
    sp = moegen.spec("prefill")
    b = moegen.batch(sp, 8192)
    ids, _ = M.route(b["logits"], sp["k"])
    counts = np.bincount(ids.reshape(-1), minlength=sp["E"])
    assert counts.min() == 0 and counts.max() > 2000
    hot = moegen.hot_ids(moegen.spec("mixed"))
    assert len(hot) == 32 and len(set(hot.tolist())) == 32
    ranks = moegen.zipf_ranks(moegen.spec("mixed"))
    assert sorted(ranks[hot].tolist()) == list(range(1, 33))
