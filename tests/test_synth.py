"""The seeded input generators (CPU): determinism, quantiser sanity, routing skew."""
import numpy as np

from oracle import moe_oracle as O
from synth import CONFIGS, Config, zipf_logits, zipf_popularity


def test_host_generator_is_deterministic(hostgen):
    c = CONFIGS[1]
    lay = O.blob_layout(c.H, c.I)
    a = hostgen.expert_blob(c, 0, 2, lay)
    b = hostgen.expert_blob(c, 0, 2, lay)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, hostgen.expert_blob(c, 0, 3, lay))
    assert np.array_equal(hostgen.x(c, 0, 1), hostgen.x(c, 0, 1))
    assert not np.array_equal(hostgen.x(c, 0, 1), hostgen.x(c, 0, 2))


def test_quantised_weights_track_gaussian_recipe(hostgen):
    """Decoded weights: std ~0.02, and every block's values lie within one
    E2M1 step (scale * G * 2, the widest gap) of an N(0, 0.02)-like draw."""
    c = Config(cfg_id=1, name="q", T=1, H=512, I=256, E=1, k=1, L=1, router="matrix")
    lay = O.blob_layout(c.H, c.I)
    blob = hostgen.expert_blob(c, 0, 0, lay)
    for m in range(3):
        w = O.dequant(blob, lay, m)
        assert abs(w.std() / 0.02 - 1) < 0.05
        assert abs(w.mean()) < 1e-3
        assert np.abs(w).max() <= 0.12 * 1.07
        # every block has a code of magnitude >= 4 (block max maps near 6)
        rows, K = w.shape
        s = O.matrix_scales(blob, lay, m)
        G = np.frombuffer(blob[lay.off_globals + 4 * m: lay.off_globals + 4 * m + 4].tobytes(), np.float32)[0]
        blockmax = np.abs(w).reshape(rows, K // 16, 16).max(axis=2) / (O.e4m3fn_decode(s).reshape(rows, -1) * G)
        assert blockmax.min() >= 4.0 and blockmax.max() <= 6.0


def test_mx_blob_recipe(hostgen):
    """MX blobs hold the NVFP4 blobs' weights (same stream), re-quantised per 32
    values: every block's largest code magnitude is 4 or 6 (amax / 2^shared in
    [4, 8), 6 saturating), and the two decodings agree to within their
    quantisation steps."""
    c = Config(cfg_id=1, name="q", T=1, H=512, I=256, E=1, k=1, L=1, router="matrix")
    lay, mlay = O.blob_layout(c.H, c.I), O.mx_blob_layout(c.H, c.I)
    nv = hostgen.expert_blob(c, 0, 0, lay)
    mx = hostgen.expert_blob_mx(c, 0, 0, mlay)
    assert not mx[mlay.blob_bytes:].any()
    for m in range(3):
        w = O.mx_dequant(mx, mlay, m, c.H, c.I)
        sc = O.e8m0_decode(O.mx_matrix_scales(mx, mlay, m, c.H, c.I))
        top = np.abs(w).reshape(w.shape[0], -1, 32).max(axis=2) / sc
        assert set(np.unique(top)) <= {4.0, 6.0}
        w_nv = O.dequant(nv, lay, m)
        assert np.linalg.norm(w - w_nv) / np.linalg.norm(w_nv) < 0.25
        assert abs(w.std() / 0.02 - 1) < 0.06


def test_activation_statistics(hostgen):
    x = O.bf16_bits_to_f64(hostgen.x(CONFIGS[4], 0, 0, T=256))
    assert abs(x.std() - 1) < 0.01 and abs(x.mean()) < 0.01 and np.abs(x).max() <= 6


def test_zipf_first_choice_rank_slope():
    c = CONFIGS[3]
    T = 40000
    lg = zipf_logits(c, 0, 0, T=T)
    first = np.argmax(lg, axis=1)
    pop = zipf_popularity(c, 0, 0)
    rank = np.argsort(np.argsort(-pop))          # 0 = most popular
    freq = np.bincount(rank[first], minlength=c.E)
    r = np.arange(1, 21)
    slope = np.polyfit(np.log(r), np.log(freq[:20]), 1)[0]
    assert abs(slope + c.zipf_s) < 0.15, slope


def test_zipf_hot_set_drifts_per_epoch():
    c = CONFIGS[3]
    assert np.array_equal(zipf_popularity(c, 0, 0), zipf_popularity(c, 0, c.epoch(15)))
    assert not np.array_equal(zipf_popularity(c, 0, c.epoch(15)), zipf_popularity(c, 0, c.epoch(16)))
