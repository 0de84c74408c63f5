"""Seeded input generators: determinism, shapes and the stated recipe."""

import numpy as np
import torch

from mixture_experts_expert_mm_amd import workloads as wl


def test_configs_match_stated_shapes():
    c = wl.CONFIGS
    assert (c["tiny_bf16"].T, c["tiny_bf16"].H, c["tiny_bf16"].I, c["tiny_bf16"].E, c["tiny_bf16"].K) == (64, 256, 128, 8, 2)
    assert (c["mid_bf16"].T, c["mid_bf16"].H, c["mid_bf16"].I, c["mid_bf16"].E, c["mid_bf16"].K) == (2048, 4096, 1408, 16, 4)
    for n in ("dsv3_bf16", "dsv3_fp8_t128", "dsv3_fp8_t16384", "dsv3_int8", "dsv3_bf16_t16384", "dsv3_bf16_t128"):
        assert (c[n].H, c[n].I, c[n].E, c[n].K) == (7168, 2048, 32, 8)
    assert c["dsv3_fp8_t128"].seed == c["dsv3_fp8_t16384"].seed      # one weight set for the sweep
    assert c["dsv3_bf16_t128"].seed == c["dsv3_bf16_t16384"].seed == c["dsv3_bf16"].seed
    assert (c["dsv3_bf16_t16384"].T, c["dsv3_bf16_t128"].T) == (16384, 128)


def test_routing_is_deterministic_distinct_and_normalised():
    cfg = wl.CONFIGS["dsv3_bf16"].with_(T=512)
    a = wl.routing(cfg)
    b = wl.routing(cfg)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ids, w = a[0].numpy(), a[1].numpy()
    assert ids.dtype == np.int32 and w.dtype == np.float32
    for row in ids:
        assert len(set(row.tolist())) == cfg.K
    assert np.all((ids >= 0) & (ids < cfg.E))
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)                      # descending score order


def test_bias_skews_routing():
    skew = np.bincount(wl.routing(wl.CONFIGS["dsv3_bf16"])[0].numpy().ravel(), minlength=32)
    flat = np.bincount(wl.routing(wl.CONFIGS["dsv3_int8"].with_(T=4096))[0].numpy().ravel(), minlength=32)
    assert skew.max() / skew.min() > 3 * flat.max() / flat.min()


def test_masked_routes():
    cfg = wl.CONFIGS["tiny_bf16"].with_(masked_ratio=0.25)
    ids, w = (t.numpy() for t in wl.routing(cfg))
    m = ids < 0
    assert 0.1 < m.mean() < 0.4
    assert np.all(w[m] == 0)


def test_tokens_and_weights():
    cfg = wl.CONFIGS["tiny_bf16"]
    x = wl.tokens(cfg)
    assert x.dtype == torch.bfloat16 and x.shape == (cfg.T, cfg.H)
    assert torch.equal(x, wl.tokens(cfg))
    assert abs(x.float().std().item() - 1.0) < 0.05
    w1, w2, s1, s2 = wl.expert_weights(cfg, 3)
    assert w1.shape == (cfg.H, 2 * cfg.I) and w2.shape == (cfg.I, cfg.H) and s1 is None
    assert abs(w1.float().std().item() * np.sqrt(cfg.H) - 1.0) < 0.05
    assert abs(w2.float().std().item() * np.sqrt(cfg.I) - 1.0) < 0.05


def test_quantised_weights_per_channel():
    for uc, qmax in (("int8", 127), ("fp8", 448)):
        cfg = wl.CONFIGS["tiny_bf16"].with_(usecase=uc)
        q, _, s, _ = wl.expert_weights(cfg, 1)
        qv = q.float()
        assert torch.all(qv.abs().amax(0) == qmax)            # one element per channel hits Qmax
        w1, _ = wl.expert_weights_f32(cfg, 1)
        assert torch.allclose(qv * s[None, :], w1, rtol=0.07, atol=float(s.max()) * 0.51)


def test_shared_expert_weights_and_active_mask():
    cfg = wl.Config("s", "int8", 40, 256, 128, 4, 2, 0.0, 5, shared=1, inactive_ratio=0.3)
    w = wl.all_weights(cfg)
    assert w.w1.shape == (5, 256, 256) and w.s2.shape == (5, 256)
    # the shared expert is drawn like expert index E of the routed recipe
    q1, q2, s1, s2 = wl.expert_weights(cfg, 4)
    assert torch.equal(w.w1[4], q1) and torch.equal(w.s1[4], s1)
    m = wl.active_mask(cfg)
    assert m.dtype == torch.int8 and m.shape == (40,) and set(m.tolist()) <= {0, 1}
    assert torch.equal(m, wl.active_mask(cfg)) and 0 < int(m.sum()) < 40
    assert wl.active_mask(cfg.with_(inactive_ratio=0.0)) is None


def test_mx_weights_layout_and_scale_of_values():
    import oracle
    for uc in ("mxfp8", "mxfp4"):
        cfg = wl.Config("mx", uc, 8, 512, 256, 3, 2, 0.0, 9, shared=1)
        w = wl.all_weights(cfg)
        half = 2 if uc == "mxfp4" else 1
        assert w.w1.shape == (4, 512, 512 // half) and w.w2.shape == (4, 256, 512 // half)
        assert w.s1.shape == (4, 512, 16) and w.s2.shape == (4, 512, 8) and w.s1.dtype == torch.uint8
        codes = wl.unpack_codes(w.w1[0], cfg)
        assert codes.shape == (512, 512)
        fmt = oracle.MX_WEIGHT_FORMAT[uc]
        vals = oracle.mx_dequantize(codes.T, w.s1[0].numpy(), fmt)
        assert np.all(np.isfinite(vals))
        rms = np.sqrt(np.mean(vals ** 2))
        assert 0.5 / np.sqrt(512) < rms < 2.0 / np.sqrt(512), rms
