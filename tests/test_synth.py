"""The seeded generators: determinism, shapes and the stated distributions."""
import numpy as np
import torch

from synth import WORKLOADS, joint_inputs, n_tokens, shrink, sparse_inputs


def test_token_counts():
    assert n_tokens(WORKLOADS["tiny"]) == 88
    assert n_tokens(WORKLOADS["block"]) == 5850
    assert n_tokens(WORKLOADS["480p"]) == 35050
    assert n_tokens(WORKLOADS["720p"]) == 76330


def test_deterministic_and_seed_sensitive():
    w = WORKLOADS["tiny"]
    a, b = joint_inputs(w), joint_inputs(w)
    for t in "qkv":
        assert torch.equal(a[t], b[t])
        assert a[t].dtype == torch.float32 and a[t].shape == (88, 2, 64)
    c = joint_inputs(shrink("tiny", seed=1))
    assert not torch.equal(a["q"], c["q"])


def test_scaled_bf16_inputs():
    w = shrink("block", T=2, H=4, W=4, n_audio=10, n_text=6)
    x = joint_inputs(w)
    assert x["q"].dtype == torch.bfloat16 and x["q"].shape == (48, 24, 128)
    s = x["k"].float().std().item()
    assert abs(s - 128 ** -0.5) < 0.01


def test_bf16_rounding_is_nearest_even():
    vals = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=torch.float32)
    got = vals.to(torch.bfloat16).float().tolist()
    assert got == [1.0, 1.0 + 2 ** -6, 1.0]


def test_outliers():
    w = shrink("720p", T=2, H=5, W=8, n_audio=7, n_text=3, heads=2, head_dim=16)
    n = n_tokens(w)
    x = joint_inputs(w)
    idx = x["outliers"]
    assert idx.numel() == round(0.1 * n) and len(set(idx.tolist())) == idx.numel()
    mask = torch.zeros(n, dtype=torch.bool)
    mask[idx] = True
    big = x["v"][mask].float().abs().mean().item()
    small = x["v"][~mask].float().abs().mean().item()
    assert 3.0 < big / small < 5.0


def test_sparse_fields():
    w = shrink("sparse2k", T=16, H=16, W=32, heads=2, head_dim=16)
    x = sparse_inputs(w)
    q = x["q"].float().numpy().reshape(16, 16, 32, 32)
    k = x["k"].float().numpy().reshape(16, 16, 32, 32)
    v = x["v"].float().numpy().reshape(16, 16, 32, 32)
    # per-channel variance 1 + 0.01 of noise
    assert abs(q.var(axis=(0, 1, 2)).mean() - 1.01) < 0.03
    # Q and K share a field, V does not
    cqk = np.mean([np.corrcoef(q[..., c].ravel(), k[..., c].ravel())[0, 1] for c in range(32)])
    cqv = np.mean([np.corrcoef(q[..., c].ravel(), v[..., c].ravel())[0, 1] for c in range(32)])
    assert cqk > 0.98 and abs(cqv) < 0.1
    # Gaussian covariance with length 4: correlation at a lag of 4 along w is about e^-0.5
    lag = np.mean(q * np.roll(q, 4, axis=2)) / np.mean(q * q)
    assert abs(lag - np.exp(-0.5) / 1.01) < 0.08
    assert torch.equal(sparse_inputs(w)["v"], x["v"])


def test_adaptive_inputs():
    from synth import adaptive_inputs
    w = shrink("adaptive2k", T=8, H=32, W=32, heads=2, head_dim=16, fg_radius=6.0, audio_radius=4.0)
    x = adaptive_inputs(w)
    n = 8 * 32 * 32
    assert x["q"].shape == (n, 2, 16) and x["q"].dtype == torch.bfloat16
    assert x["a"].shape == (n,) and x["a"].dtype == torch.float32
    a = x["a"].numpy().reshape(8, 32, 32)
    assert a.min() >= 0.0 and abs(a.max() - 4.0) < 0.3
    # the audio pulse has period 6 frames: frames 0 and 6 peak, frame 3 is silent
    assert a[3].max() < 1e-6 and abs(a[0].max() - a[6].max()) < 1e-5
    # Q and K share their field as in the uniform workload
    q, k = x["q"].float().numpy(), x["k"].float().numpy()
    assert np.corrcoef(q.ravel(), k.ravel())[0, 1] > 0.98
    # V: the foreground blob carries more local variation than the background
    v = x["v"].float().numpy().reshape(8, 32, 32, 32)
    dv = np.abs(np.diff(v, axis=0)).mean(axis=(0, 3))
    assert dv.max() > 3 * dv.min()
    again = adaptive_inputs(w)
    for t in "qkva":
        assert torch.equal(again[t], x[t])
