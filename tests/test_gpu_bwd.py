"""GPU parity of the training calls: mmdit_joint_attn_fwd (output and
log-sum-exp) and mmdit_joint_attn_bwd (dq, dk, dv) against the fp64 oracle
(oracle.attention_bwd), which forms the gradients from q, k, v and dO alone.

Tolerances: forward outputs take the stated floating-point bars, max-abs 2e-2
for bf16 inputs with fp32 outputs and 1e-4 for the fp32 path (and the fp32
path's gradients, 1e-4).  bf16 gradients are held entry by entry to the
allowance of grad_bounds (the bf16 rounding of P and dS carried through |dO|,
|V|, |K| and |Q|), and at unit-scale inputs also to max-abs 2e-2.  The
log-sum-exp: the forward sums the fp16-rounded probabilities (relative 2^-11
each), so 2e-3 absolute."""
import math

import numpy as np
import pytest
import torch

import joint_video_audio_rope_amd as J
from oracle import attention_bwd as AB
from synth import WORKLOADS, joint_inputs, normal_tensors, upstream_grad

import grad_bounds as GB

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16, TOL_FP32, TOL_LSE = 2e-2, 1e-4, 2e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_sum(name, got, ref):
    """sum_j dv_j = sum_i dO_i (each query's probabilities sum to one): an
    invariant over all keys, whose per-entry errors largely cancel; held to
    1e-3 of its largest entry."""
    err, peak = float(np.max(np.abs(got - ref))), float(np.max(np.abs(ref)))
    print("%s: max-abs %.3e, max |ref| %.3e" % (name, err, peak), flush=True)
    assert err <= 1e-3 * peak, (name, err, peak)


def check(name, got, ref, tol):
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    peak = float(np.max(np.abs(ref))) if ref.size else 0.0
    print("%s: max-abs %.3e, max |ref| %.3e" % (name, err, peak), flush=True)
    assert err <= tol, (name, err)


def run(q, k, v, g, scale=None):
    o, lse = J.mmdit_joint_attn_fwd(q, k, v, softmax_scale=scale)
    dq, dk, dv = J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def test_bwd_single_key():
    """One key: every softmax row is the constant 1, so dv is the sum of dO over
    the queries and dq, dk are exactly zero: dS = P (dP - D) with dP = dO . v
    and D = dO . o, o = v.  The zeros come out of cancelling fp32 sums of 128
    products, so they are held to the error bound of two such sums (3 gamma_128
    times the sum of |dO_c v_c|, plus the bf16 rounding of dS), propagated
    through |k| and |q|, not to a fraction of their own largest entry."""
    nq, h, d = 160, 2, 128
    q, k, v, g = normal_tensors([(nq, h, d), (1, h, d), (1, h, d), (nq, h, d)], seed=41, device=DEV)
    o, lse, dq, dk, dv = run(q, k, v, g)
    qq, kk, vv, gg = f64(q), f64(k), f64(v), f64(g)
    check("o", f64(o), np.broadcast_to(vv, qq.shape), TOL_BF16)
    GB.check("dv", f64(dv), gg.sum(axis=0, keepdims=True), GB.bwd_allowances(qq, kk, vv, gg)[2])
    u = 2.0 ** -24
    gamma = 128 * u / (1 - 128 * u)
    ds_bound = 3 * gamma * np.einsum("ihc,hc->ih", np.abs(gg), np.abs(vv[0])) * (1 + 2.0 ** -8)   # [nq, h]
    scale = 1.0 / math.sqrt(d)
    dq_bound = scale * ds_bound[:, :, None] * np.abs(kk)                                        # [nq, h, d]
    dk_bound = scale * np.einsum("ih,ihc->hc", ds_bound, np.abs(qq))[None]                      # [1, h, d]
    print("dq max %.2e (bound %.2e), dk max %.2e (bound %.2e)" % (
        np.abs(f64(dq)).max(), dq_bound.max(), np.abs(f64(dk)).max(), dk_bound.max()), flush=True)
    assert (np.abs(f64(dq)) <= dq_bound).all()
    assert (np.abs(f64(dk)) <= dk_bound).all()


@pytest.mark.parametrize("nq,nk,h,d", [
    (300, 333, 3, 128),    # several 64-query / 64-key tiles, ragged tails on both sides
    (130, 70, 2, 64),      # head_dim 64
    (64, 64, 1, 128),      # exactly one tile
    (1, 5, 1, 128),        # one query, fewer keys than a tile
    (257, 1000, 2, 128),   # one query past a 256-query dQ workgroup
    (520, 129, 2, 128),    # keys one past a 128-key dK/dV workgroup
])
def test_bwd_bf16_matches_oracle(nq, nk, h, d):
    q, k, v, g = normal_tensors([(nq, h, d), (nk, h, d), (nk, h, d), (nq, h, d)], seed=nq * 7 + nk, device=DEV)
    o, lse, dq, dk, dv = run(q, k, v, g)
    qq, kk, vv, gg = f64(q), f64(k), f64(v), f64(g)
    o_ref, lse_ref = AB.attention_fwd_lse(qq, kk, vv)
    check("o", f64(o), o_ref, TOL_BF16)
    check("lse", f64(lse), lse_ref, TOL_LSE)
    rq, rk, rv = AB.attention_bwd(qq, kk, vv, gg)
    aq, ak, av = GB.bwd_allowances(qq, kk, vv, gg)
    GB.check("dq", f64(dq), rq, aq)
    GB.check("dk", f64(dk), rk, ak)
    GB.check("dv", f64(dv), rv, av)


def test_bwd_bf16_explicit_scale():
    q, k, v, g = normal_tensors([(200, 2, 128), (150, 2, 128), (150, 2, 128), (200, 2, 128)], seed=11, device=DEV)
    o, lse, dq, dk, dv = run(q, k, v, g, scale=0.05)
    qq, kk, vv, gg = f64(q), f64(k), f64(v), f64(g)
    check("lse", f64(lse), AB.attention_fwd_lse(qq, kk, vv, scale=0.05)[1], TOL_LSE)
    allow = GB.bwd_allowances(qq, kk, vv, gg, scale=0.05)
    for name, got, ref, a in zip(("dq", "dk", "dv"), (dq, dk, dv), AB.attention_bwd(qq, kk, vv, gg, scale=0.05),
                                 allow):
        GB.check(name, f64(got), ref, a)


@pytest.mark.parametrize("shape", [(88, 88, 2, 64), (200, 150, 2, 128)])
def test_bwd_fp32_matches_oracle(shape):
    nq, nk, h, d = shape
    q, k, v, g = normal_tensors([(nq, h, d), (nk, h, d), (nk, h, d), (nq, h, d)], seed=5, dtype="fp32", device=DEV)
    o, lse, dq, dk, dv = run(q, k, v, g)
    qq, kk, vv, gg = f64(q), f64(k), f64(v), f64(g)
    o_ref, lse_ref = AB.attention_fwd_lse(qq, kk, vv)
    check("o", f64(o), o_ref, TOL_FP32)
    check("lse", f64(lse), lse_ref, TOL_FP32)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), AB.attention_bwd(qq, kk, vv, gg)):
        check(name, f64(got), ref, TOL_FP32)


def test_bwd_tiny_workload_fp32():
    w = WORKLOADS["tiny"]
    x = joint_inputs(w, DEV)
    g = upstream_grad(w, DEV)
    o, lse, dq, dk, dv = run(x["q"], x["k"], x["v"], g)
    ref = AB.attention_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g))
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check(name, f64(got), r, TOL_FP32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_without_queries_gives_zero_key_gradients(dtype):
    q, k, v, g = normal_tensors([(0, 2, 64), (70, 2, 64), (70, 2, 64), (0, 2, 64)], seed=3, dtype=dtype, device=DEV)
    o = torch.empty((0, 2, 64), dtype=torch.float32, device=DEV)
    lse = torch.empty((2, 0), dtype=torch.float32, device=DEV)
    dk = torch.full((70, 2, 64), 7.0, device=DEV)
    dv = torch.full((70, 2, 64), 7.0, device=DEV)
    J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_repeat_is_bitwise_identical():
    q, k, v, g = normal_tensors([(700, 3, 128), (650, 3, 128), (650, 3, 128), (700, 3, 128)], seed=9, device=DEV)
    _, _, dq1, dk1, dv1 = run(q, k, v, g)
    _, _, dq2, dk2, dv2 = run(q, k, v, g)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def test_bwd_joint_480p_sampled():
    """The full 480p-latent joint sequence (35050 tokens, 24 x 128) in the
    launch configuration the bench times: dq on sampled queries of every head,
    dk and dv on sampled keys of two heads (their queries' log-sum-exp and D
    formed over all keys by the oracle), and sum_j dv_j = sum_i dO_i over
    every head."""
    w = WORKLOADS["480p"]
    x = joint_inputs(w, DEV)
    g = upstream_grad(w, DEV)
    o, lse, dq, dk, dv = run(x["q"], x["k"], x["v"], g)
    n = x["q"].shape[0]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, n - 1, 34319, 34320], rng.choice(n, 8, replace=False)]))
    qq, kk, vv, gg = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g)
    rq, _, _ = AB.attention_bwd(qq[rows], kk, vv, gg[rows])
    GB.check("dq rows", f64(dq)[rows], rq, GB.bwd_allowances(qq[rows], kk, vv, gg[rows])[0])
    keys = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 6, replace=False)]))
    heads = [0, 23]
    rk, rv = AB.key_rows_grads(qq, kk, vv, gg, keys, heads)
    ak, av = GB.key_rows_allowances(qq, kk, vv, gg, keys, heads)
    GB.check("dk rows", f64(dk)[keys][:, heads], rk, ak)
    GB.check("dv rows", f64(dv)[keys][:, heads], rv, av)
    sums = dv.double().sum(dim=0).cpu().numpy()
    check_sum("sum dv", sums, gg.sum(axis=0))


def test_bwd_audio_video_480p_shapes():
    """The cross-attention shapes of the 480p-latent layer: 218 audio queries
    against the 34320 video-stream keys (the forward splits the key range and
    merges the partials, so the log-sum-exp comes from the merge) and the
    reverse direction, forward with lse and backward."""
    w = WORKLOADS["480p"]
    x = joint_inputs(w, DEV)
    g = upstream_grad(w, DEV)
    n_vs = (w["n_cond_frames"] + w["T"]) * w["H"] * w["W"]
    a0, a1 = n_vs, n_vs + w["n_audio"]
    q, k, v = x["q"], x["k"], x["v"]
    # audio -> video
    qa, ga = q[a0:a1].contiguous(), g[a0:a1].contiguous()
    kv, vv = k[:n_vs].contiguous(), v[:n_vs].contiguous()
    o, lse, dq, dk, dv = run(qa, kv, vv, ga)
    qq, kk, vv64, gg = f64(qa), f64(kv), f64(vv), f64(ga)
    o_ref, lse_ref = AB.attention_fwd_lse(qq, kk, vv64)
    check("a->v o", f64(o), o_ref, TOL_BF16)
    check("a->v lse", f64(lse), lse_ref, TOL_LSE)
    rq, _, _ = AB.attention_bwd(qq, kk, vv64, gg)
    GB.check("a->v dq", f64(dq), rq, GB.bwd_allowances(qq, kk, vv64, gg)[0])
    keys = np.array([0, 1, 1559, 1560, 17000, n_vs - 1])
    rk, rv = AB.key_rows_grads(qq, kk, vv64, gg, keys, list(range(w["heads"])))
    ak, av = GB.key_rows_allowances(qq, kk, vv64, gg, keys, list(range(w["heads"])))
    GB.check("a->v dk rows", f64(dk)[keys], rk, ak)
    GB.check("a->v dv rows", f64(dv)[keys], rv, av)
    # video -> audio: sampled video queries, every audio key
    ka, va = k[a0:a1].contiguous(), v[a0:a1].contiguous()
    qv, gv = q[:n_vs].contiguous(), g[:n_vs].contiguous()
    o, lse, dq, dk, dv = run(qv, ka, va, gv)
    rows = np.array([0, 1, 777, 1560, 20000, n_vs - 1])
    rq, _, _ = AB.attention_bwd(f64(qv)[rows], f64(ka), f64(va), f64(gv)[rows])
    GB.check("v->a dq rows", f64(dq)[rows], rq, GB.bwd_allowances(f64(qv)[rows], f64(ka), f64(va), f64(gv)[rows])[0])
    rk, rv = AB.key_rows_grads(f64(qv), f64(ka), f64(va), f64(gv), np.arange(w["n_audio"]), [0, 11])
    ak, av = GB.key_rows_allowances(f64(qv), f64(ka), f64(va), f64(gv), np.arange(w["n_audio"]), [0, 11])
    GB.check("v->a dk", f64(dk)[:, [0, 11]], rk, ak)
    GB.check("v->a dv", f64(dv)[:, [0, 11]], rv, av)


def test_bwd_joint_720p_sampled():
    """The 720p-latent joint sequence (76330 tokens) with its 10 % outlier
    tokens scaled by 4 (large logits: the forward's lazy rescale and the
    log-sum-exp carry them): dq on sampled queries of every head, outliers
    included, and dk, dv on sampled keys of one head."""
    w = WORKLOADS["720p"]
    x = joint_inputs(w, DEV)
    g = upstream_grad(w, DEV)
    o, lse, dq, dk, dv = run(x["q"], x["k"], x["v"], g)
    n = x["q"].shape[0]
    out = x["outliers"].cpu().numpy()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, n - 1], out[:4], rng.choice(n, 4, replace=False)]))
    qq, kk, vv, gg = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g)
    o_ref, lse_ref = AB.attention_fwd_lse(qq[rows], kk, vv)
    check("720p lse rows", f64(lse)[:, rows], lse_ref, TOL_LSE)
    rq, _, _ = AB.attention_bwd(qq[rows], kk, vv, gg[rows])
    # the outlier tokens (x4) make gradient entries of 30 and more: the
    # allowance alone, no absolute bar
    GB.check("720p dq rows", f64(dq)[rows], rq, GB.bwd_allowances(qq[rows], kk, vv, gg[rows])[0], unit=False)
    keys = np.unique(np.concatenate([[0, n - 1], out[4:7], rng.choice(n, 3, replace=False)]))
    rk, rv = AB.key_rows_grads(qq, kk, vv, gg, keys, [5])
    ak, av = GB.key_rows_allowances(qq, kk, vv, gg, keys, [5])
    GB.check("720p dk rows", f64(dk)[keys][:, [5]], rk, ak, unit=False)
    GB.check("720p dv rows", f64(dv)[keys][:, [5]], rv, av, unit=False)
