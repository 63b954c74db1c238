"""The C ABI on the host: the library loads, exports what include/mmdit.h
declares, builds the RoPE table the oracle's angles define, plans workspaces,
and rejects bad arguments before touching the GPU (CPU only)."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import joint_video_audio_rope_amd as J
from joint_video_audio_rope_amd import _lib as L
from oracle import rope as R
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmdit.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mmdit_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("mmdit_rope3d", "mmdit_joint_attn", "mmdit_av_cross_attn", "mmdit_block_sparse_attn",
              "mmdit_joint_attn_fwd", "mmdit_joint_attn_bwd", "mmdit_block_sparse_attn_fwd",
              "mmdit_block_sparse_attn_bwd", "mmdit_block_sparse_attn_adaptive", "mmdit_token_norms",
              "mmdit_block_sparse_attn_adaptive_bwd", "mmdit_adaptive_tile_table",
              "mmdit_workspace_bytes", "mmdit_last_error", "mmdit_abi_version",
              "mmdit_rope3d_table_floats", "mmdit_rope3d_build_table", "mmdit_joint_attn_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = J.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_abi_version_and_empty_error():
    assert J.mmdit_abi_version() == 4
    assert isinstance(J.mmdit_last_error(), str)


def test_struct_layout_matches_header():
    # the binding's ctypes structs follow the C layout on x86-64
    assert ctypes.sizeof(L.Segment) == 48
    assert L.Segment.t_scale.offset == 40
    assert ctypes.sizeof(L.SparseDesc) == 48
    assert L.SparseDesc.top_p.offset == 32 and L.SparseDesc.wait_limit.offset == 40
    assert L.RopeDesc.segs.offset == 32 and L.RopeDesc.n_tokens.offset == 48


@pytest.mark.parametrize("name", ["tiny", "block", "480p", "720p"])
def test_rope_table_matches_oracle_angles(name):
    w = WORKLOADS[name]
    spec = J.rope_spec_for(w)
    tab = spec.host_table().numpy().reshape(-1, 2)
    ref = R.rope_table(w)
    parts = []
    if w["n_cond_frames"]:
        parts += [ref["cond_t"], ref["h"], ref["w"]]
    parts += [ref["video_t"], ref["h"], ref["w"], ref["audio_t"]]
    want = np.concatenate([p.reshape(-1, 2) for p in parts]).astype(np.float32)
    assert tab.shape == want.shape
    assert np.array_equal(tab.view(np.uint32), want.view(np.uint32))


def test_layout_segments_follow_the_sequence_order():
    segs, n = J.layout_segments(3, 4, 4, 1, 16, 8, (3, 16))
    assert n == 88
    assert [s["kind"] for s in segs] == [0, 0, 1, 2]
    assert segs[0]["t0"] == -1 and segs[0]["count"] == 16
    assert segs[1]["offset"] == 16 and segs[1]["t0"] == 0
    assert segs[2]["offset"] == 64 and segs[2]["t_scale"] == 3 / 16
    assert segs[3]["offset"] == 80


def test_workspace_plans():
    ws = J.mmdit_workspace_bytes
    # bf16 joint attention: V^T in fp16, key count padded to 64
    n = 35050
    # (plus the per-head partial maxima of V for its prescale: 24 x 64 uint32)
    assert ws(J.MMDIT_OP_JOINT_ATTN, n, n, 24, 128, J.MMDIT_BF16) == 24 * 128 * 35072 * 2 + 24 * 64 * 4
    assert ws(J.MMDIT_OP_JOINT_ATTN, 88, 88, 2, 64, J.MMDIT_FP32) == 0
    # audio queries against video keys split the keys and add partials
    big = ws(J.MMDIT_OP_AV_CROSS_ATTN, 34320, 218, 24, 128, J.MMDIT_BF16)
    assert big > 24 * 128 * 34368 * 2
    sd = J.sparse_desc()
    b = ws(J.MMDIT_OP_BLOCK_SPARSE_ATTN, 172032, 172032, 24, 128, J.MMDIT_BF16, sd)
    # block logits are computed and selected 2048 query blocks at a time (1 GiB for all heads)
    assert b >= 24 * 2048 * 2688 * 8 + 24 * 2688 * 84 * 4 + 2 * 24 * 2688 * 128 * 64 * 2
    assert b < 24 * 2688 * 2688 * 8 + 2 * 24 * 2688 * 128 * 64 * 2 + (1 << 28)
    # a million-token grid: the logits stay within the 1 GiB chunk
    big = ws(J.MMDIT_OP_BLOCK_SPARSE_ATTN, 32 * 128 * 256, 0, 24, 128, J.MMDIT_BF16, sd)
    assert big < 2 * 24 * 16384 * 128 * 64 * 2 + (3 << 30)


def _call_joint(**over):
    a = dict(q=16, n_q=10, k=32, v=48, n_kv=10, heads=2, hd=64, dtype=J.MMDIT_BF16, scale=0.125,
             o=1 << 20, ws=1 << 24, ws_bytes=1 << 20)
    a.update(over)
    lib = J.lib()
    return lib.mmdit_joint_attn(a["q"], a["n_q"], a["k"], a["v"], a["n_kv"], a["heads"], a["hd"],
                                a["dtype"], a["scale"], a["o"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(hd=96), L.MMDIT_ERR_UNSUPPORTED),
    (dict(dtype=7), L.MMDIT_ERR_INVALID_ARG),
    (dict(n_kv=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(n_q=-1), L.MMDIT_ERR_INVALID_ARG),
    (dict(heads=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(k=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(q=8), L.MMDIT_ERR_INVALID_ARG),                     # misaligned
    (dict(o=16), L.MMDIT_ERR_INVALID_ARG),                    # output aliases q
    (dict(scale=math.inf), L.MMDIT_ERR_INVALID_ARG),
    (dict(scale=-0.125), L.MMDIT_ERR_INVALID_ARG),
    (dict(scale=math.nan), L.MMDIT_ERR_INVALID_ARG),
    (dict(ws=0), L.MMDIT_ERR_WORKSPACE),
    (dict(ws_bytes=100), L.MMDIT_ERR_WORKSPACE),
])
def test_joint_attn_rejects_bad_arguments(over, status):
    # fake, never-dereferenced addresses: validation fails before any HIP call
    assert _call_joint(**over) == status
    assert J.mmdit_last_error() != ""


def _call_bwd(**over):
    # q, k, v, d_o: 10 x 2 x 64 bf16 = 2560 B; o, dq, dk, dv: 5120 B; lse: 80 B
    a = dict(q=1 << 20, n_q=10, k=2 << 20, v=3 << 20, n_kv=10, heads=2, hd=64, dtype=J.MMDIT_BF16,
             scale=0.125, o=4 << 20, lse=5 << 20, d_o=6 << 20, dq=7 << 20, dk=8 << 20, dv=9 << 20,
             ws=1 << 30, ws_bytes=1 << 28)
    a.update(over)
    return J.lib().mmdit_joint_attn_bwd(a["q"], a["n_q"], a["k"], a["v"], a["n_kv"], a["heads"], a["hd"],
                                        a["dtype"], a["scale"], a["o"], a["lse"], a["d_o"], a["dq"], a["dk"],
                                        a["dv"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(hd=96), L.MMDIT_ERR_UNSUPPORTED),
    (dict(n_kv=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(dk=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(dv=(9 << 20) + 8), L.MMDIT_ERR_INVALID_ARG),          # misaligned
    (dict(lse=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(d_o=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(dk=(7 << 20) + 2048), L.MMDIT_ERR_INVALID_ARG),      # dk overlaps dq
    (dict(dv=(6 << 20) + 1024), L.MMDIT_ERR_INVALID_ARG),      # dv overlaps d_o
    (dict(dq=(5 << 20) - 1024), L.MMDIT_ERR_INVALID_ARG),      # dq overlaps lse
    (dict(n_q=1 << 24), L.MMDIT_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), L.MMDIT_ERR_WORKSPACE),
])
def test_joint_attn_bwd_rejects_bad_arguments(over, status):
    assert _call_bwd(**over) == status
    assert J.mmdit_last_error() != ""


def test_joint_attn_fwd_rejects_bad_lse():
    lib = J.lib()
    args = [1 << 20, 10, 2 << 20, 3 << 20, 10, 2, 64, J.MMDIT_BF16, 0.125, 4 << 20]
    assert lib.mmdit_joint_attn_fwd(*args, 0, 1 << 30, 1 << 28, None) == L.MMDIT_ERR_INVALID_ARG
    assert lib.mmdit_joint_attn_fwd(*args, (5 << 20) + 2, 1 << 30, 1 << 28, None) == L.MMDIT_ERR_INVALID_ARG
    assert lib.mmdit_joint_attn_fwd(*args, (4 << 20) + 64, 1 << 30, 1 << 28, None) == L.MMDIT_ERR_INVALID_ARG


def test_bwd_workspace_plan():
    ws = J.mmdit_workspace_bytes
    n = 35050
    pad = 35072
    a256 = lambda x: (x + 255) // 256 * 256
    want = 2 * a256(24 * pad * 4) + 3 * a256(24 * 128 * pad * 2)
    assert ws(J.MMDIT_OP_JOINT_ATTN_BWD, n, n, 24, 128, J.MMDIT_BF16) == want
    assert ws(J.MMDIT_OP_JOINT_ATTN_BWD, 88, 88, 2, 64, J.MMDIT_FP32) == a256(2 * 88 * 4)
    assert ws(J.MMDIT_OP_JOINT_ATTN_BWD, 0, 64, 2, 64, J.MMDIT_BF16) == a256(2 * 64 * 64 * 2)


def test_rope_rejects_bad_descriptors():
    w = dict(WORKLOADS["480p"])
    lib = J.lib()
    good = J.rope_spec_for(w)
    bad_split = J.RopeSpec(*J.layout_segments(21, 30, 52, 1, 218, 512, (21, 218)), 24, 128, (36, 46, 46))
    assert lib.mmdit_rope3d(ctypes.byref(bad_split.desc), 256, 512, 1024, 1, None) == L.MMDIT_ERR_UNSUPPORTED
    segs, n = J.layout_segments(21, 30, 52, 1, 218, 512, (21, 218))
    segs[1]["offset"] -= 1                                            # overlaps the cond frame
    ov = J.RopeSpec(segs, n, 24, 128, (32, 48, 48))
    assert lib.mmdit_rope3d(ctypes.byref(ov.desc), 256, 512, 1024, 1, None) == L.MMDIT_ERR_INVALID_ARG
    assert "overlap" in J.mmdit_last_error()
    assert lib.mmdit_rope3d(ctypes.byref(good.desc), 256, 512, 1024, 9, None) == L.MMDIT_ERR_INVALID_ARG
    assert lib.mmdit_rope3d(ctypes.byref(good.desc), 0, 512, 1024, 1, None) == L.MMDIT_ERR_INVALID_ARG
    assert lib.mmdit_rope3d(None, 256, 512, 1024, 1, None) == L.MMDIT_ERR_INVALID_ARG


@pytest.mark.parametrize("over,status", [
    (dict(zone=(8, 8, 6)), L.MMDIT_ERR_INVALID_ARG),
    (dict(block=(2, 4, 4)), L.MMDIT_ERR_UNSUPPORTED),
    (dict(top_k=-1), L.MMDIT_ERR_INVALID_ARG),
    (dict(top_p=1.5), L.MMDIT_ERR_INVALID_ARG),
    (dict(top_p=float("nan")), L.MMDIT_ERR_INVALID_ARG),
    (dict(T=20), L.MMDIT_ERR_INVALID_ARG),
    (dict(hd=64), L.MMDIT_ERR_UNSUPPORTED),
    (dict(ws_bytes=10), L.MMDIT_ERR_WORKSPACE),
    (dict(T=32, H=256, W=272), L.MMDIT_ERR_UNSUPPORTED),    # 34816 blocks per head (max 32768)
    (dict(wait_limit=-1), L.MMDIT_ERR_INVALID_ARG),
    (dict(wait_limit=(1 << 18) + 1), L.MMDIT_ERR_INVALID_ARG),
])
def test_block_sparse_rejects_bad_arguments(over, status):
    a = dict(T=24, H=64, W=112, heads=24, hd=128, zone=(8, 8, 8), block=(4, 4, 4), top_k=32,
             top_p=0.9, ws_bytes=1 << 40, wait_limit=0)
    a.update(over)
    sd = J.sparse_desc(a["zone"], a["block"], a["top_k"], a["top_p"], a["wait_limit"])
    lib = J.lib()
    st = lib.mmdit_block_sparse_attn(1 << 20, 1 << 30, 1 << 31, a["T"], a["H"], a["W"], a["heads"],
                                     a["hd"], ctypes.byref(sd), 0.088, 1 << 36, None, None,
                                     1 << 40, a["ws_bytes"], None)
    assert st == status


def _sparse_bwd_call(**over):
    # 24 x 64 x 112 grid, 24 heads: bf16 tensors 1.06 GB, fp32 tensors 2.1 GB each
    a = dict(q=1 << 32, k=2 << 32, v=3 << 32, o=4 << 32, lse=5 << 32, d_o=6 << 32, mask=7 << 32,
             dq=8 << 32, dk=9 << 32, dv=10 << 32, T=24, H=64, W=112, heads=24, hd=128, scale=0.088,
             ws=1 << 40, ws_bytes=1 << 38)
    a.update(over)
    sd = J.sparse_desc()
    return J.lib().mmdit_block_sparse_attn_bwd(a["q"], a["k"], a["v"], a["T"], a["H"], a["W"], a["heads"],
                                               a["hd"], ctypes.byref(sd), a["scale"], a["o"], a["lse"],
                                               a["d_o"], a["mask"], a["dq"], a["dk"], a["dv"], a["ws"],
                                               a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(hd=64), L.MMDIT_ERR_UNSUPPORTED),
    (dict(T=20), L.MMDIT_ERR_INVALID_ARG),
    (dict(scale=-1.0), L.MMDIT_ERR_INVALID_ARG),
    (dict(mask=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(lse=(5 << 32) + 2), L.MMDIT_ERR_INVALID_ARG),
    (dict(dv=(10 << 32) + 8), L.MMDIT_ERR_INVALID_ARG),     # misaligned
    (dict(dk=(8 << 32) + 4096), L.MMDIT_ERR_INVALID_ARG),   # dk overlaps dq
    (dict(dq=(6 << 32) + 4096), L.MMDIT_ERR_INVALID_ARG),   # dq overlaps d_o
    (dict(dv=(7 << 32) - 4096), L.MMDIT_ERR_INVALID_ARG),   # dv runs into the mask
    (dict(ws_bytes=1000), L.MMDIT_ERR_WORKSPACE),
])
def test_block_sparse_bwd_rejects_bad_arguments(over, status):
    assert _sparse_bwd_call(**over) == status
    assert J.mmdit_last_error() != ""


def test_block_sparse_fwd_requires_lse_and_mask():
    lib = J.lib()
    sd = J.sparse_desc()
    args = [1 << 32, 2 << 32, 3 << 32, 24, 64, 112, 24, 128, ctypes.byref(sd), 0.088, 4 << 32]
    assert lib.mmdit_block_sparse_attn_fwd(*args, 0, 7 << 32, None, 1 << 40, 1 << 38, None) == L.MMDIT_ERR_INVALID_ARG
    assert lib.mmdit_block_sparse_attn_fwd(*args, 5 << 32, 0, None, 1 << 40, 1 << 38, None) == L.MMDIT_ERR_INVALID_ARG
    # lse inside o
    assert lib.mmdit_block_sparse_attn_fwd(*args, (4 << 32) + 256, 7 << 32, None, 1 << 40, 1 << 38,
                                           None) == L.MMDIT_ERR_INVALID_ARG


def test_sparse_bwd_workspace_plan():
    a256 = lambda x: (x + 255) // 256 * 256
    n, nb, h = 172032, 2688, 24
    # D, lse2; Q^T, dO^T, K^T block images; transposed bitmask; dispatch orders of the
    # 672 groups of 4 query blocks and of 4 key blocks per head; Q, dO, K, V row images
    want = (2 * a256(h * n * 4) + 7 * a256(h * nb * 128 * 64 * 2) + a256(h * nb * 84 * 4)
            + 2 * a256(h * 672 * 4))
    sd = J.sparse_desc()
    assert J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, n, n, h, 128, J.MMDIT_BF16, sd) == want


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.lib()


def test_block_sparse_workspace_query_matches_the_call():
    # the call's own requirement (quoted in its error) equals the size query
    sd = J.sparse_desc()
    T, H, W, h = 24, 64, 112, 24
    need = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN, T * H * W, T * H * W, h, 128, J.MMDIT_BF16, sd)
    lib = J.lib()
    st = lib.mmdit_block_sparse_attn(1 << 20, 1 << 30, 1 << 31, T, H, W, h, 128, ctypes.byref(sd), 0.088,
                                     1 << 36, None, None, 1 << 40, need - 1, None)
    assert st == L.MMDIT_ERR_WORKSPACE
    assert int(re.search(r"required (\d+)", J.mmdit_last_error()).group(1)) == need


def _adaptive_call(**over):
    # 24 x 64 x 112 grid, 24 heads: bf16 tensors 1.06 GB, fp32 o 2.1 GB
    a = dict(q=1 << 32, k=2 << 32, v=3 << 32, a=4 << 32, T=24, H=64, W=112, heads=24, hd=128, top_k=32,
             top_p=0.9, scale=0.088, o=5 << 32, lse=None, shape=6 << 32, tblock=7 << 32, nblocks=8 << 32,
             mask=None, count=None, ws=1 << 40, ws_bytes=1 << 38)
    a.update(over)
    return J.lib().mmdit_block_sparse_attn_adaptive(
        a["q"], a["k"], a["v"], a["a"], a["T"], a["H"], a["W"], a["heads"], a["hd"], a["top_k"], a["top_p"],
        a["scale"], a["o"], a["lse"], a["shape"], a["tblock"], a["nblocks"], a["mask"], a["count"], a["ws"],
        a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(T=20), L.MMDIT_ERR_INVALID_ARG),                  # not whole 8 x 8 x 8 zones
    (dict(W=100), L.MMDIT_ERR_INVALID_ARG),
    (dict(hd=64), L.MMDIT_ERR_UNSUPPORTED),
    (dict(T=64, H=128, W=272), L.MMDIT_ERR_UNSUPPORTED),    # 4352 zones, 34816 tiles (max 32768)
    (dict(top_k=-1), L.MMDIT_ERR_INVALID_ARG),
    (dict(top_p=1.5), L.MMDIT_ERR_INVALID_ARG),
    (dict(scale=-0.5), L.MMDIT_ERR_INVALID_ARG),
    (dict(a=(4 << 32) + 2), L.MMDIT_ERR_INVALID_ARG),       # misaligned norms
    (dict(lse=(9 << 32) + 2), L.MMDIT_ERR_INVALID_ARG),
    (dict(tblock=(5 << 32) + 1024), L.MMDIT_ERR_INVALID_ARG),   # tile_block inside o
    (dict(shape=(1 << 32) + 64), L.MMDIT_ERR_INVALID_ARG),      # zone_shape inside q
    (dict(a=(5 << 32) + 4096), L.MMDIT_ERR_INVALID_ARG),         # o overwrites the norms
    (dict(nblocks=(7 << 32) + 2), L.MMDIT_ERR_INVALID_ARG),
    (dict(o=(2 << 32) + 1024), L.MMDIT_ERR_INVALID_ARG),         # o aliases k
    (dict(ws_bytes=1000), L.MMDIT_ERR_WORKSPACE),
])
def test_block_sparse_adaptive_rejects_bad_arguments(over, status):
    assert _adaptive_call(**over) == status
    assert J.mmdit_last_error() != ""


def test_adaptive_workspace_plan_and_query():
    a256 = lambda x: (x + 255) // 256 * 256
    n, h = 172032, 24
    nt, nz = n // 64, n // 512
    sd = J.sparse_desc()
    uniform = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN, n, n, h, 128, J.MMDIT_BF16, sd)
    extra = a256(nz * 6 * 3 * 8) + a256(nz * 4 * 8) + a256(nz) + a256(nt) + 2 * a256(nt * 4) + 256
    need = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, n, 0, h, 128, J.MMDIT_BF16, None)
    assert need == uniform + extra
    assert _adaptive_call(ws_bytes=need - 1) == L.MMDIT_ERR_WORKSPACE
    assert int(re.search(r"required (\d+)", J.mmdit_last_error()).group(1)) == need


@pytest.mark.parametrize("args,status", [
    ((1 << 32, 10, 6, 2 << 32), L.MMDIT_ERR_INVALID_ARG),          # width not a multiple of 4
    ((1 << 32, 10, 0, 2 << 32), L.MMDIT_ERR_INVALID_ARG),
    ((1 << 32, -1, 8, 2 << 32), L.MMDIT_ERR_INVALID_ARG),
    (((1 << 32) + 8, 10, 8, 2 << 32), L.MMDIT_ERR_INVALID_ARG),    # x not 16-byte aligned
    ((1 << 32, 10, 8, (1 << 32) + 64), L.MMDIT_ERR_INVALID_ARG),   # out inside x
    ((None, 10, 8, 2 << 32), L.MMDIT_ERR_INVALID_ARG),
    ((None, 0, 8, None), L.MMDIT_OK),                               # nothing to do
])
def test_token_norms_checks(args, status):
    assert J.lib().mmdit_token_norms(*args, None) == status


def _adaptive_bwd_call(**over):
    a = dict(q=1 << 32, k=2 << 32, v=3 << 32, o=4 << 32, lse=5 << 32, d_o=6 << 32, shape=7 << 32,
             mask=(7 << 32) + (1 << 20), dq=8 << 32, dk=9 << 32, dv=10 << 32, T=24, H=64, W=112, heads=24, hd=128,
             scale=0.088, ws=1 << 40, ws_bytes=1 << 39)
    a.update(over)
    return J.lib().mmdit_block_sparse_attn_adaptive_bwd(
        a["q"], a["k"], a["v"], a["T"], a["H"], a["W"], a["heads"], a["hd"], a["scale"], a["o"], a["lse"],
        a["d_o"], a["shape"], a["mask"], a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(T=20), L.MMDIT_ERR_INVALID_ARG),
    (dict(T=64, H=128, W=272), L.MMDIT_ERR_UNSUPPORTED),    # 4352 zones (max 4096)
    (dict(hd=64), L.MMDIT_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), L.MMDIT_ERR_INVALID_ARG),
    (dict(shape=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(lse=0), L.MMDIT_ERR_INVALID_ARG),
    (dict(mask=(7 << 32) + (1 << 20) + 2), L.MMDIT_ERR_INVALID_ARG),
    (dict(dq=(8 << 32) + 8), L.MMDIT_ERR_INVALID_ARG),
    (dict(dk=(8 << 32) + 4096), L.MMDIT_ERR_INVALID_ARG),          # dk overlaps dq
    (dict(dv=(7 << 32) - 1024), L.MMDIT_ERR_INVALID_ARG),          # dv runs into zone_shape
    (dict(ws_bytes=1000), L.MMDIT_ERR_WORKSPACE),
])
def test_block_sparse_adaptive_bwd_rejects_bad_arguments(over, status):
    assert _adaptive_bwd_call(**over) == status
    assert J.mmdit_last_error() != ""


def test_adaptive_bwd_workspace_plan():
    a256 = lambda x: (x + 255) // 256 * 256
    n, nb, h = 172032, 2688, 24
    hb = n * h * 128 * 2
    uniform_bwd = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, n, n, h, 128, J.MMDIT_BF16,
                                          J.sparse_desc())
    # the tile table (first token int32, log2 edges uint8 per 64-token tile)
    # and the uniform backward's workspace over the tiles: no permuted copies
    want = a256(nb * 4) + a256(nb) + a256(uniform_bwd)
    need = J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD, n, 0, h, 128, J.MMDIT_BF16, None)
    assert need == want
    assert need < uniform_bwd + hb
    assert _adaptive_bwd_call(ws_bytes=need - 1) == L.MMDIT_ERR_WORKSPACE


def _tile_tokens(H, W, base, dims):
    """Tokens of one tile from its first token and log2 edges (the header's formula)."""
    lt, lh, lw = dims & 3, (dims >> 2) & 3, (dims >> 4) & 3
    out = []
    for r in range(64):
        a, b, c = r >> (lh + lw), (r >> lw) & ((1 << lh) - 1), r & ((1 << lw) - 1)
        out.append(int(base) + (a * H + b) * W + c)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_adaptive_tile_table_matches_oracle_partition(seed):
    """The library's tile arithmetic (the same functions its kernels run)
    reproduces the oracle's blocks: the tiles of block b hold exactly the
    oracle's tokens of block b, and every zone has 8 tiles."""
    from oracle import adaptive_blocks as AD
    rng = np.random.default_rng(seed)
    T, H, W = 8 * int(rng.integers(1, 3)), 8 * int(rng.integers(1, 4)), 8 * int(rng.integers(1, 4))
    nz = T * H * W // 512
    codes = np.arange(nz) % 16 if seed == 0 else rng.integers(0, 16, nz)
    base, dims, block = J.mmdit_adaptive_tile_table(T, H, W, codes.astype(np.uint8))
    blocks, _ = AD.adaptive_block_tokens(T, H, W, codes)
    assert block.max() + 1 == len(blocks) and np.all(np.diff(block) >= 0)
    got = {}
    for s in range(len(base)):
        got.setdefault(int(block[s]), []).extend(_tile_tokens(H, W, base[s], int(dims[s])))
    for b, toks in enumerate(blocks):
        assert sorted(got[b]) == sorted(toks.tolist()), (seed, b)


def test_adaptive_tile_table_rejects_bad_input():
    with pytest.raises(L.MmditError, match="multiples of 8"):
        J.mmdit_adaptive_tile_table(8, 8, 12, [3])
    with pytest.raises(L.MmditError, match="shape code"):
        J.mmdit_adaptive_tile_table(8, 8, 16, [3, 16])


def test_noalloc_checks_run_before_any_device_call():
    """The allocation-free joint attention validates its arguments and the
    scratch size on the host first: these fail without touching a GPU."""
    lib = J.lib()
    call = lambda n_q, n_kv, heads, hd, q=1 << 30, o=1 << 34: lib.mmdit_joint_attn_noalloc(
        q, n_q, 2 << 30, 3 << 30, n_kv, heads, hd, J.MMDIT_BF16, 0.0, o, None)
    assert call(8, 11000, 24, 128) == L.MMDIT_ERR_WORKSPACE
    assert "scratch" in J.mmdit_last_error() and str(64 << 20) in J.mmdit_last_error()
    assert call(8, 1000, 24, 96) == L.MMDIT_ERR_UNSUPPORTED
    assert call(8, 1000, 24, 128, q=(1 << 30) + 8) == L.MMDIT_ERR_INVALID_ARG
    assert call(8, 1000, 24, 128, o=(1 << 30) + 256) == L.MMDIT_ERR_INVALID_ARG     # o aliases q
    assert J.MMDIT_NOALLOC_SCRATCH_BYTES == 64 << 20


def test_fused_rope_attention_checks():
    """mmdit_joint_attn_rope validates on the host before enqueueing anything."""
    w = WORKLOADS["block"]
    spec = J.rope_spec_for(w)
    lib = J.lib()
    n, h, d = 5850, 24, 128
    tb = n * h * d * 2
    need = J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_ROPE, n, n, h, d, J.MMDIT_BF16)
    assert need == J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16) + \
        (tb + 255) // 256 * 256

    def call(q=1 << 32, k=2 << 32, v=3 << 32, o=4 << 32, qr=5 << 32, kr=6 << 32, dtype=J.MMDIT_BF16, tab=7 << 32,
             ws=8 << 32, wsb=need):
        return lib.mmdit_joint_attn_rope(ctypes.byref(spec.desc), tab, q, k, v, dtype, 0.0, o, qr, kr, ws, wsb, None)
    assert call(dtype=J.MMDIT_FP32) == L.MMDIT_ERR_UNSUPPORTED
    assert call(qr=1 << 32) == L.MMDIT_ERR_INVALID_ARG                    # q_rot = q (in place) is refused
    assert call(kr=(5 << 32) + 4096) == L.MMDIT_ERR_INVALID_ARG           # k_rot overlaps q_rot
    assert call(qr=(4 << 32) + tb) == L.MMDIT_ERR_INVALID_ARG             # q_rot inside o
    assert call(kr=(6 << 32) + 8) == L.MMDIT_ERR_INVALID_ARG              # misaligned
    assert call(tab=0) == L.MMDIT_ERR_INVALID_ARG
    assert call(wsb=need - 1) == L.MMDIT_ERR_WORKSPACE
    assert call(ws=(5 << 32) - 4096) == L.MMDIT_ERR_INVALID_ARG           # workspace runs into q_rot
