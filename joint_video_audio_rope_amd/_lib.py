"""ctypes binding of libmmdit.so (include/mmdit.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Tensors are torch tensors used as device memory.  Calls run on
`stream` when given (outputs and workspace the wrapper allocates are then
taken on that stream), else on torch's current stream.  softmax_scale=None
passes 0, for which the library uses 1/sqrt(head_dim).  There is no
fallback: if the library is missing, every call raises.
"""
import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmdit.so")

MMDIT_OK, MMDIT_ERR_INVALID_ARG, MMDIT_ERR_UNSUPPORTED, MMDIT_ERR_WORKSPACE, MMDIT_ERR_HIP = range(5)
MMDIT_NOALLOC_SCRATCH_BYTES = 64 << 20
MMDIT_FP32, MMDIT_BF16 = 0, 1
MMDIT_SEG_VIDEO, MMDIT_SEG_AUDIO, MMDIT_SEG_TEXT = 0, 1, 2
(MMDIT_OP_JOINT_ATTN, MMDIT_OP_AV_CROSS_ATTN, MMDIT_OP_BLOCK_SPARSE_ATTN, MMDIT_OP_JOINT_ATTN_BWD,
 MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD,
 MMDIT_OP_JOINT_ATTN_ROPE) = range(8)

# (b_T, b_H, b_W) of the content-adaptive shape codes, in code order
ADAPTIVE_SHAPES = ((2, 4, 8), (2, 8, 4), (4, 2, 8), (4, 4, 4), (4, 8, 2), (8, 2, 4), (8, 4, 2),
                   (2, 8, 8), (4, 4, 8), (4, 8, 4), (8, 2, 8), (8, 4, 4), (8, 8, 2),
                   (4, 8, 8), (8, 4, 8), (8, 8, 4))
MMDIT_MAX_SEGMENTS = 16

_STATUS = {1: "MMDIT_ERR_INVALID_ARG", 2: "MMDIT_ERR_UNSUPPORTED", 3: "MMDIT_ERR_WORKSPACE",
           4: "MMDIT_ERR_HIP"}


class MmditError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), msg))
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("offset", ctypes.c_int64), ("count", ctypes.c_int64),
                ("t0", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("t_scale", ctypes.c_double)]


class RopeDesc(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_t", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32), ("theta", ctypes.c_double),
                ("segs", ctypes.POINTER(Segment)), ("n_segs", ctypes.c_int32),
                ("n_tokens", ctypes.c_int64)]


class SparseDesc(ctypes.Structure):
    _fields_ = [("zone", ctypes.c_int32 * 3), ("block", ctypes.c_int32 * 3),
                ("top_k", ctypes.c_int32), ("top_p", ctypes.c_double), ("wait_limit", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmmdit.so is not built (%s); run "
                               "`python -m joint_video_audio_rope_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_size_t, ctypes.c_float, ctypes.c_double)
        L.mmdit_abi_version.restype = i32
        L.mmdit_abi_version.argtypes = []
        L.mmdit_last_error.restype = ctypes.c_char_p
        L.mmdit_last_error.argtypes = []
        L.mmdit_rope3d_table_floats.restype = sz
        L.mmdit_rope3d_table_floats.argtypes = [ctypes.POINTER(RopeDesc)]
        L.mmdit_rope3d_build_table.restype = i32
        L.mmdit_rope3d_build_table.argtypes = [ctypes.POINTER(RopeDesc), vp]
        L.mmdit_workspace_bytes.restype = sz
        L.mmdit_workspace_bytes.argtypes = [i32, i64, i64, i32, i32, i32, ctypes.POINTER(SparseDesc)]
        L.mmdit_rope3d.restype = i32
        L.mmdit_rope3d.argtypes = [ctypes.POINTER(RopeDesc), vp, vp, vp, i32, vp]
        L.mmdit_joint_attn.restype = i32
        L.mmdit_joint_attn.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, f32, vp, vp, sz, vp]
        L.mmdit_joint_attn_rope.restype = i32
        L.mmdit_joint_attn_rope.argtypes = [ctypes.POINTER(RopeDesc), vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, sz,
                                            vp]
        L.mmdit_joint_attn_noalloc.restype = i32
        L.mmdit_joint_attn_noalloc.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, f32, vp, vp]
        L.mmdit_joint_attn_fwd.restype = i32
        L.mmdit_joint_attn_fwd.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, f32, vp, vp, vp, sz, vp]
        L.mmdit_joint_attn_bwd.restype = i32
        L.mmdit_joint_attn_bwd.argtypes = [vp, i64, vp, vp, i64, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                           vp, sz, vp]
        L.mmdit_av_cross_attn.restype = i32
        L.mmdit_av_cross_attn.argtypes = [vp, vp, vp, i64, vp, vp, vp, i64, i32, i32, i32, f32,
                                          vp, vp, vp, sz, vp]
        L.mmdit_block_sparse_attn.restype = i32
        L.mmdit_block_sparse_attn.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(SparseDesc), f64, vp, vp, vp, vp, sz, vp]
        L.mmdit_block_sparse_attn_fwd.restype = i32
        L.mmdit_block_sparse_attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(SparseDesc),
                                                  f64, vp, vp, vp, vp, vp, sz, vp]
        L.mmdit_block_sparse_attn_bwd.restype = i32
        L.mmdit_block_sparse_attn_bwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(SparseDesc),
                                                  f64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mmdit_adaptive_tile_table.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.mmdit_adaptive_tile_table.restype = i32
        L.mmdit_token_norms.argtypes = [vp, i64, i64, vp, vp]
        L.mmdit_token_norms.restype = i32
        L.mmdit_block_sparse_attn_adaptive.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, f64,
                                                       vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mmdit_block_sparse_attn_adaptive.restype = i32
        L.mmdit_block_sparse_attn_adaptive_bwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f64, vp, vp, vp, vp,
                                                           vp, vp, vp, vp, vp, sz, vp]
        L.mmdit_block_sparse_attn_adaptive_bwd.restype = i32
        _lib = L
    return _lib


def _check(status):
    if status != MMDIT_OK:
        raise MmditError(status, lib().mmdit_last_error().decode())


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return MMDIT_BF16
    if t.dtype == torch.float32:
        return MMDIT_FP32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for the tensors a wrapper allocates (outputs, workspace): they
    are taken on the stream the kernels run on, so the caching allocator does
    not hand a freed workspace to other work before those kernels are done."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace of %d bytes needed" % nbytes)
    return ws, ws.numel() * ws.element_size()


# ---- host-only calls ---------------------------------------------------------
def mmdit_abi_version():
    return lib().mmdit_abi_version()


def mmdit_last_error():
    return lib().mmdit_last_error().decode()


def layout_segments(T, H, W, n_cond_frames=0, n_audio=0, n_text=0, audio_scale=None):
    """Segments of one joint sequence [cond | video | audio | text].

    Conditioning frames form a VIDEO segment at t0 = -n_cond_frames (so one
    frame sits at t = -1); generated frames start at t = 0; audio token j sits
    at j * audio_scale, audio_scale given as (num, den) (e.g. (21, 218) for
    218 audio tokens over 21 frames); required when n_audio > 0.
    """
    segs = []
    off = 0
    if n_cond_frames:
        n = n_cond_frames * H * W
        segs.append(dict(kind=MMDIT_SEG_VIDEO, offset=off, count=n, t0=-n_cond_frames,
                         T=n_cond_frames, H=H, W=W))
        off += n
    n = T * H * W
    segs.append(dict(kind=MMDIT_SEG_VIDEO, offset=off, count=n, t0=0, T=T, H=H, W=W))
    off += n
    if n_audio:
        if audio_scale is None:
            raise ValueError("layout_segments: audio_scale (num, den) is required with audio tokens")
        num, den = audio_scale
        segs.append(dict(kind=MMDIT_SEG_AUDIO, offset=off, count=n_audio, t_scale=num / den))
        off += n_audio
    if n_text:
        segs.append(dict(kind=MMDIT_SEG_TEXT, offset=off, count=n_text))
        off += n_text
    return segs, off


class RopeSpec:
    """A RoPE descriptor kept alive together with its segment array."""

    def __init__(self, segments, n_tokens, heads, head_dim, split, theta=10000.0):
        arr = (Segment * max(1, len(segments)))()
        for i, s in enumerate(segments):
            arr[i] = Segment(s["kind"], s["offset"], s["count"], s.get("t0", 0), s.get("T", 0),
                             s.get("H", 0), s.get("W", 0), float(s.get("t_scale", 0.0)))
        self._segs = arr
        self.desc = RopeDesc(heads, head_dim, split[0], split[1], split[2], float(theta),
                             ctypes.cast(arr, ctypes.POINTER(Segment)), len(segments), n_tokens)
        self._dev_table = {}

    def table_floats(self):
        return lib().mmdit_rope3d_table_floats(ctypes.byref(self.desc))

    def host_table(self):
        n = self.table_floats()
        buf = torch.empty(max(n, 1), dtype=torch.float32)
        _check(lib().mmdit_rope3d_build_table(ctypes.byref(self.desc), ctypes.c_void_p(buf.data_ptr())))
        return buf[:n]

    def device_table(self, device):
        dev = torch.device(device)
        if dev not in self._dev_table:
            self._dev_table[dev] = self.host_table().to(dev)
        return self._dev_table[dev]


def mmdit_rope3d_table_floats(spec):
    return spec.table_floats()


def mmdit_rope3d_build_table(spec):
    """Host (cos, sin) table as a CPU float32 tensor."""
    return spec.host_table()


def mmdit_workspace_bytes(op, n_q, n_kv, heads, head_dim, dtype, sparse=None):
    sp = None if sparse is None else ctypes.byref(sparse)
    return lib().mmdit_workspace_bytes(op, n_q, n_kv, heads, head_dim, dtype, sp)


# ---- device calls ------------------------------------------------------------
def mmdit_rope3d(spec, q, k, stream=None):
    """Rotate q and k in place ([n_tokens, heads, head_dim], same dtype)."""
    assert q.is_contiguous() and k.is_contiguous() and q.dtype == k.dtype and q.shape == k.shape
    tab = spec.device_table(q.device)
    _check(lib().mmdit_rope3d(ctypes.byref(spec.desc), _ptr(tab), _ptr(q), _ptr(k), _dtype(q),
                              _stream(stream)))
    return q, k


def _scale(softmax_scale):
    """0 asks the library for its default, 1/sqrt(head_dim)."""
    return 0.0 if softmax_scale is None else float(softmax_scale)


def mmdit_joint_attn(q, k, v, softmax_scale=None, o=None, ws=None, stream=None):
    """Softmax attention of q [n_q, h, d] against k, v [n_kv, h, d]; fp32 output."""
    n_q, h, d = q.shape
    n_kv = k.shape[0]
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    assert k.shape == v.shape == (n_kv, h, d) and q.dtype == k.dtype == v.dtype
    with _on(stream):
        if o is None:
            o = torch.empty((n_q, h, d), dtype=torch.float32, device=q.device)
        need = mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN, n_q, n_kv, h, d, _dtype(q))
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_joint_attn(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, h, d, _dtype(q), _scale(softmax_scale),
                                      _ptr(o), _ptr(ws), wsb, _stream(stream)))
    return o


def mmdit_joint_attn_rope(spec, q, k, v, softmax_scale=None, o=None, q_rot=None, k_rot=None, want_rotated=True,
                          ws=None, stream=None):
    """Joint self-attention with the RoPE of `spec` fused in: returns (o fp32,
    q_rot, k_rot), o the attention of the rotated q, k (bf16, unchanged) over
    v, and q_rot, k_rot the rotated tensors (None unless want_rotated or
    given)."""
    n, h, d = q.shape
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16 and q.shape == k.shape == v.shape
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    tab = spec.device_table(q.device)
    with _on(stream):
        if o is None:
            o = torch.empty((n, h, d), dtype=torch.float32, device=q.device)
        if want_rotated and q_rot is None:
            q_rot = torch.empty_like(q)
        if want_rotated and k_rot is None:
            k_rot = torch.empty_like(k)
        need = mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN_ROPE, n, n, h, d, MMDIT_BF16)
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_joint_attn_rope(ctypes.byref(spec.desc), _ptr(tab), _ptr(q), _ptr(k), _ptr(v), MMDIT_BF16,
                                           _scale(softmax_scale), _ptr(o), _ptr(q_rot), _ptr(k_rot), _ptr(ws), wsb,
                                           _stream(stream)))
    return o, q_rot, k_rot


def mmdit_joint_attn_noalloc(q, k, v, softmax_scale=None, o=None, stream=None):
    """mmdit_joint_attn with the library's fixed per-GPU scratch instead of a
    workspace (for callers that cannot allocate; pass o to allocate nothing
    here either).  Calls that overlap on one GPU race."""
    n_q, h, d = q.shape
    n_kv = k.shape[0]
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    assert k.shape == v.shape == (n_kv, h, d) and q.dtype == k.dtype == v.dtype
    with _on(stream):
        if o is None:
            o = torch.empty((n_q, h, d), dtype=torch.float32, device=q.device)
        _check(lib().mmdit_joint_attn_noalloc(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, h, d, _dtype(q),
                                              _scale(softmax_scale), _ptr(o), _stream(stream)))
    return o


def mmdit_joint_attn_fwd(q, k, v, softmax_scale=None, o=None, lse=None, ws=None, stream=None):
    """mmdit_joint_attn plus the log-sum-exp: returns (o fp32 [n_q, h, d],
    lse fp32 [h, n_q], natural log)."""
    n_q, h, d = q.shape
    n_kv = k.shape[0]
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    assert k.shape == v.shape == (n_kv, h, d) and q.dtype == k.dtype == v.dtype
    with _on(stream):
        if o is None:
            o = torch.empty((n_q, h, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((h, n_q), dtype=torch.float32, device=q.device)
        need = mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN, n_q, n_kv, h, d, _dtype(q))
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_joint_attn_fwd(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, h, d, _dtype(q),
                                          _scale(softmax_scale), _ptr(o), _ptr(lse), _ptr(ws), wsb, _stream(stream)))
    return o, lse


def mmdit_joint_attn_bwd(q, k, v, o, lse, d_o, softmax_scale=None, dq=None, dk=None, dv=None, ws=None,
                         stream=None):
    """Gradients (dq, dk, dv), fp32, of the attention that mmdit_joint_attn_fwd
    computed as (o, lse); d_o has the dtype of q."""
    n_q, h, d = q.shape
    n_kv = k.shape[0]
    for t in (q, k, v, o, lse, d_o):
        assert t.is_contiguous()
    assert k.shape == v.shape == (n_kv, h, d) and q.dtype == k.dtype == v.dtype == d_o.dtype
    assert o.shape == d_o.shape == (n_q, h, d) and o.dtype == torch.float32
    assert lse.shape == (h, n_q) and lse.dtype == torch.float32
    with _on(stream):
        if dq is None:
            dq = torch.empty((n_q, h, d), dtype=torch.float32, device=q.device)
        if dk is None:
            dk = torch.empty((n_kv, h, d), dtype=torch.float32, device=q.device)
        if dv is None:
            dv = torch.empty((n_kv, h, d), dtype=torch.float32, device=q.device)
        need = mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN_BWD, n_q, n_kv, h, d, _dtype(q))
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_joint_attn_bwd(_ptr(q), n_q, _ptr(k), _ptr(v), n_kv, h, d, _dtype(q),
                                          _scale(softmax_scale), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(ws), wsb, _stream(stream)))
    return dq, dk, dv


def mmdit_av_cross_attn(q_v, k_v, v_v, q_a, k_a, v_a, softmax_scale=None, o_video=None,
                        o_audio=None, ws=None, stream=None):
    """Video queries -> audio keys and audio queries -> video keys; fp32 outputs."""
    n_v, h, d = q_v.shape
    n_a = q_a.shape[0]
    for t in (q_v, k_v, v_v, q_a, k_a, v_a):
        assert t.is_contiguous() and t.dtype == q_v.dtype
    with _on(stream):
        if o_video is None:
            o_video = torch.empty((n_v, h, d), dtype=torch.float32, device=q_v.device)
        if o_audio is None:
            o_audio = torch.empty((n_a, h, d), dtype=torch.float32, device=q_v.device)
        need = mmdit_workspace_bytes(MMDIT_OP_AV_CROSS_ATTN, n_v, n_a, h, d, _dtype(q_v))
        ws, wsb = _ws(need, q_v.device, ws)
        _check(lib().mmdit_av_cross_attn(_ptr(q_v), _ptr(k_v), _ptr(v_v), n_v, _ptr(q_a), _ptr(k_a),
                                         _ptr(v_a), n_a, h, d, _dtype(q_v), _scale(softmax_scale), _ptr(o_video),
                                         _ptr(o_audio), _ptr(ws), wsb, _stream(stream)))
    return o_video, o_audio


def sparse_desc(zone=(8, 8, 8), block=(4, 4, 4), top_k=32, top_p=0.9, wait_limit=0):
    sd = SparseDesc()
    for i in range(3):
        sd.zone[i] = zone[i]
        sd.block[i] = block[i]
    sd.top_k = top_k
    sd.top_p = top_p
    sd.wait_limit = wait_limit
    return sd


def mmdit_block_sparse_attn(q, k, v, T, H, W, zone=(8, 8, 8), block=(4, 4, 4), top_k=32,
                            top_p=0.9, softmax_scale=None, o=None, sel_mask=None, sel_count=None,
                            ws=None, stream=None, want_selection=True, wait_limit=0):
    """Block-sparse self-attention over a T x H x W raster grid.

    Returns (o fp32, sel_mask uint32-as-int32 [h, nb, ceil(nb/32)], sel_count int32 [h, nb]).
    wait_limit: see mmdit_sparse_desc (0: the library's bound; tests of the
    failure path only).
    """
    n, h, d = q.shape
    assert n == T * H * W and q.dtype == torch.bfloat16
    sd = sparse_desc(zone, block, top_k, top_p, wait_limit)
    nb = n // (block[0] * block[1] * block[2])
    with _on(stream):
        if o is None:
            o = torch.empty((n, h, d), dtype=torch.float32, device=q.device)
        if want_selection and sel_mask is None:
            sel_mask = torch.empty((h, nb, (nb + 31) // 32), dtype=torch.int32, device=q.device)
        if want_selection and sel_count is None:
            sel_count = torch.empty((h, nb), dtype=torch.int32, device=q.device)
        need = mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN, n, n, h, d, MMDIT_BF16, sd)
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_block_sparse_attn(_ptr(q), _ptr(k), _ptr(v), T, H, W, h, d,
                                             ctypes.byref(sd), _scale(softmax_scale), _ptr(o), _ptr(sel_mask),
                                             _ptr(sel_count), _ptr(ws), wsb, _stream(stream)))
    return o, sel_mask, sel_count


def mmdit_block_sparse_attn_fwd(q, k, v, T, H, W, zone=(8, 8, 8), block=(4, 4, 4), top_k=32, top_p=0.9,
                                softmax_scale=None, o=None, lse=None, sel_mask=None, sel_count=None, ws=None,
                                stream=None, wait_limit=0):
    """Block-sparse attention for a training step: (o fp32, lse fp32 [h, n],
    sel_mask, sel_count); sel_mask feeds mmdit_block_sparse_attn_bwd."""
    n, h, d = q.shape
    assert n == T * H * W and q.dtype == torch.bfloat16
    sd = sparse_desc(zone, block, top_k, top_p, wait_limit)
    nb = n // (block[0] * block[1] * block[2])
    with _on(stream):
        if o is None:
            o = torch.empty((n, h, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((h, n), dtype=torch.float32, device=q.device)
        if sel_mask is None:
            sel_mask = torch.empty((h, nb, (nb + 31) // 32), dtype=torch.int32, device=q.device)
        if sel_count is None:
            sel_count = torch.empty((h, nb), dtype=torch.int32, device=q.device)
        need = mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN, n, n, h, d, MMDIT_BF16, sd)
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), T, H, W, h, d, ctypes.byref(sd),
                                                 _scale(softmax_scale), _ptr(o), _ptr(lse), _ptr(sel_mask),
                                                 _ptr(sel_count), _ptr(ws), wsb, _stream(stream)))
    return o, lse, sel_mask, sel_count


def mmdit_adaptive_tile_table(T, H, W, zone_shape):
    """Host-side tile table of an adaptive grid: (tile_base int32 [nt],
    tile_dims uint8 [nt], tile_block int32 [nt]) numpy arrays for the zone
    shape codes (uint8, any array-like of T*H*W/512 entries)."""
    import numpy as np
    codes = np.ascontiguousarray(np.asarray(zone_shape, dtype=np.uint8))
    nt = T * H * W // 64
    base = np.empty(nt, dtype=np.int32)
    dims = np.empty(nt, dtype=np.uint8)
    block = np.empty(nt, dtype=np.int32)
    cp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().mmdit_adaptive_tile_table(T, H, W, cp(codes), cp(base), cp(dims), cp(block)))
    return base, dims, block


def mmdit_token_norms(x, out=None, stream=None):
    """out[t] = ||x[t]||_2 over all other dimensions of an fp32 tensor
    [n, ...] (e.g. the video output of mmdit_av_cross_attn)."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    n = x.shape[0]
    width = x.numel() // max(n, 1)
    with _on(stream):
        if out is None:
            out = torch.empty(n, dtype=torch.float32, device=x.device)
        _check(lib().mmdit_token_norms(_ptr(x), n, width, _ptr(out), _stream(stream)))
    return out


def mmdit_block_sparse_attn_adaptive(q, k, v, T, H, W, a_norm=None, top_k=32, top_p=0.9, softmax_scale=None,
                                     o=None, lse=None, want_lse=False, ws=None, stream=None):
    """Block-sparse attention with content-adaptive block shapes.  Returns a
    dict: o fp32 [n, h, d], lse ([h, n] or None), zone_shape uint8 [nz] codes
    into ADAPTIVE_SHAPES, tile_block int32 [nt], n_blocks int32 [1], sel_mask
    int32 [h, nt, ceil(nt/32)] (tile level), sel_count int32 [h, nt]."""
    n, h, d = q.shape
    assert n == T * H * W and q.dtype == k.dtype == v.dtype == torch.bfloat16
    for t in (q, k, v):
        assert t.is_contiguous()
    if a_norm is not None:
        assert a_norm.dtype == torch.float32 and a_norm.numel() == n and a_norm.is_contiguous()
    nt, nz = n // 64, n // 512
    dev = q.device
    with _on(stream):
        if o is None:
            o = torch.empty((n, h, d), dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty((h, n), dtype=torch.float32, device=dev)
        out = dict(o=o, lse=lse,
                   zone_shape=torch.empty(nz, dtype=torch.uint8, device=dev),
                   tile_block=torch.empty(nt, dtype=torch.int32, device=dev),
                   n_blocks=torch.empty(1, dtype=torch.int32, device=dev),
                   sel_mask=torch.empty((h, nt, (nt + 31) // 32), dtype=torch.int32, device=dev),
                   sel_count=torch.empty((h, nt), dtype=torch.int32, device=dev))
        need = mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, n, 0, h, d, MMDIT_BF16, None)
        ws, wsb = _ws(need, dev, ws)
        _check(lib().mmdit_block_sparse_attn_adaptive(
            _ptr(q), _ptr(k), _ptr(v), _ptr(a_norm), T, H, W, h, d, top_k, top_p, _scale(softmax_scale), _ptr(o),
            _ptr(lse), _ptr(out["zone_shape"]), _ptr(out["tile_block"]), _ptr(out["n_blocks"]),
            _ptr(out["sel_mask"]), _ptr(out["sel_count"]), _ptr(ws), wsb, _stream(stream)))
    return out


def mmdit_block_sparse_attn_adaptive_bwd(q, k, v, fwd, d_o, T, H, W, softmax_scale=None, dq=None, dk=None,
                                         dv=None, ws=None, stream=None):
    """Gradients (dq, dk, dv), fp32, of the adaptive block-sparse attention
    whose forward returned `fwd` (the dict of mmdit_block_sparse_attn_adaptive,
    called with want_lse=True); shapes and selection are held fixed."""
    n, h, d = q.shape
    assert n == T * H * W and q.dtype == k.dtype == v.dtype == d_o.dtype == torch.bfloat16
    assert fwd["lse"] is not None, "the forward must keep the log-sum-exp (want_lse=True)"
    for t in (q, k, v, d_o, fwd["o"], fwd["lse"], fwd["zone_shape"], fwd["sel_mask"]):
        assert t.is_contiguous()
    with _on(stream):
        dq, dk, dv = (torch.empty((n, h, d), dtype=torch.float32, device=q.device) if t is None else t
                      for t in (dq, dk, dv))
        need = mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD, n, 0, h, d, MMDIT_BF16, None)
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_block_sparse_attn_adaptive_bwd(
            _ptr(q), _ptr(k), _ptr(v), T, H, W, h, d, _scale(softmax_scale), _ptr(fwd["o"]), _ptr(fwd["lse"]),
            _ptr(d_o), _ptr(fwd["zone_shape"]), _ptr(fwd["sel_mask"]), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsb,
            _stream(stream)))
    return dq, dk, dv


def mmdit_block_sparse_attn_bwd(q, k, v, o, lse, d_o, sel_mask, T, H, W, zone=(8, 8, 8), block=(4, 4, 4),
                                softmax_scale=None, dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients (dq, dk, dv), fp32, of the block-sparse attention whose
    forward returned (o, lse, sel_mask); the selection is held fixed."""
    n, h, d = q.shape
    assert n == T * H * W and q.dtype == k.dtype == v.dtype == d_o.dtype == torch.bfloat16
    for t in (q, k, v, o, lse, d_o, sel_mask):
        assert t.is_contiguous()
    sd = sparse_desc(zone, block, 0, 1.0)
    with _on(stream):
        dq, dk, dv = (torch.empty((n, h, d), dtype=torch.float32, device=q.device) if t is None else t
                      for t in (dq, dk, dv))
        need = mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, n, n, h, d, MMDIT_BF16, sd)
        ws, wsb = _ws(need, q.device, ws)
        _check(lib().mmdit_block_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), T, H, W, h, d, ctypes.byref(sd),
                                                 _scale(softmax_scale), _ptr(o), _ptr(lse), _ptr(d_o),
                                                 _ptr(sel_mask), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsb,
                                                 _stream(stream)))
    return dq, dk, dv
