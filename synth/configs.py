"""The synthetic workloads, as plain numbers.

Each entry is raw workload data: token grid sizes, modality counts, head
geometry, dtype, seed and the input distribution.  Nothing here computes any
step of the method.  Both the product path (through the Python binding, which
turns these numbers into C-ABI segment descriptors) and the oracle (which turns
them into per-token positions by its own rules) read the same numbers.

Token order inside one joint sequence is [cond | video | audio | text]:
conditioning frames first (raster h, w per frame), then the generated video
frames in raster (t, h, w) order, then audio tokens, then text tokens.
"""

WORKLOADS = {
    "tiny": dict(
        id=1, dtype="fp32", seed=0,
        T=3, H=4, W=4, n_cond_frames=1, n_audio=16, n_text=8,
        heads=2, head_dim=64, split=(16, 24, 24), theta=10000.0,
        audio_scale=(3, 16), input_scale=1.0, outlier_frac=0.0, outlier_gain=1.0,
    ),
    "block": dict(
        id=2, dtype="bf16", seed=1,
        T=21, H=16, W=16, n_cond_frames=0, n_audio=218, n_text=256,
        heads=24, head_dim=128, split=(32, 48, 48), theta=10000.0,
        audio_scale=(21, 218), input_scale=128 ** -0.5, outlier_frac=0.0, outlier_gain=1.0,
    ),
    "480p": dict(
        id=3, dtype="bf16", seed=2,
        T=21, H=30, W=52, n_cond_frames=1, n_audio=218, n_text=512,
        heads=24, head_dim=128, split=(32, 48, 48), theta=10000.0,
        audio_scale=(21, 218), input_scale=1.0, outlier_frac=0.0, outlier_gain=1.0,
    ),
    "720p": dict(
        id=4, dtype="bf16", seed=3,
        T=21, H=45, W=80, n_cond_frames=0, n_audio=218, n_text=512,
        heads=24, head_dim=128, split=(32, 48, 48), theta=10000.0,
        audio_scale=(21, 218), input_scale=1.0, outlier_frac=0.10, outlier_gain=4.0,
    ),
    "sparse2k": dict(
        id=5, dtype="bf16", seed=4,
        T=24, H=64, W=112, heads=24, head_dim=128,
        zone=(8, 8, 8), block=(4, 4, 4), top_k=32, top_p=0.9,
        field_length=4.0, noise_std=0.1,
    ),
    "adaptive2k": dict(
        id=6, dtype="bf16", seed=5,
        T=24, H=64, W=112, heads=24, head_dim=128,
        top_k=32, top_p=0.9,
        field_length=4.0, noise_std=0.1,
        bg_length=16.0, bg_amp=1.0, fg_lengths=(2.0, 4.0, 8.0), fg_radius=20.0,
        audio_radius=10.0, audio_gain=4.0, audio_period=6.0,
    ),
}

BY_ID = {w["id"]: name for name, w in WORKLOADS.items()}


def layout_counts(w):
    """Token counts of each modality segment, in sequence order."""
    frame = w["H"] * w["W"]
    n_cond = w.get("n_cond_frames", 0) * frame
    n_video = w["T"] * frame
    return dict(cond=n_cond, video=n_video, audio=w.get("n_audio", 0), text=w.get("n_text", 0))


def n_tokens(w):
    c = layout_counts(w)
    return c["cond"] + c["video"] + c["audio"] + c["text"]


def shrink(name, **over):
    """A copy of a workload with some sizes overridden (small parity cases)."""
    w = dict(WORKLOADS[name])
    w.update(over)
    return w
