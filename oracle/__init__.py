"""fp64 CPU oracle for the joint video-audio attention hot path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import anything under this package; the library (HIP
kernels, C ABI and its Python binding) never does, and this package imports
nothing from the library.  It computes the plain definitions in float64 with
numpy so that a reader can check each step against the pages by eye:

  rope.py          time-shifted 3D RoPE (SkyReels-V4 pages)
  attention.py     dense softmax attention: joint, A<->V and video->text
  attention_bwd.py log-sum-exp and gradients of (masked) softmax attention
  block_sparse.py  Prism block pooling, hybrid top-k/top-p, sparse attention
  adaptive_blocks.py  Prism variation indicator and content-adaptive block shapes
  brute.py         pure-Python loop versions used to cross-check the above
"""
from . import rope, attention, attention_bwd, block_sparse, adaptive_blocks, brute  # noqa: F401
