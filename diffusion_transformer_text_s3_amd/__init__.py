"""MI355X (gfx950) S3-DiT hot path: HIP kernels behind the C ABI of include/zdit.h, and a
ctypes binding (`binding`).  Build the library with
`python -m diffusion_transformer_text_s3_amd.build`."""
from . import binding  # noqa: F401

__all__ = ["binding"]
