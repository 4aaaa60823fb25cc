"""MI355X-native persistent decode megakernel (HIP, gfx950).

Submodules:
  inputs  - seeded synthetic model weights, prompts and KV contexts (no GPU needed)
  mk      - the Python binding of include/mk.h (loads libmk.so; no fallback)
  _build  - hipcc build of libmk.so
"""
__all__ = ["inputs", "mk"]
