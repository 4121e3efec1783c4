"""MI355X-native ESM-2 encoder forward: a C-ABI library of gfx950 HIP kernels
(libesmenc.so) with a thin Python binding.

Submodules: `esm` (the binding: Encoder and host-only checks), `datagen`
(seeded synthetic inputs), `build` (compiles the library with hipcc)."""

__all__ = ["esm", "datagen", "build"]
