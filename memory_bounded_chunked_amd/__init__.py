"""Token-chunked, activation-bounded DiT block forward on MI355X (gfx950).

The compute path is the HIP library built from ``csrc/`` and called through its
C ABI (``include/dit_block.h``); this package only marshals arguments.
"""
__all__ = ["DitBlock", "load_library"]


def __getattr__(name):
    # Lazy: importing the package (e.g. for ``synth``) does not load torch or the library.
    if name in ("DitBlock", "load_library"):
        from . import block
        return getattr(block, name)
    raise AttributeError(name)
