"""MI355X-native single-token multi-head latent attention (MLA) decode.

The compute path is the C-ABI library ``libmla_decode.so`` (hand-written HIP for
gfx950) declared in ``include/mla_decode.h``; :mod:`.binding` is its thin Python
binding and raises if the library is not built.  :mod:`.synth` makes seeded
synthetic inputs and imports nothing else from this package.

Importing the package itself loads nothing, so the input generator can be used
on hosts where the library has not been built.
"""

__all__ = ["binding", "synth"]
