"""TokenGate gated-prefill hot path on MI355X (gfx950).

The four steps -- gate scoring, document-only top-K selection, gather of the
kept rows, token-gated attention -- run in hand-written HIP kernels behind the
C-ABI library ``libtokengate.so``.  ``learned_token_pruning_scorer_amd.binding``
holds the thin Python wrappers (same names as the C entry points); importing
the package itself loads neither torch nor the library.
"""
import importlib

__all__ = ["configs", "inputs", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
