"""MI355X (gfx950) TTT-layer forward pass: HIP kernels behind a C ABI (libttt.so).

    from weights_ttt_layer_amd import linear_fwd, mlp_fwd

``linear_fwd`` runs TTT-Linear (plain or LayerNorm+residual inner model) and
``mlp_fwd`` runs TTT-MLP, both in the mini-batch dual form, on device tensors.
``linear_fwd_block`` gives block-causal large-chunk outputs and
``linear_decode`` takes one online step per (sequence, head) stream.
``layer_fwd`` runs the whole layer: projections, key normalisation, the inner
TTT-Linear model, output LayerNorm + residual and the output projection.
``linear_bwd`` is the backward of ``linear_fwd`` (small-b combinations).
``linear_fwd_noalloc`` is ``linear_fwd`` for callers that cannot allocate: its
large-chunk workspace is a static device array inside the library.
Build the library first with ``python -m weights_ttt_layer_amd.build``.
"""
from .binding import (  # noqa: F401
    TTTError,
    layer_fwd,
    layer_parts,
    layer_workspace_bytes,
    linear_bwd,
    linear_decode,
    linear_fwd,
    linear_fwd_block,
    linear_fwd_noalloc,
    linear_path,
    linear_workspace_bytes,
    load_library,
    mlp_fwd,
    status_string,
)

__all__ = ["TTTError", "layer_fwd", "layer_parts", "layer_workspace_bytes", "linear_bwd",
           "linear_decode", "linear_fwd", "linear_fwd_block", "linear_fwd_noalloc", "linear_path",
           "linear_workspace_bytes", "load_library", "mlp_fwd", "status_string"]
