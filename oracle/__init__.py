"""fp64 CPU oracle for the selective-scan backward and the layer around it.

TEST INFRASTRUCTURE. Only the test-suite, the package entry's smoke check and
the bench's CPU-baseline leg may import, call or run anything in this package.
The HIP library and its Python binding never import it, and it imports nothing
from them: the two sides share no code.  Inputs come from ``synth`` (random
draws and storage rounding only).

Sources (pages, by title and section):
  * mamba-rs 0.5.1, ``src/mamba_ssm/cpu/backward.rs``: module notes O2-O5 and
    ``backward_mamba_layer_batched`` Phases B1-B8 (the layer backward, with the
    sequential SSM BPTT in Phase B3) and ``backward_mamba_backbone_batched``.
  * luma-tensor 0.0.1, ``src/grad/backprop.rs``: the reverse-mode rules used by
    the independent tape in ``oracle.tape``.
  * rlx-cpu 0.2.17, ``src/training_bwd.rs``: ``rms_norm_backward_row`` and
    ``cumsum_backward_row``.

Every function here is pinned by a CPU test against something other than
itself (finite differences, the tape, closed forms, invariants); there is no
function marked "parity unpinned".
"""
