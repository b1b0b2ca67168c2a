"""CPU oracle for one training step of a pre-LayerNorm decoder-only transformer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

The oracle is the plain definition of the step in float64 numpy, written
function by function from the pages (see the docstrings for the passage each
one follows). Matrix products use numpy's matmul as a library primitive; there
is no blocking, fusion or reordering beyond what each definition states.
"""
from .model import (  # noqa: F401
    index_layout,
    embedding_fwd,
    embedding_bwd,
    layernorm_fwd,
    layernorm_bwd,
    linear_fwd,
    linear_bwd,
    gelu,
    gelu_grad,
    attention_probs,
    attention_fwd,
    attention_bwd,
    xent_fwd_bwd,
    forward,
    loss_and_grads,
    grad_norm_and_scale,
    adamw,
    train_step,
    csr_by_key,
)
from .schedule import lr_schedule  # noqa: F401
from .generate import next_token, kept_ids, cdf_bounds  # noqa: F401
from .scaler import loss_scale_update, loss_scale_trace  # noqa: F401
