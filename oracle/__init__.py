"""fp64 oracle of the optimizer step (test infrastructure only).

``oracle.optimizers``: Adafactor, CAME, LAMB. ``oracle.galore``: the GaLore step
(low-rank projected AdamW with a periodic SVD refresh of the projector).

Only the test suite, the package smoke check and the bench's CPU-baseline leg may
import this package. It is independent of the HIP library: no shared code,
headers, helpers or constants.
"""
from .optimizers import (  # noqa: F401
    ADAFACTOR_DEFAULTS, CAME_DEFAULTS, LAMB_DEFAULTS, INIT_STATE, STEP, STEP_TENSOR,
    MSG_LR_WITH_RELATIVE, MSG_WARMUP_NEEDS_RELATIVE,
    adafactor_beta2t, adafactor_hparams, adafactor_init_state, adafactor_step,
    adafactor_step_size, adafactor_step_tensor, came_hparams, came_init_state, came_step,
    came_step_tensor, is_factored, lamb_hparams, lamb_init_state, lamb_step, lamb_step_tensor,
    rms, round_bf16, quantize_i8, dequantize_i8, I8_GROUP,
)
