"""fp64 CPU oracle for the joint sCM target, its training backward, the joint DMD term and
the stage-3 mix.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.
"""
from .scm_oracle import (  # noqa: F401
    Dual, attention, attention_fwd_jvp, attention_lse, block_x0, boost_factor, joint_block,
    l2_normalise, scm_direction, scm_sample, scm_target, student_field, time_embedding,
    rf_wrap, rf_x0, trigflow_field, trigflow_noise,
)
from .dmd_oracle import (  # noqa: F401
    dmd_sample, dmd_target, guided, residual_scale, stage3_loss, teacher_prediction,
)
from .grad_oracle import scm_loss_and_grads, student_fields, student_x0_torch  # noqa: F401
