"""Plain fp64 CPU oracle for the fused chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table
or helper with the HIP library; the only thing both sides consume is the
seeded input generator ``sparse_top_kl_amd.synth``, which holds none of the
method's arithmetic.

Every function in ``kl_oracle`` is pinned by a CPU test against something
other than itself (library routines, closed forms, brute force, finite
differences); see ``tests/test_oracle.py``. ``topk_oracle`` (the teacher
top-K cache) is pinned the same way in ``tests/test_oracle_topk.py``, and
``renorm_oracle`` (the student-renormalised loss option) in
``tests/test_oracle_renorm.py``.
"""

from .kl_oracle import (  # noqa: F401
    brute_force,
    forward_backward,
    logsumexp_rows,
    student_logits,
    teacher_log_probs,
)
from .topk_oracle import teacher_logits, teacher_topk, topk_rows  # noqa: F401,E402
from .renorm_oracle import renorm_brute_force, renorm_forward_backward  # noqa: F401,E402
