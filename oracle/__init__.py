"""FP64 CPU oracle for the recurrent KDA training recurrence.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it. The HIP path never does.
"""
from .kda_oracle import (  # noqa: F401
    EPS, LOWER_BOUND, SCALE, prologue, recurrence, forward_task, backward_task,
    recurrence_backward, prologue_backward, chunk_quantities, chunk_recurrence,
    chunk_forward_task, chunk_recurrence_backward, chunk_backward_task,
    forward, backward, forward_tasks, backward_tasks, task_list, default_workers,
)
