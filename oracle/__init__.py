"""CPU oracle for the Gated DeltaNet recurrent forward step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it. The product path (the HIP library and its binding)
never imports it.
"""

from .gdn_oracle import (HEAD_MAP_DIV, HEAD_MAP_MOD, build, reference, reference_bf16,
                         reference_threads, rollback, rollback_threads, to_bf16)

__all__ = ["HEAD_MAP_DIV", "HEAD_MAP_MOD", "build", "reference", "reference_bf16",
           "reference_threads", "rollback", "rollback_threads", "to_bf16"]
