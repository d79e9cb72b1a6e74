"""fp64 CPU oracle of the JointSchemaHead forward pass (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the library never does.
"""
from .head import forward, forward_record, load_params, from_bf16  # noqa: F401
