"""CPU oracle for MLA absorb attention and latent-KV expansion (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the product path never does.
"""
from . import bruteforce, mla_oracle  # noqa: F401
