"""CPU oracle of QK-Normed MLA absorbed-latent decode (test infrastructure only).

Importable only from the tests, the smoke check and the benchmark's CPU-baseline
leg.  The HIP library and its Python binding never import it.
"""
from . import qkn_oracle  # noqa: F401
