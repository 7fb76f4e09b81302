"""CPU oracle for the MLA latent-KV hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import OracleError  # noqa: F401
from .dsa_oracle import dsa_rank_keys, dsa_select, dsa_select_rows  # noqa: F401
from .append_oracle import append_compressed, o_proj, rms_norm  # noqa: F401
