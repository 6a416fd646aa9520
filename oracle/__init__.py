"""CPU float64 oracle (test infrastructure; never used by the product path)."""
from .mla_oracle import (attend, causal_window_visible, materialize_kv, mla_decode_step,
                         q_absorb, latent_partial, lse_combine, v_up,
                         latent_bytes_per_token, block_bytes)

__all__ = ["attend", "causal_window_visible", "materialize_kv", "mla_decode_step",
           "q_absorb", "latent_partial", "lse_combine", "v_up",
           "latent_bytes_per_token", "block_bytes"]
