"""fp64 CPU oracle of the HiMuon step -- test infrastructure only (see himuon_oracle)."""
from .himuon_oracle import (  # noqa: F401
    COEFFS_CUBIC, COEFFS_QUINTIC, TILE_FULL, tiles, frobenius_normalise, ns_iterate,
    ns_tile, tiled_ns, tiled_ns_loop, phi, phi_iterate, momentum,
    bf16_round, momentum_stored, apply_update, step, tile_flops, ns_flops, step_bytes,
)
from . import diagnostics  # noqa: F401,E402
