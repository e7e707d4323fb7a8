"""libtpmlp: one tensor-parallel rank's share of the transformer MLP on MI355X (gfx950)."""
