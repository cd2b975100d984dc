"""MI355X (gfx950) engine for KeOps-style Gaussian map-reductions (placeholder; binding below)."""
