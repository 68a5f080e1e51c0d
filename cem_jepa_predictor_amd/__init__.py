"""MI355X (gfx950) CEM plan step over an action-conditioned predictor.

The compute path is the HIP library `libcem_jepa.so` (built by
`cem_jepa_predictor_amd.build`), called through the thin ctypes binding in
`cem_jepa_predictor_amd._lib`.  `inputs` holds the seeded synthetic workloads.
"""
