"""MI355X (gfx950) causal / sliding-window grouped-query attention, forward and backward."""
