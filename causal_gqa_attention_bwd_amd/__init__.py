"""Causal grouped-query attention backward with a per-query document-start mask, for MI355X (gfx950)."""
