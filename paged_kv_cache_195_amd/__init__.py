"""Paged attention over a block-table K/V cache for AMD MI355X (gfx950)."""
