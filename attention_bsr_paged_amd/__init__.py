"""attention_bsr_paged_amd: paged block-sparse-row attention for MI355X (gfx950)."""
