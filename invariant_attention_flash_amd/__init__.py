"""Batch-invariant attention forward for MI355X (gfx950): packed varlen
prefill and paged-KV decode behind a C-ABI library (``libinvattn.so``)."""
