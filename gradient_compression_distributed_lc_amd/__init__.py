"""3LC state-change codec for MI355X (gfx950): HIP kernels behind a C-ABI."""
