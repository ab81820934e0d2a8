"""Stage-pipelined half-precision TN GEMM for MI355X (gfx950)."""
