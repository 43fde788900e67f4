"""MI355X (gfx950) dense row-major GEMM: C = A x B with FP32 accumulation."""
