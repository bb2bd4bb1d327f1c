"""CPU oracle for the GPTQ layer path (numpy fp64). Test infrastructure: imported only by tests/,
the smoke entry and the benchmark's CPU-baseline leg; it shares no code with the GPU library."""
