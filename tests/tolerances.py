"""Parity tolerances: maximum absolute difference between a HIP output and
the fp64 oracle's, by the element type the path computes from (fp32 1e-5,
bf16 2e-2, fp8 key/value cache 6e-2).  Cache contents, slots, tables and
free lists are compared bit for bit instead."""

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
