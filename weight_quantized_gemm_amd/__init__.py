"""libqgemm: weight-quantized GEMM (fp32 / Int4-Block64 / Int8-Block0 / W4A8)
for AMD MI355X (gfx950), behind a C ABI (include/qgemm.h).

The Python face is weight_quantized_gemm_amd.qgemm (a thin ctypes binding);
weight_quantized_gemm_amd.synth holds the seeded synthetic inputs.
"""
