"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the oracle side and the GPU side of every test and by
the benchmark.  It holds no arithmetic of the method itself: it only draws
random numbers (numpy PCG64), rounds them to bfloat16 where a workload asks
for bf16 storage, and lays them out.  The one formula here is the bias
initialisation (inverse softplus of a log-uniform time step), which is part
of the input recipe, not of the scan.

Layouts: u, delta_raw, z: (batch, dim, L) with L fastest; B, C: (batch, N, L);
A: (dim, N) fp32; delta_bias, D: (dim,) fp32; decode state: (batch, dim, N)
fp32.  bf16 tensors are returned as uint16 bit patterns (round to nearest
even from the fp32 draw).

Fixed draw order from ``default_rng(seed)``:
  A jitter -> dt (-> bias) -> D -> delta_raw -> u -> B -> C -> z
and for the decode workload, after D: h0; each decode step s then draws
  delta_raw -> u -> B -> C -> z  from ``default_rng([seed, s])``.
The convolution prologue's taps, bias and carried state come from
``default_rng([seed, 1_000_003])`` (make_conv_params), a key no decode
step uses; its input x is the workload's u draw.
"""
from .configs import (ScanConfig, DecodeConfig, SsdConfig, SCAN_CONFIGS, DECODE_CONFIG,  # noqa: F401
                      SSD_CONFIG, CONFIGS, get_config)
from .inputs import (bf16_bits, bf16_to_f32, make_scan_inputs, make_decode_params,  # noqa: F401
                     make_decode_step, impulse_inputs, widen, inv_softplus_bias,
                     make_conv_params, make_ssd_inputs)
