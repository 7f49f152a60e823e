"""fp64 CPU oracle for the selective state-space scan (S6).

TEST INFRASTRUCTURE ONLY: the plain sequential definition that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
library (``selective_state_space_28_amd``) and neither imports the other.

The arithmetic lives in ``ssm_oracle.c`` (plain C, double precision); this
module only converts numpy arrays to float64 and calls it through ctypes.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against values and identities fixed by the pages (worked impulse response,
printed exp/softplus values, convolution = recurrence, brute-force
semiseparable sums, stability bound, chunking/decode identities).  The D-skip
term and the silu gate are pinned only by their definitions (the pages do not
state them): parity unpinned by the pages for those two terms.  The
convolution prologue (causal_conv1d_silu, conv_step) is pinned against numpy's
convolution with the taps reversed, its identity and delay special cases,
and its own chunking and decode identities; its tap order, width and
non-linearity are readings of the pages, not printed on them.  The backward
(scan_bwd) is pinned by central finite differences of the forward, in fp64.
ssd_scan_fwd is the scan with a scalar A per head ("Mamba" paper review,
"Mamba 2"; NN LAB "Mamba" page, "Bridging Tensor Cores and Recurrence"),
pinned against an independent chunked evaluation and linear attention.
"""
from .oracle import (build, causal_conv1d_silu, conv_scan_fwd, conv_step,  # noqa: F401
                     lib_path, scan_bwd, scan_fwd, ssd_scan_fwd, state_update)
