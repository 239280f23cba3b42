"""Plain fp64 CPU oracle for the spectral-domain FP4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP library under
``fp4_spectral_split_amd/`` and imports nothing from it.

Modules
-------
formats  E2M1 / E8M0 / E4M3 scalars, MXFP4 and NVFP4 block codecs.
split    Randomized spectral split A = U_k S_k V_k^T + R (Householder QR,
         one-sided Jacobi SVD), and the quantized split record.
linear   Y = X W^T, dX = dY W, dW = dY^T X on the dequantized split operands
         (reconstruction route, plus the four-term expansion as a second route).
optim    The adaptive spectral learning rate (rescaling a gradient's mid and
         low singular directions) and the dual-range regularizer.

Every floating-point step runs in fp64 unless a step is defined as an fp32
operation (the NVFP4 scale arithmetic), which is emulated exactly as an fp64
operation followed by one rounding to fp32.

Pinning status (what each function is checked against, outside itself) is
listed in each module's header. Items "parity unpinned": the method-level
claim that the split lowers tail-spectrum distortion is tested for direction
only, because the pages print no values for it; and the functional forms of
the adaptive spectral learning rate and the dual-range regularizer, which the
pages describe in words only (each kernel is pinned to its stated reading).
"""
