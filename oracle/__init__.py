"""CPU oracle for the low-bit routed-expert MoE FFN -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy (fp64) definitions of every step of the layer:
routing, grouping, low-bit dequantisation, MXFP4 -> FP8 conversion, MXFP8 activation
quantisation, the SwiGLU expert FFN and the gate-weighted combine; and of the quantisers that
produce the low-bit formats from fp32 weights (``quant``: decisions taken in fp32, in a fixed
order, so that a GPU quantiser can match them bit for bit).  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it;
the HIP library never does, and this package imports nothing from it (no shared code,
tables or constants).

Sources, cited by page title and section:

* [Moet-QA]      mhpn.cn Q&A on the vLLM-Moet project, section on what the project
                 teaches: 2-bit expert quantisation on a sign-symmetric codebook, the
                 FP4 cache of hot experts, hand-written matmul kernels.
* [Moet-README]  ossradar.top page "vLLM-Moet": release notes of v2026.11.03-r23 (the
                 prefill MoE as FC1 + SwiGLU + MXFP8 quantisation, then FC2) and the
                 README tables (routed experts per layer, MXFP4 checkpoint bytes).
* [Strata-R9700] lcz.me thread "移植Strata技术路线到vLLM以适配R9700…", the post listing
                 the tried paths, path 6 (the 3-bit expert layout: 8 levels, e4m3
                 scale over 64, 32 codes in three 32-bit words).
* [Day0-MXFP4]   ruibaoantu.com article "国产GPU完成MoE大模型Day-0适配…", section 4
                 (MXFP4 expert weights converted online to FP8 into a reused workspace).
* [OCP-MX]       OCP Microscaling Formats (MX) Specification v1.0 (public spec): e8m0,
                 e2m1, e4m3fn element encodings and the shared-scale rule.

Readings taken where the pages are silent or ambiguous are stated next to the code
that takes them.  Every function here is pinned by tests in ``tests/test_oracle_*.py``
against worked examples, brute force, closed forms or invariants.
"""
from . import formats, moe, quant  # noqa: F401
