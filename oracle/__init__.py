"""Oracle: a plain, slow CPU definition of the frame-synchronous decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import or run anything in this package.  The
product path (the HIP library and its Python binding) never imports it and
shares no code with it; the only code both sides use is the seeded input
generator package ``synth``.

Modules:

* ``fp8``     - OCP E4M3 codec from the format definition (pinned against
                torch's independent float8_e4m3fn conversion, the format's
                published special values, exhaustive midpoint rounding and
                the analytic round-trip bound).
* ``decoder`` - the incremental step (per-slot cache, one frame per step,
                optional depth loop).  Pinned by: equality with the full
                causal recompute, session isolation, closed-form special
                cases, float64-vs-float32 agreement; its bf16 rounding of
                activations by torch's bfloat16 conversion and a one-layer
                position-0 closed form.
* ``full``    - the full causal recompute, pinned against a library-built
                reference (torch CPU rms_norm, scaled_dot_product_attention,
                silu and complex-multiplication rotary embedding, float64).

Decoded outputs of the pages' own models are not printed anywhere in the
pages, so no function here is pinned to a printed output value; every pin
is one of the independent checks above.
"""
from . import fp8  # noqa: F401
from .decoder import Oracle, Cache, rmsnorm, rope, rope_table, round_bf16, silu  # noqa: F401
from .full import forward_full, depth_full  # noqa: F401
