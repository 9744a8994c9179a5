"""fp64 CPU oracle for the TurboQuant hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library (``decode_tq_quantize_amd``) never imports
it, and this package imports nothing from the library: the two share only
the written specification and the seeded inputs of ``synth``.

Everything is plain numpy/scipy in float64, written step by step in the
order the pages give the method:

* ``codebook``  — the rotated-coordinate marginal and the Lloyd-Max scalar
  quantiser built on it (riverfrot "TurboQuant" post, sections 4.1-4.2);
* ``tq``        — per-vector quantisation (normalise, rotate, scalar-quantise,
  residual, QJL sign sketch; section 4.3), the packed layouts, the
  inner-product estimator, decode attention over the compressed cache
  (sections 2.2 and 4.3) and top-k inner-product search (uiyeonassociation
  post, results section), plus the KV-cache size formula (section 2.4).

Parity status of each function (what pins it) is listed in its docstring.
The packed layouts are this library's own choice (the pages only require
that no per-block scale or zero-point be stored): "parity unpinned by the
pages", pinned instead by hand-written bit fixtures and round trips.
"""
from . import codebook, tq  # noqa: F401
