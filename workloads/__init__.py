"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no step of the method: it draws random bit streams, scales, signs,
activations, routes, gates and width assignments, and lays expert units out in one
buffer. The oracle and the GPU path both consume what it returns; neither is imported
here.

Seeding: tensor j of workload k is drawn from ``numpy.random.default_rng([k, j, *extra])``
with j = 0 codes, 1 scales, 2 signs, 3 activations, 4 routes, 5 gates, 6 widths.

Distributions (the pages' own tensors are real DeepSeek experts, which are not
available; these stand in with the pages' shapes: 128 x 5120 units, 384 experts per
layer, top-8 routing, 8,192-token prefill chunks):
- trellis bit streams: uniform random uint32 words;
- fp16 per-channel scales: U(0.5, 1.5) / sqrt(in), rounded to fp16;
- signs: uniform +-1 (int8);
- activations: N(0, 1) drawn in fp32, rounded to bf16 (nearest-even);
- MXFP4: codes uniform over the 16 nibbles, E8M0 bytes uniform in 119..125
  (exponents -8..-2);
- fp8b32: codes uniform over the 254 non-NaN E4M3 bytes, E8M0 bytes uniform in
  113..119 (exponents -14..-8);
- routes: top-k distinct experts per token, uniform or Zipf-skewed;
- gates: softmax of topk N(0, 1) logits per token (fp32).
"""

from .gen import *  # noqa: F401,F403
from .gen import __all__  # noqa: F401
