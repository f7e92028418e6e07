"""CPU fp64 oracle for compressed-domain decode attention on a TurboQuant-style packed cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or constant generator with the HIP
library; the only thing both sides consume is the seeded input generator in
``workloads.py``, which holds none of the method's arithmetic.

What it computes, and where the pages define it (page title, then section):

* ``codebook``  -- the coordinate law of a uniformly rotated unit vector and its Lloyd-Max
  scalar codebook ("TurboQuant ... MNN on phones", 2.2 and 2.3).
* ``rotation``  -- sign flips, the normalised Walsh-Hadamard transform on blocks of 32 or
  on the whole head ("TurboQuant ... MNN on phones", 3.1) and the IsoQuant SO(4)
  block rotation v -> q_L v conj(q_R) ("RotaryQuant ... Fused Compressed-Space
  Attention", key design 2).
* ``quant``     -- norm -> normalise -> rotate -> per-coordinate codebook search, and the
  inverse lookup -> inverse rotation -> times norm ("TurboQuant ... MNN on phones", 2.1;
  compare-count search rule, 3.4).
* ``layout``    -- the packed byte layout (8 codes in 3 bytes, or 2 per byte;
  "TurboQuant ... MNN on phones", 3.3) as this library fixes it.
* ``attention`` -- plain softmax attention over explicitly dequantised K/V, key-axis
  splits with a log-sum-exp merge ("RoPE-Aware Bit Allocation for KV-Cache
  Quantization", packed-cache implementation details), and the rotated-domain
  rewrite used as a self-check ("RotaryQuant ...", key design 3); attention over a row's
  quantised and unquantised token stores.
* ``blockgtq``  -- Block-GTQ keys: RoPE-block energies, the greedy integer bit allocation,
  one TQ-MSE encoder per width (rotation, codebook, compare-count), nibble records
  ("RoPE-Aware Bit Allocation ...", overview, energy score, greedy allocation, grouping and
  packed-cache paragraphs).
* ``qjl``       -- two-stage keys: (b-1)-bit TQ-MSE plus the sign bits of a Gaussian projection
  of the residual, and the unbiased inner-product estimate they give ("TurboQuant ... MNN on
  phones", 2.4 and 3.2).
* ``zipcodec``  -- the lossless BF16 exponent codec of the KV cache: chunk rule, 4-bit
  codes, page metadata and the decode by integer adds ("ZipFusion ...", compression format
  and register decode sections).

Every function works in float64 unless it is explicitly producing a stored fp32 value.
Parity pins for each function live in ``tests/test_oracle_*.py``; nothing here is
"parity unpinned".
"""

from . import codebook, rotation, quant, layout, attention, zipcodec, blockgtq, qjl  # noqa: F401
