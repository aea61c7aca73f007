"""CPU oracle for the FP8 (e4m3) fine-grained-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code, tables or helpers with the HIP
library; the only module both sides use is ``synth`` (seeded random inputs,
which holds none of the method's arithmetic).

What it computes, and where the pages define it (pages are cited by title and
section; the texts are machine-extracted and partly machine-translated):

* e4m3fn decode / round-to-nearest-even encode (``oracle.e4m3``): the pages
  only name the E4M3 format ("DeepGEMM: Ince olceklendirmeyle temiz ve verimli
  FP8 GEMM cekirdekleri", section on the v3.2 MQA kernels, which types q as
  E4M3).  The bit layout is the OCP 8-bit e4m3fn one (bias 7, no infinities,
  NaN = S.1111.111), the format gfx950 implements natively.
* fine-grained quantisation (``oracle.quant``): one fp32 scale per 1x128
  activation group and per 128x128 weight block, scale = amax / 448
  (DeepSeek-V3 fine-grained scaling named in the release summary, GeekNews
  topic 19444, opening bullets; the same digest, "GEMM arayuzu ve yerlesim
  kisitlari", says SM90 scale factors are FP32 and that casting is the user's
  job, done by simple helpers).
* power-of-two (UE8M0) factors (``oracle.quant``, ``*_ue8m0``): the same
  digest section says the newer architecture takes UE8M0 factors packed four
  to an int32; the fp32 factor is rounded up to a power of two and packed
  along K (readings stated in ``oracle.quant``).
* the GEMM D = bf16(A . B^T) with per-128-K-slice promotion (``oracle.gemm``):
  "GEMM arayuzu ve yerlesim kisitlari" (NT layout, D = C + A @ B.T, no C here)
  and the two-level promotion described in the release summary's opening
  bullets and in 7minutos.es, "Detalles y beneficios tecnicos".
* the M-grouped contiguous and masked forms (``oracle.gemm``): "Dense ve
  Grouped GEMM" of the same digest.
* acceptance metrics (``oracle.metrics``).

Every function is pinned by tests in ``tests/test_oracle.py`` against
something other than itself (torch's own float8/bfloat16 conversions, exact
rational brute force, closed forms and invariants).
"""

from . import e4m3, quant, gemm, metrics  # noqa: F401

__all__ = ["e4m3", "quant", "gemm", "metrics"]
