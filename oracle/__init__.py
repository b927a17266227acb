"""CPU oracle of the CSA/HCA compressed-attention path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import anything under this directory; the product path
(the HIP library and its Python binding) never does, and the two share no
code.  Everything here is float64 NumPy written from the pages' description of
the method and from the published definitions of the number formats.
"""
from . import codecs, csa  # noqa: F401
