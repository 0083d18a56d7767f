"""MI355X-native ranking head: fused catalog scoring, logsumexp and top-K.

``genrec`` holds the ctypes binding of the HIP library (libgenrec.so);
``synth`` holds the seeded input generators.  Import them explicitly:
``from full_catalog_ranking_amd import genrec``.
"""
__version__ = "1.0.0"
