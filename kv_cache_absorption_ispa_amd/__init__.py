"""ISPA hot path on MI355X: decomposable attention, Gram accumulation and the closed-form absorb.

The compute runs in the HIP library ``libispa.so`` (built from ``csrc/``); this
package is its thin Python binding.  ``inputs`` holds the seeded synthetic
input generator.
"""
