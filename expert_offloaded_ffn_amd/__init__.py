"""MI355X-native forward pass of one Mixture-of-Experts FFN layer with an expert slot pool.

The compute path is a HIP library (``libmoeffn.so``, built from ``csrc/``) behind a C ABI;
``binding`` marshals torch tensors and streams into its calls. ``synth`` draws the seeded
synthetic inputs. Importing this package loads nothing; the library is loaded on first use.
"""
__all__ = ["binding", "synth"]
