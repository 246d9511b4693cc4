"""MI355X (gfx950) nearest-centroid assignment and Lloyd centroid update.

The compute path is a C-ABI HIP library (``libkmeans_mi355x.so``, built from
``csrc/``); ``binding`` marshals torch tensors to it. ``datagen`` draws seeded
synthetic inputs.
"""
