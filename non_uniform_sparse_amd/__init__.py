"""MI355X-native sparse, head-ragged decode attention.

The compute path is the HIP library ``libkvs.so`` built from ``csrc/``; the
Python side only marshals arguments (see ``kvs``).  ``workloads`` draws the
seeded synthetic inputs.
"""
