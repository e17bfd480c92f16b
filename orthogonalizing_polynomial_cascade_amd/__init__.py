"""MI355X-native ANVIL bank step: twin-rail momentum and the orthogonalising polynomial cascade.

The compute path is the HIP library `libanvil.so` (csrc/), reached through the ctypes binding in
`anvil.py`.  `workloads.py` draws the seeded synthetic gradient stacks.
"""
