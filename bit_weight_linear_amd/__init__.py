"""MI355X-native sign-binarised linear layers (OneBit and Double Binary Factorization).

The compute path lives in the HIP library ``lib/libobl.so`` built from
``csrc/`` (see ``build.py``); :mod:`bit_weight_linear_amd.binding` is the thin
ctypes binding over its C ABI (``include/obl.h``).  Importing this package does
not load the library; importing ``binding`` does, and fails loudly when it is
missing.
"""
__all__ = ["binding", "workloads", "build"]
