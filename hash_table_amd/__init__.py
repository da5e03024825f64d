"""MI355X-native hash-blocked TSDF integration (allocate + update).

The compute path lives in the HIP library built from ``csrc/`` and is reached
through :mod:`hash_table_amd.tsdf`, a ctypes binding of its C ABI.  Importing
the package loads nothing; :mod:`hash_table_amd.scenes` generates the
seeded synthetic inputs.
"""
