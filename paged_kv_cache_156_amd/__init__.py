"""Paged KV-cache decode attention for MI355X (gfx950).

The compute path lives in the HIP library ``libpkv.so`` (sources under
``csrc/``); ``binding`` marshals arguments to its C ABI. ``workloads`` draws
seeded synthetic inputs. Importing this package loads nothing: the library is
opened on first use, and every entry point raises if it is missing.
"""
