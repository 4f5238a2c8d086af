"""kvdec: single-query grouped-query decode attention over long KV caches on
MI355X (gfx950).

The compute path is the C-ABI library ``libkvdec.so`` built from ``csrc/``;
``long_context_decode_kv_amd.kvdec`` is its Python binding (argument
marshalling only).  ``long_context_decode_kv_amd.synth`` holds the seeded
input generators.  Importing this package loads nothing; importing the
binding loads the library and raises if it has not been built.
"""
