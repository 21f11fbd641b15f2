"""MI355X-native factored recurrent states: buffered decode, factored readout,
Brand compaction and a dense fallback behind the C-ABI of libsinkstate.so.

``sinkstate`` is the ctypes binding (it imports torch to share its HIP
runtime); ``workloads`` holds the seeded synthetic inputs; ``build`` compiles
the library for gfx950.
"""
