"""Slow, obviously correct CPU oracle (float64 attention, naive radix tree).

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import anything under this directory.  The
product path never does, and this package never imports the native library.
"""
