"""CPU oracle for the grouped top-k W4A16 MoE FFN.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import, call, link or execute anything in
this directory; the HIP product path never does, and shares no code with it.

Every function here is pinned by the CPU tests against closed forms, format
definitions, library routines and exact rational brute force (the full-shape
layer output itself has no printed value on the pages: it is the same code
at a larger size).
"""
