"""CPU oracle of the MXFP4 block-scaled Hadamard-32 path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.
"""
