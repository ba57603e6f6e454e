"""CPU oracle for the AFD FFN-rank hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from here.  The product path never does.
"""
