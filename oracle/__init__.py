"""CPU oracle of the delta-prefetched sparse FFN -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. The HIP product path never imports, links or calls it.
"""
