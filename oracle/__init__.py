"""CPU fp64 oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from this package.  It shares no code with the HIP library
or its Python binding, and neither imports the other.
"""
