"""fp64 CPU oracle of the two-branch video sparse attention forward.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path."""
