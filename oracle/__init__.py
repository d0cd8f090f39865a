"""CPU oracle of the DMS decode path.  Test infrastructure: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it."""
