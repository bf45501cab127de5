"""CPU oracle for the binary-weight x ternary-activation product.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py.  Nothing in the GPU library imports it.
"""
