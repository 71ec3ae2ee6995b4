"""CPU oracle for the embedding-bag + dot-interaction core (test infrastructure only).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import this package.
"""
