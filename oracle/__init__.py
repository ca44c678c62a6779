"""CPU oracle of the compressed sparse attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg; never by the product package.
"""
