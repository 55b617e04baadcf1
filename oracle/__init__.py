"""Test infrastructure only: the fp64 CPU oracle of the Muon step.

Imported by the tests, the package smoke check and the benchmark's CPU
baseline; never by the product path.
"""
