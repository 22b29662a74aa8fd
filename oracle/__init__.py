"""CPU oracle for the Gated DeltaNet verify path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's cpu_baseline leg are the
only users.  The product library never imports, links or runs anything here, and nothing here
imports the product library.
"""
