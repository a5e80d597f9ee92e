"""fp64 CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU-baseline leg of the
benchmark may import it.  The product package (kda_gated_delta_rule_amd) never
imports, links or runs anything under this directory.
"""
