"""CPU oracle for the dynamic draft-tree round -- test infrastructure only.

Imported by the test suite, the package smoke check and the bench's CPU
baseline leg, never by the library or its binding.
"""
