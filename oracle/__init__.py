"""CPU oracle for the code-predictor loop (test infrastructure only: imported
by tests, the smoke check and the benchmark's CPU baseline, never by the
library)."""
