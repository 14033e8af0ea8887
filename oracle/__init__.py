"""CPU oracle of the paged decode path. Test infrastructure only: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg."""
