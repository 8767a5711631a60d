"""CPU oracle for the routed FP4 expert FFN. Test infrastructure only: imported by the
tests, the smoke check and the CPU-baseline leg of the bench, never by the product path."""
