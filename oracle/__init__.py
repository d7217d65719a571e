"""fp64 CPU oracle of the MoE layer. TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline)."""
