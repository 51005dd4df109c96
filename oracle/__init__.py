"""fp64 CPU oracle of the paged-KV decode step: test infrastructure only (tests,
package smoke check and the benchmark's CPU baseline); never on the product path."""
