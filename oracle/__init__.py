"""CPU oracle: test infrastructure only (tests, smoke check, CPU baseline of the benchmark).

The library never imports this package and this package imports nothing from the library.
"""
