"""CPU fp64 oracle of the gated delta rule (token recurrence, chunkwise stage model and
its C twin).

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU baseline
leg of the benchmark may import, call, link or run anything in this directory. The HIP
library and its Python binding never import it, and it imports nothing from them.
"""
