"""CPU oracle for the QuoKA chunked-prefill hot path (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
package; the library itself never does.  `quoka` is the fp64 numpy oracle,
`brute` a pure-Python brute force for tiny inputs.
"""
