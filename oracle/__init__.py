"""Float64 CPU oracle for sparse MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library and its Python binding never call it, and
nothing here shares code with the HIP kernels: no kernels, headers, helpers,
tables or constant generators.

Modules:

* ``oracle.ref``       the decode itself (gather, full softmax with sink, PV),
                       split partials and their merge, row decoding of bf16
                       and fp8-e4m3 / UE8M0 pools;
* ``oracle.plan_ref``  the integer plans: the host split-count cost model and
                       the persistent kernel's balanced tile partition;
* ``oracle.writer_ref`` the fp8/UE8M0 cache writer's rule;
* ``oracle.a8_ref``    the fp8 ("a8w8") QK: q quantised as the writer
                       quantises, then the decode of ``oracle.ref``;
* ``oracle.paged_ref`` the dense paged GQA decode (separate K and V caches,
                       a block table, MTP tokens causal among themselves).

Parity status of each function is stated in its docstring.  The host
planner's exact split count with the library's fitted coefficients is
"parity unpinned": the pages say the coefficients were fitted but do not
print them, so only the cost formula and its properties are pinned.
"""
