"""Plain, slow CPU oracle of the DeepSeekMoE layer forward pass (float64 numpy).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The GPU product path never does; it shares no
code with this package (both read their inputs from ``synth`` only).

Each function cites the passage of the pages it follows, by page title and section:

* [TR]  "DeepSeek Technical Report: MoE Architecture" (rooftopsnow.tistory.com/291)
* [YJ]  "DeepSeek model complete analysis" (youngju.dev)
* [HB]  DeepSeek-V3 report digest (honbul.tistory.com/207)
* [PW]  "DeepSeek-V3 walkthrough" (factory.pai-world.com)

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*``,
except that no pin reaches the pages' whole-model FLOP figure (parity unpinned; it needs the whole
16B model and its FLOP convention, which are outside this layer).
"""
from . import formats, quant, moe  # noqa: F401
