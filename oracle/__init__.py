"""Plain, slow CPU oracle for OSCAR-style INT2 KV-cache write and decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports,
calls or links it, and shares no code, table or constant generator with it.

What it computes, and where each piece comes from (sources are the public
pages describing OSCAR; "axbrief" is the article "Together AI's OSCAR breaks
the 2-bit KV cache accuracy barrier", "techllm" is the post "KV cache
compression: TurboQuant, OSCAR, EpiCache", "gist" is the gist.science summary
of the OptR paper, arXiv 2608.02691):

* ``calibration``  key rotation R_K = U_Q . H . P_br from the query second
  moment C_Q (axbrief, section "어텐션 통계 기반 회전과 Triton 커널의 결합";
  techllm, section "OSCAR — INT2를 실전으로 끌어내린 캘리브레이션 회전").
* ``quantizer``    range clipping with c_K = 0.96 / c_V = 0.92 and per-token
  asymmetric INT2 in 64-channel groups (axbrief, same section).
* ``layout``       byte layout of one INT2 page (4 codes per byte, fp16 scale
  and minimum per group).  The pages say the cache stays paged-attention
  compatible but do not give a layout; this is the layout the library
  documents in ``include/oscar.h``.
* ``store``        routing of tokens to BF16 sink / INT2 history / BF16 recent
  window, window eviction and the FIFO page allocator (axbrief, section
  "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개"; techllm OSCAR section on the
  mixed-precision paged cache).
* ``attention``    GQA decode attention over the mixed-precision cache and the
  split-softmax combine, by their plain definitions (axbrief, rotation
  section: the read path unpacks, dequantizes, undoes the rotation and
  attends in one pass).

Every function is pinned by ``tests/test_oracle_pins.py`` against facts the
pages or the mathematics fix (closed forms, invariants, brute force,
hand-worked examples in ``tests/golden/``).  Parity status per function is
listed in each module header; none is "parity unpinned" except where stated.
"""
from . import calibration, quantizer, layout, store, attention  # noqa: F401
