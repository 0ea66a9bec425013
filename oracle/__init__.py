"""CPU oracle for FP64 GEMM emulation by Ozaki Scheme II (``ozaki2``) and by
the Scheme I slice split (``ozaki1``).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this directory.  The only permitted users are the
tests under ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``.  The oracle shares no code, tables or constant
generators with the HIP library: it is written independently from the
mathematics of the method so that the two can check each other.

Citations in this package name the web pages the method is taken from:

* "Ozaki II notes" -- the page *Ozaki Scheme II：用 CRT 把高精度 GEMM 映射成少量
  INT8 GEMM* (chatdocs.ruinique.com/nla/ozaki-scheme-ii), with its numbered
  sections §1-§16;
* "Ozaki I notes" -- the course page *Ozaki Scheme*
  (zsc0tt.pages.dev/courses/hpc-summer/ozaki-scheme), with its named sections.
"""
