"""Float64 CPU oracle for paged K/V split-K decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, no
headers, no constants and no helpers with the HIP library; it is written from
the source pages directly so that it can check that library independently.

What it computes is the plain definition of the method: split-K flash
decoding with an exact log-sum-exp merge reaches the same numbers as one
softmax over all keys, so the oracle is that one softmax, evaluated in float64
over K/V rows that it decodes and gathers through the block table itself.

Source pages cited throughout (title, then the section used):

* lucebox#555 -- Luce-Org/lucebox pull 555, "feat(qwen35): add
  paged-attention monolithic decode-only AR foundation".  Sections: Summary,
  Benchmark results (Uniform batches, Ragged 8-request workload, K/V
  capacity), Validation.
* llama.cpp-PR2 -- achyudh/llama.cpp pull 2, "hip: add RDNA2 gfx1030 paged
  attention fallback for adaptive KV streaming".  Its body is a series of
  commit messages; a citation names the commit by its topic (the split-K
  decode commit, the page-table commit, the log-sum-exp output commit, the
  pd_combine fix, the LDS-read commit).
* TensorFold#1156 -- ashhart/TensorFold issue 1156, "CUDA: Qwen3.5/3.6
  attention caches on the core KV pool".  Sections: Design / Kernels,
  Verification, Activity.
* colibri#372 -- JustVugg/colibri pull 372, "cuda: keep paged ragged KV
  resident across decode steps".  Sections: Summary, Validation.

Modules:

* ``quant``       -- decoding of F16 / BF16 / Q8_0 / Q4_0 rows to float64.
* ``encode``      -- encoding of float32 rows into those four formats (the
                     quantiser of a device-side append).
* ``attention``   -- block-table gather, plain causal GQA softmax attention,
                     the log-sum-exp merge of chunk partials.
* ``pool_model``  -- byte-level model of the paged pool (append scatter,
                     logical gather).
* ``alloc_model`` -- model of the exact transactional block allocator.

Every function is pinned by ``tests/test_oracle_*.py`` to something other than
itself (values printed on the pages, closed forms, a library routine, brute
force on tiny inputs, invariants).
"""

from . import quant, encode, attention, pool_model, alloc_model  # noqa: F401

# Names of the four K/V encodings the pages list (lucebox#555, Summary, for
# F16 / Q4_0 / Q8_0; TensorFold#1156, Summary, for bf16 K/V).
F16, BF16, Q8_0, Q4_0 = "f16", "bf16", "q8_0", "q4_0"
TYPES = (F16, BF16, Q8_0, Q4_0)
