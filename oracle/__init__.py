"""CPU oracle for the 4-bit KV-cache codecs and paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``bit_quantized_kv_amd``) never imports it, and this
package never imports the product path: the two share no code, tables, constants
or helpers.  The only module both sides use is ``workloads`` (seeded synthetic
inputs, none of the method's arithmetic).

What it computes, plainly and slowly (numpy, fp64 unless a decision is taken):

* ``lloyd_max``  - the 16-level Lloyd-Max quantizer of N(0,1) (the default
                   16-entry key codebook).
* ``wht``        - the orthonormal Walsh-Hadamard rotation (explicit matrix and
                   staged butterflies).
* ``tq4``        - the TQ4/4 codecs: rotated keys coded against the 16-entry
                   table with a per-(token, head) scale; values with a
                   per-32-channel asymmetric uniform 4-bit code.
* ``mxfp4``      - the FP4 (e2m1) / UE8M0 / FP8 (e4m3) stretch codecs.
* ``layout``     - the packed byte layout of one (16-token block, kv-head)
                   record.
* ``paged``      - the paged cache: slot mapping, block table, gather.
* ``attention``  - exact fp64 decode attention over the dequantized cache, and
                   the split/merge (log-sum-exp) algebra.

Where floating point decides an integer (a key code, a value code, an FP4/FP8
code, a rounded scale) the oracle takes the decision in the same precision as
the kernels (fp32 with a fixed operation order, stated in each function), so
codes can be compared bit for bit.  Each such rule is also checked against the
exact (fp64) rule, which it matches except at flagged near-ties.

Pages cited, by title (the text of each is the method's only source):

* [TQ-AMD] "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來" - a summary of AMD's
  ROCm TurboQuant integration in vLLM.  Sections: spec table; 2 "TQ4/4 是最穩的
  預設值" (4-bit K / 4-bit V, K = rotation + LUT, V = uniform); 4
  "Walsh-Hadamard 比隨機 rotation 更實用" (WHT instead of random rotation);
  5 "4-bit 路徑先別加 QJL" (no QJL at 4 bits).
* [UQ] "UltraQuant：4-bit KV 快取加速長代理" - a summary of the UltraQuant
  paper.  Sections: "方法怎麼做，白話講" (how the method works: WHT, no QJL,
  K/V asymmetry, Lloyd-Max / calibrated 16-entry table, FP8 queries, FP4 KV,
  UE8M0 group scales, scaled MFMA); "它實際證明了什麼" (results, the K MSE
  figures).
* [ST] "StateTree-Representation：讓 LLM 壓縮後仍保留 BF16 精度" - paged KV
  blocks of 16 tokens in vLLM (first body paragraph after the summary).

Parity status of each function is stated in its docstring as "pinned by ..."
(the tests under ``tests/test_oracle_*.py`` that tie it to something other than
itself).  One quantity is parity unpinned: the per-element key MSE figures that
[UQ] "它實際證明了什麼" prints (1.32e-4 -> 1.18e-4 with calibrated centroids)
were measured on real activations that are not available, so the MSE this
oracle reports on synthetic rows is compared only with the Lloyd-Max value.
"""
