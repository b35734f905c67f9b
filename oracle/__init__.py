"""Plain CPU oracle for STAR-KV latent-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package;
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
it.  It shares no code with the HIP library (decode_attention_starkv_amd):
the byte format is implemented here again, from its written specification.

What it computes (sources are the pages' sections, equations and algorithms):

* quant.py    -- asymmetric b-bit group quantizer with fp16 scale/zero
                 (technical review of arXiv 2606.08382, section 6.1, eq. 14:
                 leading channels at 4 bits, the rest at 3 bits), emulated
                 bit-for-bit in IEEE float32/float16 arithmetic;
* hadamard.py -- block-wise Walsh-Hadamard rotation (review section 6.1,
                 eq. 13), as a matrix and as the float32 fast transform that
                 defines the stored latents;
* cache.py    -- the packed cache format (pack, unpack, append), dequantize;
* attention.py-- reconstruction K = Z_k B_k^T, V = Z_v B_v^T (review eq. 2)
                 followed by plain softmax attention a = q K^T * scale,
                 p = softmax(a), o = p V (review section 2.3), in float64;
                 the causal prefill variant; the split-T merge of the
                 attention decomposition theorem (CaliDrop review, "What
                 carries the argument");
* sizes.py    -- cache-size formulas (review eq. 1 and eq. 15).

Every function is pinned by tests/test_oracle_*.py against closed forms,
special cases, brute force or numbers the pages print.  Parity unpinned:
nothing (the byte order inside the packed format is pinned only by its
written specification and hand-derived examples, since the pages fix none).
"""
