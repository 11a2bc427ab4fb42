"""CPU oracle for the USP (Ulysses + zigzag Ring-Attention) forward hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never calls into it, and this package never
imports the product path.  The two share no code: only the seeded input
generator, which holds none of the method's arithmetic, feeds both.

Everything here is plain, slow and meant to be checked by eye against the
source pages.  Floating point is float64 throughout.

Sources (cited by title and section in every function):

* [USP review] "USP: 统一序列并行方法用于长上下文生成式AI" -- the xllm-io
  paper-review blog on Fang & Zhao, "USP: A Unified Sequence Parallelism
  Approach for Long Context Generative AI".  Section 三 (技术架构) holds the
  Ulysses 4D layout, Algorithm 1 (USP-Attention) and Algorithm 2 (the
  load-balanced "zigzag" split); section 四 holds the degenerate cases.
* [CP vs Ulysses] "Context Parallel 与 Ulysses" -- the ml-interview blog.  Its
  concepts section states the ring schedule and the online-softmax LSE merge;
  Figure 1 is the cp=4 ring schedule; Figure 2 and the section
  "为什么要一头一尾配对" give the causal per-rank loads; "推导 / 关键公式" and
  "对比与手算例子" give the communication volumes.
* [ByteScale notes] the Notion notes on ByteScale (sequence packing).
* [YunChang] the YunChang (long-context-attention) README translation, for the
  user-facing layout [batch, seq_len, num_heads, head_dim].
* [UPipe page] "Untied Ulysses：基于分头切分的高效上下文并行方案" -- the
  ai-stack.site summary of UPipe.  Its section 2 (核心方法与创新) names
  headwise chunking: attention heads pushed through in fine-grained chunks so
  that the attention's intermediate tensors exist for one chunk at a time.
  The rest of the page is commentary; only that idea is used.

Modules:

* ``attention`` -- masked softmax attention by its definition (one shot), and
  a brute-force scalar version for tiny shapes.
* ``merge``     -- the LSE merge rule of [CP vs Ulysses].
* ``index``     -- zigzag split, Ulysses layout, ring schedule, tile classes,
  causal load accounting.
* ``usp``       -- Algorithms 1 and 2 composed over a virtual (ud x rd) grid,
  also with the head blocks pushed through in chunks ([UPipe page]).
* ``comm``      -- the per-GPU communication-volume formulas (design input only).
* ``backward``  -- gradients of the attention (dQ, dK, dV): of the whole
  sequence, of one ring step given the forward's lse, and of one ring rank.

Parity status: every function is pinned by the ``-m "not gpu"`` tests against
facts the pages print or against mathematics (closed forms, brute force, a
library routine); the backward is pinned to finite differences of the forward
and to torch autograd of a plain masked softmax.  The one reading that no page fixes -- zigzag applied to a
packed variable-length stream -- is noted where it is used.
"""
