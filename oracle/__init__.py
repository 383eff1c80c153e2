"""Plain, slow, obviously-correct CPU oracle for one data-parallel rank's
sharded mixed-precision optimizer step.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it, call it or load the library
it builds.  It shares no code with the HIP library (no headers, helpers,
tables or constants), and imports nothing from it.

Sources (web pages; cited by title and section):
  * "DP, ZeRO-1/2/3, FSDP: how much memory per GPU, how much more
    communication?" (charliedreemur ml-interview notes "dp-zero-fsdp", in
    Chinese; section names translated): concepts, figures 1-2, derivation,
    worked example "7B, N = 8", follow-ups.
  * "Data Parallel, ZeRO and FSDP" (k8ai): plain DDP, communication cost, bus
    bandwidth, ZeRO/FSDP table, 70B full-shard example.
  * "Behind the scenes of distributed training and why your GPU wiring
    matters" (automationscribe): what each GPU holds; DDP; FSDP; the ZeRO dial.

Modules:
  _c            ctypes access to oracle.c (fp32 / fp64 elementwise arithmetic)
  layout        flattened, padded, sharded unit layout (own implementation)
  strategies    DDP / ZeRO-1/2/3 / FSDP / Megatron-DO steps over N simulated
                ranks, with per-rank held-bytes and collective accounting
  ring          a ring reduce-scatter / all-gather / all-reduce simulation
                that counts the bytes each rank sends
  closed_forms  the pages' memory and communication closed forms
"""
