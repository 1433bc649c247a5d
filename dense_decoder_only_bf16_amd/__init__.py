"""gfx950 (MI355X) forward pass of nanochat's GPT: batched prefill + KV-cache decode.

The product is the C-ABI library libnc.so (include/nc.h) built from csrc/ by
`python -m dense_decoder_only_bf16_amd.build`; `nc` is its ctypes binding and `inputs`
holds the seeded synthetic workloads.  Importing the package loads nothing: the library is
loaded on the first call into `nc`.
"""
