"""Plain fp64 CPU oracle for the HyperQuant hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything in this package; only the
tests, the smoke check and the CPU-baseline leg of the benchmark do.  The
oracle shares no code, constants or helpers with the HIP path.

What it restates (sources are web pages about one method, cited by title):

* [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal Quantization Pipeline
  for Large Language and Diffusion Models", arXiv abstract as shown on
  mlsanity.com (paper 2606.23406), whose enumerated ideas (i)-(iv) are the
  method's stages: per-tile randomized Hadamard transform, nearest point of a
  low-dimensional lattice (E8, D4, A2, Z), lossless bit-stripping plus Rice
  coding of the lattice indices, and KV-cache bias correction.
* [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
  Pipeline for Large Language and Diffusion Models", abstract on
  acceptodds.com (iclr2027-3515): Walsh-Hadamard rotation per tile, E8 as the
  default lattice, a lossless strip of bits fixed by lattice membership, Rice
  coding within about 0.1 bps of the lattice's rate-distortion ideal,
  algebraic (codebook-free) decoding, subtractive dither for the KV cache, one
  itemized rate accounting.
* [issue] GitHub issue "HyperQuant: A Rate-Distortion-Optimal Quantization
  Pipeline ... #9", "Additional context": a packed, Rice-coded lattice-index
  checkpoint format.

Every place where the pages are silent is a stated reading; each function's
docstring names the one it takes.  Module map:

  splitmix  SplitMix64 counter hash; RHT sign vector; KV dither box samples
  hadamard  Sylvester Hadamard matrix; forward/inverse randomized transform
  lattices  nearest-point rules for E8, D4, A2, Z; margins; brute force
  rice      zigzag map, Rice code length, parameter search, packer/unpacker
  codec     scale rule, quantizer input grid, strip/unstrip, encode/decode
"""

from . import splitmix, hadamard, lattices, rice, codec  # noqa: F401
