"""CPU oracle for the quantized-halo GNN layer -- test infrastructure, not part of the product.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run anything in this package.  The HIP library never calls into it and shares no code with it;
both sides only consume the seeded inputs of ``quantized_halo_aggregation_amd.synth``.

What it computes, and in what precision (SYLVIE guide, referred to below as "the guide"):

* ``philox``    -- Philox4x32-10 counter-based generator (Salmon et al., SC'11), the random source
                   of stochastic rounding.  Pinned against PyTorch's independent header-only Philox
                   engine and by statistical checks.
* ``quantize``  -- per-vector stochastic integer quantisation, bit packing and dequantisation
                   (guide section 6).  Runs in float32, the precision the messages live in, because
                   its floating-point values decide integer codes that must match bit for bit.
* ``aggregate`` -- normalised GCN neighbour aggregation z_v = sum over N(v) and v of
                   x_u / sqrt(d_v d_u) (guide section 2), its transpose for embedding gradients, the
                   GraphSAGE neighbour mean, and the dequantise-and-add of received halo gradients.
                   Float64 accumulation of float32 inputs.
* ``dense``     -- the dense projection h = ReLU(W a) and its gradients, including the weight
                   gradient of guide section 7.  Float64.
* ``layer``     -- whole layers (forward and backward) for one GPU's share of a partition, chained
                   from the pieces above.
* ``control``   -- the host-side width control: the Graph Extractor's importance and mask levels
                   (guide section 7), the Quant Orchestrator's per-epoch widths (section 9) and the
                   Coordinator's loss-descent-rate rule for the base width and execution mode
                   (section 8).  Exact integer decisions; the Coordinator in float64.

Readings of points the guide leaves open are stated where they are used.
"""
