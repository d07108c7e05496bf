"""MI355X (gfx950) MoE layer forward: route -> capacity-limited dispatch ->
grouped expert FFN -> combine, as hand-written HIP kernels behind a C ABI.

`top_routing_expert_02_amd.moe` is the Python binding of libmoe.so;
`top_routing_expert_02_amd.synth` generates the seeded synthetic workloads.
Nothing is imported eagerly so that the input generator can be used without
the native library.
"""
