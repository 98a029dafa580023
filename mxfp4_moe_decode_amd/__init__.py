"""MI355X-native fused MXFP4 MoE layer (router, top-k, MXFP4 routed experts,
MXFP8 shared expert, combine) behind a small C-ABI library."""
