"""MI355X-native MoE FFN layer: routing and int4 SwiGLU experts in HIP for gfx950."""
