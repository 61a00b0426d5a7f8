"""MI355X-native MoE expert-parallel layer: route, dispatch, grouped SwiGLU FFN, combine."""
