"""learnable_butterfly_rotation_amd: MI355X (gfx950) butterfly rotation + fused RTN quantization."""
