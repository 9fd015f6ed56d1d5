"""MI355X-native ConvRot quantized linear (W8A8 / W4A4)."""
