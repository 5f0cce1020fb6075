"""MI355X-native W4A16 group-quantized projection (qmv / qmm) — Python binding."""
