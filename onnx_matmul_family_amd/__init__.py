"""ONNX MatMul-family operators for AMD Instinct MI355X (gfx950)."""
