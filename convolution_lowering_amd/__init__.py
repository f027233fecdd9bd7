"""MI355X-native batched 2-D convolution forward pass without im2col (binding lands next)."""
