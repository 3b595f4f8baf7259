"""MI355X-native differentiable Fourier-slice projection (binding placeholder)."""
