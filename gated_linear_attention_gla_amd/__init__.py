"""MI355X-native GLA forward + SREM (DiG token mixer) behind a C-ABI HIP library."""
