"""MI355X-native (gfx950) Mamba-2 SSD chunked forward pass."""
