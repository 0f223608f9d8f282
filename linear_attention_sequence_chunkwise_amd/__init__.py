"""MI355X-native Kimi Delta Attention (KDA) forward pass (see kda.py for the binding)."""
